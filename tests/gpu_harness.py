"""Runs a workload case through the library on the GPU (test infrastructure)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from workloads import POISON_BF16, POISON_F16, POISON_I8, DecodeCase


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev16(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def dev32(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def _fill16(n, pattern, device):
    return torch.full((n,), int(np.uint16(pattern).view(np.int16)), dtype=torch.int16, device=device)


class GpuCase:
    """Device pools (poisoned), tables, q and output for one DecodeCase."""

    def __init__(self, kvp, case: DecodeCase, device="cuda", block_tables=None):
        self.kvp = kvp
        self.case = case
        c = case.cfg
        self.desc = kvp.make_desc(case.num_pages, c.page_size, c.num_kv_heads, c.head_dim,
                                  c.kv_dtype)
        self.pool = kvp.kvp_pool_create(self.desc)
        kv_bytes, meta_bytes = kvp.kvp_pool_bytes(self.desc)
        self.quant = c.kv_dtype != "bf16"
        # host dtype of code pools as the oracle holds them (INT8 signed, packed
        # INT4 nibbles and FP8 bytes unsigned)
        self.code_np = np.int8 if c.kv_dtype == "int8" else np.uint8
        if self.quant:
            fill = int(np.uint8(POISON_I8).view(np.int8))
            self.k_pool = torch.full((kv_bytes,), fill, dtype=torch.int8, device=device)
            self.v_pool = torch.full((kv_bytes,), fill, dtype=torch.int8, device=device)
            self.k_meta = _fill16(meta_bytes // 2, POISON_F16, device)
            self.v_meta = _fill16(meta_bytes // 2, POISON_F16, device)
        else:
            self.k_pool = _fill16(kv_bytes // 2, POISON_BF16, device)
            self.v_pool = _fill16(kv_bytes // 2, POISON_BF16, device)
            self.k_meta = self.v_meta = None
        bt = case.block_tables if block_tables is None else block_tables
        self.bt_host = bt
        self.bt = dev32(bt, device)
        self.ctx = dev32(case.ctx, device)
        self.q = dev16(case.q, device) if case.q is not None else None
        self.device = device

    def append_history(self):
        c = self.case
        self.kvp.kvp_kv_append(self.pool, self.k_pool, self.v_pool, self.k_meta, self.v_meta,
                               dev16(c.hist_k, self.device), dev16(c.hist_v, self.device),
                               dev32(c.hist_seq, self.device), dev32(c.hist_pos, self.device),
                               self.bt)

    def append_new(self):
        c = self.case
        self.kvp.kvp_kv_append(self.pool, self.k_pool, self.v_pool, self.k_meta, self.v_meta,
                               dev16(c.new_k, self.device), dev16(c.new_v, self.device),
                               dev32(c.new_seq, self.device), dev32(c.new_pos, self.device),
                               self.bt)

    def upload(self, k, v, km, vm):
        """Replace the device pools by host pools (e.g. the oracle's)."""
        if self.quant:
            self.k_pool.copy_(torch.from_numpy(np.ascontiguousarray(k).view(np.int8)))
            self.v_pool.copy_(torch.from_numpy(np.ascontiguousarray(v).view(np.int8)))
            self.k_meta.copy_(torch.from_numpy(np.ascontiguousarray(km).view(np.int16)))
            self.v_meta.copy_(torch.from_numpy(np.ascontiguousarray(vm).view(np.int16)))
        else:
            self.k_pool.copy_(torch.from_numpy(np.ascontiguousarray(k).view(np.int16)))
            self.v_pool.copy_(torch.from_numpy(np.ascontiguousarray(v).view(np.int16)))

    def pools_host(self):
        if self.quant:
            return (self.k_pool.cpu().numpy().view(self.code_np),
                    self.v_pool.cpu().numpy().view(self.code_np),
                    self.k_meta.cpu().numpy().view(np.uint16),
                    self.v_meta.cpu().numpy().view(np.uint16))
        return (self.k_pool.cpu().numpy().view(np.uint16),
                self.v_pool.cpu().numpy().view(np.uint16), None, None)

    def decode(self, num_splits=0, max_context_len=None, q=None, ctx=None) -> np.ndarray:
        c = self.case
        q = self.q if q is None else q
        ctx_t = self.ctx if ctx is None else ctx
        mx = int(c.ctx.max()) if max_context_len is None else int(max_context_len)
        ws_bytes = self.kvp.kvp_decode_workspace_bytes(self.pool, c.B, c.cfg.num_q_heads, mx,
                                                       num_splits)
        ws = None
        if ws_bytes:
            # NaN everywhere: the kernels must overwrite every partial they read
            ws = torch.full((ws_bytes // 4,), float("nan"), dtype=torch.float32,
                            device=self.device)
        out = _fill16(q.numel(), POISON_BF16, self.device).view(q.shape)
        self.kvp.kvp_paged_attention_decode(self.pool, q, self.k_pool, self.v_pool, self.k_meta,
                                            self.v_meta, self.bt, ctx_t, mx, float(c.scale), out,
                                            num_splits_req=num_splits, workspace=ws)
        torch.cuda.synchronize()
        return out.cpu().numpy().view(np.uint16)

    def decode_scheduled(self, max_bins=None, sink=0, window=0, ctx_host=None, q=None,
                         max_context_len=None) -> np.ndarray:
        """The decode (window decode when window > 0) along a balanced
        schedule built from the host lengths (the case's, or ctx_host); by
        default the bins the library picks for the pool."""
        c = self.case
        q = self.q if q is None else q
        ctx = c.ctx if ctx_host is None else ctx_host
        if max_bins is None:
            max_bins = self.kvp.kvp_decode_schedule_bins(self.pool, c.cfg.num_q_heads)
        mx = int(ctx.max()) if max_context_len is None else int(max_context_len)
        sched = self.kvp.kvp_decode_schedule(self.pool, ctx, c.cfg.num_q_heads,
                                             int(self.bt_host.shape[1]), max_bins, sink, window)
        sdev = dev32(sched.used, self.device)
        ws = None
        if sched.info.workspace_bytes:
            ws = torch.full((sched.info.workspace_bytes // 4 + 1,), float("nan"),
                            dtype=torch.float32, device=self.device)
        out = _fill16(q.numel(), POISON_BF16, self.device).view(q.shape)
        self.kvp.kvp_paged_attention_decode_scheduled(
            self.pool, q, self.k_pool, self.v_pool, self.k_meta, self.v_meta, self.bt,
            dev32(ctx, self.device), mx, float(c.scale), sdev, sched, out, workspace=ws)
        torch.cuda.synchronize()
        self.last_schedule = sched
        return out.cpu().numpy().view(np.uint16)

    def close(self):
        self.pool.close()
