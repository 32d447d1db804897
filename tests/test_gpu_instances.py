"""Every compiled decode and multi-query instance on the GPU against the oracle.

The header accepts pages of 16 or 32 tokens, head dims 64 and 128, four KV
formats and query groups up to 64 ("Understanding KV-Cache Optimization in
Modern LLM Serving", section "PagedAttention Solution": fixed-size blocks of
16 or 32 tokens; "KV-Cache Optimization Techniques", section "Multi-Query and
Grouped-Query Caching", eq. 7; section "KV-Cache Quantization", eq. 3).  The
library compiles one kernel instance per (format, P, D) and per query-group
class: the vector-ALU kernel for g = 1, 2, 3 and the matrix-core kernels with
one (g <= 16), two (g <= 32) or four (g <= 64) 16-head tiles, each in a
uniform-plan and a balanced-schedule form.  The matrix below reaches every one
of them: format x P x D x g in {1, 2, 3, 4, 8, 20, 40, 64}, each case a
ragged batch spanning several pages, checked

  - bit for bit on every pool byte kv_append writes or must leave alone,
  - against the oracle (max-abs 1e-2, rel-L2 5e-3) for the uniform plan with
    one and three splits and for the balanced schedule with the library's
    bin count and with three bins (items cut across bins, merged afterwards).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from workloads import TINY, make_case, variant

from .casetools import assert_close, assert_within_one_rounding, layout_of, oracle_pools
from .gpu_harness import GpuCase, dev32, log

pytestmark = pytest.mark.gpu

FORMATS = ("bf16", "int8", "int4", "fp8")
PAGES = (16, 32)
DIMS = (64, 128)
# query heads per KV head -> (H_q, H_kv): every vector-ALU group and every
# head-tile count, with two KV heads where the query heads stay few
GROUPS = {1: (2, 2), 2: (4, 2), 3: (6, 2), 4: (8, 2), 8: (16, 2), 20: (40, 2), 40: (40, 1),
          64: (64, 1)}


def _kernel_of(g):
    if g < 4:
        return f"valu_g{g}"
    return f"mfma_nt{1 if g <= 16 else 2 if g <= 32 else 4}"


def _cfg(fmt, P, D, g, seed, suffix="", **kw):
    hq, hkv = GROUPS[g]
    # several pages, a one-token sequence, an exact page multiple and a long
    # ragged one: every ring slot, the masked tail and the split boundaries
    ctx = (7 * P + 3, 1, 2 * P, 13 * P - 1)
    quant = fmt != "bf16"
    return variant(TINY, name=f"{fmt}_p{P}_d{D}_g{g}{suffix}", batch=len(ctx), ctx_fixed=ctx,
                   num_q_heads=hq, num_kv_heads=hkv, head_dim=D, page_size=P, kv_dtype=fmt,
                   pool_pages=None, outlier_channels=3 if quant else 0,
                   outlier_gain=8.0 if quant else 1.0, seed=seed, **kw)


MATRIX = [_cfg(f, P, D, g, 466000 + i) for i, (f, P, D, g) in
          enumerate(itertools.product(FORMATS, PAGES, DIMS, sorted(GROUPS)))]


@pytest.fixture(scope="module")
def kvp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_465_amd as m
    return m


def _pools_equal(got, ref, what):
    for name, g, r in zip(("K", "V", "K meta", "V meta"), got, ref):
        if r is None:
            assert g is None
            continue
        gb = g.reshape(-1).view(np.uint8)
        rb = r.reshape(-1).view(np.uint8)
        bad = np.nonzero(gb != rb)[0]
        assert bad.size == 0, f"{what}: {name} pool differs at {bad.size} bytes, first {bad[:5]}"


def _run_matrix_case(kvp, cfg):
    case = make_case(cfg)
    g = cfg.num_q_heads // cfg.num_kv_heads
    log(f"[instance] {cfg.name} kernel={_kernel_of(g)} seed={cfg.seed} ctx={case.ctx.tolist()} "
        f"pages={case.num_pages}")
    k, v, km, vm = oracle_pools(case)
    ref = oracle.paged_decode(layout_of(case), case.q, k, v, km, vm, case.block_tables, case.ctx,
                              case.scale)
    gc = GpuCase(kvp, case)
    gc.append_history()
    gc.append_new()
    torch.cuda.synchronize()
    _pools_equal(gc.pools_host(), (k, v, km, vm), cfg.name)
    one = gc.decode(num_splits=1)
    assert_close(one, ref, f"{cfg.name} S=1")
    three = gc.decode(num_splits=3)
    assert_close(three, ref, f"{cfg.name} S=3")
    assert_within_one_rounding(one, three, f"{cfg.name} S=3 vs S=1")
    for bins in (None, 3):
        out = gc.decode_scheduled(max_bins=bins)
        i = gc.last_schedule.info
        m, r = assert_close(out, ref, f"{cfg.name} scheduled bins<={bins}")
        log(f"  sched bins={i.num_bins} items={i.num_items} merge={i.num_merge}: "
            f"max_abs={m:.2e} rel_l2={r:.2e}")
    gc.close()


@pytest.mark.parametrize("cfg", MATRIX, ids=lambda c: c.name)
def test_every_decode_instance(kvp, cfg):
    _run_matrix_case(kvp, cfg)


# Queries four times larger: sharper softmax (the running maximum moves, the
# accumulators rescale) on the quantized formats, whose kernels take q as
# float16 matrix-core operands.
QGAIN = [_cfg(f, P, 128, g, 467000 + i, suffix="_qgain4", q_gain=4.0)
         for i, (f, P, g) in enumerate(itertools.product(("int8", "int4", "fp8"), (16, 32),
                                                          (2, 8, 40)))]


@pytest.mark.parametrize("cfg", QGAIN, ids=lambda c: c.name)
def test_quantized_instances_with_sharp_queries(kvp, cfg):
    _run_matrix_case(kvp, cfg)


# ---- multi-query attention (chunked prefill, verification) -----------------------
# "KV-Cache Optimization Techniques", section "Cache-Aware Scheduling": chunks of
# q_len new tokens attend causally over the cache.  With g = 4 query heads per
# KV head, chunks of 3, 6, 20 and 40 tokens give 12, 24, 80 and 160 rows per
# (sequence, KV head): the page-split kernel with one and two head tiles (rows
# fit one wavefront) and the row-tiled kernel with one and two tiles per
# wavefront, for every format, page size and head dim.
PREFILL_MODES = {3: "split_nt1", 6: "split_nt2", 20: "tiled_nt1", 40: "tiled_nt2"}


def _prefill_cfg(fmt, P, D, q_len, seed):
    ctx = (9 * P + 5, 50, 2 * P + 40, 13 * P - 1)
    quant = fmt != "bf16"
    return variant(TINY, name=f"{fmt}_p{P}_d{D}_{PREFILL_MODES[q_len]}", batch=len(ctx),
                   ctx_fixed=ctx, num_q_heads=8, num_kv_heads=2, head_dim=D, page_size=P,
                   kv_dtype=fmt, pool_pages=None, outlier_channels=3 if quant else 0,
                   outlier_gain=8.0 if quant else 1.0, q_len=q_len, seed=seed)


PREFILL_MATRIX = [_prefill_cfg(f, P, D, L, 469000 + i) for i, (f, P, D, L) in
                  enumerate(itertools.product(FORMATS, PAGES, DIMS, sorted(PREFILL_MODES)))]


@pytest.mark.parametrize("cfg", PREFILL_MATRIX, ids=lambda c: c.name)
def test_every_prefill_instance(kvp, cfg):
    case = make_case(cfg)
    log(f"[prefill instance] {cfg.name} seed={cfg.seed} ctx={case.ctx.tolist()} "
        f"q_len={cfg.q_len}")
    k, v, km, vm = oracle_pools(case)
    ref = oracle.paged_prefill(layout_of(case), case.q, case.q_start, k, v, km, vm,
                               case.block_tables, case.ctx, case.scale)
    gc = GpuCase(kvp, case)
    gc.append_history()
    gc.append_new()
    torch.cuda.synchronize()
    _pools_equal(gc.pools_host(), (k, v, km, vm), cfg.name)
    out = torch.full_like(gc.q, int(np.uint16(0x7FC0).view(np.int16)))
    kvp.kvp_paged_attention_prefill(gc.pool, gc.q, dev32(case.q_start), gc.k_pool, gc.v_pool,
                                    gc.k_meta, gc.v_meta, gc.bt, gc.ctx, cfg.q_len,
                                    int(case.ctx.max()), float(case.scale), out)
    torch.cuda.synchronize()
    m, r = assert_close(out.cpu().numpy().view(np.uint16), ref, cfg.name)
    log(f"  max_abs={m:.2e} rel_l2={r:.2e}")
    gc.close()
