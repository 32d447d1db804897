"""Balanced decode schedules on the GPU against the oracle, through the C ABI.

"KV-Cache Optimization Techniques", section "PagedAttention": the decode
reads each sequence's pages through its table; the balanced schedule only
changes which workgroup streams which blocks.  The result must be eq. 1 over
each sequence's tokens (within the attention tolerance against the oracle)
and within one bfloat16 rounding of the uniform plan's result, for any number
of bins, with sinks + window, empty sequences and shared pages.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import INT4_LONG, INT8_LONG, LLAMA3_8B_LAYER, make_case, variant
from workloads.generate import f32_to_bf16_bits

from .casetools import assert_close, assert_within_one_rounding, layout_of
from .gpu_harness import GpuCase, dev32, log
from .test_gpu_parity import SMALL, _case, _evicted_case, _oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_465_amd as m
    return m


def _info(s):
    i = s.info
    return f"bins={i.num_bins} items={i.num_items} merge={i.num_merge} slots={i.num_slots}"


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("max_bins", [3, 1024])
def test_scheduled_decode_matches_oracle(kvp, cfg, max_bins):
    case = _case(cfg)
    k, v, km, vm, ref = _oracle(case)
    gc = GpuCase(kvp, case)
    gc.upload(k, v, km, vm)
    out = gc.decode_scheduled(max_bins=max_bins)
    log(f"[sched] {cfg.name} bins<={max_bins} {_info(gc.last_schedule)}")
    m, r = assert_close(out, ref, f"{cfg.name} scheduled bins<={max_bins}")
    log(f"  max_abs={m:.2e} rel_l2={r:.2e}")
    assert_within_one_rounding(out, gc.decode(), f"{cfg.name} scheduled vs uniform")
    # the same schedule again: the same bits
    assert np.array_equal(out, gc.decode_scheduled(max_bins=max_bins))
    gc.close()


@pytest.mark.parametrize("cfg", [variant(INT4_LONG, name="int4_sched", batch=5, ctx_lo=1,
                                         ctx_hi=2500),
                                 variant(INT4_LONG, name="fp8_sched_g2", batch=4, kv_dtype="fp8",
                                         num_q_heads=16, ctx_lo=100, ctx_hi=1500)],
                         ids=lambda c: c.name)
def test_scheduled_decode_lowbit(kvp, cfg):
    case = make_case(cfg)
    from .casetools import oracle_pools
    k, v, km, vm = oracle_pools(case)
    ref = oracle.paged_decode(layout_of(case), case.q, k, v, km, vm, case.block_tables, case.ctx,
                              case.scale)
    gc = GpuCase(kvp, case)
    gc.upload(k, v, km, vm)
    for bins in (5, 1024):
        out = gc.decode_scheduled(max_bins=bins)
        log(f"[sched lowbit] {cfg.name} bins<={bins} {_info(gc.last_schedule)}")
        assert_close(out, ref, f"{cfg.name} bins<={bins}")
    gc.close()


def test_int4_lds_ring_short_streams(kvp):
    """INT4 pools with 32-token pages of 128 channels (g <= 16) stream their
    pages through a three-slot LDS ring per wavefront, with filler copies once
    a stream's pages are all issued: sequences of one to three pages and just
    past them, cut into 1 to 1024 bins (one-page items, bins holding a single
    page, streams shorter than the ring), against the oracle and within one
    bfloat16 rounding of the uniform plan."""
    from .casetools import oracle_pools
    cfg = variant(INT4_LONG, name="int4_ring", batch=12, ctx_lo=0, ctx_hi=0,
                  ctx_fixed=(1, 31, 32, 33, 64, 65, 95, 96, 97, 130, 700, 2049))
    case = make_case(cfg)
    k, v, km, vm = oracle_pools(case)
    ref = oracle.paged_decode(layout_of(case), case.q, k, v, km, vm, case.block_tables, case.ctx,
                              case.scale)
    gc = GpuCase(kvp, case)
    gc.upload(k, v, km, vm)
    uniform = gc.decode()
    for bins in (1, 2, 7, 64, 1024):
        out = gc.decode_scheduled(max_bins=bins)
        log(f"[int4 ring] bins<={bins} {_info(gc.last_schedule)}")
        assert_close(out, ref, f"int4 ring bins<={bins}")
        assert_within_one_rounding(out, uniform, f"int4 ring bins<={bins} vs uniform")
    gc.close()


@pytest.mark.parametrize("name", ["l8b_small", "int8_small", "prefix_small"])
def test_one_device_schedule_serves_many_calls(kvp, name):
    """One device copy of a schedule that cuts pairs across bins serves calls
    in stream order (the layers of a step): four calls with different
    queries on one copy, each against the oracle; the schedule words are
    left as they were."""
    cfg = next(c for c in SMALL if c.name == name)
    case = _case(cfg)
    k, v, km, vm, _ = _oracle(case)
    gc = GpuCase(kvp, case)
    gc.upload(k, v, km, vm)
    sched = kvp.kvp_decode_schedule(gc.pool, case.ctx, cfg.num_q_heads,
                                    int(case.block_tables.shape[1]), 7)
    i = sched.info
    log(f"[sched reuse] {name} {_info(sched)}")
    assert i.num_merge > 0, "the case must cut pairs across bins"
    sdev = dev32(sched.used)
    ws = torch.full((i.workspace_bytes // 4 + 1,), float("nan"), dtype=torch.float32,
                    device="cuda")
    rng = np.random.default_rng(4650)
    lay = layout_of(case)
    for call in range(4):
        qh = case.q if call == 0 else f32_to_bf16_bits(
            rng.standard_normal(case.q.shape).astype(np.float32))
        ref = oracle.paged_decode(lay, qh, k, v, km, vm, case.block_tables, case.ctx, case.scale)
        q = torch.from_numpy(qh.view(np.int16)).cuda()
        out = torch.full_like(q, int(np.uint16(0x7FC0).view(np.int16)))
        kvp.kvp_paged_attention_decode_scheduled(
            gc.pool, q, gc.k_pool, gc.v_pool, gc.k_meta, gc.v_meta, gc.bt, gc.ctx,
            int(case.ctx.max()), float(case.scale), sdev, sched, out, workspace=ws)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy().view(np.uint16), ref, f"{name} call {call}")
        assert np.array_equal(sdev.cpu().numpy(), sched.used), f"call {call}: schedule changed"
    gc.close()


def test_schedule_bins_fill_the_device(kvp):
    """Four bins per compute unit (one wavefront per SIMD); eight for INT8
    and FP8 pools and twelve for INT4 pools on the matrix-core path with
    g <= 16, whose stream kernel runs two (INT4: three) wavefronts per SIMD;
    the vector path (g < 4) and larger groups keep four."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for dtype, hq, want in (("bf16", 32, 4), ("int8", 32, 8), ("fp8", 32, 8), ("int4", 32, 12),
                            ("int4", 16, 4), ("bf16", 8, 4), ("int8", 128, 8), ("int8", 256, 4),
                            ("int4", 512, 4)):
        pool = kvp.kvp_pool_create(kvp.make_desc(64, 32, 8, 128, dtype))
        assert kvp.kvp_decode_schedule_bins(pool, hq) == want * cus, (dtype, hq)
        pool.close()


WINDOW = [c for c in SMALL if c.name in ("tiny", "tiny_g1", "l8b_small", "int8_small",
                                          "prefix_small")]


@pytest.mark.parametrize("cfg", WINDOW, ids=lambda c: c.name)
@pytest.mark.parametrize("sink,window", [(4, 64), (0, 17), (3, 200)])
def test_scheduled_window_decode(kvp, cfg, sink, window):
    """Sinks + window along a schedule built for that selection; the dropped
    pages are freed (-1) and poisoned, so a block outside the streamed list
    that were read would show."""
    case = _case(cfg)
    k, v, km, vm, bt, n_poisoned = _evicted_case(case, sink, window)
    ref = oracle.paged_decode_window(layout_of(case), case.q, k, v, km, vm, bt, case.ctx,
                                     case.scale, sink, window)
    gc = GpuCase(kvp, case, block_tables=bt)
    gc.upload(k, v, km, vm)
    for bins in (4, 1024):
        out = gc.decode_scheduled(max_bins=bins, sink=sink, window=window)
        log(f"[sched window] {cfg.name} s={sink} w={window} bins<={bins} "
            f"{_info(gc.last_schedule)}")
        assert_close(out, ref, f"{cfg.name} s={sink} w={window} bins<={bins}")
    gc.close()


def test_scheduled_empty_and_edge_lengths(kvp):
    """Lengths 0, 1, P-1, P, P+1, 2P, 5P+3 and 0 again over sequences that
    hold 200 tokens each: empty sequences give exactly 0, the rest the
    oracle's attention over their first n tokens, for several bin counts."""
    cfg = variant(LLAMA3_8B_LAYER, name="l8b_edges_sched", batch=8, ctx_fixed=(200,) * 8,
                  ctx_lo=0, ctx_hi=0)
    case = make_case(cfg)
    from .casetools import oracle_pools
    k, v, km, vm = oracle_pools(case)
    P = cfg.page_size
    lens = np.array([0, 1, P - 1, P, P + 1, 2 * P, 5 * P + 3, 0], dtype=np.int32)
    ref = oracle.paged_decode(layout_of(case), case.q, k, v, km, vm, case.block_tables, lens,
                              case.scale)
    gc = GpuCase(kvp, case)
    gc.upload(k, v, km, vm)
    for bins in (1, 2, 7, 1024):
        out = gc.decode_scheduled(max_bins=bins, ctx_host=lens)
        log(f"[sched edges] bins<={bins} {_info(gc.last_schedule)}")
        assert_close(out, ref, f"edges bins<={bins}")
        assert (out[lens == 0] == 0).all()
    gc.close()


def test_scheduled_items_outside_the_call_are_skipped(kvp):
    """An item naming a sequence outside the batch is skipped by the kernel
    (checked before any access): its own output row keeps the poison, every
    other row is the oracle's."""
    cfg = SMALL[6]
    case = _case(cfg)
    k, v, km, vm, ref = _oracle(case)
    gc = GpuCase(kvp, case)
    gc.upload(k, v, km, vm)
    sched = kvp.kvp_decode_schedule(gc.pool, case.ctx, cfg.num_q_heads,
                                    int(case.block_tables.shape[1]), 1024)
    i = sched.info
    items = sched.words[i.items_offset:i.items_offset + 8 * i.num_items].reshape(-1, 8)
    direct = np.nonzero(items[:, 4] == -1)[0]
    victim = int(direct[len(direct) // 2])
    b, h = int(items[victim, 0]), int(items[victim, 1])
    items[victim, 0] = case.B + 5
    log(f"[sched skip] item {victim} (seq {b}, head {h}) -> seq {case.B + 5}")
    out = torch.full_like(gc.q, int(np.uint16(0x7FC0).view(np.int16)))
    ws = torch.empty(max(i.workspace_bytes, 4) // 4 + 1, dtype=torch.float32, device="cuda")
    kvp.kvp_paged_attention_decode_scheduled(
        gc.pool, gc.q, gc.k_pool, gc.v_pool, gc.k_meta, gc.v_meta, gc.bt, gc.ctx,
        int(case.ctx.max()), float(case.scale), dev32(sched.used), sched, out, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    g = cfg.num_q_heads // cfg.num_kv_heads
    mask = np.ones(got.shape[:2], bool)
    mask[b, h * g:(h + 1) * g] = False
    assert (got[b, h * g:(h + 1) * g] == 0x7FC0).all()
    assert_close(got[mask], ref[mask], "rows of the other items")
    gc.close()


def _sampled_scheduled(kvp, cfg, seqs):
    case = make_case(cfg)
    log(f"[full sched] {cfg.name} B={case.B} max_ctx={int(case.ctx.max())} sampled={list(seqs)}")
    gc = GpuCase(kvp, case)
    gc.append_history()
    gc.append_new()
    out = gc.decode_scheduled()
    log(f"  {_info(gc.last_schedule)}")
    lay = layout_of(case)
    from workloads import POISON_BF16, POISON_F16, POISON_I8
    k, v, km, vm = lay.empty_pools(POISON_BF16 if lay.dtype == "bf16" else POISON_I8, POISON_F16)
    sel = np.isin(case.hist_seq, list(seqs))
    oracle.append(lay, k, v, km, vm, case.hist_k[sel], case.hist_v[sel], case.hist_seq[sel],
                  case.hist_pos[sel], case.block_tables)
    nsel = np.isin(case.new_seq, list(seqs))
    oracle.append(lay, k, v, km, vm, case.new_k[nsel], case.new_v[nsel], case.new_seq[nsel],
                  case.new_pos[nsel], case.block_tables)
    ref = oracle.paged_decode(lay, case.q, k, v, km, vm, case.block_tables, case.ctx, case.scale,
                              seqs=seqs)
    seqs = list(seqs)
    m, r = assert_close(out[seqs], ref[seqs], cfg.name + " scheduled")
    log(f"  max_abs={m:.2e} rel_l2={r:.2e}")
    assert_within_one_rounding(out, gc.decode(), cfg.name + " scheduled vs uniform")
    gc.close()


def test_full_llama3_8b_layer_scheduled(kvp):
    _sampled_scheduled(kvp, LLAMA3_8B_LAYER, seqs=(0, 9, 33, 63))


def test_full_int8_long_scheduled(kvp):
    _sampled_scheduled(kvp, INT8_LONG, seqs=(0, 6, 15))
