"""Plant plausible mistakes in the CPU oracle and check that a pin catches each.

The mistakes are planted with monkeypatch in this process only; the oracle's
files are never changed.  A mutant that no pin notices would mean the pins
leave that part of the oracle unchecked.
"""
import numpy as np
import pytest

import oracle
from oracle import accounting as oacc
from oracle import paged_attention as opa
from oracle import quantize as oq
from workloads import INT8_LONG, TINY, make_case, variant

from . import pins

_CASES = {}


def _case(cfg):
    if cfg.name not in _CASES:
        _CASES[cfg.name] = make_case(cfg)
    return _CASES[cfg.name]


def _all_pins():
    small = pins.small_cases()
    int8rows = make_case(variant(INT8_LONG, name="int8_rows", batch=1, ctx_lo=64, ctx_hi=64))
    checks = [
        ("block_table", pins.pin_block_table_worked_example),
        ("special", pins.pin_special_cases),
        ("q_exact", pins.pin_quantize_exact_rational),
        ("q_ties", pins.pin_quantize_ties_and_grid),
        ("q_round_trip", lambda: pins.pin_quantize_round_trip(int8rows.hist_k)),
        ("closed_forms", pins.pin_memory_closed_forms),
        ("prefix", pins.pin_shared_prefix_memory),
        ("waste", lambda: pins.pin_waste_bound(_case(TINY))),
    ]
    for c in small:
        checks.append((f"layout_{c.name}",
                       lambda c=c: pins.pin_append_and_gather_layout(_case(c))))
        checks.append((f"sdpa_{c.name}", lambda c=c: pins.pin_attention_vs_sdpa(_case(c))))
    for sink, window in ((4, 16), (0, 7)):
        checks.append((f"window_{sink}_{window}",
                       lambda s=sink, w=window: pins.pin_window_vs_sdpa(_case(TINY), s, w)))
    checks.append(("window_degenerate", lambda: pins.pin_window_degenerate(_case(TINY))))
    checks.append(("window_memory", pins.pin_window_memory_bound))
    checks.append(("int4_layout", pins.pin_quantized_layout))
    checks.append(("int4_round_trip", pins.pin_int4_round_trip_and_ties))
    checks.append(("fp8_vs_torch", pins.pin_fp8_encode_vs_torch))
    checks.append(("fp8_rows", pins.pin_fp8_rows))
    for c in pins.prefill_cases()[:2]:
        checks.append((f"prefill_{c.name}", lambda c=c: pins.pin_prefill_vs_sdpa(_case(c))))
    return checks


def _failing(checks):
    failed = []
    for name, fn in checks:
        try:
            fn()
        except (AssertionError, ValueError, IndexError) as e:  # noqa: PERF203
            failed.append(name)
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert _failing(_all_pins()) == []


# ---- mutants -----------------------------------------------------------------
def _attend_wrong_group(q, K, V, scale):
    Hq, D = q.shape
    Hkv = K.shape[0]
    out = np.zeros((Hq, D))
    if K.shape[1] == 0:
        return out
    for j in range(Hq):
        h = j % Hkv                      # mistake: interleaved instead of consecutive groups
        s = (K[h] @ q[j]) * scale
        p = np.exp(s - s.max())
        out[j] = (p @ V[h]) / p.sum()
    return out


def _attend_no_scale(q, K, V, scale):
    return _ORIG_ATTEND(q, K, V, 1.0)


def _attend_denominator_off(q, K, V, scale):
    Hq, D = q.shape
    Hkv = K.shape[0]
    g = Hq // Hkv
    out = np.zeros((Hq, D))
    if K.shape[1] == 0:
        return out
    for j in range(Hq):
        s = (K[j // g] @ q[j]) * scale
        p = np.exp(s - s.max())
        out[j] = (p @ V[j // g]) / (p.sum() + 1e-3)   # mistake: perturbed normalizer
    return out


def _gather_drop_last(layout, k, v, km, vm, row, ctx):
    K, V = _ORIG_GATHER(layout, k, v, km, vm, row, ctx)
    return K[:, :-1] if ctx else K, V[:, :-1] if ctx else V


def _gather_v_untransposed(layout, k, v, km, vm, row, ctx):
    # mistake: read V as if stored [page][h][t][d] like K
    K, _ = _ORIG_GATHER(layout, k, v, km, vm, row, ctx)
    V, _ = _ORIG_GATHER(layout, v, v, km, vm, row, ctx)
    return K, V


def _slot_swapped(row, pos, P):
    return int(row[pos % P if pos % P < len(row) else 0]), pos // P


def _quant_floor(x_bits):
    x = oq.bf16_bits_to_f32(x_bits)
    mn, mx = x.min(-1), x.max(-1)
    z16 = ((mx + mn) * np.float32(0.5)).astype(np.float16)
    s16 = ((mx - mn) / np.float32(254.0)).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1), s16)
    q = np.floor((x - z16.astype(np.float32)[..., None]) / s16.astype(np.float32)[..., None] + 0.5)
    return np.clip(q, -128, 127).astype(np.int8), s16.view(np.uint16), z16.view(np.uint16)


def _quant_unrounded_scale(x_bits):
    x = oq.bf16_bits_to_f32(x_bits)
    mn, mx = x.min(-1), x.max(-1)
    z16 = ((mx + mn) * np.float32(0.5)).astype(np.float16)
    s32 = (mx - mn) / np.float32(254.0)
    s32 = np.where(s32 == 0, np.float32(1), s32)
    q = np.rint((x - z16.astype(np.float32)[..., None]) / s32[..., None])   # mistake
    s16 = s32.astype(np.float16)
    return np.clip(q, -128, 127).astype(np.int8), s16.view(np.uint16), z16.view(np.uint16)


def _quant_zero_at_min(x_bits):
    x = oq.bf16_bits_to_f32(x_bits)
    mn, mx = x.min(-1), x.max(-1)
    z16 = mn.astype(np.float16)                                             # mistake
    s16 = ((mx - mn) / np.float32(254.0)).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1), s16)
    q = np.rint((x - z16.astype(np.float32)[..., None]) / s16.astype(np.float32)[..., None])
    return np.clip(q, -128, 127).astype(np.int8), s16.view(np.uint16), z16.view(np.uint16)


def _dequant_swapped(codes, s_bits, z_bits):
    return _ORIG_DEQUANT(codes, z_bits, s_bits)


def _append_v_untransposed(layout, k, v, km, vm, k_rows, v_rows, seq_idx, pos, bt):
    # mistake: write V rows in K's [page][h][t][d] layout
    spare_meta = None if vm is None else np.empty_like(vm)
    _ORIG_APPEND(layout, k, np.empty_like(v), km, spare_meta, k_rows, v_rows, seq_idx, pos, bt)
    _ORIG_APPEND(layout, v, np.empty_like(v), vm, spare_meta, v_rows, v_rows, seq_idx, pos, bt)


def _append_meta_swapped(layout, k, v, km, vm, k_rows, v_rows, seq_idx, pos, bt):
    # mistake: the zero point stored in the scale's slot and the scale in the
    # zero's (paired with _dequant_swapped this stays self-consistent)
    if km is None:
        return _ORIG_APPEND(layout, k, v, km, vm, k_rows, v_rows, seq_idx, pos, bt)
    tk, tv = km.copy(), vm.copy()
    _ORIG_APPEND(layout, k, v, tk, tv, k_rows, v_rows, seq_idx, pos, bt)
    P, H = layout.page_size, layout.num_kv_heads
    seq_idx, pos = np.asarray(seq_idx, np.int64), np.asarray(pos, np.int64)
    pages = np.asarray(bt, np.int64)[seq_idx, pos // P]
    rows = ((pages[:, None] * H + np.arange(H)[None, :]) * P + (pos % P)[:, None]).reshape(-1)
    for dst, src in ((km, tk), (vm, tv)):
        d2, s2 = dst.reshape(-1, 2), src.reshape(-1, 2)
        d2[rows, 0] = s2[rows, 1]
        d2[rows, 1] = s2[rows, 0]


def _kv_bytes_missing_two(layers, kv_heads, head_dim, tokens, elem_bytes):
    return layers * kv_heads * head_dim * tokens * elem_bytes


def _prefix_no_shared_copy(requests, tokens, shared, c):
    return requests * (tokens - shared) * c


def _waste_mod(n, P):
    return n % P


_ORIG_ATTEND = opa.attend
_ORIG_GATHER = opa.gather_sequence
_ORIG_DEQUANT = oq.dequantize
_ORIG_APPEND = opa.append

def _kept_off_by_one(n, sink, window):
    if window <= 0 or sink + window >= n:
        return np.arange(n)
    return np.concatenate([np.arange(sink), np.arange(n - window + 1, n)])


def _kept_no_sinks(n, sink, window):
    if window <= 0 or sink + window >= n:
        return np.arange(n)
    return np.arange(n - window, n)


def _kept_overlap_twice(n, sink, window):
    if window <= 0:
        return np.arange(n)
    return np.concatenate([np.arange(min(sink, n)), np.arange(max(n - window, 0), n)])


def _prefill_causal_off_by_one(layout, q_bits, q_start, k_pool, v_pool, k_meta, v_meta,
                               block_tables, context_lens, scale, seqs=None):
    q = opa._to_f64(q_bits)
    out = np.zeros(q.shape)
    for b in range(len(q_start) - 1):
        r0, r1 = int(q_start[b]), int(q_start[b + 1])
        n = int(context_lens[b])
        K, V = opa.gather_sequence(layout, k_pool, v_pool, k_meta, v_meta, block_tables[b], n)
        for i in range(r1 - r0):
            pos = n - (r1 - r0) + i
            out[r0 + i] = opa.attend(q[r0 + i], K[:, :pos], V[:, :pos], float(np.float32(scale)))
    return out


def _prefill_anchored_at_zero(layout, q_bits, q_start, k_pool, v_pool, k_meta, v_meta,
                              block_tables, context_lens, scale, seqs=None):
    q = opa._to_f64(q_bits)
    out = np.zeros(q.shape)
    for b in range(len(q_start) - 1):
        r0, r1 = int(q_start[b]), int(q_start[b + 1])
        n = int(context_lens[b])
        K, V = opa.gather_sequence(layout, k_pool, v_pool, k_meta, v_meta, block_tables[b], n)
        for i in range(r1 - r0):
            out[r0 + i] = opa.attend(q[r0 + i], K[:, :i + 1], V[:, :i + 1],
                                     float(np.float32(scale)))
    return out


def _int4_fifteen_steps(x_bits):
    x = oq.bf16_bits_to_f32(x_bits)
    mn, mx = x.min(axis=-1), x.max(axis=-1)
    z16 = ((mx + mn) * np.float32(0.5)).astype(np.float16)
    s16 = ((mx - mn) / np.float32(15.0)).astype(np.float16)
    s16 = np.where(s16 == np.float16(0.0), np.float16(1.0), s16)
    q = np.rint((x - z16.astype(np.float32)[..., None]) / s16.astype(np.float32)[..., None])
    return np.clip(q, -8, 7).astype(np.int8), s16.view(np.uint16), z16.view(np.uint16)


def _e4m3_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    lo = np.clip(np.searchsorted(oq._E4M3_POS, a, side="right") - 1, 0, 0x7E).astype(np.uint8)
    return np.where(np.signbit(x), lo | np.uint8(0x80), lo).astype(np.uint8)


def _pack_swapped(codes):
    c = (np.asarray(codes, dtype=np.int64) + 8).astype(np.uint8)
    return (c[..., 1::2] | (c[..., 0::2] << 4)).astype(np.uint8)


def _unpack_swapped(b):
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
    out[..., 1::2] = (b & 0xF).astype(np.int64) - 8
    out[..., 0::2] = (b >> 4).astype(np.int64) - 8
    return out


MUTANTS = {
    "int4_fifteen_steps": [(oq, "quantize_rows_int4", _int4_fifteen_steps),
                           (opa, "quantize_rows_int4", _int4_fifteen_steps)],
    "fp8_truncating_round": [(oq, "e4m3_encode", _e4m3_truncate)],
    "int4_nibbles_swapped": [(opa, "_pack_nibbles", _pack_swapped),
                             (opa, "_unpack_nibbles", _unpack_swapped)],
    "prefill_causal_off_by_one": [(opa, "paged_prefill", _prefill_causal_off_by_one),
                                  (oracle, "paged_prefill", _prefill_causal_off_by_one)],
    "prefill_anchored_at_zero": [(opa, "paged_prefill", _prefill_anchored_at_zero),
                                 (oracle, "paged_prefill", _prefill_anchored_at_zero)],
    "window_off_by_one": [(opa, "kept_positions", _kept_off_by_one),
                          (oracle, "kept_positions", _kept_off_by_one)],
    "window_sinks_dropped": [(opa, "kept_positions", _kept_no_sinks),
                             (oracle, "kept_positions", _kept_no_sinks)],
    "window_overlap_counted_twice": [(opa, "kept_positions", _kept_overlap_twice),
                                     (oracle, "kept_positions", _kept_overlap_twice)],
    "gqa_interleaved_groups": [(opa, "attend", _attend_wrong_group),
                               (oracle, "attend", _attend_wrong_group)],
    "scale_dropped": [(opa, "attend", _attend_no_scale), (oracle, "attend", _attend_no_scale)],
    "softmax_normalizer": [(opa, "attend", _attend_denominator_off),
                           (oracle, "attend", _attend_denominator_off)],
    "last_token_dropped": [(opa, "gather_sequence", _gather_drop_last),
                           (oracle, "gather_sequence", _gather_drop_last)],
    "v_layout_untransposed": [(opa, "gather_sequence", _gather_v_untransposed),
                              (oracle, "gather_sequence", _gather_v_untransposed)],
    "slot_block_row_swapped": [(opa, "slot", _slot_swapped), (oracle, "slot", _slot_swapped)],
    "round_half_up": [(oq, "quantize_rows", _quant_floor), (opa, "quantize_rows", _quant_floor)],
    "unrounded_scale": [(oq, "quantize_rows", _quant_unrounded_scale),
                        (opa, "quantize_rows", _quant_unrounded_scale)],
    "zero_point_at_min": [(oq, "quantize_rows", _quant_zero_at_min),
                          (opa, "quantize_rows", _quant_zero_at_min)],
    "dequant_swapped": [(oq, "dequantize", _dequant_swapped), (opa, "dequantize", _dequant_swapped)],
    "meta_pair_misplaced": [(opa, "append", _append_meta_swapped),
                            (oracle, "append", _append_meta_swapped),
                            (oq, "dequantize", _dequant_swapped),
                            (opa, "dequantize", _dequant_swapped)],
    "append_v_untransposed": [(opa, "append", _append_v_untransposed),
                              (oracle, "append", _append_v_untransposed)],
    "memory_missing_factor_two": [(oacc, "kv_bytes", _kv_bytes_missing_two),
                                  (oracle, "kv_bytes", _kv_bytes_missing_two)],
    "prefix_copy_not_counted": [(oacc, "prefix_cached_bytes", _prefix_no_shared_copy),
                                (oracle, "prefix_cached_bytes", _prefix_no_shared_copy)],
    "waste_mod": [(oacc, "waste", _waste_mod), (oracle, "waste", _waste_mod)],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    _CASES.clear()
    for mod, attr, fn in MUTANTS[name]:
        monkeypatch.setattr(mod, attr, fn)
    # tests/casetools imports oracle lazily through the package, so patched
    # package attributes are what the pins see.
    failed = _failing(_all_pins())
    _CASES.clear()
    assert failed, f"no pin caught mutant {name}"
