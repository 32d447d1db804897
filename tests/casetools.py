"""Test-side helpers: assemble a case's logical rows, build oracle pools,
compare outputs to the tolerance the workloads are held to."""
from __future__ import annotations

import numpy as np

import oracle
from workloads import POISON_BF16, POISON_F16, POISON_I8, DecodeCase

# Attention outputs (bfloat16, float32 accumulation) against the float64 oracle.
MAX_ABS_TOL = 1e-2
REL_L2_TOL = 5e-3


def layout_of(case: DecodeCase) -> oracle.PoolLayout:
    c = case.cfg
    return oracle.PoolLayout(case.num_pages, c.page_size, c.num_kv_heads, c.head_dim, c.kv_dtype)


def logical_rows(case: DecodeCase, b: int):
    """K and V rows of sequence b in position order: uint16 [ctx, H_kv, D]."""
    c = case.cfg
    n = int(case.ctx[b])
    K = np.zeros((n, c.num_kv_heads, c.head_dim), dtype=np.uint16)
    V = np.zeros_like(K)
    filled = np.zeros(n, dtype=bool)
    src = [b] if not c.shared_prefix or b == 0 else [0, b]
    for s in src:
        sel = np.nonzero(case.hist_seq == s)[0]
        p = case.hist_pos[sel]
        keep = p < n - 1 if s == b else p < c.shared_prefix
        K[p[keep]] = case.hist_k[sel[keep]]
        V[p[keep]] = case.hist_v[sel[keep]]
        filled[p[keep]] = True
    mine = np.nonzero(case.new_seq == b)[0]
    K[case.new_pos[mine]] = case.new_k[mine]
    V[case.new_pos[mine]] = case.new_v[mine]
    filled[case.new_pos[mine]] = True
    assert filled.all()
    return K, V


def oracle_pools(case: DecodeCase, with_new: bool = True):
    """Poisoned pools with every history row (and the new rows) appended by the oracle."""
    lay = layout_of(case)
    fill = POISON_BF16 if lay.dtype == "bf16" else POISON_I8
    k, v, km, vm = lay.empty_pools(fill, POISON_F16)
    oracle.append(lay, k, v, km, vm, case.hist_k, case.hist_v, case.hist_seq, case.hist_pos,
                  case.block_tables)
    if with_new:
        oracle.append(lay, k, v, km, vm, case.new_k, case.new_v,
                      case.new_seq, case.new_pos, case.block_tables)
    return k, v, km, vm


def compare_outputs(out_bf16_bits: np.ndarray, ref_f64: np.ndarray):
    """(max_abs, rel_l2, worst index, max_ulps_big) of bfloat16 outputs against float64.

    bfloat16 keeps 8 significant bits, so an output of magnitude >= 4 is stored
    with a rounding step of at least 1/32: no bfloat16 result can be within
    1e-2 of it in general.  max_abs is therefore taken over outputs with
    |ref| < 4, and outputs with |ref| >= 4 are measured in bfloat16 ulps of
    their magnitude (max_ulps_big).  rel_l2 covers every output."""
    got = (np.asarray(out_bf16_bits, dtype=np.uint16).astype(np.uint32) << 16) \
        .view(np.float32).astype(np.float64)
    if not np.isfinite(got).all():
        return float("inf"), float("inf"), None, float("inf")
    d = np.abs(got - ref_f64)
    big = np.abs(ref_f64) >= 4.0
    small_d = np.where(big, 0.0, d)
    max_abs = float(small_d.max()) if d.size else 0.0
    den = float(np.linalg.norm(ref_f64))
    rel = float(np.linalg.norm(got - ref_f64) / den) if den > 0 else float(np.linalg.norm(d))
    worst = np.unravel_index(int(small_d.argmax()), d.shape) if d.size else None
    max_ulps = 0.0
    if big.any():
        ulp = np.exp2(np.floor(np.log2(np.abs(ref_f64[big]))) - 7)
        max_ulps = float((d[big] / ulp).max())
    return max_abs, rel, worst, max_ulps


def assert_close(out_bf16_bits, ref_f64, what=""):
    max_abs, rel, worst, ulps = compare_outputs(out_bf16_bits, ref_f64)
    assert max_abs <= MAX_ABS_TOL and rel <= REL_L2_TOL and ulps <= 1.0, \
        f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} worst={worst} big_ulps={ulps:.2f}"
    return max_abs, rel


def assert_within_one_rounding(a_bits, b_bits, what=""):
    """Two bfloat16 results of the same attention computed with different
    summation orders (split counts, kernels): every element pair differs by at
    most 1e-2 or by one bfloat16 rounding step at its magnitude, whichever is
    larger (two float32 values a hair apart can round to neighbouring
    bfloat16 values, which are 1/64 apart in [2, 4))."""
    a = (np.asarray(a_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    b = (np.asarray(b_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    a, b = a.astype(np.float64), b.astype(np.float64)
    assert np.isfinite(a).all() and np.isfinite(b).all(), what
    mag = np.maximum(np.abs(a), np.abs(b))
    step = np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7)
    bound = np.maximum(MAX_ABS_TOL, step)
    bad = np.abs(a - b) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements differ by more than one rounding"
