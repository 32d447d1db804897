"""Checks that pin the CPU oracle to the pages and to mathematics.

Each ``pin_*`` raises AssertionError when the oracle disagrees with something
fixed outside it: values the pages print, a library routine that computes the
same definition, exact-rational arithmetic, closed forms and invariants.
test_oracle_pins runs them on the oracle; test_oracle_mutations plants
plausible mistakes in the oracle and checks that some pin catches each one.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle import paged_attention as opa
from oracle import quantize as oq
from workloads import TINY, f32_to_bf16_bits, make_case, variant

from .casetools import layout_of, logical_rows, oracle_pools
from .exact_ieee import fp8_scale_exact, quantize_row_exact

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32) \
        .astype(np.float64)


def prefill_cases():
    """Small chunked cases: fixed and ragged chunk lengths, g = 1, 2, 4, 8, INT8."""
    return [
        variant(TINY, name="tiny_chunk5", q_len=5),
        variant(TINY, name="tiny_chunk_ragged", q_len=1, q_len_hi=9, batch=3, ctx_fixed=(37, 100, 8),
                pool_pages=24),
        variant(TINY, name="tiny_chunk_g1", q_len=4, num_q_heads=2, num_kv_heads=2, pool_pages=32),
        variant(TINY, name="tiny_chunk_g8_p32_int8", q_len=6, page_size=32, kv_dtype="int8",
                num_q_heads=16, num_kv_heads=2, head_dim=128, pool_pages=16, outlier_channels=3,
                outlier_gain=8.0),
    ]


# Small cases: the tiny workload and its MHA (g=1), g=2, H_kv=2 and peaky variants.
def small_cases():
    return [
        TINY,
        variant(TINY, name="tiny_g1", num_q_heads=2, num_kv_heads=2, pool_pages=32),
        variant(TINY, name="tiny_g2", num_q_heads=4, num_kv_heads=2, pool_pages=32),
        variant(TINY, name="tiny_h2g4", num_q_heads=8, num_kv_heads=2, pool_pages=32,
                head_dim=128),
        variant(TINY, name="tiny_peaky", q_gain=4.0),
        variant(TINY, name="tiny_p32_int8", page_size=32, kv_dtype="int8", num_q_heads=8,
                num_kv_heads=2, head_dim=128, pool_pages=16, outlier_channels=3,
                outlier_gain=8.0),
        variant(TINY, name="tiny_p16_int4_h2", kv_dtype="int4", num_q_heads=8,
                num_kv_heads=2, pool_pages=24, outlier_channels=3, outlier_gain=8.0),
        variant(TINY, name="tiny_p32_fp8_h2", page_size=32, kv_dtype="fp8", num_q_heads=4,
                num_kv_heads=2, head_dim=128, pool_pages=16),
    ]


# ---------------------------------------------------------------- layout / gather
_EXACT_MEMO = {}


def _memo_exact(fn):
    """Cache an exact-row-model function by its input bits: the model does not
    depend on the oracle, so its answers hold across planted oracle mistakes."""
    def wrapped(rows_bits, dtype="int8"):
        a = np.ascontiguousarray(rows_bits)
        key = (fn.__name__, dtype, a.shape, a.tobytes())
        if key not in _EXACT_MEMO:
            _EXACT_MEMO[key] = fn(a, dtype)
        return _EXACT_MEMO[key]
    return wrapped


@_memo_exact
def _row_codes_exact(row_bits, dtype):
    """One (token, head) row of D bfloat16 values -> (codes, scale bits, zero
    bits) by the exact-rational model of the row contract (INT8 / INT4), or
    the exact scale and torch's e4m3 cast (FP8): independent of the oracle's
    quantizer."""
    x = _bf16_f64(np.asarray(row_bits).reshape(-1))
    if dtype == "fp8":
        sc = fp8_scale_exact(x.tolist())
        q = (x.astype(np.float32) / np.float32(float(sc))).astype(np.float32)
        codes = torch.from_numpy(np.clip(q, -448, 448)).to(torch.float8_e4m3fn) \
            .view(torch.uint8).numpy().astype(np.int64)
        return codes, int(np.float16(float(sc)).view(np.uint16)), 0
    if dtype == "int4":
        codes, sc, z = quantize_row_exact(x.tolist(), steps=14, lo=-8, hi=7)
    else:
        codes, sc, z = quantize_row_exact(x.tolist())
    return (np.asarray(codes, dtype=np.int64), int(np.float16(float(sc)).view(np.uint16)),
            int(np.float16(float(z)).view(np.uint16)))


def loop_scatter(case):
    """Pools written one element at a time from the header's index formulas:
    bfloat16 rows, or for the quantized formats each row's codes and its
    (scale, zero) float16 pair from the exact row model."""
    from workloads import POISON_F16, POISON_I8
    lay = layout_of(case)
    c = case.cfg
    P, H, D = c.page_size, c.num_kv_heads, c.head_dim
    dt = c.kv_dtype
    km = vm = None
    if dt == "bf16":
        k = np.full(lay.elems, 0x7FC0, dtype=np.uint16)
        v = np.full(lay.elems, 0x7FC0, dtype=np.uint16)
    else:
        nbytes = lay.elems // 2 if dt == "int4" else lay.elems
        k = np.full(nbytes, POISON_I8, dtype=np.uint8)
        v = np.full(nbytes, POISON_I8, dtype=np.uint8)
        km = np.full(lay.meta_elems, POISON_F16, dtype=np.uint16)
        vm = np.full(lay.meta_elems, POISON_F16, dtype=np.uint16)
    for b in range(case.B):
        K, V = logical_rows(case, b)
        for pos in range(int(case.ctx[b])):
            page = int(case.block_tables[b][pos // P])
            t = pos % P
            for h in range(H):
                if dt == "bf16":
                    for d in range(D):
                        k[((page * H + h) * P + t) * D + d] = K[pos, h, d]
                        v[((page * H + h) * D + d) * P + t] = V[pos, h, d]
                    continue
                for rows, pool, meta, is_v in ((K, k, km, False), (V, v, vm, True)):
                    codes, s_bits, z_bits = _row_codes_exact(rows[pos, h], dt)
                    for d in range(D):
                        if dt == "int4":
                            idx = (((page * H + h) * (D // 2) + d // 2) * P + t if is_v
                                   else ((page * H + h) * P + t) * (D // 2) + d // 2)
                            sh = 4 * (d % 2)
                            pool[idx] = (int(pool[idx]) & ~(0xF << sh) & 0xFF) | \
                                (((int(codes[d]) + 8) & 0xF) << sh)
                        else:
                            idx = (((page * H + h) * D + d) * P + t if is_v
                                   else ((page * H + h) * P + t) * D + d)
                            pool[idx] = int(codes[d]) & 0xFF
                    meta[((page * H + h) * P + t) * 2 + 0] = s_bits
                    meta[((page * H + h) * P + t) * 2 + 1] = z_bits
    return k, v, km, vm


def pin_block_table_worked_example():
    g = _golden("block_table_p2.json")
    row = np.array(g["block_table"], dtype=np.int32)
    for c in g["cases"]:
        assert oracle.slot(row, c["pos"], c["page_size"]) == (c["page"], c["row"]), c


def pin_append_and_gather_layout(case):
    """oracle.append writes, byte for byte, what the element loop writes (codes,
    scales and zero points included); gather returns the rows (for the
    quantized formats, the exact row model's dequantized values)."""
    loop = loop_scatter(case)
    pools = oracle_pools(case)
    for name, got, want in zip(("K", "V", "K meta", "V meta"), pools, loop):
        if want is None:
            assert got is None, name
            continue
        assert np.array_equal(np.asarray(got).view(np.uint8), want.view(np.uint8)), \
            f"{name} pool differs from the header layout"
    k, v, km, vm = pools
    lay = layout_of(case)
    dt = case.cfg.kv_dtype
    for b in range(case.B):
        K, V = logical_rows(case, b)
        Kg, Vg = oracle.gather_sequence(lay, k, v, km, vm, case.block_tables[b],
                                        int(case.ctx[b]))
        if dt == "bf16":
            Kw, Vw = _bf16_f64(K), _bf16_f64(V)
        else:
            Kw = np.stack([_dequant_exact(K[t], dt) for t in range(K.shape[0])])
            Vw = np.stack([_dequant_exact(V[t], dt) for t in range(V.shape[0])])
        assert np.array_equal(Kg, Kw.transpose(1, 0, 2)), f"K gather seq {b}"
        assert np.array_equal(Vg, Vw.transpose(1, 0, 2)), f"V gather seq {b}"


# ---------------------------------------------------------------- attention
def _sdpa(q, K, V, scale):
    """torch's scaled_dot_product_attention in float64 on the CPU (GQA: query
    head j reads KV head j // g)."""
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale,
                                                         enable_gqa=True)
    return o[0, :, 0, :].numpy()


def pin_attention_vs_sdpa(case, tol=1e-12):
    k, v, km, vm = oracle_pools(case)
    lay = layout_of(case)
    out = oracle.paged_decode(lay, case.q, k, v, km, vm, case.block_tables, case.ctx,
                              case.scale)
    for b in range(case.B):
        K, V = logical_rows(case, b)
        dt = case.cfg.kv_dtype
        if dt != "bf16":
            # the library routine sees the dequantized rows of the row contract
            Kf = np.stack([_dequant_exact(K[t], dt) for t in range(K.shape[0])])
            Vf = np.stack([_dequant_exact(V[t], dt) for t in range(V.shape[0])])
        else:
            Kf, Vf = _bf16_f64(K), _bf16_f64(V)
        ref = _sdpa(_bf16_f64(case.q[b]), Kf, Vf, float(np.float32(case.scale)))
        err = np.abs(out[b] - ref).max()
        assert err <= tol, f"seq {b}: oracle vs sdpa {err:.3e}"


@_memo_exact
def _dequant_exact(rows_bits, dtype="int8"):
    """[H, D] bfloat16 rows -> float64 values after the exact row contract of
    ``dtype`` (exact-rational IEEE steps for INT8/INT4; for FP8 the
    exact-rational scale and torch's float8_e4m3fn conversion of x / s)."""
    xs = _bf16_f64(rows_bits)
    res = np.zeros_like(xs)
    for h in range(xs.shape[0]):
        if dtype == "fp8":
            s = fp8_scale_exact(xs[h].tolist())
            q = (xs[h].astype(np.float32) / np.float32(float(s))).astype(np.float32)
            e4 = torch.from_numpy(np.clip(q, -448, 448)).to(torch.float8_e4m3fn)
            res[h] = float(s) * e4.to(torch.float64).numpy()
            continue
        if dtype == "int4":
            codes, s, z = quantize_row_exact(xs[h].tolist(), steps=14, lo=-8, hi=7)
        else:
            codes, s, z = quantize_row_exact(xs[h].tolist())
        res[h] = [float(s * c + z) for c in codes]
    return res


def pin_special_cases():
    rng = np.random.default_rng(7)
    D, n = 64, 21
    V = rng.standard_normal((1, n, D))
    K = rng.standard_normal((1, n, D))
    q = rng.standard_normal((2, D))
    # one token: the output is that token's V row, exactly
    o = oracle.attend(q, K[:, :1], V[:, :1], 0.125)
    assert np.array_equal(o, np.repeat(V[:, 0], 2, axis=0))
    # zero query or identical keys: uniform weights, the mean of V
    o = oracle.attend(np.zeros((2, D)), K, V, 0.125)
    assert np.allclose(o, V[0].mean(axis=0), rtol=0, atol=1e-14)
    Keq = np.repeat(K[:, :1], n, axis=1)
    o = oracle.attend(q, Keq, V, 0.125)
    assert np.allclose(o, V[0].mean(axis=0), rtol=0, atol=1e-14)
    # empty context: zero
    o = oracle.attend(q, K[:, :0], V[:, :0], 0.125)
    assert np.array_equal(o, np.zeros((2, D)))


def pin_page_relabel_invariance(case, seed=11):
    """Relabelling physical pages leaves every output bit unchanged."""
    lay = layout_of(case)
    k, v, km, vm = oracle_pools(case)
    out = oracle.paged_decode(lay, case.q, k, v, km, vm, case.block_tables, case.ctx,
                              case.scale)
    perm = np.random.default_rng(seed).permutation(case.num_pages)
    c = case.cfg
    per_page = c.num_kv_heads * c.page_size * c.head_dim

    def relabel(a, n):
        if a is None:
            return None
        src = a.reshape(case.num_pages, -1)   # one page's bytes per row, any format
        dst = np.empty_like(src)
        dst[perm] = src
        return dst.reshape(-1)

    bt = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1)
    meta_n = c.num_kv_heads * c.page_size * 2
    out2 = oracle.paged_decode(lay, case.q, relabel(k, per_page), relabel(v, per_page),
                               relabel(km, meta_n), relabel(vm, meta_n), bt, case.ctx,
                               case.scale)
    assert np.array_equal(out, out2)


# ---------------------------------------------------------------- quantization
def _quant_rows_for_pins():
    rng = np.random.default_rng(3)
    rows = [rng.standard_normal(64).astype(np.float32) for _ in range(40)]
    x = rng.standard_normal(64).astype(np.float32)
    x[[3, 17]] *= 8
    rows.append(x)
    rows.append(np.full(64, 0.375, np.float32))               # constant row
    rows.append(np.linspace(-1e-6, 1e-6, 64).astype(np.float32))  # tiny range
    rows.append((rng.standard_normal(64) * 300).astype(np.float32))  # wide range
    rows.append((rng.standard_normal(64) + 40).astype(np.float32))   # offset row
    return [f32_to_bf16_bits(r) for r in rows]


def pin_quantize_exact_rational():
    """The float32/float16 pipeline equals the exact-rational IEEE model, bit for bit."""
    for bits in _quant_rows_for_pins():
        codes, s16, z16 = oq.quantize_rows(bits[None, :])
        xs = [Fraction(float(v)) for v in _bf16_f64(bits)]
        ecodes, es, ez = quantize_row_exact(xs)
        assert codes[0].tolist() == ecodes
        assert Fraction(float(s16.view(np.float16)[0])) == es
        assert Fraction(float(z16.view(np.float16)[0])) == ez


def pin_quantize_ties_and_grid():
    # mn = -127, mx = 127: z = 0, s = 1, codes = x rounded half to even
    x = np.zeros(16, np.float32)
    x[:8] = [-127, 127, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5]
    codes, s16, z16 = oq.quantize_rows(f32_to_bf16_bits(x)[None])
    assert s16.view(np.float16)[0] == 1.0 and z16.view(np.float16)[0] == 0.0
    assert codes[0, :8].tolist() == [-127, 127, 2, 4, -2, 0, 0, 2]
    # a row already on the grid of its own scale comes back exactly
    grid = np.arange(-127, 128, 17, dtype=np.float32)
    grid = np.concatenate([grid, [-127.0, 127.0]]).astype(np.float32)
    codes, s16, z16 = oq.quantize_rows(f32_to_bf16_bits(grid)[None])
    back = oq.dequantize(codes, s16, z16)[0]
    assert np.array_equal(back, grid.astype(np.float64))
    # a constant row: codes 0, value recovered exactly
    c = np.full(32, -0.71875, np.float32)
    codes, s16, z16 = oq.quantize_rows(f32_to_bf16_bits(c)[None])
    assert (codes == 0).all()
    assert np.array_equal(oq.dequantize(codes, s16, z16)[0], c.astype(np.float64))


def pin_quantize_round_trip(rows_bits):
    """|x - (s*code + z)| <= s * (1/2 + 2^-15) on normal-like rows (so no code clamps)."""
    codes, s16, z16 = oq.quantize_rows(rows_bits)
    x = _bf16_f64(rows_bits)
    back = oq.dequantize(codes, s16, z16)
    s = s16.view(np.float16).astype(np.float64)[..., None]
    assert (np.abs(x - back) <= s * (0.5 + 2.0 ** -15)).all()


# ---------------------------------------------------------------- closed forms
def pin_memory_closed_forms():
    g = _golden("memory_closed_forms.json")
    e = g["llama3_70b"]
    one = oracle.kv_bytes(e["layers"], e["kv_heads"], e["head_dim"], e["tokens"],
                          e["elem_bytes"])
    assert one == e["bytes_printed"]
    assert one * e["batch"] == 85_899_345_920
    # the printed 85.7 GB is 2.68 GB (rounded first) x 32 = 85.76, cut to one decimal
    assert int(round(one / 1e9, 2) * e["batch"] * 10) / 10 == e["batch_gb_printed"]
    q = g["gqa_llama2_70b"]
    assert 1 / oracle.gqa_ratio(q["kv_groups"], q["q_heads"]) == q["reduction_printed"]
    assert q["reduction_printed"] * q["int4_reduction_printed"] == q["int4_times_gqa_printed"]
    x3 = g["exercise3"]
    L, H, D, T = x3["layers"], x3["heads"], x3["head_dim"], x3["tokens"]
    assert oracle.kv_bytes(L, H, D, T, 2) == x3["fp16_bytes"]
    assert oracle.kv_bytes(L, H, D, T, 1) == x3["int8_bytes"]
    assert oracle.kv_bytes(L, 4, D, T, 0.5) == x3["int4_gqa4_bytes"]
    assert oracle.kv_bytes(L, H, D, T, 2) / oracle.kv_bytes(L, H, D, T, 1) == \
        q["int8_reduction_printed"]
    p = g["prefix_l81"]
    c = 1.0
    saved = oracle.paged_bytes(p["requests"], 2500, c) - \
        oracle.prefix_cached_bytes(p["requests"], 2500, p["shared"], c)
    assert saved == (p["requests"] - 1) * p["shared"] * c
    assert saved + p["shared"] * c == p["savings_printed_in_units_of_c"]
    x2 = g["exercise2"]
    for own in (0, 1, 500, 4096):   # any per-request suffix length: the saving is the same
        n = x2["shared"] + own
        saved = oracle.paged_bytes(x2["requests"], n, 1) - \
            oracle.prefix_cached_bytes(x2["requests"], n, x2["shared"], 1)
        assert saved == x2["savings_in_units_of_c"], own
    c70 = oracle.bytes_per_token(80, 8, 128, 2)
    assert c70 == x2["llama3_70b_c_bytes"]
    assert x2["savings_in_units_of_c"] * c70 == x2["llama3_70b_savings_bytes"]
    x1 = g["exercise1"]
    worst = max(oracle.waste(n, x1["page_size"]) for n in range(1, 4 * x1["page_size"] + 1))
    assert worst == x1["max_waste_tokens"]
    assert x1["static_max_tokens"] - 1 == x1["static_max_waste_tokens"]


def pin_waste_bound(case):
    """Paging wastes at most P-1 slots per sequence ("PagedAttention" section)."""
    P = case.cfg.page_size
    for n in case.ctx:
        n = int(n)
        a = oracle.alloc_tokens(n, P)
        assert a % P == 0 and a >= n and a - P < n
        w = oracle.waste(n, P)
        assert 0 <= w <= P - 1 and (n + w) % P == 0


def pin_shared_prefix_memory():
    """Unique bytes of the shared-prefix workload equal eq. 2's prefix-cached value."""
    from workloads import SHARED_PREFIX_MQA as cfg
    case = make_case(cfg, with_data=False)
    c = oracle.bytes_per_token(1, cfg.num_kv_heads, cfg.head_dim, 2)
    assert c == 512
    pages = np.unique(case.block_tables[case.block_tables >= 0])
    assert pages.size == 125 + 100 * 32 == 3325
    unique_tokens = cfg.shared_prefix + int((case.ctx - cfg.shared_prefix).sum())
    assert unique_tokens * c == oracle.prefix_cached_bytes(cfg.batch, 2500, cfg.shared_prefix, c) \
        == 26_624_000
    saved = oracle.paged_bytes(cfg.batch, 2500, c) - unique_tokens * c
    assert saved == 101_376_000
    slots = pages.size * cfg.page_size
    assert slots - unique_tokens == 1200
    # only each sequence's own last page has empty slots
    assert sum(oracle.waste(int(n), cfg.page_size) for n in case.ctx) == 1200


# ---------------------------------------------------------------- sinks + window
def pin_window_vs_sdpa(case, sink, window, tol=1e-12):
    """Eq. 5: with s sinks and a w-token window the output is attention over
    the rows t < s and t >= n - w of the contiguous sequence, computed by the
    library routine on rows chosen by a boolean mask over 0..n-1."""
    k, v, km, vm = oracle_pools(case)
    lay = layout_of(case)
    out = oracle.paged_decode_window(lay, case.q, k, v, km, vm, case.block_tables, case.ctx,
                                     case.scale, sink, window)
    for b in range(case.B):
        K, V = logical_rows(case, b)
        n = K.shape[0]
        t = np.arange(n)
        keep = (t < sink) | (t >= n - window) if sink + window < n else np.ones(n, bool)
        dt = case.cfg.kv_dtype
        if dt != "bf16":
            Kf = np.stack([_dequant_exact(K[i], dt) for i in np.nonzero(keep)[0]])
            Vf = np.stack([_dequant_exact(V[i], dt) for i in np.nonzero(keep)[0]])
        else:
            Kf, Vf = _bf16_f64(K[keep]), _bf16_f64(V[keep])
        ref = _sdpa(_bf16_f64(case.q[b]), Kf, Vf, float(np.float32(case.scale)))
        err = np.abs(out[b] - ref).max()
        assert err <= tol, f"seq {b} (s={sink}, w={window}): oracle vs sdpa {err:.3e}"


def pin_window_degenerate(case):
    """No window (w = 0) or s + w >= n: exactly the full decode.  s = 0: exactly
    attention over the last w rows (eq. 6, K_{t-w+1:t})."""
    k, v, km, vm = oracle_pools(case)
    lay = layout_of(case)
    full = oracle.paged_decode(lay, case.q, k, v, km, vm, case.block_tables, case.ctx, case.scale)
    n_max = int(case.ctx.max())
    for s, w in ((0, 0), (5, 0), (0, n_max), (3, n_max - 3), (n_max, 1)):
        got = oracle.paged_decode_window(lay, case.q, k, v, km, vm, case.block_tables, case.ctx,
                                         case.scale, s, w)
        assert np.array_equal(got, full), (s, w)
    w = 7
    got = oracle.paged_decode_window(lay, case.q, k, v, km, vm, case.block_tables, case.ctx,
                                     case.scale, 0, w)
    qf = _bf16_f64(case.q)
    sc = float(np.float32(case.scale))
    for b in range(case.B):
        n = int(case.ctx[b])
        K, V = oracle.gather_sequence(lay, k, v, km, vm, case.block_tables[b], n)
        ref = oracle.attend(qf[b], K[:, max(n - w, 0):], V[:, max(n - w, 0):], sc)
        assert np.array_equal(got[b], ref), b


def pin_window_memory_bound(page_size=16, sink=4, window=40, steps=400):
    """Eq. 6: memory is bounded whatever the context.  A sequence grown one
    token at a time, evicting after each step, never holds more than
    ceil(s/P) + ceil(w/P) + 1 pages, and always holds every page a kept
    position lies in (so at least the w * 2 * L * d_k values of eq. 6)."""
    model = oracle.PoolModel(10_000)
    held = {}
    bound = -(-sink // page_size) + -(-window // page_size) + 1
    next_id = 0
    for n in range(1, steps + 1):
        blk = (n - 1) // page_size
        if blk not in held:
            model.check_alloc(1, [next_id])
            held[blk] = next_id
            next_id += 1
        drop = [b for b in oracle.window_evicted_blocks(n, page_size, sink, window) if b in held]
        model.free([held.pop(b) for b in drop])
        assert len(held) <= bound, (n, len(held), bound)
        kept_blocks = set((oracle.kept_positions(n, sink, window) // page_size).tolist())
        assert kept_blocks <= set(held), n
        # the pages held carry at least eq. 6's |cache| (one layer, d_k = 128)
        assert len(held) * page_size * 2 * 128 >= oracle.window_cache_elems(min(n, window), 1, 128)
    assert model.free_count == 10_000 - len(held)


# ---------------------------------------------------------------- multi-query chunks
def pin_prefill_vs_sdpa(case, tol=1e-12):
    """Chunk rows of a sequence of n tokens: torch's SDPA in float64 over the
    contiguous rows with an explicit boolean mask (row i may see column t iff
    t <= n - q_len + i), per query head."""
    k, v, km, vm = oracle_pools(case)
    lay = layout_of(case)
    out = oracle.paged_prefill(lay, case.q, case.q_start, k, v, km, vm, case.block_tables,
                               case.ctx, case.scale)
    g = case.cfg.num_q_heads // case.cfg.num_kv_heads
    for b in range(case.B):
        K, V = logical_rows(case, b)
        n = K.shape[0]
        r0, r1 = int(case.q_start[b]), int(case.q_start[b + 1])
        L = r1 - r0
        dt = case.cfg.kv_dtype
        if dt != "bf16":
            Kf = np.stack([_dequant_exact(K[t], dt) for t in range(n)])
            Vf = np.stack([_dequant_exact(V[t], dt) for t in range(n)])
        else:
            Kf, Vf = _bf16_f64(K), _bf16_f64(V)
        qf = _bf16_f64(case.q[r0:r1])                       # [L, H_q, D]
        mask = np.arange(n)[None, :] <= (n - L + np.arange(L))[:, None]   # [L, n]
        qt = torch.from_numpy(np.ascontiguousarray(qf.transpose(1, 0, 2)))[None]  # [1,Hq,L,D]
        kt = torch.from_numpy(np.ascontiguousarray(Kf.transpose(1, 0, 2)))[None]  # [1,Hkv,n,D]
        vt = torch.from_numpy(np.ascontiguousarray(Vf.transpose(1, 0, 2)))[None]
        kt = kt.repeat_interleave(g, dim=1)
        vt = vt.repeat_interleave(g, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=float(np.float32(case.scale)))
        ref = ref[0].numpy().transpose(1, 0, 2)              # [L, Hq, D]
        err = np.abs(out[r0:r1] - ref).max() if L else 0.0
        assert err <= tol, f"seq {b}: oracle prefill vs sdpa {err:.3e}"


def pin_prefill_single_row_is_decode(case):
    """A chunk of one token is the decode step, bit for bit."""
    assert (np.diff(case.q_start) == 1).all()
    k, v, km, vm = oracle_pools(case)
    lay = layout_of(case)
    a = oracle.paged_prefill(lay, case.q, case.q_start, k, v, km, vm, case.block_tables,
                             case.ctx, case.scale)
    d = oracle.paged_decode(lay, case.q, k, v, km, vm, case.block_tables, case.ctx, case.scale)
    assert np.array_equal(a, d)


# ---------------------------------------------------------------- prefix caching
def pin_prefix_eq2(N=100, T=2512, shared=2000, P=16):
    """Eq. 2 with the worked numbers of "Prefix Caching" (N = 100 requests,
    P_shared = 2000 tokens; T = 2512, a whole number of pages):
    caching every request's full blocks leaves P_shared/P + N*(T-P_shared)/P
    distinct pages, i.e. the prefix-cached memory of eq. 2 divided by the
    bytes of one page, and each later request matches exactly the prefix."""
    rng = np.random.default_rng(3)
    prefix = rng.integers(0, 50_000, shared).tolist()
    model = oracle.PrefixModel(P)
    next_page = 0
    for r in range(N):
        toks = prefix + rng.integers(0, 50_000, T - shared).tolist()
        got = model.match(toks)
        assert len(got) == (shared // P if r > 0 else 0), (r, len(got))
        pages = got + list(range(next_page, next_page + T // P - len(got)))
        next_page += T // P - len(got)
        model.insert(toks, pages)
    c = 1.0  # bytes per token: any unit
    expect = oracle.prefix_cached_bytes(N, T, shared, c) / (c * P)
    assert model.unique_pages() == expect == shared // P + N * (T - shared) // P


def pin_prefix_longest_match(trials=300, P=4):
    """The model's match is the longest common whole-block prefix with any
    inserted sequence, found by brute force over the inserted token lists."""
    rng = np.random.default_rng(5)
    model = oracle.PrefixModel(P)
    seqs = []
    base = rng.integers(0, 3, 64).tolist()        # small alphabet: many shared prefixes
    for t in range(trials):
        cut = int(rng.integers(0, 64))
        toks = base[:cut] + rng.integers(0, 3, int(rng.integers(0, 40))).tolist()
        best = 0
        for s in seqs:
            k = 0
            while (k + 1) * P <= min(len(s), len(toks)) and s[:(k + 1) * P] == toks[:(k + 1) * P]:
                k += 1
            best = max(best, k)
        assert len(model.match(toks)) == best, t
        model.insert(toks, list(range(1000 * t, 1000 * t + len(toks) // P)))
        seqs.append(toks)


# ---------------------------------------------------------------- INT4 and FP8 rows
def pin_int4_exact_rational(rows_bits):
    """quantize_rows_int4 equals the exact-rational IEEE model of its contract."""
    from oracle import quantize as oq
    codes, s16, z16 = oq.quantize_rows_int4(rows_bits)
    x = _bf16_f64(rows_bits)
    for i in range(x.shape[0]):
        c, s, z = quantize_row_exact(x[i].tolist(), steps=14, lo=-8, hi=7)
        assert codes[i].tolist() == c, i
        assert float(np.uint16(s16[i]).view(np.float16)) == float(s)
        assert float(np.uint16(z16[i]).view(np.float16)) == float(z)


def pin_int4_round_trip_and_ties():
    """Round trip within s*(1/2 + 2^-15) when nothing clamps; tie rows round
    half to even; a row already on the grid reconstructs exactly."""
    from oracle import quantize as oq
    rng = np.random.default_rng(12)
    x = rng.standard_normal((200, 128)).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    codes, s16, z16 = oq.quantize_rows_int4(bits)
    s = s16.view(np.float16).astype(np.float64)[:, None]
    z = z16.view(np.float16).astype(np.float64)[:, None]
    err = np.abs(_bf16_f64(bits) - (s * codes + z))
    unclamped = (codes > -8) & (codes < 7)
    assert (err[unclamped] <= (s * (0.5 + 2.0 ** -15) * np.ones_like(err))[unclamped]).all()
    # range -7..7 with s = 1, z = 0: ties 2.5 -> 2, 3.5 -> 4, -0.5 -> -0
    tie = np.zeros(128, np.float32)
    tie[:6] = [-7, 7, 2.5, 3.5, -0.5, 1.5]
    c, s1, z1 = oq.quantize_rows_int4(f32_to_bf16_bits(tie)[None])
    assert c[0, :6].tolist() == [-7, 7, 2, 4, 0, 2]
    grid = (np.arange(128) % 15 - 7).astype(np.float32) * 0.25
    c, s1, z1 = oq.quantize_rows_int4(f32_to_bf16_bits(grid)[None])
    back = s1.view(np.float16).astype(np.float64) * c[0] + z1.view(np.float16).astype(np.float64)
    assert np.array_equal(back, grid.astype(np.float64))


def pin_fp8_encode_vs_torch():
    """e4m3 codes: torch's float8_e4m3fn conversion (a library routine) gives
    the same code for every |value| <= 448; larger magnitudes saturate to
    +-448; the code table decodes as torch decodes."""
    from oracle import quantize as oq
    rng = np.random.default_rng(13)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * np.float32(40),
                        rng.standard_normal(20_000).astype(np.float32) * np.float32(0.01),
                        np.float32([0.0, -0.0, 448, -448, 2.0 ** -9, 2.0 ** -10, 1.5 * 2 ** -9,
                                    2.0 ** -6, 240.0, 232.0, 248.0])])
    enc = oq.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc, ref)
    big = np.float32([449.0, 464.0, 479.0, 1e6, -512.0])
    assert oq.e4m3_encode(big).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    dec = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    dec = dec.to(torch.float64).numpy()
    t = oq.e4m3_table()
    assert np.array_equal(np.isnan(t), np.isnan(dec)) and np.array_equal(t[~np.isnan(t)],
                                                                         dec[~np.isnan(dec)])


def pin_fp8_rows():
    """FP8 rows: the scale is the exact-rational f16(f32(amax/448)); every code
    is the e4m3 rounding of the float32 quotient x / s; |x| / s <= 448 up to
    the scale's own rounding, so only the extreme element can saturate."""
    from oracle import quantize as oq
    rng = np.random.default_rng(14)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[:, 5] *= 8
    bits = f32_to_bf16_bits(x)
    codes, s16, z16 = oq.quantize_rows_fp8(bits)
    assert (z16 == 0).all()
    xf = _bf16_f64(bits)
    for i in range(64):
        s = fp8_scale_exact(xf[i].tolist())
        assert float(np.uint16(s16[i]).view(np.float16)) == float(s)
        q = (bf16_bits_to_f32_np(bits[i]) / np.float32(float(s))).astype(np.float32)
        ref = torch.from_numpy(np.clip(q, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8)
        assert np.array_equal(codes[i], ref.numpy()), i
    # relative error of the nearest e4m3 value is at most 2^-4 in the normal range
    back = oq.dequantize_fp8(codes, s16)
    s = s16.view(np.float16).astype(np.float64)[:, None]
    normal = np.abs(xf) >= s * 2.0 ** -6
    assert (np.abs(back - xf)[normal] <= 2.0 ** -4 * np.abs(xf)[normal] + 1e-300).all()


def bf16_bits_to_f32_np(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def pin_int4_memory_ratios():
    """"KV-Cache Quantization": FP16 -> INT4 is 4x; "Multi-Query and Grouped-Query
    Caching": GQA with the LLaMA-2 70B numbers (H = 64, G = 8) times INT4 is the
    printed 32x.  With float16 scale and zero per row the INT4 row is (D/2+4)/(2D)
    of bfloat16 (0.266 at D = 128)."""
    g = _golden("memory_closed_forms.json")["gqa_llama2_70b"]
    int4_over_fp16 = 0.5 / 2
    total = oracle.gqa_ratio(g["kv_groups"], g["q_heads"]) * int4_over_fp16
    assert 1 / total == g["int4_times_gqa_printed"]
    assert 1 / int4_over_fp16 == g["int4_reduction_printed"]
    from oracle.accounting import int4_row_ratio
    assert int4_row_ratio(128) == 68 / 256


def pin_quantized_layout():
    """INT4 and FP8 pool bytes sit where the header's index formulas put them:
    INT4 K byte ((page*H + h)*P + t)*(D/2) + d/2 and V byte
    ((page*H + h)*(D/2) + d/2)*P + t, channel d in the low nibble when d is
    even, holding code + 8; FP8 codes in the INT8 layout."""
    from oracle import quantize as oq
    P, H, D, NP = 16, 2, 64, 3
    x = np.zeros((1, H, D), np.float32)
    x[0, 0, :15] = np.arange(-7, 8)          # row range -7..7: s = 1, z = 0, codes = x
    x[0, 0, 15:] = 0
    x[0, 1, :] = np.linspace(-3, 3, D)
    bits = f32_to_bf16_bits(x)
    bt = np.array([[2, 0]], np.int32)
    for dt in ("int4", "fp8"):
        lay = oracle.PoolLayout(NP, P, H, D, dt)
        k, v, km, vm = lay.empty_pools(0x7F, 0)
        oracle.append(lay, k, v, km, vm, bits, bits, np.array([0]), np.array([5]), bt)
        page, t = 2, 5
        quant = oq.quantize_rows_int4 if dt == "int4" else oq.quantize_rows_fp8
        codes, s16, z16 = quant(bits[0])
        for h in range(H):
            for d in range(D):
                if dt == "int4":
                    kb = k[((page * H + h) * P + t) * (D // 2) + d // 2]
                    vb = v[((page * H + h) * (D // 2) + d // 2) * P + t]
                    nib = lambda b: (int(b) >> (4 * (d % 2))) & 0xF  # noqa: E731
                    assert nib(kb) == codes[h, d] + 8 and nib(vb) == codes[h, d] + 8, (h, d)
                else:
                    assert k[((page * H + h) * P + t) * D + d] == codes[h, d]
                    assert v[((page * H + h) * D + d) * P + t] == codes[h, d]
            assert km[((page * H + h) * P + t) * 2] == s16[h]
            assert vm[((page * H + h) * P + t) * 2 + 1] == z16[h]
        if dt == "int4":
            assert codes[0, :15].tolist() == list(range(-7, 8))
        # every byte outside the written row keeps its fill
        touched = np.zeros(k.size, bool)
        for h in range(H):
            per = D // 2 if dt == "int4" else D
            touched[((page * H + h) * P + t) * per:((page * H + h) * P + t + 1) * per] = True
        assert (k[~touched] == 0x7F).all()
