"""The CPU oracle against what the pages and mathematics fix (no GPU)."""
import numpy as np
import pytest

import oracle
from workloads import INT8_LONG, LLAMA3_8B_LAYER, SHARED_PREFIX_MQA, TINY, make_case, variant

from . import pins


@pytest.fixture(scope="module", params=pins.small_cases(), ids=lambda c: c.name)
def small_case(request):
    return make_case(request.param)


def test_block_table_worked_example():
    pins.pin_block_table_worked_example()


def test_append_and_gather_follow_layout(small_case):
    pins.pin_append_and_gather_layout(small_case)


def test_attention_vs_library_sdpa(small_case):
    pins.pin_attention_vs_sdpa(small_case)


def test_special_cases():
    pins.pin_special_cases()


def test_page_relabel_invariance(small_case):
    pins.pin_page_relabel_invariance(small_case)


def test_quantize_matches_exact_rational_ieee():
    pins.pin_quantize_exact_rational()


def test_quantize_ties_grid_constant():
    pins.pin_quantize_ties_and_grid()


def test_quantize_round_trip_on_outlier_rows():
    """Rows shaped like the INT8 workload (N(0,1), 1% channels x8)."""
    c = variant(INT8_LONG, batch=2, ctx_lo=300, ctx_hi=400)
    case = make_case(c)
    pins.pin_quantize_round_trip(case.hist_k)
    pins.pin_quantize_round_trip(case.hist_v)


def test_memory_closed_forms():
    pins.pin_memory_closed_forms()


def test_int8_row_ratio():
    # Section "KV-Cache Quantization" prints a 2x reduction FP16 -> INT8; the
    # stored float16 scale and zero add 4 bytes per 128-channel row.
    assert oracle.int8_row_ratio(128) == 132 / 256 == 0.515625


@pytest.mark.parametrize("cfg", [TINY, LLAMA3_8B_LAYER, INT8_LONG, SHARED_PREFIX_MQA],
                         ids=lambda c: c.name)
def test_waste_bound(cfg):
    pins.pin_waste_bound(make_case(cfg, with_data=False))


def test_shared_prefix_memory():
    pins.pin_shared_prefix_memory()


def test_pool_model_semantics():
    m = oracle.PoolModel(4)
    m.check_alloc(3, [0, 1, 2])
    with pytest.raises(oracle.NoPages):
        m.check_alloc(2, [3, 0])
    m.share([0, 1])
    assert m.refcount(0) == 2 and m.free_count == 1
    with pytest.raises(oracle.AllocError):
        m.free([2, 2])
    m.free([0, 1, 2])
    assert m.refcount(0) == 1 and m.refcount(2) == 0 and m.free_count == 2
    with pytest.raises(oracle.AllocError):
        m.share([2])


@pytest.mark.parametrize("sink,window", [(0, 7), (4, 16), (1, 1), (16, 33), (3, 50)])
def test_window_vs_library_sdpa(small_case, sink, window):
    pins.pin_window_vs_sdpa(small_case, sink, window)


def test_window_degenerate_cases(small_case):
    pins.pin_window_degenerate(small_case)


def test_window_memory_bound():
    pins.pin_window_memory_bound()
    pins.pin_window_memory_bound(page_size=32, sink=0, window=100, steps=700)


@pytest.mark.parametrize("cfg", pins.prefill_cases(), ids=lambda c: c.name)
def test_prefill_vs_library_sdpa(cfg):
    pins.pin_prefill_vs_sdpa(make_case(cfg))


def test_prefill_single_row_is_decode(small_case):
    pins.pin_prefill_single_row_is_decode(small_case)


def test_prefix_cache_model_eq2():
    pins.pin_prefix_eq2()


def test_prefix_cache_model_longest_match():
    pins.pin_prefix_longest_match()


def test_int4_matches_exact_rational_ieee():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((48, 128)).astype(np.float32)
    x[:, [3, 70]] *= 8
    from workloads import f32_to_bf16_bits
    pins.pin_int4_exact_rational(f32_to_bf16_bits(x))


def test_int4_round_trip_and_ties():
    pins.pin_int4_round_trip_and_ties()


def test_fp8_encode_vs_torch():
    pins.pin_fp8_encode_vs_torch()


def test_fp8_rows():
    pins.pin_fp8_rows()


def test_int4_memory_ratios():
    pins.pin_int4_memory_ratios()


@pytest.mark.parametrize("dtype", ["int4", "fp8"])
def test_quantized_attention_vs_library_sdpa(dtype):
    """Attention over INT4 / FP8 pools equals torch SDPA over the rows the
    row contract reconstructs (exact-rational dequantization for INT4; the
    e4m3 value table times the scale for FP8)."""
    cfg = variant(TINY, name="tiny_" + dtype, kv_dtype=dtype, num_q_heads=8, num_kv_heads=2,
                  head_dim=128, pool_pages=32, outlier_channels=3, outlier_gain=8.0)
    pins.pin_attention_vs_sdpa(make_case(cfg))


def test_quantized_pool_layout():
    pins.pin_quantized_layout()
