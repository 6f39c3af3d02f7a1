"""Plant plausible mistakes in the CPU oracle (on the CPU, via monkeypatch) and
check that at least one pin catches each. Guards against pins too weak to notice
a dropped term, a wrong index or sign, or a transposed operand."""
import numpy as np
import pytest

import oracle
from tests import pins


def _fails(pin_list):
    failed = []
    for p in pin_list:
        try:
            p()
        except AssertionError:
            failed.append(p.__name__)
    return failed


ATTN_PINS = [pins.pin_decode_vs_sdpa, pins.pin_prefill_vs_sdpa, pins.pin_chunk_is_tail_of_full_prefill,
             pins.pin_decode_closed_forms, pins.pin_gqa_equals_replicated_mha]
FP8_PINS = [pins.pin_fp8_code_table, pins.pin_fp8_encode_vs_torch, pins.pin_fp8_hand_cases,
            pins.pin_fp8_roundtrip]
CACHE_PINS = [pins.pin_store_roundtrip, pins.pin_layout_offsets, pins.pin_store_skip_and_sentinel]
NORM_PINS = [pins.pin_bf16_round_hand_cases, pins.pin_bf16_round_vs_torch, pins.pin_rmsnorm_vs_torch,
             pins.pin_residual_sum_vs_torch_bf16_add, pins.pin_rmsnorm_closed_forms]


def _interleaved_heads(h, group, num_kv_heads):
    return h % num_kv_heads


def _top_left_mask(Lq, Lk):
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    return j <= i


def _strict_mask(Lq, Lk):
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    return j < (Lk - Lq) + i


def _no_max_shift_wrong_norm(z, mask=None):
    if mask is not None:
        z = np.where(mask, z, -np.inf)
    p = np.exp(z)
    return p / p.shape[-1]          # divides by the count instead of the sum


def _ties_up(lo, hi):
    return np.ones_like(hi, dtype=bool)


def _decode_off_by_one_exponent(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 8.0))
    return np.where((e == 15) & (m == 7), np.nan, sign * val)


def _depage_swapped_v(k_cache, v_cache, table_row, length, block_size, k_scale=None, v_scale=None):
    import math
    nb = math.ceil(length / block_size)
    blocks = np.asarray(table_row[:nb], dtype=np.int64)
    H = k_cache.shape[1]
    x = 16 // k_cache.itemsize
    D = k_cache.shape[2] * x
    K = k_cache[blocks].transpose(0, 3, 1, 2, 4).reshape(nb * block_size, H, D)[:length]
    V = v_cache[blocks].transpose(0, 4, 2, 1, 3).reshape(nb * block_size, H, D)[:length]  # o//x, o%x swapped
    return K, V


def _residual_dropped(x, r):
    return x


def _mean_over_h_minus_1(h):
    return np.sum(h * h, axis=-1, keepdims=True) / (h.shape[-1] - 1)


def _bf16_via_float32(v):
    import workloads as W
    with np.errstate(over="ignore"):
        return W.f32_to_bf16_bits(np.asarray(v, dtype=np.float64).astype(np.float32))


def _bf16_ties_away(v):
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    step = np.exp2(np.maximum(ex - 1, -126) - 7.0)
    q = np.floor(a / step + 0.5) * step
    q = np.where(np.signbit(v), -q, q)
    with np.errstate(over="ignore"):
        return (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


MUTATIONS = [
    ("attention._kv_head", _interleaved_heads, ATTN_PINS),
    ("attention._causal_mask", _top_left_mask, ATTN_PINS),
    ("attention._causal_mask", _strict_mask, ATTN_PINS),
    ("attention._softmax_rows", _no_max_shift_wrong_norm, ATTN_PINS),
    ("fp8._tie_break", _ties_up, FP8_PINS),
    ("fp8.decode", _decode_off_by_one_exponent, FP8_PINS),
    ("cache.depage_raw", _depage_swapped_v, CACHE_PINS),
    ("norm._residual_sum", _residual_dropped, NORM_PINS),
    ("norm._mean_square", _mean_over_h_minus_1, NORM_PINS),
    ("norm.f64_to_bf16_bits", _bf16_via_float32, NORM_PINS),
    ("norm.f64_to_bf16_bits", _bf16_ties_away, NORM_PINS),
]


@pytest.mark.parametrize("target,bad,pin_list", MUTATIONS,
                         ids=[f"{t}:{b.__name__}" for t, b, _ in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, target, bad, pin_list):
    mod_name, attr = target.split(".")
    mod = getattr(oracle, mod_name)
    monkeypatch.setattr(mod, attr, bad)
    if mod_name == "fp8" and attr == "decode":
        # encode's table is built from decode at import time; rebuild it too
        monkeypatch.setattr(mod, "_POS_VALUES", bad(np.arange(0x7F, dtype=np.uint8)))
    if mod_name == "cache":
        # attention imports depage by name
        pass
    failed = _fails(pin_list)
    assert failed, f"no pin caught the planted mistake {bad.__name__} in {target}"
