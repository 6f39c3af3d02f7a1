"""OCP FP8 E4M3 ("e4m3fn") codec, written from the format's definition.

Test infrastructure (see the package docstring): not used by the product path.

The pages name an FP8 KV cache with 2x compression but not its sub-format
("nano-vllm-lite：深入理解LLM推理机制的教育级开源项目", 核心技术改进 §3 FP8 KV
Cache量化). The reading taken is OCP E4M3 without infinities, the format
CDNA4 converts natively:
* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field e > 0: value (1 + m/8) * 2**(e - 7);
* exponent field 0: value (m/8) * 2**-6 (subnormals);
* S.1111.111 is NaN; there is no infinity; the largest finite value is 448.

Encoding picks the finite code nearest to the input, ties to the code whose
last bit is 0, and saturates anything beyond +-448 to +-448.
"""
import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def decode(codes) -> np.ndarray:
    """float64 value of each e4m3fn byte."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * val
    return np.where((e == 15) & (m == 7), np.nan, val)


# the 127 non-negative finite codes 0x00..0x7E, in increasing value order
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = decode(_POS_CODES.astype(np.uint8))


def _tie_break(lo_code, hi_code):
    """At an exact midpoint the even code (last bit 0) wins."""
    return (hi_code & 1) == 0


def encode(x) -> np.ndarray:
    """Nearest e4m3fn code to each float32 input (ties to even, saturating)."""
    x = np.asarray(x, dtype=np.float32)
    mag = np.minimum(np.abs(x.astype(np.float64)), MAX_FINITE)
    hi = np.clip(np.searchsorted(_POS_VALUES, mag, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & _tie_break(lo, hi))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(np.isnan(x), NAN_CODE, code)
    return code.astype(np.uint8)


def quantize(values_f32, scale_f32) -> np.ndarray:
    """Bytes stored for float32 values with one float32 dequantisation scale:
    the float32 quotient value / scale (IEEE, correctly rounded), then encode."""
    q = np.asarray(values_f32, dtype=np.float32) / np.float32(scale_f32)
    return encode(q.astype(np.float32))


def quantize_bf16(bits, scale_f32) -> np.ndarray:
    """quantize() of bf16 inputs (uint16 bit patterns) with one scale, looked up
    in a table of quantize() over all 65536 bf16 patterns. quantize() acts on
    each value alone, so the table gives the same bytes; it only saves the
    encoding of values that repeat (large pools)."""
    key = np.float32(scale_f32).tobytes()
    table = _QUANT_TABLES.get(key)
    if table is None:
        every = (np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)).view(np.float32)
        with np.errstate(over="ignore", invalid="ignore"):   # inf / NaN patterns: saturate / NaN code
            table = _QUANT_TABLES[key] = quantize(every, np.float32(scale_f32))
    return table[np.asarray(bits, dtype=np.uint16)]


_QUANT_TABLES = {}


def decode_table() -> np.ndarray:
    """decode() of all 256 codes, indexed by code (the same values, looked up)."""
    return decode(np.arange(256, dtype=np.uint8))
