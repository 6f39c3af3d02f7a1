"""Residual add + RMSNorm — TEST INFRASTRUCTURE (see the package docstring).

What the pages fix: every transformer layer applies a residual connection
(Add) followed by RMSNorm, and doing both in one kernel saves the trip of the
intermediate sum through memory ("nano-vllm-lite：深入理解LLM推理机制的教育级开源项目",
核心技术改进 §1 CUDA融合内核：Add+RMSNorm).

Reading (the pages print no formula; this is the standard RMSNorm):
    h = x + r                                 (r absent: h = x)
    y = h / sqrt(mean(h^2) + eps) * w         (mean over the hidden dimension)
The sum h is the new residual stream; it is returned as bf16, rounded to
nearest with ties to even directly from the exact sum. y is returned unrounded
in float64.
"""
import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """Nearest bf16 (8 significant bits, exponent range of float32) to each
    float64 value, ties to even, in one rounding step (no detour through
    float32). Magnitudes that round beyond the largest finite bf16 give inf."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    finite = np.isfinite(a) & (a > 0)
    safe = np.where(finite, a, 1.0)
    _, ex = np.frexp(safe)                         # safe = m * 2^ex, m in [0.5, 1)
    step = np.exp2(np.maximum(ex - 1, -126) - 7.0)  # bf16 spacing in that binade
    q = np.rint(safe / step) * step                # exact scaling; rint ties to even
    q = np.where(finite, q, a)
    q = np.where(q > _BF16_MAX, np.inf, q)
    q = np.where(np.signbit(v), -q, q)
    bits = (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(v), np.uint16(0x7FC0), bits)


def _residual_sum(x, r):
    return x if r is None else x + r


def _mean_square(h):
    return np.mean(h * h, axis=-1, keepdims=True)


def add_rmsnorm(x_bits, w_bits, eps, r_bits=None):
    """x_bits, r_bits: bf16 bits [T, H]; w_bits: bf16 bits [H].
    Returns (y float64 [T, H], h as bf16 bits [T, H] or None when r is absent)."""
    x = bf16_bits_to_f64(x_bits)
    r = None if r_bits is None else bf16_bits_to_f64(r_bits)
    w = bf16_bits_to_f64(w_bits)
    h = _residual_sum(x, r)
    y = h / np.sqrt(_mean_square(h) + float(eps)) * w
    return y, (None if r is None else f64_to_bf16_bits(h))
