"""GPU parity of pa_add_rmsnorm (residual add fused with RMSNorm) against the CPU
oracle. The new residual is compared bit for bit. The normalised output is
float32 arithmetic rounded once to bf16, so it must lie within bf16 rounding of
the float64 result: |gpu - oracle| <= 1e-6 + 2^-8·|oracle| element-wise."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import dev_bf16, host_bits
from tests.util import assert_close, bf16_f64

pytestmark = pytest.mark.gpu

TOL = (1e-6, 2.0 ** -8)
EPS = 1e-6


def _run(x, r, w, eps=EPS):
    import paged_kv_cache_store_amd as pa
    xd, wd = dev_bf16(x), dev_bf16(w)
    if r is None:
        return host_bits(pa.add_rmsnorm(xd, wd, eps)), None
    out, hres = pa.add_rmsnorm(xd, wd, eps, residual=dev_bf16(r))
    return host_bits(out), host_bits(hres)


def _check(T, H, residual, seed, eps=EPS):
    x, r, w = W.norm_inputs(seed, T, H)
    if not residual:
        r = None
    got, hres = _run(x, r, w, eps)
    y, hbits = oracle.norm.add_rmsnorm(x, w, eps, r)
    ma, mr = assert_close(bf16_f64(got), y, *TOL, what=f"T={T} H={H} res={residual}")
    if residual:
        assert np.array_equal(hres, hbits), f"residual bits differ at T={T} H={H}"
    return ma, mr


# every lanes-per-row configuration, ragged row lengths inside each, 1..260 rows
SIZES = [8, 128, 136, 256, 264, 512, 1000, 1024, 1032, 2048, 2056, 3584, 4096, 4104, 5120, 8192,
         8200, 16384]


@pytest.mark.parametrize("H", SIZES)
def test_add_rmsnorm_sizes(H):
    print(f"H={H}", flush=True)
    for i, T in enumerate((1, 3, 37, 260)):
        _check(T, H, True, seed=400 + H + i)
    _check(37, H, False, seed=500 + H)


@pytest.mark.parametrize("name", list(W.NORM_WORKLOADS))
def test_norm_workloads_full(name):
    """The benchmark shapes, every element checked."""
    T, H = W.NORM_WORKLOADS[name]
    print(name, flush=True)
    ma, mr = _check(T, H, True, seed=7)
    print(f"max_abs={ma:.3e} max_rel={mr:.3e}")


def test_in_place_matches_out_of_place():
    import paged_kv_cache_store_amd as pa
    x, r, w = W.norm_inputs(31, 50, 1024)
    ref_out, ref_h = _run(x, r, w)
    xd, rd, wd = dev_bf16(x), dev_bf16(r), dev_bf16(w)
    pa.add_rmsnorm(xd, wd, EPS, residual=rd, out=xd, residual_out=rd)
    assert np.array_equal(host_bits(xd), ref_out) and np.array_equal(host_bits(rd), ref_h)
    # crossed: out over the residual, new residual over x
    xd, rd = dev_bf16(x), dev_bf16(r)
    pa.add_rmsnorm(xd, wd, EPS, residual=rd, out=rd, residual_out=xd)
    assert np.array_equal(host_bits(rd), ref_out) and np.array_equal(host_bits(xd), ref_h)


def test_guard_rows_untouched_and_deterministic():
    import paged_kv_cache_store_amd as pa
    T, H = 9, 4104
    x, r, w = W.norm_inputs(32, T, H)
    buf = torch.full((T + 2, H), -5.0, dtype=torch.bfloat16, device="cuda")
    hbuf = torch.full((T + 2, H), -5.0, dtype=torch.bfloat16, device="cuda")
    xd, rd, wd = dev_bf16(x), dev_bf16(r), dev_bf16(w)
    pa.add_rmsnorm(xd, wd, EPS, residual=rd, out=buf[1:T + 1], residual_out=hbuf[1:T + 1])
    first, hfirst = host_bits(buf), host_bits(hbuf)
    pa.add_rmsnorm(xd, wd, EPS, residual=rd, out=buf[1:T + 1], residual_out=hbuf[1:T + 1])
    assert np.array_equal(first, host_bits(buf)) and np.array_equal(hfirst, host_bits(hbuf))
    sentinel = host_bits(torch.full((H,), -5.0, dtype=torch.bfloat16))
    for b in (first, hfirst):
        assert np.array_equal(b[0], sentinel) and np.array_equal(b[T + 1], sentinel)


def test_large_eps_and_zero_rows():
    """A large eps (its placement matters) and all-zero rows (output 0, no NaN)."""
    T, H = 6, 256
    x, r, w = W.norm_inputs(33, T, H)
    r[2] = x[2] ^ np.uint16(0x8000)       # h = 0 on row 2
    x[4] = 0
    r[4] = 0
    got, hres = _run(x, r, w, eps=3.0)
    y, hbits = oracle.norm.add_rmsnorm(x, w, 3.0, r)
    assert_close(bf16_f64(got), y, *TOL, what="eps=3")
    assert np.array_equal(hres, hbits)
    assert not np.any(bf16_f64(got)[[2, 4]])


def test_zero_tokens_is_noop_and_errors():
    import paged_kv_cache_store_amd as pa
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    pa.add_rmsnorm(x, w, EPS)
    with pytest.raises(pa.PaError):
        pa.add_rmsnorm(torch.zeros((2, 12), dtype=torch.bfloat16, device="cuda"),
                       torch.ones(12, dtype=torch.bfloat16, device="cuda"), EPS)
    flat = torch.zeros(2 * 64 + 1, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pa.PaError):                 # 2-byte misaligned rows
        pa.add_rmsnorm(flat[1:].view(2, 64), w, EPS)
