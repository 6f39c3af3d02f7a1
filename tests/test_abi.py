"""The C-ABI library loads, exports what include/pa.h declares, and rejects bad
arguments on the host before any launch (no GPU needed: every call here fails
validation, so nothing reaches the HIP runtime)."""
import ctypes

import pytest

pa = pytest.importorskip("paged_kv_cache_store_amd")

OK, NULL, SHAPE, UNSUP, WS = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def desc(nb=8, bs=16, hkv=2, d=64, dtype=0, ks=None, vs=None):
    return pa.CacheDesc(nb, bs, hkv, d, dtype, ks, vs)


@pytest.fixture(scope="module")
def lib():
    return pa.library()


def test_exports_every_declared_symbol(lib):
    names = pa.header_functions()
    assert {"pa_store_kv", "pa_decode", "pa_store_decode", "pa_prefill_varlen", "pa_decode_workspace_size",
            "pa_decode_partition_size", "pa_status_string", "pa_last_hip_error", "pa_copy_blocks",
            "pa_bm_create", "pa_bm_add_sequence", "pa_bm_append_token"} <= set(names)
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5, -6, -7, 7):
        assert lib.pa_status_string(s)
    assert lib.pa_last_hip_error() == b""


def store(lib, d, k=FAKE, v=FAKE, slots=FAKE, T=4, kc=FAKE, vc=FAKE):
    return lib.pa_store_kv(k, v, slots, T, kc, vc, ctypes.byref(d) if d is not None else None, None)


def test_store_validation(lib):
    assert store(lib, None) == NULL
    assert store(lib, desc(), k=None) == NULL
    assert store(lib, desc(), kc=None) == NULL
    assert store(lib, desc(), T=-1) == SHAPE
    assert store(lib, desc(), T=0, k=None, v=None, slots=None) == OK      # no-op
    assert store(lib, desc(bs=48)) == UNSUP
    assert store(lib, desc(d=96)) == UNSUP
    assert store(lib, desc(dtype=3)) == UNSUP
    assert store(lib, desc(nb=0)) == SHAPE
    assert store(lib, desc(hkv=1025)) == UNSUP                            # at most 1024 KV heads
    assert store(lib, desc(dtype=1)) == NULL                              # fp8 needs scales


def decode(lib, d, q=FAKE, S=4, hq=4, maxctx=100, mb=8, P=0, ws=None, wsb=0, scale=0.125):
    return lib.pa_decode(q, FAKE, FAKE, FAKE, mb, FAKE, S, hq, maxctx, scale, FAKE,
                         ctypes.byref(d) if d is not None else None, P, ws, wsb, None)


def test_decode_validation(lib):
    assert decode(lib, None) == NULL
    assert decode(lib, desc(), q=None) == NULL
    assert decode(lib, desc(), hq=3) == SHAPE                 # Hq % Hkv
    assert decode(lib, desc(hkv=1), hq=3) == UNSUP            # group 3 not built
    assert decode(lib, desc(), S=-1) == SHAPE
    assert decode(lib, desc(), P=100) == SHAPE                # not a multiple of 256
    for bad in (float("nan"), float("inf"), float("-inf")):
        assert decode(lib, desc(), scale=bad) == SHAPE
    # any finite scale passes the scale check (q = NULL then fails, so nothing launches)
    assert decode(lib, desc(), scale=-0.125, q=None) == NULL
    assert decode(lib, desc(), S=0, q=None) == OK             # nothing to do
    # a split decode needs its workspace
    assert decode(lib, desc(bs=256), maxctx=2048, P=256) == WS
    need = lib.pa_decode_workspace_size(4, 4, 64, 2048, 256)
    assert need == 4 * 4 * 8 * (64 + 2) * 4
    assert decode(lib, desc(bs=256), maxctx=2048, P=256, ws=FAKE, wsb=need - 1) == WS
    # partition block ids must fit the 256-entry LDS table
    assert decode(lib, desc(bs=16), maxctx=8192, mb=512, P=8192, ws=FAKE, wsb=1 << 30) == UNSUP


def decode_noalloc(lib, d, q=FAKE, S=4, hq=4, maxctx=100, mb=8, P=0, scale=0.125):
    return lib.pa_decode_noalloc(q, FAKE, FAKE, FAKE, mb, FAKE, S, hq, maxctx, scale, FAKE,
                                 ctypes.byref(d) if d is not None else None, P, None)


def test_decode_noalloc_validation(lib):
    """The allocation-free decode checks its arguments as pa_decode does, and
    refuses a call whose scratch would exceed the library's array (64 MiB)
    before anything runs."""
    assert decode_noalloc(lib, None) == NULL
    assert decode_noalloc(lib, desc(), q=None) == NULL
    assert decode_noalloc(lib, desc(), hq=3) == SHAPE
    assert decode_noalloc(lib, desc(), P=100) == SHAPE
    assert decode_noalloc(lib, desc(), S=0, q=None) == OK
    big = desc(nb=8, bs=256, hkv=8, d=128)
    assert lib.pa_decode_workspace_size(4096, 32, 128, 32768, 256) > (64 << 20)
    assert decode_noalloc(lib, big, S=4096, hq=32, maxctx=32768, mb=128, P=256) == WS


def store_decode(lib, d, nk=FAKE, nv=FAKE, sm=FAKE, S=4, hq=4, maxctx=100, mb=8, P=0):
    return lib.pa_store_decode(FAKE, nk, nv, sm, FAKE, FAKE, FAKE, mb, FAKE, S, hq, maxctx, 0.125,
                               FAKE, ctypes.byref(d) if d is not None else None, P, None, 0, None)


def test_store_decode_validation(lib):
    assert store_decode(lib, None) == NULL
    assert store_decode(lib, desc(), nk=None) == NULL
    assert store_decode(lib, desc(), nv=None) == NULL
    assert store_decode(lib, desc(), sm=None) == NULL
    assert store_decode(lib, desc(), hq=3) == SHAPE
    assert store_decode(lib, desc(), P=100) == SHAPE
    assert store_decode(lib, desc(dtype=1)) == NULL                    # fp8 needs scales
    assert store_decode(lib, desc(), S=0, nk=None, nv=None, sm=None) == OK
    assert store_decode(lib, desc(bs=256), maxctx=2048, P=256) == WS


def test_workspace_and_partition_rules(lib):
    assert lib.pa_decode_workspace_size(4, 4, 64, 200, 0) == 0          # one partition: no workspace
    assert lib.pa_decode_workspace_size(0, 4, 64, 200, 0) == 0
    assert lib.pa_decode_partition_size(64, 32, 32768, 1024) == 1024
    for ctx in (1, 100, 1016, 2042, 32657):
        p = lib.pa_decode_partition_size(1, 1, ctx, 0)
        assert p % 256 == 0 and 256 <= p <= 2048
        assert lib.pa_decode_partition_size(1024, 32, ctx, 0) == min(4096, max(256, -(-ctx // 256) * 256))
    assert lib.pa_decode_partition_size(256, 16, 1016, 0) == 1024      # contexts kept whole
    assert lib.pa_decode_partition_size(64, 32, 32657, 0) == 2048      # few rows: split
    P = lib.pa_decode_partition_size(64, 32, 32768, 0)
    assert lib.pa_decode_workspace_size(64, 32, 128, 32768, 0) == 64 * 32 * (32768 // P) * 130 * 4


def prefill(lib, d, q=FAKE, S=2, hq=4, mq=16, mk=64, mb=8, scale=0.125, bt=FAKE):
    return lib.pa_prefill_varlen(q, FAKE, FAKE, FAKE, FAKE, bt, mb, S, hq, mq, mk, scale, FAKE,
                                 ctypes.byref(d) if d is not None else None, None)


def test_prefill_validation(lib):
    assert prefill(lib, None) == NULL
    assert prefill(lib, desc(), q=None) == NULL
    assert prefill(lib, desc(), hq=5) == SHAPE
    assert prefill(lib, desc(dtype=1)) == NULL                         # fp8 needs scales
    assert prefill(lib, desc(dtype=1, ks=FAKE, vs=FAKE), hq=5) == SHAPE
    assert prefill(lib, desc(), mq=-1) == SHAPE
    assert prefill(lib, desc(hkv=1025), hq=1025) == UNSUP
    assert prefill(lib, desc(), S=0, q=None) == OK
    for bad in (0.0, -0.5, float("inf"), float("nan")):
        assert prefill(lib, desc(), scale=bad) == SHAPE


def test_prefill_packed_validation(lib):
    """No block table: packed bf16 keys/values; only head counts, head_dim and
    dtype of the descriptor matter (no pool, no max_blocks_per_seq)."""
    assert prefill(lib, None, bt=None) == NULL
    assert prefill(lib, desc(dtype=1, ks=FAKE, vs=FAKE), bt=None) == UNSUP   # packed is bf16 only
    nopool = desc()
    nopool.num_blocks, nopool.block_size = 0, 0
    assert prefill(lib, nopool, bt=None, S=0, q=None) == OK
    assert prefill(lib, nopool, bt=None, mb=0, S=0, q=None) == OK
    assert prefill(lib, nopool, bt=None, hq=5) == SHAPE
    assert prefill(lib, nopool, bt=None, q=None) == NULL
    assert prefill(lib, nopool, bt=None, q=ctypes.c_void_p(0x1008)) == UNSUP
    d64 = desc()
    d64.head_dim = 96
    assert prefill(lib, d64, bt=None) == UNSUP
    wide = desc(hkv=1025)
    wide.num_blocks, wide.block_size = 0, 0
    assert prefill(lib, wide, bt=None, hq=1025) == UNSUP                  # at most 1024 KV heads
    # with a table, the pool must be a valid one
    assert prefill(lib, nopool) == SHAPE


def norm(lib, x=FAKE, r=FAKE, w=FAKE, T=4, H=64, eps=1e-6, out=ctypes.c_void_p(0x2000),
         rout=ctypes.c_void_p(0x3000)):
    return lib.pa_add_rmsnorm(x, r, w, T, H, eps, out, rout, None)


def test_add_rmsnorm_validation(lib):
    assert norm(lib, T=-1) == SHAPE
    assert norm(lib, H=0) == SHAPE
    assert norm(lib, H=12) == UNSUP                          # not a multiple of 8
    assert norm(lib, H=16392) == UNSUP                       # above 16384
    for bad in (0.0, -1e-6, float("inf"), float("nan")):
        assert norm(lib, eps=bad) == SHAPE
    assert norm(lib, T=0, x=None, r=None, w=None, out=None, rout=None) == OK
    assert norm(lib, x=None) == NULL
    assert norm(lib, w=None) == NULL
    assert norm(lib, rout=None) == NULL                      # residual given, no residual_out
    assert norm(lib, rout=ctypes.c_void_p(0x2000)) == SHAPE  # residual_out == out
    assert norm(lib, x=ctypes.c_void_p(0x1002)) == UNSUP     # not 16-byte aligned
    assert norm(lib, rout=ctypes.c_void_p(0x3008)) == UNSUP


def test_alignment_rules(lib):
    """bf16 / fp8 data must be 16-byte aligned, int32 arrays 4-byte aligned."""
    odd16, odd4 = ctypes.c_void_p(0x1008), ctypes.c_void_p(0x1002)
    assert store(lib, desc(), k=odd16) == UNSUP
    assert store(lib, desc(), kc=odd16) == UNSUP
    assert store(lib, desc(), slots=odd4) == UNSUP
    assert decode(lib, desc(), q=odd16) == UNSUP
    assert store_decode(lib, desc(), nk=odd16) == UNSUP
    assert store_decode(lib, desc(), sm=odd4) == UNSUP
    assert prefill(lib, desc(), q=odd16) == UNSUP
    assert lib.pa_copy_blocks(odd16, FAKE, FAKE, 1, ctypes.byref(desc()), None) == UNSUP


def test_decode_vector_alu_form_compiles(tmp_path):
    """The decode kernel's other form (PA_DECODE_MFMA=0: the products on the
    VALU with v_dot2) still compiles for gfx950 (device code only)."""
    import os
    import shutil
    import subprocess

    import paged_kv_cache_store_amd.build as B
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path / "decode_valu.o"
    cmd = [B.HIPCC, *B.DEVICE_FLAGS, "-DPA_DECODE_MFMA=0", "--cuda-device-only", "-I", B.INCLUDE, "-I", B.CSRC,
           "-c", os.path.join(B.CSRC, "decode.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    assert out.stat().st_size > 0
