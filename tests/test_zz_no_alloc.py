"""pa_decode_noalloc — the decode for callers that cannot allocate — against
pa_decode with a caller's workspace, through the C ABI: bit-identical output on
two calls in a row, the second with a smaller input (the library's scratch
array keeps the first call's contents), bf16 and fp8, split and whole
contexts, many sequences (ranked longest first) and few. A call that would
need more scratch than the array holds is refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_store_amd as pa
import workloads as W
from tests.gpu_util import GpuCase, host_bits

pytestmark = pytest.mark.gpu

WORKSPACE = -4


def _noalloc(case, partition_size, out):
    w = case.w
    return pa.decode_noalloc(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                             float(w.scale), w.max_context_len, out, k_scale=case.k_scale,
                             v_scale=case.v_scale, partition_size=partition_size)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_noalloc_matches_decode_two_calls(kv):
    rng = np.random.default_rng(500)
    big = W.custom(seed=501, Hq=16, Hkv=4, D=128, bs=64, kv_dtype=kv,
                   context_lens=tuple(int(x) for x in rng.integers(0, 3000, 300)))
    small = W.custom(seed=502, Hq=8, Hkv=2, D=64, bs=16, kv_dtype=kv, context_lens=(1, 40, 700, 2100, 5))
    for w, ps in ((big, 256), (small, 512)):       # the second call is smaller
        print(f"{kv}: {w.num_seqs} sequences, partition {ps}", flush=True)
        case = GpuCase(w)
        want = host_bits(case.decode(partition_size=ps))
        out = torch.full_like(case.q, -3.0)
        _noalloc(case, ps, out)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), want)
        # and again with the contexts kept whole where they fit
        want0 = host_bits(case.decode(partition_size=0))
        _noalloc(case, 0, out)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), want0)


def test_noalloc_refuses_beyond_the_array():
    """4096 sequences x 32 query heads x 128 partitions of 256 tokens need far
    more than the array: PA_ERR_WORKSPACE, returned before any launch."""
    lib = pa.library()
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    desc = pa.CacheDesc(8, 256, 8, 128, 0, None, None)
    need = lib.pa_decode_workspace_size(4096, 32, 128, 32768, 256)
    assert need > (64 << 20)
    st = lib.pa_decode_noalloc(p, p, p, p, 128, p, 4096, 32, 32768, 0.088, p, ctypes.byref(desc), 256, None)
    assert st == WORKSPACE
