"""A captured step (store + prefill + decode) replayed as a HIP graph gives the
eager results bit for bit, on every replay, with eager work between replays."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import GpuCase, host_bits

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    import paged_kv_cache_store_amd as pa
    w = W.custom(seed=401, Hq=8, Hkv=2, D=128, bs=64, context_lens=(5, 300, 1300),
                 prefill=[(64, 100)], partition_size=512)
    case = GpuCase(w, store_new=False)
    S, Hq, D = w.q.shape
    out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device="cuda")
    pout = torch.empty_like(case.pq)
    need = pa.decode_workspace_size(S, Hq, D, w.max_context_len, 512)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def step():
        case.store_new()
        case.prefill(out=pout)
        pa.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, float(w.scale),
                  w.max_context_len, out=out, partition_size=512, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager_out, eager_pout = host_bits(out), host_bits(pout)
    eager_k, eager_v = host_bits(case.k_cache), host_bits(case.v_cache)
    graph = pa.capture_step(step)
    for r in range(3):
        out.fill_(0)
        pout.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), eager_out), f"decode differs on replay {r}"
        assert np.array_equal(host_bits(pout), eager_pout), f"prefill differs on replay {r}"
        assert np.array_equal(host_bits(case.k_cache), eager_k)
        assert np.array_equal(host_bits(case.v_cache), eager_v)
        # eager work between replays
        case.decode(partition_size=512)
        torch.cuda.synchronize()
