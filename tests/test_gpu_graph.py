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


def test_graph_replay_store_decode_matches_eager():
    """The decode step as the benchmark captures it (pa_store_decode, split
    contexts, bf16 and fp8): every replay equals the eager call, pools included."""
    import paged_kv_cache_store_amd as pa
    from tests.gpu_util import dev_bf16, dev_i32
    for kv in ("bf16", "fp8"):
        w = W.custom(seed=402, Hq=16, Hkv=4, D=128, bs=64, context_lens=(1, 64, 65, 700, 2000),
                     partition_size=512, kv_dtype=kv)
        case = GpuCase(w, store_new=False)
        S, Hq, D = w.q.shape
        live = np.flatnonzero(w.context_lens > 0)
        k = np.zeros((S,) + w.new_k.shape[1:], np.uint16)
        v = np.zeros_like(k)
        slots = np.full(S, -1, np.int32)
        k[live], v[live], slots[live] = w.new_k, w.new_v, w.new_slots
        kd, vd, sd = dev_bf16(k), dev_bf16(v), dev_i32(slots)
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device="cuda")
        need = pa.decode_workspace_size(S, Hq, D, w.max_context_len, 512)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

        def step():
            pa.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                      float(w.scale), w.max_context_len, out=out, k_scale=case.k_scale,
                      v_scale=case.v_scale, partition_size=512, workspace=ws, new_k=kd, new_v=vd,
                      slot_mapping=sd)

        step()
        torch.cuda.synchronize()
        eager_out = host_bits(out)
        eager_k, eager_v = host_bits(case.k_cache), host_bits(case.v_cache)
        graph = pa.capture_step(step)
        for r in range(3):
            out.fill_(0)
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host_bits(out), eager_out), f"{kv}: output differs on replay {r}"
            assert np.array_equal(host_bits(case.k_cache), eager_k)
            assert np.array_equal(host_bits(case.v_cache), eager_v)
            case.decode(partition_size=512)     # eager work between replays
            torch.cuda.synchronize()
