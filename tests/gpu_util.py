"""GPU-side set-up shared by the GPU tests: upload a workload, fill NaN-poisoned
pools through pa_store_kv, run the calls. Only argument plumbing lives here."""
import numpy as np
import torch

import workloads as W


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host_bits(t):
    """uint16 (bf16) or uint8 (fp8) bit patterns of a device tensor."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class GpuCase:
    """Device copies of a workload with pools filled by the library's store."""

    def __init__(self, w, store_new=True):
        import paged_kv_cache_store_amd as pa
        self.w = w
        self.pa = pa
        self.k_cache, self.v_cache = pa.empty_pools(w.num_blocks, w.num_kv_heads, w.block_size,
                                                    w.head_dim, w.kv_dtype)
        if w.kv_dtype == "fp8":
            self.k_cache.fill_(int(W.FP8_NAN))
            self.v_cache.fill_(int(W.FP8_NAN))
            self.k_scale = torch.from_numpy(w.k_scale).cuda()
            self.v_scale = torch.from_numpy(w.v_scale).cuda()
        else:
            self.k_cache.view(torch.int16).fill_(int(W.BF16_NAN))
            self.v_cache.view(torch.int16).fill_(int(W.BF16_NAN))
            self.k_scale = self.v_scale = None
        self.q = dev_bf16(w.q)
        self.block_tables = dev_i32(w.block_tables)
        self.context_lens = dev_i32(w.context_lens)
        self.new_k, self.new_v = dev_bf16(w.new_k), dev_bf16(w.new_v)
        self.new_slots = dev_i32(w.new_slots)
        if w.fill_slots.size:
            self.store(dev_bf16(w.fill_k), dev_bf16(w.fill_v), dev_i32(w.fill_slots))
        if store_new:
            self.store_new()
        if w.has_prefill:
            self.pq = dev_bf16(w.pq)
            self.cu_q = dev_i32(w.cu_seqlens_q)
            self.cu_k = dev_i32(w.cu_seqlens_k)
            self.p_block_tables = dev_i32(w.p_block_tables)
        torch.cuda.synchronize()

    def store(self, k, v, slots):
        self.pa.store_kv(k, v, slots, self.k_cache, self.v_cache, self.k_scale, self.v_scale)

    def store_new(self):
        if self.w.new_slots.size:
            self.store(self.new_k, self.new_v, self.new_slots)

    def decode(self, partition_size=None, out=None):
        w = self.w
        ps = w.partition_size if partition_size is None else partition_size
        return self.pa.decode(self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
                              float(w.scale), w.max_context_len, out=out, k_scale=self.k_scale,
                              v_scale=self.v_scale, partition_size=ps)

    def prefill(self, out=None):
        w = self.w
        return self.pa.prefill_varlen(self.pq, self.k_cache, self.v_cache, self.cu_q, self.cu_k,
                                      self.p_block_tables, float(w.scale), w.max_seqlen_q,
                                      w.max_seqlen_k, out=out, k_scale=self.k_scale,
                                      v_scale=self.v_scale)
