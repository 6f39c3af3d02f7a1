// Internal launch wrappers of libpa: one per kernel family. Arguments have been
// validated by the C ABI layer (api.hip); each wrapper only enqueues work.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace pa {

struct PoolDims {
  int num_blocks, block_size, num_kv_heads, head_dim;
  bool fp8;
};

hipError_t launch_store_kv(const uint16_t* k, const uint16_t* v, const int32_t* slots,
                           int num_tokens, uint8_t* k_cache, uint8_t* v_cache,
                           const PoolDims& pool, const float* k_scale, const float* v_scale,
                           hipStream_t stream);

hipError_t launch_copy_blocks(uint8_t* k_cache, uint8_t* v_cache, const int32_t* pairs, int num_pairs,
                              const PoolDims& pool, hipStream_t stream);

// Workspace layout for a decode with num_parts partitions per sequence:
//   float o[num_seqs][num_q_heads][num_parts][head_dim]   (unnormalised partial output)
//   float m[num_seqs][num_q_heads][num_parts]              (partial max, log2 units)
//   float l[num_seqs][num_q_heads][num_parts]              (partial sum of weights)
//   int32 order[num_seqs] (256-byte aligned, after the partials) when the
//   sequences are ranked longest first (many sequences, long contexts)
size_t decode_workspace_bytes(int num_seqs, int num_q_heads, int head_dim, int num_parts, int ctx_cap);

hipError_t launch_decode(const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int num_q_heads,
                         int max_context_len, float scale, uint16_t* out, const PoolDims& pool,
                         const float* k_scale, const float* v_scale, int partition_size,
                         void* workspace, hipStream_t stream, const uint16_t* new_k = nullptr,
                         const uint16_t* new_v = nullptr, const int32_t* new_slots = nullptr);

hipError_t launch_prefill(const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                          const int32_t* cu_q, const int32_t* cu_k, const int32_t* block_tables,
                          int max_blocks_per_seq, int num_seqs, int num_q_heads,
                          int max_seqlen_q, int max_seqlen_k, float scale, uint16_t* out,
                          const PoolDims& pool, const float* k_scale, const float* v_scale,
                          hipStream_t stream);

// resident workgroups of a persistent prefill launch (0: two per CU; < 0: one
// workgroup per work item)
void set_prefill_slots(int n);

hipError_t launch_add_rmsnorm(const uint16_t* x, const uint16_t* r, const uint16_t* w, uint16_t* out,
                              uint16_t* r_out, int num_tokens, int hidden, float eps, hipStream_t stream);

}  // namespace pa
