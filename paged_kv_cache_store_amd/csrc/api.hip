// C ABI of libpa (declared in include/pa.h): argument checks, then launches.
// Every check below runs on the host before anything is enqueued, so a bad
// argument never reaches the GPU and the checks can be exercised without one.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "pa.h"
#include "pa_block_manager.h"
#include "pa_launch.h"

namespace {

thread_local char g_hip_error[256] = "";

pa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  snprintf(g_hip_error, sizeof(g_hip_error), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return PA_ERR_HIP;
}

constexpr int kMaxKvHeads = 1024;

bool supported_block_size(int bs) {
  return bs == 16 || bs == 32 || bs == 64 || bs == 128 || bs == 256;
}

pa_status check_cache(const pa_cache_desc* c, pa::PoolDims* dims) {
  if (!c) return PA_ERR_NULL;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->block_size <= 0 || c->head_dim <= 0)
    return PA_ERR_SHAPE;
  if (!supported_block_size(c->block_size)) return PA_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return PA_ERR_UNSUPPORTED;
  // a block (every KV head) stays far below 2 GiB: kernels size it in 32 bits
  if (c->num_kv_heads > kMaxKvHeads) return PA_ERR_UNSUPPORTED;
  if (c->dtype != PA_KV_BF16 && c->dtype != PA_KV_FP8_E4M3) return PA_ERR_UNSUPPORTED;
  if (c->dtype == PA_KV_FP8_E4M3 && (!c->k_scale || !c->v_scale)) return PA_ERR_NULL;
  dims->num_blocks = c->num_blocks;
  dims->block_size = c->block_size;
  dims->num_kv_heads = c->num_kv_heads;
  dims->head_dim = c->head_dim;
  dims->fp8 = c->dtype == PA_KV_FP8_E4M3;
  return PA_OK;
}

bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

}  // namespace

// Scratch of pa_decode_noalloc: a file-scope device array, one per GPU, held
// until the process ends. In host code `scratch` is only the symbol's
// stand-in; kernels are given its device address on the device concerned,
// looked up once per device with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that owns `stream` (the current
// device for the null stream), looked up the first time with that device current.
pa_status scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return hip_status(e);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

// The kernels move bf16 / fp8 data in 16-byte vectors and read int32 arrays as
// dwords: data pointers must be 16-byte aligned, int32 arrays 4-byte aligned.
bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

int32_t round_up(int32_t x, int32_t m) { return (x + m - 1) / m * m; }

// Automatic partition size. With enough (sequence, query head) rows to fill the
// GPU, contexts stay whole (no partial results, no reduce); otherwise long
// contexts are cut into 2048-token partitions. Never above 4096 tokens, so the
// partition's block ids fit the 256-entry table in LDS for every block size.
int32_t auto_partition(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len) {
  int32_t whole = round_up(max_context_len, 256);
  if (whole < 256) whole = 256;
  const long long rows = (long long)num_seqs * num_q_heads;
  const int32_t cap = rows >= 4096 ? 4096 : 2048;
  return whole < cap ? whole : cap;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "sizes are negative or inconsistent";
    case PA_ERR_UNSUPPORTED: return "head_dim, block_size, group size or dtype not supported";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP error (see pa_last_hip_error)";
    case PA_ERR_NO_BLOCKS: return "not enough free KV blocks";
    case PA_ERR_NOT_FOUND: return "unknown sequence id";
  }
  return "unknown status";
}

const char* pa_last_hip_error(void) { return g_hip_error; }

pa_status pa_store_kv(const void* k, const void* v, const int32_t* slot_mapping,
                      int32_t num_tokens, void* k_cache, void* v_cache,
                      const pa_cache_desc* cache, hipStream_t stream) {
  pa::PoolDims dims;
  pa_status st = check_cache(cache, &dims);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (!k_cache || !v_cache) return PA_ERR_NULL;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping) return PA_ERR_NULL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 4))
    return PA_ERR_UNSUPPORTED;
  return hip_status(pa::launch_store_kv(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                        slot_mapping, num_tokens, static_cast<uint8_t*>(k_cache),
                                        static_cast<uint8_t*>(v_cache), dims, cache->k_scale,
                                        cache->v_scale, stream));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                         const pa_cache_desc* cache, hipStream_t stream) {
  pa::PoolDims dims;
  pa_status st = check_cache(cache, &dims);
  if (st != PA_OK) return st;
  if (num_pairs < 0 || num_pairs > 65535) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return PA_ERR_NULL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(pairs, 4)) return PA_ERR_UNSUPPORTED;
  return hip_status(pa::launch_copy_blocks(static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                                           pairs, num_pairs, dims, stream));
}

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                 int32_t partition_size) {
  if (partition_size > 0) return partition_size;
  return auto_partition(num_seqs, num_q_heads, max_context_len < 0 ? 0 : max_context_len);
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  const int32_t ctx = max_context_len < 0 ? 0 : max_context_len;
  const int32_t P = pa_decode_partition_size(num_seqs, num_q_heads, ctx, partition_size);
  if (P <= 0) return 0;
  const int32_t np = ctx > 0 ? (ctx + P - 1) / P : 1;
  return pa::decode_workspace_bytes(num_seqs, num_q_heads, head_dim, np, ctx);
}

namespace {

// pa_decode and pa_store_decode: the same checks and decode launch; the second
// hands the newest tokens to the decode kernel (which reads position n-1 from
// them) and then launches their store.
pa_status decode_impl(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_context_len, float scale, void* out, const pa_cache_desc* cache,
                      int32_t partition_size, void* workspace, size_t workspace_bytes,
                      hipStream_t stream, const void* new_k, const void* new_v,
                      const int32_t* slot_mapping, bool with_new, bool noalloc = false) {
  pa::PoolDims dims;
  pa_status st = check_cache(cache, &dims);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % dims.num_kv_heads != 0) return PA_ERR_SHAPE;
  if (!supported_group(num_q_heads / dims.num_kv_heads)) return PA_ERR_UNSUPPORTED;
  if (partition_size < 0 || partition_size % 256 != 0) return PA_ERR_SHAPE;
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PA_ERR_NULL;
  if (with_new && (!new_k || !new_v || !slot_mapping)) return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(workspace, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PA_ERR_UNSUPPORTED;
  if (with_new && (!aligned(new_k, 16) || !aligned(new_v, 16) || !aligned(slot_mapping, 4)))
    return PA_ERR_UNSUPPORTED;
  // the grid covers contexts up to the smaller of the two host bounds
  const long long cap_ll = (long long)max_blocks_per_seq * dims.block_size;
  const int32_t cap = int32_t(cap_ll < max_context_len ? cap_ll : max_context_len);
  const int32_t P = pa_decode_partition_size(num_seqs, num_q_heads, cap, partition_size);
  if (P / dims.block_size > 256) return PA_ERR_UNSUPPORTED;  // block ids of a partition live in LDS
  const int32_t np = cap > 0 ? (cap + P - 1) / P : 1;
  const size_t need = pa::decode_workspace_bytes(num_seqs, num_q_heads, dims.head_dim, np, cap);
  if (noalloc) {
    // the library's own scratch array instead of a caller's workspace
    if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
    workspace = nullptr;
    if (need > 0) {
      const pa_status st2 = scratch_address(stream, &workspace);
      if (st2 != PA_OK) return st2;
    }
  } else if (need > 0 && (!workspace || workspace_bytes < need)) {
    return PA_ERR_WORKSPACE;
  }
  const hipError_t e = pa::launch_decode(
      static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(k_cache),
      static_cast<const uint8_t*>(v_cache), block_tables, max_blocks_per_seq, context_lens, num_seqs,
      num_q_heads, cap, scale, static_cast<uint16_t*>(out), dims, cache->k_scale, cache->v_scale, P,
      workspace, stream, with_new ? static_cast<const uint16_t*>(new_k) : nullptr,
      with_new ? static_cast<const uint16_t*>(new_v) : nullptr, with_new ? slot_mapping : nullptr);
  if (e != hipSuccess || !with_new) return hip_status(e);
  // the store of the newest tokens, after the decode that took them from new_k / new_v
  return hip_status(pa::launch_store_kv(static_cast<const uint16_t*>(new_k), static_cast<const uint16_t*>(new_v),
                                        slot_mapping, num_seqs, static_cast<uint8_t*>(const_cast<void*>(k_cache)),
                                        static_cast<uint8_t*>(const_cast<void*>(v_cache)), dims,
                                        cache->k_scale, cache->v_scale, stream));
}

}  // namespace

pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t max_context_len, float scale, void* out,
                    const pa_cache_desc* cache, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                     num_q_heads, max_context_len, scale, out, cache, partition_size, workspace,
                     workspace_bytes, stream, nullptr, nullptr, nullptr, false);
}

pa_status pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t max_context_len, float scale, void* out,
                            const pa_cache_desc* cache, int32_t partition_size, hipStream_t stream) {
  return decode_impl(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                     num_q_heads, max_context_len, scale, out, cache, partition_size, nullptr, 0, stream,
                     nullptr, nullptr, nullptr, false, true);
}

pa_status pa_store_decode(const void* q, const void* new_k, const void* new_v,
                          const int32_t* slot_mapping, void* k_cache, void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                          int32_t max_context_len, float scale, void* out,
                          const pa_cache_desc* cache, int32_t partition_size, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                     num_q_heads, max_context_len, scale, out, cache, partition_size, workspace,
                     workspace_bytes, stream, new_k, new_v, slot_mapping, true);
}

pa_status pa_prefill_varlen(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            int32_t num_seqs, int32_t num_q_heads, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, float scale, void* out,
                            const pa_cache_desc* cache, hipStream_t stream) {
  pa::PoolDims dims;
  const bool packed = block_tables == nullptr;
  if (packed) {
    // packed keys/values: only the head counts, head_dim and dtype of the
    // descriptor are read
    if (!cache) return PA_ERR_NULL;
    if (cache->num_kv_heads <= 0 || cache->head_dim <= 0) return PA_ERR_SHAPE;
    if (cache->head_dim != 64 && cache->head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (cache->num_kv_heads > kMaxKvHeads) return PA_ERR_UNSUPPORTED;
    if (cache->dtype != PA_KV_BF16) return PA_ERR_UNSUPPORTED;
    dims.num_blocks = 0;
    dims.block_size = 0;
    dims.num_kv_heads = cache->num_kv_heads;
    dims.head_dim = cache->head_dim;
    dims.fp8 = false;
  } else {
    pa_status st = check_cache(cache, &dims);
    if (st != PA_OK) return st;
  }
  if (num_seqs < 0 || num_q_heads <= 0 || max_seqlen_q < 0 || max_seqlen_k < 0 ||
      (!packed && max_blocks_per_seq <= 0))
    return PA_ERR_SHAPE;
  if (num_q_heads % dims.num_kv_heads != 0) return PA_ERR_SHAPE;
  if (!supported_group(num_q_heads / dims.num_kv_heads)) return PA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || scale == INFINITY) return PA_ERR_SHAPE;
  if (num_seqs == 0 || max_seqlen_q == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !cu_seqlens_q || !cu_seqlens_k || !out) return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || (!packed && !aligned(block_tables, 4)))
    return PA_ERR_UNSUPPORTED;
  int32_t cap_k = max_seqlen_k;
  if (!packed) {
    const long long cap_ll = (long long)max_blocks_per_seq * dims.block_size;
    cap_k = int32_t(cap_ll < max_seqlen_k ? cap_ll : max_seqlen_k);
  }
  return hip_status(pa::launch_prefill(static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(k_cache),
                                       static_cast<const uint8_t*>(v_cache), cu_seqlens_q, cu_seqlens_k,
                                       block_tables, packed ? 0 : max_blocks_per_seq, num_seqs, num_q_heads,
                                       max_seqlen_q, cap_k, scale, static_cast<uint16_t*>(out), dims,
                                       packed ? nullptr : cache->k_scale, packed ? nullptr : cache->v_scale,
                                       stream));
}

pa_status pa_prefill_set_slots(int32_t slots) {
  pa::set_prefill_slots(slots);
  return PA_OK;
}

pa_status pa_add_rmsnorm(const void* x, const void* residual, const void* weight, int32_t num_tokens,
                         int32_t hidden, float eps, void* out, void* residual_out, hipStream_t stream) {
  if (num_tokens < 0 || hidden <= 0) return PA_ERR_SHAPE;
  if (hidden % 8 != 0 || hidden > 16384) return PA_ERR_UNSUPPORTED;
  if (!(eps > 0.f) || eps == INFINITY) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!x || !weight || !out || (residual && !residual_out)) return PA_ERR_NULL;
  if (residual && residual_out == out) return PA_ERR_SHAPE;
  const void* ptrs[5] = {x, residual, weight, out, residual ? residual_out : nullptr};
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return PA_ERR_UNSUPPORTED;
  return hip_status(pa::launch_add_rmsnorm(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(residual),
      static_cast<const uint16_t*>(weight), static_cast<uint16_t*>(out),
      residual ? static_cast<uint16_t*>(residual_out) : nullptr, num_tokens, hidden, eps, stream));
}

}  // extern "C"
