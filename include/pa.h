/*
 * pa.h — C ABI of the paged KV-cache attention library (libpa.so, gfx950).
 *
 * The operations come from the pages' description of PagedAttention:
 *  - the KV cache is cut into fixed-size blocks stored non-contiguously in one
 *    pool ("nano-vllm：轻量级大模型推理引擎的技术探索与实践", PagedAttention 原理回顾;
 *    "Nano-vLLM：轻量高效的大模型推理框架…", 三.1 推理引擎架构, 块管理器);
 *  - a per-sequence block table maps logical blocks to physical blocks, and
 *    blocks may be shared within and across requests ("DeepSeek复刻vLLM反超原版：
 *    AI推理新标杆", section vLLM：大模型推理的加速引擎与挑战; prefix caching in
 *    "Nano-vLLM…", 三.2 (1) 前缀缓存);
 *  - attention is exact, memory-efficient ("FlashAttention idea", "Nano-vLLM…",
 *    三.3 模型层适配); decode is bound by KV-cache reads and prefill by compute,
 *    and prefill may come in chunks mixed with decode ("nano-vllm-lite：深入理解
 *    LLM推理机制的教育级开源项目", 核心技术改进 §2 Chunked Prefill);
 *  - the KV cache may be stored as FP8 with 2x compression (same page, §3).
 *
 * Conventions common to every call
 *  - Ownership: the caller owns all memory. Every pointer marked "device" is
 *    device memory on the device that owns `stream`; "host" pointers are read
 *    during the call only. The library allocates nothing, frees nothing and
 *    keeps no pointer after returning.
 *  - Asynchrony: all GPU work is enqueued on `stream`; calls return before it
 *    completes and never synchronise or copy device->host. Host-known bounds
 *    (max_context_len, max_seqlen_q/k) are arguments for that reason.
 *  - Errors: every call checks its host-visible arguments before enqueuing
 *    anything and returns a pa_status; nothing throws or aborts. A failed
 *    launch returns PA_ERR_HIP and pa_last_hip_error() gives the HIP text.
 *    Device-side contents (table entries, slots, lengths) are not validated:
 *    an out-of-range block id read through a table, a slot_mapping with
 *    duplicate slots, or lengths above the stated bounds are undefined
 *    behaviour, except where a call below says otherwise.
 *  - Element types: "bf16" is bfloat16 (2 bytes); "fp8" is OCP FP8 E4M3 with
 *    no infinities (bias 7, largest finite 448, 0x7F/0xFF NaN).
 *
 * KV pool layout (one pool for K, one for V, per layer), x = 16 / element size
 * (8 for bf16, 16 for fp8), token slot s -> block s / block_size, offset
 * o = s % block_size:
 *   K [num_blocks][num_kv_heads][head_dim/x][block_size][x]
 *     element (b, h, o, d) at ((((b*Hkv + h)*(D/x) + d/x)*block_size + o)*x + d%x
 *   V [num_blocks][num_kv_heads][block_size/x][head_dim][x]
 *     element (b, h, o, d) at ((((b*Hkv + h)*(block_size/x) + o/x)*D + d)*x + o%x
 * Each (block, head) slab of block_size*head_dim elements is contiguous. K
 * keeps x consecutive head-dim values of one token in 16 bytes; V keeps x
 * consecutive tokens of one head-dim index in 16 bytes.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                          */
  PA_ERR_SHAPE = -2,       /* sizes are negative or inconsistent                   */
  PA_ERR_UNSUPPORTED = -3, /* head_dim, block_size, group size or dtype not built  */
  PA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required           */
  PA_ERR_HIP = -5,         /* a HIP call failed; see pa_last_hip_error()            */
  PA_ERR_NO_BLOCKS = -6,   /* block manager: the pool cannot hold the request        */
  PA_ERR_NOT_FOUND = -7    /* block manager: unknown sequence id                     */
} pa_status;

typedef enum { PA_KV_BF16 = 0, PA_KV_FP8_E4M3 = 1 } pa_kv_dtype;

/* Alignment, for every call below: device pointers to bf16 / fp8 data (queries,
 * keys, values, outputs, pools, workspace) must be 16-byte aligned and int32
 * arrays 4-byte aligned; anything else is PA_ERR_UNSUPPORTED.
 * Device-side contents are not validated (that would need a host
 * synchronisation): every block-table entry a call reads must lie in
 * [0, num_blocks), and cu_seqlens_q / cu_seqlens_k must be non-decreasing. An
 * entry outside the pool makes the kernel read outside it. Slots outside the
 * pool are the one exception: stores skip them. */

/* One layer's pool. Supported: block_size in {16,32,64,128,256}, head_dim in
 * {64,128}, num_kv_heads at most 1024 (else PA_ERR_UNSUPPORTED). For PA_KV_FP8_E4M3, k_scale/v_scale are device float32 arrays of
 * num_kv_heads dequantisation scales (stored byte b means value(b) * scale[h]);
 * both are ignored (may be NULL) for PA_KV_BF16. */
typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  pa_kv_dtype dtype;
  const float* k_scale;
  const float* v_scale;
} pa_cache_desc;

/* pa_store_kv — write new tokens' keys and values into their cache slots.
 * The slot mapping is the per-token result of the block manager's allocation
 * (blocks hold a fixed number of tokens: "Nano-vLLM…", 三.1, 块管理器).
 *   k, v          device bf16 [num_tokens][num_kv_heads][head_dim], contiguous
 *   slot_mapping  device int32 [num_tokens]; token t goes to slot slot_mapping[t];
 *                 a slot < 0 or >= num_blocks*block_size is skipped (padding)
 *   k_cache, v_cache  device pools in the layout above
 * bf16 pools receive the bf16 bits unchanged. fp8 pools receive the E4M3 code
 * nearest to the float32 quotient value/scale[h] (IEEE correctly-rounded
 * division), ties to even, magnitudes beyond 448 saturated to 448.
 * Only the addressed slots are written. Duplicate slots: one of the writers wins.
 * num_tokens == 0 is a no-op. */
pa_status pa_store_kv(const void* k, const void* v, const int32_t* slot_mapping,
                      int32_t num_tokens, void* k_cache, void* v_cache,
                      const pa_cache_desc* cache, hipStream_t stream);

/* Bytes of device workspace pa_decode needs for these bounds: the split-context
 * partials when a context can span more than one partition, plus, for
 * num_seqs >= 128 with max_context_len > 1024, the order in which the
 * sequences are processed (longest first, ranked on the device by a small
 * kernel launched before the decode). 0 when neither applies. partition_size
 * as in pa_decode. */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t partition_size);

/* Partition size pa_decode uses for these bounds (resolves 0 = automatic: whole
 * contexts when num_seqs*num_q_heads >= 4096, else partitions of up to 2048
 * tokens; never above 4096). */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_context_len, int32_t partition_size);

/* pa_decode — one query token per sequence attends to its sequence's cached
 * keys/values through its block table (PagedAttention, "DeepSeek复刻vLLM…",
 * section vLLM：大模型推理的加速引擎与挑战).
 *   q             device bf16 [num_seqs][num_q_heads][head_dim]
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; entries at or past
 *                 ceil(context_lens[s]/block_size) are never read
 *   context_lens  device int32 [num_seqs]; sequence s attends to logical
 *                 positions 0..context_lens[s]-1 (its newest token included);
 *                 0 gives a zero output row; values are clamped to
 *                 min(max_context_len, max_blocks_per_seq*block_size)
 *   max_context_len  host bound >= every context_lens[s]; sizes the grid
 *   scale         softmax scale (e.g. 1/sqrt(head_dim)), finite (else PA_ERR_SHAPE)
 *   out           device bf16 [num_seqs][num_q_heads][head_dim], fully written
 *   partition_size   0 = automatic, else a multiple of 256 tokens: contexts
 *                 longer than one partition are split and merged by a
 *                 log-sum-exp reduce. A partition's block ids are staged in
 *                 a 256-entry table: partition/block_size > 256 is
 *                 PA_ERR_UNSUPPORTED
 *   workspace     device scratch of at least pa_decode_workspace_size(...) bytes
 *                 (may be NULL when that size is 0); contents on entry ignored.
 *                 With num_seqs >= 128 and contexts possibly longer than 1024
 *                 tokens an extra kernel first ranks the sequences by context
 *                 length into it (longest first), so the launch does not end
 *                 on a tail of long sequences
 * Query head h reads KV head h / (num_q_heads / num_kv_heads); the group size
 * num_q_heads / num_kv_heads must be 1, 2, 4 or 8. Output: softmax(scale*q.k)
 * weighted sum of v, float32 accumulation, rounded to nearest-even bf16. */
pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t max_context_len, float scale, void* out,
                    const pa_cache_desc* cache, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of the device scratch array behind pa_decode_noalloc, per GPU. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* pa_decode_noalloc — pa_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments as pa_decode without the workspace; same kernels,
 * same results bit for bit. The scratch pa_decode would take from the
 * workspace (pa_decode_workspace_size bytes: split-context partials, the
 * sequence order) comes from a device array of PA_NOALLOC_SCRATCH_BYTES
 * (64 MiB) inside the library, one per GPU the library runs on, held until the
 * process ends; a call that would need more returns PA_ERR_WORKSPACE before
 * enqueuing anything. The call allocates nothing. The first call on a device
 * looks up the array's device address (hipGetSymbolAddress) with that device
 * current. Every call on a GPU shares that GPU's array and it keeps the last
 * call's contents: calls that overlap on one GPU (other streams, other
 * threads) race and their results are undefined; calls on one stream are
 * ordered and safe. No scratch byte needs to start at zero: a call writes
 * every scratch byte it reads. */
pa_status pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t max_context_len, float scale, void* out,
                            const pa_cache_desc* cache, int32_t partition_size, hipStream_t stream);

/* pa_store_decode — a decode step: pa_store_kv of each sequence's newest token
 * and pa_decode, in one call (the store and the decode are the two halves of a
 * decode step: "Nano-vLLM…", 三.1 and 三.3).
 *   new_k, new_v  device bf16 [num_seqs][num_kv_heads][head_dim]: sequence s's
 *                 newest token
 *   slot_mapping  device int32 [num_seqs]: its slot; < 0 or >= num_blocks*block_size
 *                 skips the write (as in pa_store_kv)
 *   k_cache, v_cache  read by the decode, then written at those slots
 *   every other argument, the workspace rule and the status codes as in
 *   pa_decode; NULL new_k / new_v / slot_mapping with num_seqs > 0 -> PA_ERR_NULL.
 * Two launches on `stream`: the decode, which takes position
 * context_lens[s]-1 of sequence s from new_k / new_v (in the pool's
 * representation: the bf16 bits, or the fp8 code pa_store_kv would store)
 * when slot_mapping[s] is that position's slot, then the store of the tokens.
 * The decode thus never reads pool lines the step has just written, which is
 * faster than storing first. Result: the pool bytes and the output of
 * pa_store_kv(new_k, new_v, slot_mapping) followed by pa_decode on the same
 * stream, bit for bit, when every written slot is either the slot of position
 * context_lens[s]-1 of its own sequence s (through block_tables) or a slot no
 * sequence reads in this call; otherwise the output is undefined (a block
 * shared by several sequences is copied before it is written into). */
pa_status pa_store_decode(const void* q, const void* new_k, const void* new_v,
                          const int32_t* slot_mapping, void* k_cache, void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                          int32_t max_context_len, float scale, void* out,
                          const pa_cache_desc* cache, int32_t partition_size, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* pa_prefill_varlen — causal attention of packed query chunks over their
 * sequences' keys (cached prefix plus the chunk itself): chunked prefill
 * ("nano-vllm-lite…", 核心技术改进 §2). Two sources of keys/values:
 *  - paged (block_tables != NULL): k_cache, v_cache are the pools, bf16 or fp8,
 *    already holding the chunk's tokens (written by pa_store_kv). An fp8 pool is
 *    read through cache->k_scale / v_scale exactly as pa_decode reads it: each
 *    E4M3 byte widened to bf16 without rounding, k_scale[h] folded into the
 *    softmax scale, v_scale[h] into the output;
 *  - packed (block_tables == NULL): k_cache, v_cache are device bf16
 *    [total_k][num_kv_heads][head_dim], sequence s owning rows
 *    cu_seqlens_k[s] .. cu_seqlens_k[s+1]-1 (a contiguous KV buffer, no pool).
 *    Only cache->num_kv_heads, head_dim and dtype are read; dtype must be
 *    PA_KV_BF16 (else PA_ERR_UNSUPPORTED); max_blocks_per_seq is ignored.
 *   q             device bf16 [total_q][num_q_heads][head_dim]; sequence s owns
 *                 rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1
 *   cu_seqlens_q, cu_seqlens_k  device int32 [num_seqs+1] prefix sums; sequence s
 *                 has Lq = cu_q[s+1]-cu_q[s] queries and Lk = cu_k[s+1]-cu_k[s]
 *                 keys (logical positions 0..Lk-1 of its block table when paged)
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq], or NULL (packed)
 *   max_seqlen_q, max_seqlen_k  host bounds >= every Lq, Lk; Lq is clamped to
 *                 max_seqlen_q and Lk to max_seqlen_k (paged: also to
 *                 max_blocks_per_seq*block_size)
 *   scale         softmax scale, finite and > 0 (else PA_ERR_SHAPE)
 *   out           device bf16 [total_q][num_q_heads][head_dim]
 * Query i of sequence s sits at position Lk-Lq+i and attends to keys 0..Lk-Lq+i
 * (mask aligned bottom-right); a row that sees no key is written as zeros.
 * Packed keys are read only at rows below cu_seqlens_k[s+1]. */
pa_status pa_prefill_varlen(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            int32_t num_seqs, int32_t num_q_heads, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, float scale, void* out,
                            const pa_cache_desc* cache, hipStream_t stream);

/* pa_prefill_set_slots — how many workgroups a pa_prefill_varlen launch over a
 * bf16 pool with blocks of at least 64 tokens keeps resident. That launch is
 * persistent: each workgroup takes a run of work items (sequence, KV head,
 * block of query rows) and starts the next item's copies while it finishes the
 * current one, so the per-item start-up latency (block ids, first K/V tiles,
 * Q rows) is paid once per workgroup instead of once per item (chunked
 * prefill, "nano-vllm-lite…", 核心技术改进 §2: prefill is compute-bound, so
 * the matrix cores are kept busy across items).
 *   slots  0 (the default): two per compute unit, what the kernel's registers
 *          and LDS allow; > 0: that many; < 0: no persistent launch (one
 *          workgroup per work item, the other paths' kernel).
 * The output is the same bit for bit for every setting (each item's tiles are
 * visited in the same order with the same arithmetic). The setting is
 * process-wide, read at each later launch; it is not synchronised with launches
 * on other host threads. Always PA_OK. */
pa_status pa_prefill_set_slots(int32_t slots);

/* pa_add_rmsnorm — residual add fused with RMSNorm in one pass over each row, so
 * the sum is normalised without a round trip through memory ("nano-vllm-lite…",
 * 核心技术改进 §1):
 *     h = x + residual        (residual NULL: h = x, plain RMSNorm)
 *     out = h * weight / sqrt(mean(h^2) + eps),  mean over the hidden dimension
 *   x             device bf16 [num_tokens][hidden], contiguous
 *   residual      device bf16 [num_tokens][hidden], or NULL
 *   weight        device bf16 [hidden]
 *   out           device bf16 [num_tokens][hidden]
 *   residual_out  device bf16 [num_tokens][hidden]: receives h rounded to nearest
 *                 even bf16 (the same bits as rounding the exact sum); required
 *                 when residual is given, ignored otherwise
 *   hidden        a multiple of 8, at most 16384 (else PA_ERR_UNSUPPORTED)
 *   eps           finite and > 0 (else PA_ERR_SHAPE)
 * Float32 arithmetic: h and the sum of squares in float32, out rounded once to
 * nearest-even bf16. In place is allowed: out and residual_out may each be the
 * same pointer as x or residual (every element is read before it is written);
 * out == residual_out is PA_ERR_SHAPE and any other overlap is undefined. All
 * pointers must be 16-byte aligned (else PA_ERR_UNSUPPORTED). num_tokens == 0 is
 * a no-op. */
pa_status pa_add_rmsnorm(const void* x, const void* residual, const void* weight,
                         int32_t num_tokens, int32_t hidden, float eps, void* out,
                         void* residual_out, hipStream_t stream);

/* Static text for a status code; never NULL. */
const char* pa_status_string(pa_status s);

/* Text of the last HIP error seen by a pa_* call on this thread ("" if none). */
const char* pa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
