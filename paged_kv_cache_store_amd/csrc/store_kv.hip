// KV store: scatter new tokens' K/V rows into their block-pool slots.
//
// A slot names a fixed-size block and an offset inside it (blocks hold the KV
// of a fixed number of tokens: "Nano-vLLM：轻量高效的大模型推理框架…", 三.1 推理引擎架构,
// 块管理器). Optional FP8 E4M3 storage halves the pool ("nano-vllm-lite：深入理解
// LLM推理机制的教育级开源项目", 核心技术改进 §3).
//
// A workgroup stores 64 consecutive batch tokens of one KV head. Their K and V
// rows are first copied into LDS with coalesced reads; then a wave takes one
// 16-byte chunk of the pool's K layout at a time (8 bf16 head-dim values for a
// bf16 pool, 16 values for an fp8 one), one token per lane. K chunks are written
// whole, so tokens on consecutive slots (a prefill chunk) fill whole lines
// together. V is transposed in the pool (x consecutive positions per 16-byte
// unit): when x consecutive lanes hold tokens on the x slots of one unit, lane
// j of them writes the whole unit of head-dim (chunk * x + j), read across the
// x tokens' rows in LDS; any other value lands in its own 2-byte (bf16) or
// 1-byte (fp8) position.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kStoreThreads = 256;
constexpr int kStoreTokens = 64;   // tokens per workgroup: one per lane
constexpr int kStoreSmallGrid = 256;   // fewer tile workgroups than this: the chunk kernel

template <int kD, bool kFp8>
__global__ __launch_bounds__(kStoreThreads) void store_kv_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ slots, int num_tokens, int num_kv_heads, int block_size,
    long long num_slots, uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale) {
  constexpr int kX = kFp8 ? 16 : 8;       // elements per 16-byte pool chunk
  constexpr int kEs = kFp8 ? 1 : 2;       // bytes per pool element
  constexpr int kChunks = kD / kX;
  constexpr int kRowVecs = kD / 8;        // 16-byte vectors per bf16 input row
  constexpr int kWaves = kStoreThreads / 64;
  __shared__ __attribute__((aligned(16))) uint16_t k_s[kStoreTokens][kD];
  __shared__ __attribute__((aligned(16))) uint16_t v_s[kStoreTokens][kD];
  __shared__ long long slot_s[kStoreTokens];
  const int h = blockIdx.y;
  const long long t0 = (long long)blockIdx.x * kStoreTokens;
  const int tid = threadIdx.x;

  // ---- rows of the 64 tokens, coalesced: consecutive threads read consecutive
  // 16-byte vectors of a row
  for (int i = tid; i < kStoreTokens * kRowVecs; i += kStoreThreads) {
    const int r = i / kRowVecs, cv = i % kRowVecs;
    if (t0 + r < num_tokens) {
      const long long src = ((t0 + r) * num_kv_heads + h) * kD + cv * 8;
      *reinterpret_cast<uint4*>(&k_s[r][cv * 8]) = *reinterpret_cast<const uint4*>(k + src);
      *reinterpret_cast<uint4*>(&v_s[r][cv * 8]) = *reinterpret_cast<const uint4*>(v + src);
    }
  }
  if (tid < kStoreTokens) {
    long long slot = t0 + tid < num_tokens ? slots[t0 + tid] : -1;
    slot_s[tid] = (slot >= 0 && slot < num_slots) ? slot : -1;
  }
  __syncthreads();

  const int lane = tid % 64;
  const int w = tid / 64;
  const long long slot = slot_s[lane];
  if (slot < 0) return;   // nothing to write for this lane (no barrier follows)
  const int o = int(slot % block_size);
  const long long b = slot / block_size;
  const long long slab = (b * num_kv_heads + h) * (long long)block_size * kD;   // elements
  const int e0 = o % kX;
  const int leader = lane - e0;
  // lanes leader .. leader+x-1 hold the x slots of this lane's V unit, in order
  bool run = leader >= 0 && leader + kX <= kStoreTokens;
  if (run) {
#pragma unroll
    for (int i = 0; i < kX; ++i) run = run && slot_s[leader + i] == slot - e0 + i;
  }
  const long long v_unit = slab + (long long)(o / kX) * kD * kX;   // [b][h][o / x][d][o % x]
  const float ks = kFp8 ? k_scale[h] : 1.f;
  const float vsc = kFp8 ? v_scale[h] : 1.f;

  for (int c = w; c < kChunks; c += kWaves) {
    // K chunk c of this lane's token at [b][h][c][o][:]
    const long long k_dst = slab + ((long long)c * block_size + o) * kX;
    if constexpr (!kFp8) {
      *reinterpret_cast<uint4*>(k_cache + k_dst * kEs) = *reinterpret_cast<const uint4*>(&k_s[lane][c * kX]);
    } else {
      uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        // correctly rounded float32 division (HIP's default for '/')
        const float x = __uint_as_float(uint32_t(k_s[lane][c * kX + e]) << 16);
        out[e >> 2] |= e4m3_encode(x / ks) << (8 * (e & 3));
      }
      *reinterpret_cast<uint4*>(k_cache + k_dst) = make_uint4(out[0], out[1], out[2], out[3]);
    }
    if (run) {
      // head-dim d, positions o-e0 .. o-e0+x-1: the run's x tokens, in order
      const int d = c * kX + e0;
      uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < kX; ++i) {
        const uint32_t bits = v_s[leader + i][d];
        const uint32_t el = kFp8 ? e4m3_encode(__uint_as_float(bits << 16) / vsc) : bits;
        wv[(i * kEs) >> 2] |= el << (8 * ((i * kEs) & 3));
      }
      *reinterpret_cast<uint4*>(v_cache + (v_unit + (long long)d * kX) * kEs) =
          make_uint4(wv[0], wv[1], wv[2], wv[3]);
    } else {
#pragma unroll
      for (int e = 0; e < kX; ++e) {
        const long long el = v_unit + (long long)(c * kX + e) * kX + e0;
        const uint32_t bits = v_s[lane][c * kX + e];
        if constexpr (!kFp8)
          reinterpret_cast<uint16_t*>(v_cache)[el] = uint16_t(bits);
        else
          v_cache[el] = uint8_t(e4m3_encode(__uint_as_float(bits << 16) / vsc));
      }
    }
  }
}

// Small batches (a decode step: one token per sequence) give the tile kernel
// too few workgroups to fill the chip; they take one thread per 16-byte K chunk
// of a (token, head) instead (chunk fastest, so that a wave reads consecutive
// input), with the same V runs for bf16 found by comparing the run's slots.
template <bool kFp8>
__global__ __launch_bounds__(256) void store_kv_chunk_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ slots, int num_tokens, int num_kv_heads, int head_dim,
    int block_size, long long num_slots, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale) {
  constexpr int kX = kFp8 ? 16 : 8;  // elements per 16-byte pool chunk
  const int chunks = head_dim / kX;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)num_tokens * num_kv_heads * chunks;
  if (idx >= total) return;
  const int c = int(idx % chunks);
  const long long th = idx / chunks;
  const int h = int(th % num_kv_heads);
  const long long t = th / num_kv_heads;
  const long long slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const long long b = slot / block_size;
  const int o = int(slot % block_size);
  const long long slab = (b * num_kv_heads + h) * (long long)block_size * head_dim;  // elements
  const long long src = (t * num_kv_heads + h) * head_dim + (long long)c * kX;
  // K: chunk c of this token at [b][h][c][o][:]
  const long long k_dst = slab + ((long long)c * block_size + o) * kX;
  // V: value d at [b][h][o / x][d][o % x]
  const long long v_dst = slab + (long long)(o / kX) * head_dim * kX + (o % kX);
  if constexpr (!kFp8) {
    const uint4 kr = *reinterpret_cast<const uint4*>(k + src);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(k_cache) + k_dst) = kr;
    // V: when this token and the 7 after it in the batch fill one V chunk (8
    // consecutive slots starting at a multiple of 8, as a prefill chunk does),
    // the run's first token writes the 8 chunks of its head-dims whole; the
    // others of the run write nothing. Any other token writes its values one
    // 2-byte position at a time.
    const int e0 = o % kX;
    const long long lead = t - e0;
    bool run = lead >= 0 && lead + kX <= num_tokens;   // wave-uniform: a wave holds one token
    if (run) {
      int sv[kX];   // independent loads, compared afterwards
#pragma unroll
      for (int i = 0; i < kX; ++i) sv[i] = slots[lead + i];
#pragma unroll
      for (int i = 0; i < kX; ++i) run = run && (long long)sv[i] == slot - e0 + i;
    }
    uint16_t* vc = reinterpret_cast<uint16_t*>(v_cache) + v_dst + (long long)c * kX * kX;
    if (run) {
      if (e0 == 0) {
        uint32_t in[kX][4];   // token i of the run: head-dims c*8 .. c*8+7
#pragma unroll
        for (int i = 0; i < kX; ++i) {
          const uint4 r = *reinterpret_cast<const uint4*>(v + src + (long long)i * num_kv_heads * head_dim);
          in[i][0] = r.x; in[i][1] = r.y; in[i][2] = r.z; in[i][3] = r.w;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {          // head-dim c*8 + j: tokens 0..7 of the chunk
          uint32_t w[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t lo = (in[2 * p][j >> 1] >> (16 * (j & 1))) & 0xffffu;
            const uint32_t hi = (in[2 * p + 1][j >> 1] >> (16 * (j & 1))) & 0xffffu;
            w[p] = lo | (hi << 16);
          }
          *reinterpret_cast<uint4*>(vc + j * kX) = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    } else {
      // one 2-byte value per 16-byte unit. Lane c writes head-dims c,
      // c + chunks, ..., c + 7 chunks, so that for each e the lanes of a wave
      // write neighbouring units of the token's rows (a few lines per
      // instruction) instead of one unit in each of 64 lines
      const uint16_t* vt = v + (t * num_kv_heads + h) * head_dim;
      uint16_t* vu = reinterpret_cast<uint16_t*>(v_cache) + v_dst;
      uint16_t val[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) val[e] = vt[c + e * chunks];
#pragma unroll
      for (int e = 0; e < 8; ++e) vu[(long long)(c + e * chunks) * kX] = val[e];
    }
  } else {
    const float ks = k_scale[h];
    const float vs = v_scale[h];
    const uint4* kp = reinterpret_cast<const uint4*>(k + src);
    const uint4* vp = reinterpret_cast<const uint4*>(v + src);
    const uint4 ka = kp[0], kb = kp[1], va = vp[0], vb = vp[1];
    const uint32_t kw[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
    const uint32_t vw[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
    uint32_t kout[4] = {0u, 0u, 0u, 0u};
    uint8_t* vc = v_cache + v_dst + (long long)c * kX * kX;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t kbits = (e & 1) ? (kw[e >> 1] & 0xffff0000u) : (kw[e >> 1] << 16);
      const uint32_t vbits = (e & 1) ? (vw[e >> 1] & 0xffff0000u) : (vw[e >> 1] << 16);
      // correctly rounded float32 division (HIP's default for '/')
      const uint32_t kcode = e4m3_encode(__uint_as_float(kbits) / ks);
      const uint32_t vcode = e4m3_encode(__uint_as_float(vbits) / vs);
      kout[e >> 2] |= kcode << (8 * (e & 3));
      vc[e * kX] = uint8_t(vcode);
    }
    *reinterpret_cast<uint4*>(k_cache + k_dst) = make_uint4(kout[0], kout[1], kout[2], kout[3]);
  }
}

template <bool kFp8>
static void launch_store_d(int D, dim3 grid, hipStream_t stream, const uint16_t* k, const uint16_t* v,
                           const int32_t* slots, int num_tokens, int hkv, int bs, long long num_slots,
                           uint8_t* kc, uint8_t* vc, const float* ks, const float* vs) {
  if (D == 64)
    store_kv_kernel<64, kFp8><<<grid, kStoreThreads, 0, stream>>>(k, v, slots, num_tokens, hkv, bs,
                                                                  num_slots, kc, vc, ks, vs);
  else
    store_kv_kernel<128, kFp8><<<grid, kStoreThreads, 0, stream>>>(k, v, slots, num_tokens, hkv, bs,
                                                                   num_slots, kc, vc, ks, vs);
}

hipError_t launch_store_kv(const uint16_t* k, const uint16_t* v, const int32_t* slots,
                           int num_tokens, uint8_t* k_cache, uint8_t* v_cache,
                           const PoolDims& pool, const float* k_scale, const float* v_scale,
                           hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const dim3 grid(unsigned((num_tokens + kStoreTokens - 1) / kStoreTokens), unsigned(pool.num_kv_heads));
  const long long num_slots = (long long)pool.num_blocks * pool.block_size;
  if ((long long)grid.x * grid.y < kStoreSmallGrid) {
    const int x = pool.fp8 ? 16 : 8;
    const long long total = (long long)num_tokens * pool.num_kv_heads * (pool.head_dim / x);
    const unsigned g = unsigned((total + 255) / 256);
    if (pool.fp8)
      store_kv_chunk_kernel<true><<<g, 256, 0, stream>>>(k, v, slots, num_tokens, pool.num_kv_heads,
                                                         pool.head_dim, pool.block_size, num_slots,
                                                         k_cache, v_cache, k_scale, v_scale);
    else
      store_kv_chunk_kernel<false><<<g, 256, 0, stream>>>(k, v, slots, num_tokens, pool.num_kv_heads,
                                                          pool.head_dim, pool.block_size, num_slots,
                                                          k_cache, v_cache, k_scale, v_scale);
    return hipGetLastError();
  }
  if (pool.fp8)
    launch_store_d<true>(pool.head_dim, grid, stream, k, v, slots, num_tokens, pool.num_kv_heads,
                         pool.block_size, num_slots, k_cache, v_cache, k_scale, v_scale);
  else
    launch_store_d<false>(pool.head_dim, grid, stream, k, v, slots, num_tokens, pool.num_kv_heads,
                          pool.block_size, num_slots, k_cache, v_cache, k_scale, v_scale);
  return hipGetLastError();
}

}  // namespace pa

namespace pa {

// Copy-on-write support: copies whole blocks (all KV heads, K then V) inside a
// pool. Thread = one 16-byte unit of a block's K or V; pairs[i] = {src, dst}.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_cache,
                                                          uint4* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          long long block16) {
  const int p = blockIdx.y;
  const long long src = pairs[2 * p], dst = pairs[2 * p + 1];
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * block16;
       i += (long long)gridDim.x * blockDim.x) {
    uint4* pool = i < block16 ? k_cache : v_cache;
    const long long j = i < block16 ? i : i - block16;
    pool[dst * block16 + j] = pool[src * block16 + j];
  }
}

hipError_t launch_copy_blocks(uint8_t* k_cache, uint8_t* v_cache, const int32_t* pairs, int num_pairs,
                              const PoolDims& pool, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const long long block16 =
      (long long)pool.num_kv_heads * pool.block_size * pool.head_dim * (pool.fp8 ? 1 : 2) / 16;
  const unsigned gx = unsigned((2 * block16 + 255) / 256 < 64 ? (2 * block16 + 255) / 256 : 64);
  copy_blocks_kernel<<<dim3(gx, unsigned(num_pairs)), 256, 0, stream>>>(
      reinterpret_cast<uint4*>(k_cache), reinterpret_cast<uint4*>(v_cache), pairs, block16);
  return hipGetLastError();
}

}  // namespace pa
