// Paged decode attention (one query token per sequence) and the log-sum-exp
// reduce that merges context partitions.
//
// PagedAttention reads a sequence's keys/values from non-contiguous fixed-size
// blocks through its block table ("DeepSeek复刻vLLM反超原版：AI推理新标杆", section
// vLLM：大模型推理的加速引擎与挑战); decode is bound by the bandwidth of these
// KV-cache reads ("nano-vllm-lite：深入理解LLM推理机制的教育级开源项目", 核心技术改进
// §2), and the KV may be stored as FP8 (same page, §3). The attention itself is
// exact softmax(scale * q.k) v, computed the memory-efficient way with a running
// maximum and sum ("Nano-vLLM：轻量高效的大模型推理框架…", 三.3 模型层适配).
//
// Work decomposition (CDNA4, wave64):
// * one workgroup of 4 waves per (sequence, KV head, context partition); it
//   serves all G query heads of the KV head, so every K/V byte is read once;
// * a wave takes 64-key tiles of the partition in turn (tile t -> wave t % 4);
// * QK: lane = key. The K layout keeps 8 (bf16) or 16 (fp8) head-dim values of
//   one key in 16 bytes and consecutive keys in consecutive 16-byte slots, so a
//   wave's load of chunk c covers 1 KiB contiguous; the lane's scores of its key
//   for the G query heads come out of v_mfma_f32_4x4x4_16b_bf16 blocks that take
//   its own K registers as they were loaded (the query rows from LDS), with no
//   cross-lane reduction;
// * softmax: per tile, a DPP wave maximum per query head, running max/sum with
//   rescaling (base-2 exponentials, log2(e) folded into the scale);
// * PV: lane = head-dim index. The V layout keeps 8 (bf16) or 16 (fp8)
//   consecutive keys of one head-dim index in 16 bytes; the same 4x4x4 blocks
//   take a lane's V registers as loaded against the tile's bf16 weights (from
//   LDS). (PA_DECODE_MFMA=0 builds the earlier form: v_dot2_f32_bf16 against
//   wave-uniform query pairs and broadcast weights.)
// * the 4 waves' partial (max, sum, output) are merged in LDS; a sequence that
//   fits one partition writes its bf16 output, a longer one writes an
//   unnormalised float32 partial for the reduce kernel.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
#ifndef PA_DECODE_WAVES_PER_EU
#define PA_DECODE_WAVES_PER_EU 0
#endif

// Sequences are taken longest first when there are at least this many (0: never)
// and contexts may be longer than PA_DECODE_ORDER_MIN_CONTEXT tokens
#ifndef PA_DECODE_ORDER_MIN_SEQS
#define PA_DECODE_ORDER_MIN_SEQS 128
#endif
#ifndef PA_DECODE_ORDER_MIN_CONTEXT
#define PA_DECODE_ORDER_MIN_CONTEXT 1024
#endif

// Q.K^T and P.V on the matrix cores (4x4x4 blocks); 0: on the VALU (v_dot2)
#ifndef PA_DECODE_MFMA
#define PA_DECODE_MFMA 1
#endif

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDecodeThreads = PA_DECODE_WAVES * 64;
constexpr int kDecodeWaves = kDecodeThreads / kWave;
constexpr int kTile = 64;            // keys per wave per step
constexpr int kMaxPartBlocks = 256;  // block ids per partition staged in LDS

struct DecodeArgs {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const float* k_scale;
  const float* v_scale;
  uint16_t* out;
  float* part_o;
  float* part_m;
  float* part_l;
  const int32_t* order;    // [num_seqs] sequences longest first, or nullptr (index order)
  int max_blocks_per_seq;
  int num_q_heads;
  int num_kv_heads;
  int block_size;
  int part_size;   // P, multiple of 256
  int num_parts;   // NP = ceil(context cap / P)
  int ctx_cap;     // min(max_context_len, max_blocks_per_seq * block_size)
  float scale_log2;
  // the newest token of each sequence from the caller (nullptr: none, read the pool)
  const uint16_t* new_k;   // [num_seqs][num_kv_heads][D]
  const uint16_t* new_v;
  const int32_t* new_slots;  // [num_seqs]: its slot (the store launched after writes it there)
  long long num_slots;
};

// Inputs that no kernel writes while the decode runs, read through the constant
// address space, so that their uniform loads stay scalar loads.
template <typename T>
using const_as_ptr = const __attribute__((address_space(4))) T*;

template <typename T>
__device__ __forceinline__ const_as_ptr<T> as_constant(const T* p) {
  return (const_as_ptr<T>)p;
}

// The newest token of sequence s, KV head h, taken from the caller's buffer
// (pa_store_decode) instead of the pool. The store of these tokens runs as
// its own launch after the decode, so the decode never reads a pool line the
// step has just written: reading lines written by the store launch right
// before was measured to slow the decode by 6-8 % (Qwen3-8B layer: 628 ->
// 688 us), while the same writes into blocks nobody reads cost nothing, and
// neither does the store launched after the decode (648 us for both).
// The token is kept in LDS in the pool's representation (bf16 bits, or fp8
// codes: the nearest E4M3 code of the correctly rounded quotient value /
// scale, as the store kernel writes them): bytes [0, D·es) hold K,
// [D·es, 2·D·es) hold V, value order. The wave that reads the newest position
// puts it into that tile's registers, so the result is the one the pool will
// hold once the store has run.

// Lanes 0..D/4-1 each load 8 bf16 values (lanes below D/8: K, the rest: V).
template <int kD>
__device__ __forceinline__ uint4 load_new_token(const DecodeArgs& a, int s, int h, int lane) {
  const long long row = ((long long)s * a.num_kv_heads + h) * kD;
  if (lane >= kD / 4) return make_uint4(0, 0, 0, 0);
  const uint16_t* src = lane < kD / 8 ? a.new_k + row + lane * 8 : a.new_v + row + (lane - kD / 8) * 8;
  return *reinterpret_cast<const uint4*>(src);
}

// ... and put them into LDS in the pool's representation.
template <int kD, bool kFp8>
__device__ __forceinline__ void stage_new_token(const DecodeArgs& a, uint4 x, int h, int lane,
                                                uint8_t* tok_s) {
  if (lane >= kD / 4) return;
  if constexpr (!kFp8) {
    reinterpret_cast<uint4*>(tok_s)[lane] = x;
  } else {
    const float sc = lane < kD / 8 ? as_constant(a.k_scale)[h] : as_constant(a.v_scale)[h];
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t bits = (e & 1) ? (xw[e >> 1] & 0xffff0000u) : (xw[e >> 1] << 16);
      out[e >> 2] |= e4m3_encode(__uint_as_float(bits) / sc) << (8 * (e & 3));
    }
    reinterpret_cast<uint2*>(tok_s)[lane] = make_uint2(out[0], out[1]);
  }
}

// Waves per SIMD the compiler must leave room for. The variants that take the
// newest token from the caller need a few more registers than the plain ones
// and would drop to 2 waves; held at 3 they do not spill (fp8 with one query
// head per KV head would). The plain fp8 ones with G <= 4 fit 4 waves; left
// free, the compiler moves their accumulators to AGPRs and runs 3.
constexpr int decode_min_waves(int g, bool fp8, bool with_new) {
  return PA_DECODE_WAVES_PER_EU ? PA_DECODE_WAVES_PER_EU
         : fp8 && !with_new && g <= 4 && PA_DECODE_MFMA ? 4
         : (with_new && g < 8 && !(fp8 && g == 1) ? 3 : 1);
}

// kNew: sequence s's position context_lens[s]-1 is read from new_k / new_v
// (when new_slots[s] is that position's slot) instead of from the pool.
template <int kD, int kG, bool kFp8, bool kNew>
__global__ __launch_bounds__(kDecodeThreads)
__attribute__((amdgpu_waves_per_eu(decode_min_waves(kG, kFp8, kNew))))
void decode_kernel(const DecodeArgs a) {
  constexpr int kX = kFp8 ? 16 : 8;       // elements per 16-byte chunk
  constexpr int kKC = kD / kX;            // K chunks per key
  constexpr int kVC = kTile / kX;         // V key-chunks per tile
  constexpr int kDL = kD / kWave;         // head-dim values per lane in PV
  constexpr int kQW = kD / 2;             // query dwords (bf16 pairs) per head
  constexpr int kPW = kX / 2;             // weight dwords per V key-chunk
  // kVM: both products on v_mfma_f32_4x4x4_16b_bf16 (16 independent 4x4x4
  // blocks per instruction; in block b = lane/4, lane l holds row l%4 of A,
  // column l%4 of B and of the result), with the K and V registers used as
  // loaded.
  // * S = Q K^T, four head-dims per step: rows = the query heads, columns =
  //   the block's four keys. Lane l's B operand is its own key's K at those
  //   head-dims, its A operand head l%4's query there (from LDS), and its
  //   result the scores of its key for heads 0..3, the layout of the VALU form.
  // * O^T += V^T P^T, four keys per step: rows = head-dims 4b..4b+3 (+ 64 dl),
  //   columns = the query heads. Lane l's A operand is its own head-dim's V at
  //   those keys, its B operand head l%4's weights there, and its accumulator
  //   holds head l%4 at head-dims 4*(l/4)..+3.
  // The query heads go four to a set of rows/columns (G = 8: two sets); with
  // G < 4 the padding rows/columns repeat the last head and are never read.
  constexpr bool kVM = PA_DECODE_MFMA;
  constexpr int kHS = kG > 4 ? kG / 4 : 1;   // sets of four query heads
  constexpr int kKStep = kX / 4;             // 4x4x4 steps per 16-byte K chunk or V unit

  __shared__ int blk_s[kMaxPartBlocks];
  __shared__ __attribute__((aligned(16))) uint16_t p_s[kDecodeWaves][kG][kTile];
  __shared__ float m_s[kDecodeWaves][kG];
  __shared__ float l_s[kDecodeWaves][kG];
  __shared__ float o_s[kDecodeWaves][kG][kD];
  // kVM: the G query heads of this KV head (bf16), the A operands of S = Q K^T
  __shared__ __attribute__((aligned(16))) uint16_t q_s[kVM ? kG : 1][kVM ? kD : 8];

  const int Hkv = a.num_kv_heads;
  const int bid = blockIdx.x;
  const int h = bid % Hkv;  // KV head varies fastest: consecutive workgroups go to different XCDs
  const int rest = bid / Hkv;
  const int part = rest % a.num_parts;
  const int s = a.order ? as_constant(a.order)[rest / a.num_parts] : rest / a.num_parts;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave index, uniform
  const int lane = tid % kWave;
  const int bs = a.block_size;
  const int P = a.part_size;

  int n = as_constant(a.context_lens)[s];   // scalar load: the tile loop's bounds stay uniform
  n = n < a.ctx_cap ? n : a.ctx_cap;
  const int p0 = part * P;
  // kNew: the newest token (position n-1) is loaded by the one wave that reads
  // that position, the wave given the partition's tile holding n-1.
  __shared__ __attribute__((aligned(16))) uint8_t tok_s[kNew ? 2 * kD * (kFp8 ? 1 : 2) : 16];
  const int t_new = n > 0 ? (n - 1 - p0) / kTile : -1;   // this partition's tile holding n-1
  long long slot_new = -1;
  uint4 tok = make_uint4(0, 0, 0, 0);
  if constexpr (kNew) {
    if (n > 0 && part == (n - 1) / P && t_new % kDecodeWaves == w) {
      slot_new = as_constant(a.new_slots)[s];
      if (slot_new >= a.num_slots) slot_new = -1;
    }
    if (slot_new >= 0) tok = load_new_token<kD>(a, s, h, lane);
  }
  if (n <= 0) {
    if (part == 0) {
      for (int i = tid; i < kG * kD; i += kDecodeThreads)
        a.out[((long long)s * a.num_q_heads + h * kG) * kD + i] = 0;
    }
    return;
  }
  if (p0 >= n) return;
  const int pend = min(p0 + P, n);
  const int nsplit = (n + P - 1) / P;

  // physical block ids of this partition
  const int nb = (pend - p0 + bs - 1) / bs;
  const int* bt = a.block_tables + (long long)s * a.max_blocks_per_seq + p0 / bs;
  // kVM: wave 0 stages the query heads in LDS, its load beside the table's
  constexpr int kQ16 = kG * kD / 8;   // 16-byte pieces of the G query rows
  constexpr int kQL = (kQ16 + kWave - 1) / kWave;
  static_assert(kQL <= 2 && (kQ16 % kWave == 0 || kQL == 1), "query staging");
  uint4 qv0 = make_uint4(0, 0, 0, 0), qv1 = qv0;
  const bool qload = kVM && w == 0 && (kQ16 % kWave == 0 || lane < kQ16 % kWave);
  if (qload) {
    const uint4* qsrc = reinterpret_cast<const uint4*>(a.q + ((long long)s * a.num_q_heads + h * kG) * kD);
    qv0 = qsrc[lane];
    if (kQL > 1) qv1 = qsrc[lane + kWave];
  }
  for (int i = tid; i < nb; i += kDecodeThreads) blk_s[i] = bt[i];
  if (qload) {
    reinterpret_cast<uint4*>(&q_s[0][0])[lane] = qv0;
    if (kQL > 1) reinterpret_cast<uint4*>(&q_s[0][0])[lane + kWave] = qv1;
  }
  if (kNew && slot_new >= 0) stage_new_token<kD, kFp8>(a, tok, h, lane, tok_s);
  // (the barrier that publishes blk_s, q_s and tok_s comes after the first
  // tile's loads are issued, below)

  const auto qg = as_constant(
      reinterpret_cast<const uint32_t*>(a.q + ((long long)s * a.num_q_heads + h * kG) * kD));
  const float sc = kFp8 ? a.scale_log2 * as_constant(a.k_scale)[h] : a.scale_log2;
  const long long slab16 = (long long)bs * kD * (kFp8 ? 1 : 2) / 16;  // 16-byte units per (block, head)
  const uint4* kbase = reinterpret_cast<const uint4*>(a.k_cache) + (long long)h * slab16;
  const uint4* vbase = reinterpret_cast<const uint4*>(a.v_cache) + (long long)h * slab16;
  const long long blk_stride16 = (long long)Hkv * slab16;

  float m[kG], l[kG], acc[kVM ? 1 : kG][kDL];
  f32x4_t acc4[kHS][kDL];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < kDL; ++j) {
#pragma unroll
    for (int g = 0; g < (kVM ? 1 : kG); ++g) acc[g][j] = 0.f;
#pragma unroll
    for (int hs = 0; hs < kHS; ++hs) acc4[hs][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int hcol = lane & 3;   // kVM: this lane's query head in the 4x4 blocks (of each set)
  auto head_of = [&](int hs) { return hs * 4 + hcol < kG ? hs * 4 + hcol : kG - 1; };

  const int ntiles = (pend - p0 + kTile - 1) / kTile;

  // ---- loads of one tile: K with lane = key, V with lane = head-dim index.
  // Streaming, read-once data: non-temporal loads.
  // id >= 0: the tile lies in one block, whose id is given (not read from blk_s)
  auto load_k = [&](int t, uint4 (&kr)[kKC], int id = -1) {
    const int key0 = p0 + t * kTile;
    const int key = key0 + lane;
    const int rel = (key < pend ? key : pend - 1) - p0;
    const uint4* kp = kbase + (id >= 0 ? id : blk_s[rel / bs]) * blk_stride16 + (rel % bs);
#pragma unroll
    for (int c = 0; c < kKC; ++c) kr[c] = load_nt(kp + (long long)c * bs);
  };
  auto load_v = [&](int t, uint4 (&vr)[kVC][kDL], int id = -1) {
    const int key0 = p0 + t * kTile;
#pragma unroll
    for (int j = 0; j < kVC; ++j) {
      int kk = key0 + j * kX;
      if (kk >= pend) kk = (pend - 1) & ~(kX - 1);  // stay inside written blocks; result unused
      const int vrel = kk - p0;
      const uint4* vp = vbase + (id >= 0 ? id : blk_s[vrel / bs]) * blk_stride16 +
                        (long long)((vrel % bs) / kX) * kD;
#pragma unroll
      for (int dl = 0; dl < kDL; ++dl) vr[j][dl] = load_nt(vp + lane + dl * kWave);
    }
  };
  auto load_tile = [&](int t, uint4 (&kr)[kKC], uint4 (&vr)[kVC][kDL]) {
    load_k(t, kr);
    load_v(t, vr);
  };

  auto qk_tile = [&](int t, const uint4 (&kr)[kKC]) {
    const int key0 = p0 + t * kTile;
    const bool valid = key0 + lane < pend;
    // ---- scores
    float sv[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) sv[g] = 0.f;
    if constexpr (kVM) {
      f32x4_t sacc[kHS];
#pragma unroll
      for (int hs = 0; hs < kHS; ++hs) sacc[hs] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kKC; ++c) {
        const uint32_t kw[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
        uint32_t kb[2 * kKStep];   // the chunk's kX head-dims as bf16 pairs
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (kFp8) {
            kb[2 * i] = fp8x2_to_bf16x2<false>(kw[i]);
            kb[2 * i + 1] = fp8x2_to_bf16x2<true>(kw[i]);
          } else {
            kb[i] = kw[i];
          }
        }
#pragma unroll
        for (int hs = 0; hs < kHS; ++hs) {
          const uint4* qrow = reinterpret_cast<const uint4*>(&q_s[head_of(hs)][c * kX]);
          uint32_t qw[2 * kKStep];
#pragma unroll
          for (int u = 0; u < kKStep / 2; ++u) {
            const uint4 q4 = qrow[u];
            qw[4 * u] = q4.x; qw[4 * u + 1] = q4.y; qw[4 * u + 2] = q4.z; qw[4 * u + 3] = q4.w;
          }
#pragma unroll
          for (int i = 0; i < kKStep; ++i) {   // head-dims kX*c + 4i .. +3
            const uint2 av = make_uint2(qw[2 * i], qw[2 * i + 1]);
            const uint2 bv = make_uint2(kb[2 * i], kb[2 * i + 1]);
            sacc[hs] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(bf16x4_t, av),
                                                             __builtin_bit_cast(bf16x4_t, bv), sacc[hs], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < kG; ++g) sv[g] = sacc[g / 4][g % 4];
    } else if constexpr (kG >= 2) {
      // One query head at a time. The G heads' 64*G query dwords do not fit in
      // a wave's SGPRs; held for the whole loop they are spilled to VGPR lanes
      // and read back every tile (one v_readlane each). Here a head's dwords
      // are loaded (scalar, from the scalar cache) only after the previous
      // head's score is known: the address passes through an empty asm that
      // takes that score, so the loads can neither leave the loop nor all
      // start at once. (The asm has to sit in control flow the compiler knows
      // to be uniform, hence the scalar loads of n and of the newest slot.)
      uint64_t qa = reinterpret_cast<uint64_t>(qg);
      int dep = 0;
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        asm volatile("" : "+s"(qa) : "s"(dep));
        const auto qh = reinterpret_cast<const_as_ptr<uint32_t>>(qa) + g * kQW;
#pragma unroll
        for (int c = 0; c < kKC; ++c) {
          const uint32_t kw[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (!kFp8) {
              sv[g] = dot2_bf16(kw[i], qh[c * 4 + i], sv[g]);
            } else {
              sv[g] = dot2_bf16(fp8x2_to_bf16x2<false>(kw[i]), qh[c * 8 + 2 * i], sv[g]);
              sv[g] = dot2_bf16(fp8x2_to_bf16x2<true>(kw[i]), qh[c * 8 + 2 * i + 1], sv[g]);
            }
          }
        }
        dep = __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sv[g]));
      }
    } else
#pragma unroll
    for (int c = 0; c < kKC; ++c) {
      const uint32_t kw[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (!kFp8) {
#pragma unroll
          for (int g = 0; g < kG; ++g) sv[g] = dot2_bf16(kw[i], qg[g * kQW + c * 4 + i], sv[g]);
        } else {
          const uint32_t lo = fp8x2_to_bf16x2<false>(kw[i]);
          const uint32_t hi = fp8x2_to_bf16x2<true>(kw[i]);
#pragma unroll
          for (int g = 0; g < kG; ++g) {
            sv[g] = dot2_bf16(lo, qg[g * kQW + c * 8 + 2 * i], sv[g]);
            sv[g] = dot2_bf16(hi, qg[g * kQW + c * 8 + 2 * i + 1], sv[g]);
          }
        }
      }
    }
    // ---- online softmax (base 2)
    float alpha_col[kHS];   // kVM: the factor of this lane's column (of each set)
#pragma unroll
    for (int hs = 0; hs < kHS; ++hs) alpha_col[hs] = 1.f;
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      const float x = valid ? sv[g] * sc : -INFINITY;
      const float mn = fmaxf(m[g], wave_max(x));
      const float alpha = fast_exp2(m[g] - mn);
      const uint32_t pb = f32_to_bf16(fast_exp2(x - mn));
      l[g] = l[g] * alpha + bf16_lo(pb);
      if constexpr (kVM) {
        alpha_col[g / 4] = hcol == g % 4 ? alpha : alpha_col[g / 4];
      } else {
#pragma unroll
        for (int dl = 0; dl < kDL; ++dl) acc[g][dl] *= alpha;
      }
      m[g] = mn;
      p_s[w][g][lane] = uint16_t(pb);
    }
    if constexpr (kVM) {
#pragma unroll
      for (int hs = 0; hs < kHS; ++hs)
#pragma unroll
        for (int dl = 0; dl < kDL; ++dl) acc4[hs][dl] *= alpha_col[hs];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto pv_tile = [&](int t, const uint4 (&vr)[kVC][kDL]) {
    const int key0 = p0 + t * kTile;
#pragma unroll
    for (int j = 0; j < kVC; ++j) {
      const int kk = key0 + j * kX;
      if (kk >= pend) break;
      const int nv = pend - kk;
      if constexpr (kVM) {
        // the chunk's kX keys of each head-dim this lane holds, as bf16 pairs
        // (the values past the context's end zeroed: their weights are 0, but
        // a NaN would poison 0 * v)
        uint32_t vb[kDL][2 * kKStep];
#pragma unroll
        for (int dl = 0; dl < kDL; ++dl) {
          uint32_t vw[4] = {vr[j][dl].x, vr[j][dl].y, vr[j][dl].z, vr[j][dl].w};
          if (nv < kX) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              uint32_t mask = 0;
              if constexpr (!kFp8) {
                mask = (2 * i < nv ? 0x0000ffffu : 0u) | (2 * i + 1 < nv ? 0xffff0000u : 0u);
              } else {
#pragma unroll
                for (int b = 0; b < 4; ++b) mask |= (4 * i + b < nv) ? (0xffu << (8 * b)) : 0u;
              }
              vw[i] &= mask;
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (kFp8) {
              vb[dl][2 * i] = fp8x2_to_bf16x2<false>(vw[i]);
              vb[dl][2 * i + 1] = fp8x2_to_bf16x2<true>(vw[i]);
            } else {
              vb[dl][i] = vw[i];
            }
          }
        }
#pragma unroll
        for (int hs = 0; hs < kHS; ++hs) {
          // head head_of(hs)'s weights of the chunk's keys (B operands, four keys each)
          const uint4* pp = reinterpret_cast<const uint4*>(&p_s[w][head_of(hs)][j * kX]);
          uint32_t pq[2 * kKStep];
#pragma unroll
          for (int u = 0; u < kKStep / 2; ++u) {
            const uint4 p4 = pp[u];
            pq[4 * u] = p4.x; pq[4 * u + 1] = p4.y; pq[4 * u + 2] = p4.z; pq[4 * u + 3] = p4.w;
          }
#pragma unroll
          for (int dl = 0; dl < kDL; ++dl)
#pragma unroll
            for (int i = 0; i < kKStep; ++i) {
              const uint2 av = make_uint2(vb[dl][2 * i], vb[dl][2 * i + 1]);
              const uint2 bv = make_uint2(pq[2 * i], pq[2 * i + 1]);
              acc4[hs][dl] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
                  __builtin_bit_cast(bf16x4_t, av), __builtin_bit_cast(bf16x4_t, bv), acc4[hs][dl], 0, 0, 0);
            }
        }
        continue;
      }
      uint32_t pw[kG][kPW];
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        const uint4* pp = reinterpret_cast<const uint4*>(&p_s[w][g][j * kX]);
#pragma unroll
        for (int u = 0; u < kPW / 4; ++u) {
          const uint4 t4 = pp[u];
          pw[g][4 * u + 0] = t4.x;
          pw[g][4 * u + 1] = t4.y;
          pw[g][4 * u + 2] = t4.z;
          pw[g][4 * u + 3] = t4.w;
        }
      }
#pragma unroll
      for (int dl = 0; dl < kDL; ++dl) {
        uint32_t vw[4] = {vr[j][dl].x, vr[j][dl].y, vr[j][dl].z, vr[j][dl].w};
        if (nv < kX) {  // last chunk of the context: zero the values past its end
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t mask = 0;
            if constexpr (!kFp8) {
              mask = (2 * i < nv ? 0x0000ffffu : 0u) | (2 * i + 1 < nv ? 0xffff0000u : 0u);
            } else {
#pragma unroll
              for (int b = 0; b < 4; ++b) mask |= (4 * i + b < nv) ? (0xffu << (8 * b)) : 0u;
            }
            vw[i] &= mask;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (!kFp8) {
#pragma unroll
            for (int g = 0; g < kG; ++g) acc[g][dl] = dot2_bf16(vw[i], pw[g][i], acc[g][dl]);
          } else {
            const uint32_t lo = fp8x2_to_bf16x2<false>(vw[i]);
            const uint32_t hi = fp8x2_to_bf16x2<true>(vw[i]);
#pragma unroll
            for (int g = 0; g < kG; ++g) {
              acc[g][dl] = dot2_bf16(lo, pw[g][2 * i], acc[g][dl]);
              acc[g][dl] = dot2_bf16(hi, pw[g][2 * i + 1], acc[g][dl]);
            }
          }
        }
      }
    }
    // the next tile's weights overwrite p_s: finish this tile's reads first
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto compute_tile = [&](int t, const uint4 (&kr)[kKC], const uint4 (&vr)[kVC][kDL]) {
    qk_tile(t, kr);
    pv_tile(t, vr);
  };

  // The wave holding the newest token takes the tile with position n-1 (the
  // partition's last) after its other tiles. When the token's slot is that
  // position's slot, the wave puts the token into the tile's registers as the
  // pool will hold it after the store; any other slot is not read by this
  // sequence (the store launched after the decode writes it), so the tile is
  // read from the pool as it is.
  const bool has_new = kNew && slot_new >= 0;
  const int t_end = has_new ? t_new : ntiles;
  // This wave's first tile is loaded before the barrier that publishes blk_s:
  // with blocks of at least one tile it lies in one block, whose id is read
  // straight from the table (a scalar load), so the K/V loads need not wait
  // for the table to pass through LDS (measured 0.5-1.7 %).
  const bool early = bs >= kTile && w < t_end;
  uint4 kr0[kKC], vr0[kVC][kDL];
  if (early) {
    const int id = as_constant(bt)[(w * kTile) / bs];
    load_k(w, kr0, id);
    load_v(w, vr0, id);
  }
  if (kDecodeWaves > 1) __syncthreads();
  int t0 = w;
  if (early) {
    compute_tile(w, kr0, vr0);
    t0 += kDecodeWaves;
  }
  for (int t = t0; t < t_end; t += kDecodeWaves) {
    uint4 kr[kKC], vr[kVC][kDL];
    load_tile(t, kr, vr);
    compute_tile(t, kr, vr);
  }
  if constexpr (kNew) {
    if (has_new) {
      const int r = n - 1 - (p0 + t_new * kTile);     // the token's key index in the tile
      // uniform by construction; read as a scalar so that the branches below
      // stay uniform for the compiler
      const long long own = (long long)__builtin_amdgcn_readfirstlane(blk_s[(n - 1 - p0) / bs]) * bs + (n - 1) % bs;
      if (own != slot_new) {
        uint4 kr[kKC], vr[kVC][kDL];
        load_tile(t_new, kr, vr);
        compute_tile(t_new, kr, vr);
      } else {
        // K and V one after the other, so the tile holds no more registers
        // than an ordinary one while the token is put in
        {
          uint4 kr[kKC];
          load_k(t_new, kr);
          const uint4* tk = reinterpret_cast<const uint4*>(tok_s);
#pragma unroll
          for (int c = 0; c < kKC; ++c) {
            const uint4 nk = tk[c];
            if (lane == r) kr[c] = nk;
          }
          qk_tile(t_new, kr);
        }
        // V: element r % x of the 16-byte unit of key-chunk r / x, for each d
        uint4 vr[kVC][kDL];
        load_v(t_new, vr);
        constexpr int kEs = kFp8 ? 1 : 2;
        const int jr = r / kX;
        const int dw = (r % kX) * kEs / 4;
        const int sh = ((r % kX) * kEs % 4) * 8;
        const uint32_t keep = ~((kFp8 ? 0xffu : 0xffffu) << sh);
#pragma unroll
        for (int dl = 0; dl < kDL; ++dl) {
          const int d = lane + dl * kWave;
          const uint32_t nv = (kFp8 ? uint32_t(tok_s[kD + d])
                                    : uint32_t(reinterpret_cast<const uint16_t*>(tok_s + 2 * kD)[d])) << sh;
#pragma unroll
          for (int j = 0; j < kVC; ++j) {
            if (j == jr) {
              uint4& u = vr[j][dl];
              u.x = dw == 0 ? (u.x & keep) | nv : u.x;
              u.y = dw == 1 ? (u.y & keep) | nv : u.y;
              u.z = dw == 2 ? (u.z & keep) | nv : u.z;
              u.w = dw == 3 ? (u.w & keep) | nv : u.w;
            }
          }
        }
        pv_tile(t_new, vr);
      }
    }
  }

  // ---- merge the waves
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const float lw = wave_sum(l[g]);
    if (lane == 0) {
      m_s[w][g] = m[g];
      l_s[w][g] = lw;
    }
    if constexpr (!kVM) {
#pragma unroll
      for (int dl = 0; dl < kDL; ++dl) o_s[w][g][lane + dl * kWave] = acc[g][dl];
    }
  }
  if constexpr (kVM) {
#pragma unroll
    for (int hs = 0; hs < kHS; ++hs) {
      if (hs * 4 + hcol < kG) {
#pragma unroll
        for (int dl = 0; dl < kDL; ++dl)
#pragma unroll
          for (int i = 0; i < 4; ++i) o_s[w][hs * 4 + hcol][dl * kWave + (lane & ~3) + i] = acc4[hs][dl][i];
      }
    }
  }
  __syncthreads();
  const float vsc = kFp8 ? as_constant(a.v_scale)[h] : 1.f;
  for (int i = tid; i < kG * kD; i += kDecodeThreads) {
    const int g = i / kD;
    const int d = i % kD;
    float M = m_s[0][g];
#pragma unroll
    for (int ww = 1; ww < kDecodeWaves; ++ww) M = fmaxf(M, m_s[ww][g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecodeWaves; ++ww) {
      const float e = fast_exp2(m_s[ww][g] - M);
      L += l_s[ww][g] * e;
      O += o_s[ww][g][d] * e;
    }
    const long long row = (long long)s * a.num_q_heads + h * kG + g;
    if (nsplit == 1) {
      a.out[row * kD + d] = uint16_t(f32_to_bf16(O / L * vsc));
    } else {
      const long long pr = row * a.num_parts + part;
      a.part_o[pr * kD + d] = O * vsc;
      if (d == 0) {
        a.part_m[pr] = M;
        a.part_l[pr] = L;
      }
    }
  }
}

// Log-sum-exp merge of a sequence's partitions: with per-partition maxima m_p
// (log2 units), weight sums l_p and unnormalised outputs o_p,
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// One wave per (sequence, query head); sequences with one partition were
// finished by the decode kernel.
template <int kD>
__global__ __launch_bounds__(kWave) void decode_reduce_kernel(
    const int32_t* __restrict__ context_lens, int ctx_cap, int part_size, int num_parts,
    int num_q_heads, const float* __restrict__ part_o, const float* __restrict__ part_m,
    const float* __restrict__ part_l, uint16_t* __restrict__ out) {
  constexpr int kDL = kD / kWave;
  const int s = blockIdx.x / num_q_heads;
  const int hq = blockIdx.x % num_q_heads;
  int n = context_lens[s];
  n = n < ctx_cap ? n : ctx_cap;
  const int nsplit = (n + part_size - 1) / part_size;
  if (nsplit <= 1) return;
  const long long base = ((long long)s * num_q_heads + hq) * num_parts;
  float M = -INFINITY;
  for (int p = 0; p < nsplit; ++p) M = fmaxf(M, part_m[base + p]);
  float L = 0.f, O[kDL];
#pragma unroll
  for (int dl = 0; dl < kDL; ++dl) O[dl] = 0.f;
  for (int p = 0; p < nsplit; ++p) {
    const float e = fast_exp2(part_m[base + p] - M);
    L += part_l[base + p] * e;
#pragma unroll
    for (int dl = 0; dl < kDL; ++dl) O[dl] += part_o[(base + p) * kD + threadIdx.x + dl * kWave] * e;
  }
  const long long row = (long long)s * num_q_heads + hq;
#pragma unroll
  for (int dl = 0; dl < kDL; ++dl)
    out[row * kD + threadIdx.x + dl * kWave] = uint16_t(f32_to_bf16(O[dl] / L));
}

// Longest sequences first. Workgroups are dispatched in grid order; with the
// sequences in batch order the last ones to start are as long as any, and the
// launch ends with a tail of long workgroups on a mostly idle chip. Taken
// longest first, the tail is made of the shortest ones (measured: Qwen3-8B
// layer 631 -> 621 us, mixed-step decode 187 -> 181 us, its fp8 form 111 ->
// 98 us). One workgroup ranks the sequences by their number of 64-key tiles (a
// counting sort over 1024 buckets; longer contexts share the top bucket):
// order[rank] = sequence. Sequences of one bucket land in any order; each
// sequence's result does not depend on which workgroup computes it. The
// ranking launch takes ~5 us, more than the tail costs when contexts are short
// (Qwen3-0.6B layer, contexts up to 1024: no gain), so it runs only for many
// sequences whose contexts may be longer than that.
constexpr int kOrderBuckets = 1024;
constexpr int kOrderThreads = 1024;   // one bucket per thread
constexpr int kOrderKeep = 4;         // bucket keys of up to 4096 sequences kept in registers

bool decode_orders_sequences(int num_seqs, int ctx_cap) {
  return PA_DECODE_ORDER_MIN_SEQS > 0 && num_seqs >= PA_DECODE_ORDER_MIN_SEQS &&
         ctx_cap > PA_DECODE_ORDER_MIN_CONTEXT;
}

__global__ __launch_bounds__(kOrderThreads) void decode_order_kernel(const int32_t* __restrict__ context_lens,
                                                                     int num_seqs, int ctx_cap,
                                                                     int32_t* __restrict__ order) {
  __shared__ int cnt[kOrderBuckets];
  __shared__ int wsum[kOrderThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = tid / kWave;
  auto bucket = [&](int s) {
    int n = context_lens[s];
    n = n < ctx_cap ? n : ctx_cap;
    n = n > 0 ? n : 0;
    const int t = (n + kTile - 1) / kTile;
    return kOrderBuckets - 1 - (t < kOrderBuckets - 1 ? t : kOrderBuckets - 1);   // longest first
  };
  cnt[tid] = 0;
  int key[kOrderKeep];
#pragma unroll
  for (int k = 0; k < kOrderKeep; ++k) {
    const int s = tid + k * kOrderThreads;
    key[k] = s < num_seqs ? bucket(s) : -1;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kOrderKeep; ++k)
    if (key[k] >= 0) atomicAdd(&cnt[key[k]], 1);
  for (int s = tid + kOrderKeep * kOrderThreads; s < num_seqs; s += kOrderThreads) atomicAdd(&cnt[bucket(s)], 1);
  __syncthreads();
  // exclusive prefix sum of the bucket counts: inclusive scan inside each wave,
  // then the waves' totals
  const int c = cnt[tid];
  int x = c;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) wsum[wv] = x;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < wv; ++i) base += wsum[i];
  cnt[tid] = base + x - c;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kOrderKeep; ++k)
    if (key[k] >= 0) order[atomicAdd(&cnt[key[k]], 1)] = tid + k * kOrderThreads;
  for (int s = tid + kOrderKeep * kOrderThreads; s < num_seqs; s += kOrderThreads)
    order[atomicAdd(&cnt[bucket(s)], 1)] = s;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t decode_workspace_bytes(int num_seqs, int num_q_heads, int head_dim, int num_parts, int ctx_cap) {
  const size_t rows = (size_t)num_seqs * num_q_heads * num_parts;
  const size_t parts = num_parts > 1 ? align256(rows * ((size_t)head_dim + 2) * sizeof(float)) : 0;
  const size_t ord = decode_orders_sequences(num_seqs, ctx_cap) ? align256((size_t)num_seqs * sizeof(int32_t)) : 0;
  return parts + ord;
}

template <int kD, int kG, bool kFp8>
static void launch_decode_t(const DecodeArgs& a, unsigned grid, hipStream_t stream) {
  if (a.new_slots)
    decode_kernel<kD, kG, kFp8, true><<<grid, kDecodeThreads, 0, stream>>>(a);
  else
    decode_kernel<kD, kG, kFp8, false><<<grid, kDecodeThreads, 0, stream>>>(a);
}

template <int kD, bool kFp8>
static bool launch_decode_g(int G, const DecodeArgs& a, unsigned grid, hipStream_t stream) {
  switch (G) {
    case 1: launch_decode_t<kD, 1, kFp8>(a, grid, stream); return true;
    case 2: launch_decode_t<kD, 2, kFp8>(a, grid, stream); return true;
    case 4: launch_decode_t<kD, 4, kFp8>(a, grid, stream); return true;
    case 8: launch_decode_t<kD, 8, kFp8>(a, grid, stream); return true;
    default: return false;
  }
}

hipError_t launch_decode(const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int num_q_heads,
                         int max_context_len, float scale, uint16_t* out, const PoolDims& pool,
                         const float* k_scale, const float* v_scale, int partition_size,
                         void* workspace, hipStream_t stream, const uint16_t* new_k,
                         const uint16_t* new_v, const int32_t* new_slots) {
  if (num_seqs == 0) return hipSuccess;
  const int D = pool.head_dim;
  const int G = num_q_heads / pool.num_kv_heads;
  const long long cap_ll = (long long)max_blocks_per_seq * pool.block_size;
  const int ctx_cap = int(cap_ll < max_context_len ? cap_ll : max_context_len);
  const int P = partition_size;
  const int NP = ctx_cap > 0 ? (ctx_cap + P - 1) / P : 1;
  DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.out = out;
  // workspace: the partials (split contexts), then the sequence order
  const size_t rows = (size_t)num_seqs * num_q_heads * NP;
  float* ws = static_cast<float*>(workspace);
  a.part_o = NP > 1 ? ws : nullptr;
  a.part_m = NP > 1 ? ws + rows * D : nullptr;
  a.part_l = NP > 1 ? ws + rows * (D + 1) : nullptr;
  const size_t part_bytes = NP > 1 ? align256(rows * ((size_t)D + 2) * sizeof(float)) : 0;
  int32_t* order = decode_orders_sequences(num_seqs, ctx_cap)
                       ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + part_bytes) : nullptr;
  a.order = order;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool.num_kv_heads;
  a.block_size = pool.block_size;
  a.part_size = P;
  a.num_parts = NP;
  a.ctx_cap = ctx_cap;
  a.scale_log2 = scale * kLog2e;
  a.new_k = new_k;
  a.new_v = new_v;
  a.new_slots = new_slots;
  a.num_slots = (long long)pool.num_blocks * pool.block_size;
  const unsigned grid = unsigned((long long)num_seqs * pool.num_kv_heads * NP);
  if (order) {
    decode_order_kernel<<<1, kOrderThreads, 0, stream>>>(context_lens, num_seqs, ctx_cap, order);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  bool ok;
  if (D == 64)
    ok = pool.fp8 ? launch_decode_g<64, true>(G, a, grid, stream)
                  : launch_decode_g<64, false>(G, a, grid, stream);
  else
    ok = pool.fp8 ? launch_decode_g<128, true>(G, a, grid, stream)
                  : launch_decode_g<128, false>(G, a, grid, stream);
  if (!ok) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || NP <= 1) return e;
  const unsigned rgrid = unsigned((long long)num_seqs * num_q_heads);
  if (D == 64)
    decode_reduce_kernel<64><<<rgrid, kWave, 0, stream>>>(context_lens, ctx_cap, P, NP, num_q_heads,
                                                          a.part_o, a.part_m, a.part_l, out);
  else
    decode_reduce_kernel<128><<<rgrid, kWave, 0, stream>>>(context_lens, ctx_cap, P, NP, num_q_heads,
                                                           a.part_o, a.part_m, a.part_l, out);
  return hipGetLastError();
}

}  // namespace pa
