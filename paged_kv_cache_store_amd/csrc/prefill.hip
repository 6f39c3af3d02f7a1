// Causal varlen prefill over the paged KV cache, on the matrix cores.
//
// Chunked prefill splits a long prompt into chunks that run next to decode; a
// chunk's queries attend to the sequence's cached prefix plus the chunk itself,
// and prefill is compute-bound ("nano-vllm-lite：深入理解LLM推理机制的教育级开源项目",
// 核心技术改进 §2). The keys/values come from the block pool through the block
// table ("DeepSeek复刻vLLM反超原版：AI推理新标杆", section vLLM：大模型推理的加速引擎与挑战);
// the attention is exact, computed tile by tile with a running max and sum
// ("Nano-vLLM：轻量高效的大模型推理框架…", 三.3 模型层适配).
//
// Work decomposition (CDNA4, wave64, v_mfma_f32_32x32x16_bf16):
// * one workgroup (4 waves) per (sequence, KV head, block of 128/G query rows);
//   the G query heads of the KV head are packed into 128 columns, 32 per wave,
//   so every K/V tile staged in LDS serves all G heads;
// * K/V tiles of 64 keys are copied from the pool to LDS, double-buffered, in
//   the pool's own layouts: K [D/8][64 keys][8], V [8 chunks of 8 keys][D][8];
//   bf16 tiles go straight from the pool into LDS (buffer_load ... lds with
//   blocks of at least one tile, else global_load_lds), fp8 tiles
//   through registers, where they are widened to bf16;
// * S^T = K Q^T: A = K rows (keys) from LDS, B = Q^T from registers (loaded
//   once), so each lane owns one query column and its softmax statistics;
// * the row max needs one exchange with lane l^32; the weights P^T come out of
//   the accumulator already in the B-operand layout of the next product;
// * O^T += V^T P^T: A = V^T from LDS. The accumulator hands lane half h the keys
//   {4h..4h+3, 8+4h..8+4h+3} of each 16-key step; one v_permlane32_swap per
//   dword pair regroups them to keys 8h..8h+7, one 8-key V chunk, so every A
//   fragment is one 16-byte read.
// * packed keys/values (no block table: K and V are [Tk][Hkv][D] bf16, each
//   sequence's keys contiguous from row cu_k[s]) take the register path: K
//   chunks are copied as they are, V is transposed 8 keys x 8 head-dims at a
//   time into the same LDS layouts, so the MFMA loop is unchanged.
// * a bf16 pool with blocks of at least one tile (up to kSortMax sequences)
//   runs the persistent form (prefill_persist_kernel): the same work items and
//   the same tile loop, with at most two workgroups per CU each running a run
//   of items, the next item's first tiles copied during the current item's last
//   steps; its output is bit-identical to one workgroup per item.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 32-column blocks per wave. With 2 the pipelined loop needs more than the 512
// registers of one wave per SIMD (it spills to scratch), so 1 is the built form.
#ifndef PA_PREFILL_NB
#define PA_PREFILL_NB 1
#endif
// waves per SIMD the register budget is set for (228 VGPRs: 2)
#ifndef PA_PREFILL_WAVES_PER_EU
#define PA_PREFILL_WAVES_PER_EU 2
#endif
// LDS fragment reads kept in flight ahead of the QK^T MFMAs (0: compiler's order);
// 4 measured about 3 % faster than the compiler's order on the mixed step
#ifndef PA_PREFILL_QK_LEAD
#define PA_PREFILL_QK_LEAD 4
#endif

// LDS fragment reads kept in flight ahead of the MFMAs of a pipelined step
#ifndef PA_PREFILL_STEP_LEAD
#define PA_PREFILL_STEP_LEAD 4
#endif

constexpr int kPrefillThreads = 256;
constexpr int kPrefillWaves = kPrefillThreads / 64;
constexpr int kBN = 64;           // keys per tile
constexpr int kIdCache = 2048;    // block ids held in LDS at a time
constexpr int kSortMax = 256;     // sequences ranked by length in each workgroup

struct PrefillArgs {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* block_tables;
  const float* k_scale;
  const float* v_scale;
  uint16_t* out;
  int max_blocks_per_seq;
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int block_size;
  int max_seqlen_q;
  int cap_k;
  int block_shift;  // log2(block_size)
  int num_qblocks;
  float scale_log2;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// max / sum of x over lanes l and l^32 (v_permlane32_swap: the returned pair
// holds x of lanes l%32 and l%32+32, for every lane)
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// maximum of three floats in one instruction. fmaxf would first quiet possible
// signalling NaNs of the MFMA results (one extra instruction per operand); the
// scores here are never NaN once masked (keys past the context are masked first)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// 16 bytes per lane from global memory into LDS at lds_row + 16 * lane
// (global_load_lds: the data skips the registers; the wave's lanes land in
// lane order). Plain void pointers: with the vector-struct pointer types the
// host compilation pass drops the kernel's launch stub.
__device__ __forceinline__ void load_row_to_lds(const void* src, void* lds_row) {
  __builtin_amdgcn_global_load_lds(src, lds_row, 16, 0, 0);
}

// The same copy through a buffer descriptor (buffer_load ... lds, 16 bytes per
// lane): the lane's bytes are read at base + soff + voff (voff = 16 * lane) and
// land at lds_row + 16 * lane. The callers' offsets stay inside the block by
// construction; the descriptor's size (`bytes`) bounds only voff, the hardware
// leaving soff out of its range check. The
// compiler counts a global_load_lds (FLAT encoding, LDS written) as a pending
// FLAT access and then waits for every LDS read of the step to complete
// (lgkmcnt(0)) wherever it waits for one; the buffer form lets the fragment
// reads of the MFMA loop stay in flight.
#ifndef PA_PREFILL_COPY_BUFFER
#define PA_PREFILL_COPY_BUFFER 1
#endif
__device__ __forceinline__ __amdgpu_buffer_rsrc_t copy_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void buffer_row_to_lds(__amdgpu_buffer_rsrc_t r, int soff, int voff, void* lds_row) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_row, 16, voff,
                                           __builtin_amdgcn_readfirstlane(soff), 0, 0);
}

static constexpr bf16x2_t kOnesBf16x2 = {(__bf16)1.0f, (__bf16)1.0f};

// kNB = 32-column blocks per wave; a workgroup covers 4 * 32 * kNB packed
// (query row, head) columns, i.e. 128 * kNB / G query rows of each of the G heads.
template <int kD, int kG, int kNB, bool kFp8, bool kBig, bool kPacked = false>
__global__ __launch_bounds__(kPrefillThreads)
#if PA_PREFILL_WAVES_PER_EU
__attribute__((amdgpu_waves_per_eu(PA_PREFILL_WAVES_PER_EU)))
#endif
void prefill_kernel(const PrefillArgs a) {
  constexpr int kCols = kPrefillWaves * 32 * kNB;
  constexpr int kBM = kCols / kG;        // query rows per workgroup
  constexpr int kKS = kD / 16;           // k-steps of S^T = K Q^T
  constexpr int kDB = kD / 32;           // 32-row blocks of O^T
  constexpr int kKC = kD / 8;            // 16-byte bf16 chunks per key (LDS layout)
  constexpr int kX = kFp8 ? 16 : 8;      // elements per 16-byte chunk of the pool
  constexpr int kKLoads = (kD / kX) * kBN / kPrefillThreads;   // 16-byte K loads per thread per tile
  constexpr int kVLoads = (kBN / kX) * kD / kPrefillThreads;

  static_assert(!(kPacked && (kFp8 || kBig)), "packed keys/values are bf16, without blocks");
  constexpr bool kDirect = !kFp8 && !kPacked;   // bf16 pool tiles go straight into LDS
  constexpr int kKW = kKC / kPrefillWaves;                   // direct: K chunk rows per wave
  constexpr int kVW = (kBN / 8) * (kD / 64) / kPrefillWaves; // direct: 64-wide V rows per wave

  // Two LDS buffers per tile, each in the pool's own order: K [16-byte chunk of
  // head-dims][key] and V [8-key chunk][head-dim], 16 bytes per entry (bf16).
  // Separate arrays (not one array indexed by buffer) let the compiler see that
  // reads of one buffer never alias the copies in flight into the other, so it
  // places no wait for those copies before the reads.
  __shared__ uint4 k_a[kKC][kBN], k_b[kKC][kBN];
  __shared__ uint4 v_a[kBN / 8][kD], v_b[kBN / 8][kD];
  // a window of the sequence's block-table row: ids_s[i] = row[wbase + i]
  __shared__ int ids_s[kIdCache];

  const int Hkv = a.num_kv_heads;
  const int bid = blockIdx.x;
  const int hk = bid % Hkv;
  const int rest = bid / Hkv;
  const int tid = threadIdx.x;
  // Longest work first: sequences by decreasing key count (ties by index), and
  // within a sequence the later query blocks (they see more keys) first. Every
  // workgroup ranks the sequences itself from cu_k, staged in ids_s (not yet in
  // use); past kSortMax sequences they are taken in reverse index order.
  // The ranking pass also stages every sequence's query offset and length, so
  // the chosen sequence's are read from LDS, not with one more round trip.
  const int qb = a.num_qblocks - 1 - rest % a.num_qblocks;
  const int want = rest / a.num_qblocks;           // rank of this workgroup's sequence
  int s = a.num_seqs - 1 - want;
  int q0, Lq, Lk;
  if (a.num_seqs > 1 && a.num_seqs <= kSortMax) {
    const int S = a.num_seqs;
    for (int i = tid; i < S; i += kPrefillThreads) {
      const int lk = a.cu_k[i + 1] - a.cu_k[i];
      const int qa = a.cu_q[i];
      ids_s[i] = lk < a.cap_k ? lk : a.cap_k;
      ids_s[kSortMax + i] = qa;
      ids_s[2 * kSortMax + i] = a.cu_q[i + 1] - qa;
    }
    __syncthreads();
    for (int i = tid; i < S; i += kPrefillThreads) {
      const int li = ids_s[i];
      int rank = 0;
      for (int j = 0; j < S; ++j) {
        const int lj = ids_s[j];
        rank += (lj > li) || (lj == li && j < i);
      }
      if (rank == want) ids_s[kIdCache - 1] = i;
    }
    __syncthreads();
    s = ids_s[kIdCache - 1];
    Lk = ids_s[s];
    q0 = ids_s[kSortMax + s];
    Lq = ids_s[2 * kSortMax + s];
    __syncthreads();                                // ids_s is reused for block ids
  } else {
    q0 = a.cu_q[s];
    Lq = a.cu_q[s + 1] - q0;
    Lk = a.cu_k[s + 1] - a.cu_k[s];
    Lk = Lk < a.cap_k ? Lk : a.cap_k;
  }
  Lq = Lq < a.max_seqlen_q ? Lq : a.max_seqlen_q;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int l32 = lane % 32;
  const int half = lane / 32;
  const int row0 = qb * kBM;
  if (row0 >= Lq || Lq <= 0) return;
  const int bs = a.block_size;
  const int* bt = kPacked ? nullptr : a.block_tables + (long long)s * a.max_blocks_per_seq;
  const long long slab16 = (long long)bs * kD * (kFp8 ? 1 : 2) / 16;
  const uint4* kpool = reinterpret_cast<const uint4*>(a.k_cache) + (long long)hk * slab16;
  const uint4* vpool = reinterpret_cast<const uint4*>(a.v_cache) + (long long)hk * slab16;
  const long long blk16 = (long long)Hkv * slab16;

  // ---- this lane's query columns: packed index -> (query head, query row)
  int head[kNB], qrow[kNB], lim[kNB];
  float lim_hi = -1.f, lim_lo = 1e30f;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int pr = (w * kNB + nb) * 32 + l32;
    head[nb] = hk * kG + pr / kBM;
    qrow[nb] = row0 + pr % kBM;
    const int last = Lk - Lq + qrow[nb];                   // last key the row may see
    lim[nb] = last < Lk - 1 ? last : Lk - 1;
    const int rr = qrow[nb] < Lq - 1 ? qrow[nb] : Lq - 1;  // rows past Lq are not written
    const int needed = Lk - Lq + rr < Lk - 1 ? Lk - Lq + rr : Lk - 1;
    lim_hi = fmaxf(lim_hi, float(needed));
    lim_lo = fminf(lim_lo, float(lim[nb]));
  }
  const int wave_last = int(wave_max(lim_hi));          // keys this wave needs
  const int wave_lim_min = int(-wave_max(-lim_lo));     // tiles below it need no mask
  // keys the workgroup needs
  int wg_last = Lk - Lq + (row0 + kBM - 1 < Lq - 1 ? row0 + kBM - 1 : Lq - 1);
  wg_last = wg_last < Lk - 1 ? wg_last : Lk - 1;
  const int ntiles = wg_last >= 0 ? (wg_last + kBN) / kBN : 0;
  // ---- Q^T fragments (B operand): lane holds column qrow, head-dim 16*ks + 8*half .. +8
  uint4 qf[kNB][kKS];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int r = qrow[nb] < Lq ? qrow[nb] : Lq - 1;
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((long long)(q0 + r) * a.num_q_heads + head[nb]) * kD);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qf[nb][ks] = qp[ks * 2 + half];
  }

  // ---- tile loader.
  // Block ids come from a window of the block-table row kept in LDS (ids_s),
  // loaded before the first tile and moved forward when a tile needs blocks
  // past it. Block sizes are powers of two (shift/mask).
  // bf16 (kDirect): each wave moves whole 1 KB rows of a tile from the pool
  // into LDS, 16 bytes per lane, lane-major (buffer_load ... lds through a
  // descriptor over the tile's block when a tile lies in one block, else
  // global_load_lds): K rows are
  // (chunk c, 64 keys), V rows (8-key chunk j, 64 head-dims); no staging
  // registers and no LDS writes by the waves. fp8: loads into registers,
  // widening to bf16, LDS writes in the same layouts.
  // With blocks of at least one tile (kBig) a tile lies inside one block: its
  // base address is scalar and every lane's offset is the same for each tile.
  // Keys past Lk in the last tile then read slots of that block past the
  // context: in bounds, their scores masked, their V values zeroed before use.
  // With smaller blocks keys past Lk read key Lk-1 (K) or the chunk holding it (V).
  const int bshift = a.block_shift;
  const int bmask = bs - 1;
  // blocks the workgroup's tiles touch
  const int last_key = (ntiles * kBN < Lk ? ntiles * kBN : Lk) - 1;
  const int nblk = last_key >= 0 ? (last_key >> bshift) + 1 : 0;
  int wbase = 0;
  auto load_ids = [&](int first) {   // every thread calls it; the caller synchronises
    wbase = first;
    if constexpr (!kPacked)
      for (int i = tid; i < kIdCache && first + i < nblk; i += kPrefillThreads) ids_s[i] = bt[first + i];
  };
  auto block_of = [&](int key) { return ids_s[(key >> bshift) - wbase]; };
  // move the window so that it holds every block tiles t0..t1 read (uniform
  // branch; two tiles span at most 8 blocks, far fewer than the window)
  auto ensure_ids = [&](int t0, int t1) {
    if constexpr (kPacked) return;
    const int lastk = (t1 * kBN + kBN < Lk ? t1 * kBN + kBN : Lk) - 1;
    if ((lastk >> bshift) - wbase >= kIdCache) {
      __syncthreads();
      load_ids((t0 * kBN) >> bshift);
      __syncthreads();
    }
  };
  const int k_key = tid % kBN;            // K: this lane's key within the tile
  const int k_c0 = tid / kBN;             // staged K: first chunk (then + 4u)
  const int v_d = tid % kD;               // staged V: head-dim index
  const int v_j0 = tid / kD;              // staged V: first 16-key chunk
  // staging registers use a native vector type: with HIP's union-based uint4 the
  // array is not split into registers and the backend moves it into LDS
  constexpr int kVRegs = kDirect ? 1 : (kPacked ? 8 : kVLoads);
  u32x4_t kreg[kDirect ? 1 : kKLoads], vreg[kVRegs];
  // packed: row cu_k[s] of K / V for this KV head, rows Hkv*D elements apart
  const long long prow = (long long)Hkv * kD;
  const uint16_t* kseq = kPacked ? reinterpret_cast<const uint16_t*>(a.k_cache) +
                                       ((long long)a.cu_k[s] * Hkv + hk) * kD : nullptr;
  const uint16_t* vseq = kPacked ? reinterpret_cast<const uint16_t*>(a.v_cache) +
                                       ((long long)a.cu_k[s] * Hkv + hk) * kD : nullptr;
  // packed V: thread tid < kVItems transposes 8 keys (8-key chunk pv_j) x 8 head-dims (pv_g)
  constexpr int kVItems = (kBN / 8) * (kD / 8);
  const int pv_j = tid / (kD / 8);
  const int pv_g = tid % (kD / 8);
  // direct: the V row filled by load u of this wave: 8-key chunk j, head-dims 64*dh ..
  auto vrow = [&](int u, int& j, int& dh) {
    const int e = w * kVW + u;
    j = e / (kD / 64);
    dh = e % (kD / 64);
  };
  // direct: issue the pool -> LDS copies of tile kt's K into ks ...
  // direct: the block ids a tile's copies need, read from ids_s ahead of the
  // copies and kept raw in VGPRs so that the LDS read latency is not waited
  // for: this lane's K row (one id per tile with kBig, which also serves V)
  // and, with smaller blocks, the wave's V rows
  struct CopyIds { int k; int v[kBig ? 1 : kVW]; };
  auto copy_ids = [&](int kt, CopyIds& c) {
    kt = kt < ntiles ? kt : ntiles - 1;     // past the last tile: ids of the last (unused)
    const int key0 = kt * kBN;
    const int kkey = key0 + k_key < Lk ? key0 + k_key : Lk - 1;
    c.k = block_of(kBig ? key0 : kkey);
    if constexpr (!kBig) {
#pragma unroll
      for (int u = 0; u < kVW; ++u) {
        int j, dh;
        vrow(u, j, dh);
        const int key = key0 + j * 8;
        c.v[u] = block_of(key < Lk ? key : ((Lk - 1) & ~7));
      }
    }
  };
  auto issue_k = [&](int kt, const CopyIds& ids, uint4 (*ks)[kBN]) {
    const int key0 = kt * kBN;
    const int kkey = key0 + k_key < Lk ? key0 + k_key : Lk - 1;
    const int kblk = kBig ? __builtin_amdgcn_readfirstlane(ids.k) : ids.k;
    if constexpr (kBig && PA_PREFILL_COPY_BUFFER) {
      // the tile lies in one block: a descriptor over this KV head's slab of it
      const auto r = copy_rsrc(kpool + (long long)kblk * blk16, int(slab16 * 16));
#pragma unroll
      for (int u = 0; u < kKW; ++u) {
        const int c = w * kKW + u;
        buffer_row_to_lds(r, ((key0 & bmask) + (c << bshift)) * 16, lane * 16, &ks[c][0]);
      }
      return;
    }
    const uint4* ksrc = kpool + (long long)kblk * blk16 + (kBig ? (key0 & bmask) + k_key : (kkey & bmask));
#pragma unroll
    for (int u = 0; u < kKW; ++u) {
      const int c = w * kKW + u;
      load_row_to_lds(ksrc + ((long long)c << bshift), &ks[c][0]);
    }
  };
  // ... and of its V into vs
  auto issue_v = [&](int kt, const CopyIds& ids, uint4 (*vs)[kD]) {
    const int key0 = kt * kBN;
    const int vblk0 = __builtin_amdgcn_readfirstlane(ids.k);
    if constexpr (kBig && PA_PREFILL_COPY_BUFFER) {
      const auto r = copy_rsrc(vpool + (long long)vblk0 * blk16, int(slab16 * 16));
#pragma unroll
      for (int u = 0; u < kVW; ++u) {
        int j, dh;
        vrow(u, j, dh);
        buffer_row_to_lds(r, ((((key0 + j * 8) & bmask) >> 3) * kD + dh * 64) * 16, lane * 16, &vs[j][dh * 64]);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < kVW; ++u) {
      int j, dh;
      vrow(u, j, dh);
      const int key = key0 + j * 8;
      const int kcv = kBig ? key : (key < Lk ? key : ((Lk - 1) & ~7));
      const int vblk = kBig ? vblk0 : __builtin_amdgcn_readfirstlane(ids.v[kBig ? 0 : u]);
      const uint4* vsrc = vpool + (long long)vblk * blk16 + (long long)((kcv & bmask) >> 3) * kD + dh * 64 + k_key;
      load_row_to_lds(vsrc, &vs[j][dh * 64]);
    }
  };
  // direct: once tile kt has landed in vs (after a barrier), zero the V values
  // of keys >= Lk: their weights are 0, but a stale or NaN value would still
  // poison 0 * v. Only the last tile can hold such keys.
  auto fix_tail = [&](int kt, uint4 (*vs)[kD]) {
    const int key0 = kt * kBN;
    if (key0 + kBN <= Lk) return;
    for (int e = tid; e < (kBN / 8) * kD; e += kPrefillThreads) {
      const int j = e / kD, d = e % kD;
      const int nv = Lk - (key0 + j * 8);            // valid keys of the entry
      if (nv < 8) {
        uint4 v = vs[j][d];
        v.x &= (0 < nv ? 0x0000ffffu : 0u) | (1 < nv ? 0xffff0000u : 0u);
        v.y &= (2 < nv ? 0x0000ffffu : 0u) | (3 < nv ? 0xffff0000u : 0u);
        v.z &= (4 < nv ? 0x0000ffffu : 0u) | (5 < nv ? 0xffff0000u : 0u);
        v.w &= (6 < nv ? 0x0000ffffu : 0u) | (7 < nv ? 0xffff0000u : 0u);
        vs[j][d] = v;
      }
    }
    __syncthreads();
  };
  // staged (fp8): loads into registers ...
  auto load_tile = [&](int kt) {
    const int key0 = kt * kBN;
    if constexpr (kPacked) {
      // keys past Lk read key Lk-1 (K: scores masked) or nothing (V: zeros)
      const int key = key0 + k_key < Lk ? key0 + k_key : Lk - 1;
#pragma unroll
      for (int u = 0; u < kKLoads; ++u)
        kreg[u] = *reinterpret_cast<const u32x4_t*>(kseq + key * prow + (k_c0 + u * (kPrefillThreads / kBN)) * 8);
      if (tid < kVItems) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int vkey = key0 + pv_j * 8 + e;
          vreg[e] = vkey < Lk ? *reinterpret_cast<const u32x4_t*>(vseq + vkey * prow + pv_g * 8)
                              : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    } else if constexpr (kBig) {
      const int blk = __builtin_amdgcn_readfirstlane(block_of(key0));
      const u32x4_t* kb = reinterpret_cast<const u32x4_t*>(kpool + (long long)blk * blk16 + (key0 & bmask));
#pragma unroll
      for (int u = 0; u < kKLoads; ++u)
        kreg[u] = kb[uint32_t((k_c0 + u * (kPrefillThreads / kBN)) << bshift) + k_key];
      const u32x4_t* vb = reinterpret_cast<const u32x4_t*>(vpool + (long long)blk * blk16 +
                                                           (long long)((key0 & bmask) / kX) * kD);
#pragma unroll
      for (int u = 0; u < kVLoads; ++u) vreg[u] = vb[uint32_t((v_j0 + u * (kPrefillThreads / kD)) * kD + v_d)];
    } else {
      const int key = key0 + k_key;
      const int kc = key < Lk ? key : Lk - 1;
      const uint4* src = kpool + (long long)block_of(kc) * blk16 + (kc & bmask);
      // keys past Lk read the last key instead; their scores are masked
#pragma unroll
      for (int u = 0; u < kKLoads; ++u)
        kreg[u] = reinterpret_cast<const u32x4_t*>(src)[(long long)(k_c0 + u * (kPrefillThreads / kBN)) << bshift];
#pragma unroll
      for (int u = 0; u < kVLoads; ++u) {
        const int j = v_j0 + u * (kPrefillThreads / kD);   // x-key chunk of the tile
        const int vkey = key0 + j * kX;
        const int kcv = vkey < Lk ? vkey : ((Lk - 1) & ~(kX - 1));
        vreg[u] = reinterpret_cast<const u32x4_t*>(vpool)[(long long)block_of(kcv) * blk16 +
                                                          (long long)((kcv & bmask) / kX) * kD + v_d];
      }
    }
  };
  // ... widened to bf16 and written to LDS (every e4m3 value is a bf16 value);
  // V values past Lk are zeroed on the bytes first
  auto store_tile = [&](uint4 (*ks)[kBN], uint4 (*vs)[kD], int kt) {
    if constexpr (kPacked) {
#pragma unroll
      for (int u = 0; u < kKLoads; ++u) {
        const int c = k_c0 + u * (kPrefillThreads / kBN);
        ks[c][k_key] = make_uint4(kreg[u][0], kreg[u][1], kreg[u][2], kreg[u][3]);
      }
      if (tid < kVItems) {
        // vreg[e] holds head-dims 8*pv_g .. +7 of key 8*pv_j + e; entry
        // vs[pv_j][d] takes keys 8*pv_j .. +7 of head-dim d, two per dword
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          uint32_t wv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t lo = (vreg[2 * i][dd / 2] >> (16 * (dd % 2))) & 0xffffu;
            const uint32_t hi = (vreg[2 * i + 1][dd / 2] >> (16 * (dd % 2))) & 0xffffu;
            wv[i] = lo | (hi << 16);
          }
          vs[pv_j][pv_g * 8 + dd] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < kKLoads; ++u) {
      const int c8 = k_c0 + u * (kPrefillThreads / kBN);   // head-dims 16*c8 .. 16*c8+15
      uint32_t wv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wv[2 * i] = fp8x2_to_bf16x2<false>(kreg[u][i]);
        wv[2 * i + 1] = fp8x2_to_bf16x2<true>(kreg[u][i]);
      }
      ks[2 * c8][k_key] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      ks[2 * c8 + 1][k_key] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
    }
#pragma unroll
    for (int u = 0; u < kVLoads; ++u) {
      const int step = v_j0 + u * (kPrefillThreads / kD);  // 16-key chunk
      const int nv = Lk - (kt * kBN + step * 16);           // valid keys of the chunk
      if (nv < 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t mask = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) mask |= (4 * i + b < nv) ? (0xffu << (8 * b)) : 0u;
          vreg[u][i] &= mask;
        }
      }
      uint32_t wv[8];   // dword i holds keys 4i..4i+3
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wv[2 * i] = fp8x2_to_bf16x2<false>(vreg[u][i]);
        wv[2 * i + 1] = fp8x2_to_bf16x2<true>(vreg[u][i]);
      }
      vs[2 * step][v_d] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      vs[2 * step + 1][v_d] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
    }
  };

  f32x16_t o[kDB][kNB];
  float m[kNB], lsum[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    m[nb] = -INFINITY;
    lsum[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][nb][i] = 0.f;
  }
  const float sc = kFp8 ? a.scale_log2 * a.k_scale[hk] : a.scale_log2;

  // ---- one tile: S^T = K Q^T, online softmax, O^T += V^T P^T, from LDS buffers kc / vc
  // ---- S^T = K Q^T for the tile in kc (rows: 64 keys in two blocks of 32;
  // columns: this lane's query columns)
  auto qk_tile = [&](const uint4 (*kc)[kBN], f32x16_t (&sacc)[2][kNB]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[mb][nb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8_t af = as_bf16x8(kc[ks * 2 + half][mb * 32 + l32]);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          sacc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, as_bf16x8(qf[nb][ks]),
                                                                 sacc[mb][nb], 0, 0, 0);
      }
    }
  };
  // ---- online softmax per query column, in two parts. Scores stay unscaled
  // until one fma + exp2 per element. The reference max m of a column only
  // moves when the tile's max exceeds it by more than 8 (log2 units), so
  // weights stay <= 2^8 and O, l are rescaled rarely; O and l share the
  // reference, so the normalised result is unchanged.
  // Part 1: causal mask (diagonal tiles only), column max, move of m.
  auto softmax_max = [&](int kt, f32x16_t (&sacc)[2][kNB]) {
    const int key0 = kt * kBN;
    // ---- online softmax per query column; build P^T in the B-operand layout.
    // Scores stay unscaled until one fma + exp2 per element. The reference max
    // m of a column only moves when the tile's max exceeds it by more than 8
    // (log2 units), so weights stay <= 2^8 and O, l are rescaled rarely; O and
    // l share the reference, so the normalised result is unchanged.
    const bool diag_tile = key0 + kBN - 1 > wave_lim_min;  // some column masks keys here
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      if (diag_tile) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + mb * 32 + (i / 4) * 8 + half * 4 + (i % 4);
            if (key > lim[nb]) sacc[mb][nb][i] = -INFINITY;
          }
      }
      float smax = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) smax = max3f(smax, sacc[mb][nb][i], sacc[mb][nb][i + 1]);
      smax = pair_max(smax);
      const float mt = smax * sc;                  // sc > 0: -inf stays -inf
      const bool grow = mt > m[nb] + 8.f;
      if (__any(grow)) {
        const float mn = grow ? mt : m[nb];
        // 0 the first time (O, l are 0); 1 for a column whose max stays (also
        // one that has seen no key yet: m = -inf, where m - mn would be NaN)
        const float alpha = grow ? fast_exp2(m[nb] - mn) : 1.f;
        lsum[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][nb][i] *= alpha;
        m[nb] = mn;
      }
    }
  };
  // Part 2: weights rounded to bf16, their sum, P^T in the B-operand layout.
  uint4 pf[kNB][4];   // [nb][16-key step]
  auto softmax_exp = [&](f32x16_t (&sacc)[2][kNB]) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      // a column with no admissible key yet keeps m = -inf; its weights are 0
      const float mneg = m[nb] == -INFINITY ? 0.f : -m[nb];
      uint32_t packed[2][8];
      float ps = lsum[nb];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          f32x2_t pp;
          pp.x = fast_exp2(fmaf(sacc[mb][nb][i], sc, mneg));
          pp.y = fast_exp2(fmaf(sacc[mb][nb][i + 1], sc, mneg));
          const bf16x2_t pk = __builtin_convertvector(pp, bf16x2_t);
          ps = __builtin_amdgcn_fdot2_f32_bf16(pk, kOnesBf16x2, ps, false);  // sum of the bf16 weights
          packed[mb][i / 2] = __builtin_bit_cast(uint32_t, pk);
        }
      lsum[nb] = ps;
      // B operand of the 16-key step t = 2*mb + j: accumulator entries 8j .. 8j+7
      // hold keys {4h..4h+3, 8+4h..8+4h+3} of the step in lane half h; swapping
      // dwords 2,3 of half 0 with dwords 0,1 of half 1 (v_permlane32_swap) leaves
      // keys 8h..8h+7 in half h, the order of the V rows in LDS
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const auto r0 = __builtin_amdgcn_permlane32_swap(packed[mb][4 * j], packed[mb][4 * j + 2], false, false);
          const auto r1 = __builtin_amdgcn_permlane32_swap(packed[mb][4 * j + 1], packed[mb][4 * j + 3], false,
                                                           false);
          pf[nb][2 * mb + j] = make_uint4(r0[0], r1[0], r0[1], r1[1]);
        }
    }
  };
  auto pv_tile = [&](const uint4 (*vc)[kD]) {
    // ---- O^T += V^T P^T; step t covers tile keys 16t + 8h .. 16t + 8h + 7
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int d = db * 32 + l32;
        const bf16x8_t af = as_bf16x8(vc[2 * t + half][d]);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          o[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, as_bf16x8(pf[nb][t]), o[db][nb],
                                                              0, 0, 0);
      }
    }
  };
  // one tile, its steps in order (staged path)
  auto compute_tile = [&](int kt, const uint4 (*kc)[kBN], const uint4 (*vc)[kD]) {
    f32x16_t sacc[2][kNB];
    qk_tile(kc, sacc);
#if PA_PREFILL_QK_LEAD
    // keep PA_PREFILL_QK_LEAD fragment reads in flight ahead of the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, PA_PREFILL_QK_LEAD, 0);
#pragma unroll
    for (int i = 0; i < 2 * kKS - PA_PREFILL_QK_LEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, kNB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kNB * PA_PREFILL_QK_LEAD, 0);
#endif
    softmax_max(kt, sacc);
    softmax_exp(sacc);
    pv_tile(vc);
  };

  // Staged (fp8) loop: two LDS buffers (a, b), unrolled by two so that each
  // step names its buffers. Tile kt+1 sits in registers while tile kt is
  // computed; it is written to the other buffer after the products and the
  // loads of tile kt+2 are issued, so every load has a whole tile of work to land.
  auto staged_step = [&](int kt, uint4 (*kc)[kBN], uint4 (*vc)[kD], uint4 (*kn)[kBN], uint4 (*vn)[kD]) {
    if (kt + 2 < ntiles) ensure_ids(kt + 2, kt + 2);
    if (kt * kBN <= wave_last) {
      __builtin_amdgcn_s_setprio(1);   // MFMA issue priority, as in the direct loop
      compute_tile(kt, kc, vc);
      __builtin_amdgcn_s_setprio(0);
    }
    if (kt + 1 < ntiles) store_tile(kn, vn, kt + 1);
    if (kt + 2 < ntiles) load_tile(kt + 2);
    __syncthreads();
  };
  // Direct (bf16) loop, pipelined across tiles inside each wave: step kt runs
  // the softmax and PV of tile kt and the QK^T of tile kt+1, so the 16 QK^T
  // MFMAs of the next tile interleave with the softmax arithmetic of this one.
  // K and V of a tile therefore live in LDS at different times: step kt reads
  // K(kt+1) and V(kt) and copies K(kt+2) and V(kt+1) into the buffers the
  // previous step finished with (K(t) in k_a / k_b and V(t) in v_a / v_b by
  // the parity of t); the barrier at the end of the step waits for the copies.
  f32x16_t s_a[2][kNB], s_b[2][kNB];
  CopyIds ids_t1, ids_t2;   // ids of tiles kt+1 and kt+2 at the start of step kt
  auto pipe_step = [&](int kt, const uint4 (*k_next)[kBN], const uint4 (*v_cur)[kD], uint4 (*k_dst)[kBN],
                       uint4 (*v_dst)[kD], f32x16_t (&s_cur)[2][kNB], f32x16_t (&s_next)[2][kNB]) {
    // copies of K(kt+2) and V(kt+1) with ids read one and two steps ago; then
    // the ids of tile kt+3 for the next step
    if (kt + 2 < ntiles) issue_k(kt + 2, ids_t2, k_dst);
    if (kt + 1 < ntiles) issue_v(kt + 1, ids_t1, v_dst);
    if (kt + 3 < ntiles) ensure_ids(kt + 3, kt + 3);
    ids_t1 = ids_t2;
    copy_ids(kt + 3, ids_t2);
    if (kt * kBN <= wave_last) {
      softmax_max(kt, s_cur);
      // the two waves sharing a SIMD come from different workgroups; while this
      // one issues MFMAs it takes issue priority, so that the matrix pipe stays
      // fed when both are ready (measured: 5-6 % on the mixed step)
      __builtin_amdgcn_s_setprio(1);
      // past the last tile this reads a stale buffer; those scores are never used
      qk_tile(k_next, s_next);
      softmax_exp(s_cur);
      // issue order: a few fragment reads ahead, then each QK^T MFMA followed by
      // a share of the softmax VALU work and the next fragment read
      constexpr int kQkMfma = 2 * kKS * kNB, kQkReads = 2 * kKS, kLead = PA_PREFILL_STEP_LEAD;
      __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
      for (int i = 0; i < kQkMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 96 / kQkMfma, 0);
        if (i < kQkReads - kLead) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      pv_tile(v_cur);
      // PV: V fragment reads kept kLead ahead of their MFMAs
      constexpr int kPvReads = 4 * kDB;
      __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
      for (int i = 0; i < kPvReads - kLead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, kNB, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kNB * kLead, 0);
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
    if (kt + 1 < ntiles) fix_tail(kt + 1, v_dst);
  };
  // the loop sits inside the ntiles > 0 branch so that on every path into it
  // the Q loads are known complete: otherwise the QK^T MFMAs would carry
  // conservative waits on the global loads of the next tile
  if (ntiles > 0) {
    load_ids(0);
    __syncthreads();
    if constexpr (kDirect) {
      copy_ids(0, ids_t1);
      issue_k(0, ids_t1, k_a);
      issue_v(0, ids_t1, v_a);
      copy_ids(1, ids_t1);
      if (ntiles > 1) issue_k(1, ids_t1, k_b);
      copy_ids(2, ids_t2);
      __syncthreads();
      fix_tail(0, v_a);
      if (0 <= wave_last) qk_tile(k_a, s_a);
      // every wave is done with K(0) before step 0 copies K(2) over it
      __syncthreads();
      for (int kt = 0; kt < ntiles; kt += 2) {
        pipe_step(kt, k_b, v_a, k_a, v_b, s_a, s_b);
        if (kt + 1 < ntiles) pipe_step(kt + 1, k_a, v_b, k_b, v_a, s_b, s_a);
      }
    } else {
      load_tile(0);
      store_tile(k_a, v_a, 0);
      if (ntiles > 1) load_tile(1);
      __syncthreads();
      for (int kt = 0; kt < ntiles; kt += 2) {
        staged_step(kt, k_a, v_a, k_b, v_b);
        if (kt + 1 < ntiles) staged_step(kt + 1, k_b, v_b, k_a, v_a);
      }
    }
  }

  // ---- normalise and write this lane's query rows
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const float L = pair_sum(lsum[nb]);
    const float inv = L > 0.f ? (kFp8 ? a.v_scale[hk] : 1.f) / L : 0.f;
    if (qrow[nb] < Lq) {
      uint16_t* op = a.out + ((long long)(q0 + qrow[nb]) * a.num_q_heads + head[nb]) * kD;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + g4 * 8 + half * 4;
          // v_cvt_pk_bf16_f32: round to nearest even
          const f32x2_t lo = {o[db][nb][4 * g4 + 0] * inv, o[db][nb][4 * g4 + 1] * inv};
          const f32x2_t hi = {o[db][nb][4 * g4 + 2] * inv, o[db][nb][4 * g4 + 3] * inv};
          *reinterpret_cast<uint2*>(op + d) =
              make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t)),
                         __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t)));
        }
    }
  }
}

// ---- Persistent form of the bf16 block-table path (blocks of at least one tile,
// at most kSortMax sequences). One launch keeps at most two workgroups per CU
// resident; each takes a run of work items (sequence, KV head, query block) and
// passes from one to the next without draining its copy pipeline: the first K
// tiles and the first V tile of the next item are copied during the current
// item's last steps, with block ids from an LDS window that was filled while
// earlier items ran (three windows: the current item's, the next one's and the
// one after). The items keep the longest-first ranking of the
// one-item-per-workgroup kernel and are dealt in rounds of one per workgroup,
// each round in the reverse workgroup order of the one before, so that a
// workgroup given a long item early gets a short one late. Reversal is by
// groups of 8 workgroups when the count allows, which keeps the residue of a
// workgroup index mod 8 (and with 8 KV heads, the KV head an XCD serves) the
// same in every round.
constexpr int kWin = 256;   // block ids per window (LDS: 3 windows; longer items refill theirs)

template <int kD, int kG>
__global__ __launch_bounds__(kPrefillThreads)
__attribute__((amdgpu_waves_per_eu(2)))
void prefill_persist_kernel(const PrefillArgs a, int num_items) {
  constexpr int kBM = kPrefillWaves * 32 / kG;   // query rows per item
  constexpr int kKS = kD / 16;
  constexpr int kDB = kD / 32;
  constexpr int kKC = kD / 8;
  constexpr int kKW = kKC / kPrefillWaves;
  constexpr int kVW = (kBN / 8) * (kD / 64) / kPrefillWaves;
  static_assert(kWin % kPrefillThreads == 0, "window fill is whole rounds of the workgroup");

  __shared__ uint4 k_a[kKC][kBN], k_b[kKC][kBN];
  __shared__ uint4 v_a[kBN / 8][kD], v_b[kBN / 8][kD];
  __shared__ int win[3 * kWin];   // three windows of block ids, kWin apart
  __shared__ int seq_lk[kSortMax], seq_q0[kSortMax], seq_lq[kSortMax], seq_at[kSortMax];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int l32 = lane % 32;
  const int half = lane / 32;
  const int col = w * 32 + l32;   // this lane's packed (head, row) column of an item
  const int Hkv = a.num_kv_heads;
  const int S = a.num_seqs;
  const int bshift = a.block_shift;
  const int bmask = a.block_size - 1;
  const int slab16 = a.block_size * kD * 2 / 16;   // one KV head's slab of a block, 16-byte units
  const int blk16 = Hkv * slab16;                  // one block
  const uint4* kbase = reinterpret_cast<const uint4*>(a.k_cache);
  const uint4* vbase = reinterpret_cast<const uint4*>(a.v_cache);
  const float sc = a.scale_log2;

  // ---- sequences ranked by key count once per workgroup (ties by index)
  for (int i = tid; i < S; i += kPrefillThreads) {
    const int lk = a.cu_k[i + 1] - a.cu_k[i];
    const int qa = a.cu_q[i];
    seq_lk[i] = lk < a.cap_k ? lk : a.cap_k;
    seq_q0[i] = qa;
    const int lq = a.cu_q[i + 1] - qa;
    seq_lq[i] = lq < a.max_seqlen_q ? lq : a.max_seqlen_q;
  }
  __syncthreads();
  for (int i = tid; i < S; i += kPrefillThreads) {
    const int li = seq_lk[i];
    int rank = 0;
    for (int j = 0; j < S; ++j) {
      const int lj = seq_lk[j];
      rank += (lj > li) || (lj == li && j < i);
    }
    seq_at[rank] = i;
  }
  __syncthreads();

  // ---- work items: rank r -> KV head, query block, sequence (by its rank).
  // nt: tiles of 64 keys the item reads (0: its rows see no key; < 0: no rows)
  struct Item { int s, hk, q0, Lq, Lk, row0, nt; };
  auto item_info = [&](int r) __attribute__((always_inline)) {
    Item it;
    it.hk = r % Hkv;
    const int rest = r / Hkv;
    it.row0 = (a.num_qblocks - 1 - rest % a.num_qblocks) * kBM;
    it.s = __builtin_amdgcn_readfirstlane(seq_at[rest / a.num_qblocks]);
    it.Lk = __builtin_amdgcn_readfirstlane(seq_lk[it.s]);
    it.q0 = __builtin_amdgcn_readfirstlane(seq_q0[it.s]);
    it.Lq = __builtin_amdgcn_readfirstlane(seq_lq[it.s]);
    if (it.row0 >= it.Lq || it.Lq <= 0) {
      it.nt = -1;
    } else {
      int last = it.Lk - it.Lq + (it.row0 + kBM - 1 < it.Lq - 1 ? it.row0 + kBM - 1 : it.Lq - 1);
      last = last < it.Lk - 1 ? last : it.Lk - 1;
      it.nt = last >= 0 ? (last + kBN) / kBN : 0;
    }
    return it;
  };
  // the item of round k for this workgroup (rounds alternate direction)
  const int P = gridDim.x;
  const int b = blockIdx.x;
  auto rank_at = [&](int k) __attribute__((always_inline)) {
    int idx = b;
    if (k & 1) idx = P % 8 == 0 ? (P / 8 - 1 - b / 8) * 8 + b % 8 : P - 1 - b;
    return (long long)k * P + idx;
  };
  // this lane's output row of an item (nullptr past the item's rows)
  auto out_row = [&](const Item& it) __attribute__((always_inline)) -> uint16_t* {
    const int qr = it.row0 + col % kBM;
    if (qr >= it.Lq) return nullptr;
    return a.out + ((long long)(it.q0 + qr) * a.num_q_heads + it.hk * kG + col / kBM) * kD;
  };
  // the round of the first item at or after round k that reads keys (-1: none);
  // items whose rows see no key are written as zeros on the way
  auto find_item = [&](int k) __attribute__((always_inline)) {
    for (;; ++k) {
      const long long r = rank_at(k);
      if (r >= num_items) return -1;
      const Item it = item_info(int(r));
      if (it.nt > 0) return k;
      if (it.nt == 0) {
        uint16_t* op = out_row(it);
        if (op) {
#pragma unroll
          for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) *reinterpret_cast<uint2*>(op + db * 32 + g4 * 8 + half * 4) = make_uint2(0u, 0u);
        }
      }
    }
  };
  // blocks an item's tiles touch
  auto item_blocks = [&](int nt, int Lk) __attribute__((always_inline)) {
    const int lastk = (nt * kBN < Lk ? nt * kBN : Lk) - 1;
    return (lastk >> bshift) + 1;
  };
  // copy the first kWin block ids of the item of round k into window wi
  // (global_load_lds: the ids land without passing through registers; the
  // next barrier waits for them)
  auto window_dma = [&](int k, int wi) __attribute__((always_inline)) {
    const Item it = item_info(int(rank_at(k)));
    const int* row = a.block_tables + (long long)it.s * a.max_blocks_per_seq;
    const int nblk = item_blocks(it.nt, it.Lk);
#pragma unroll
    for (int j = 0; j < kWin / kPrefillThreads; ++j) {
      const int i = j * kPrefillThreads + w * kWave + lane;
      __builtin_amdgcn_global_load_lds(row + (i < nblk ? i : nblk - 1),
                                       &win[wi * kWin + j * kPrefillThreads + w * kWave], 4, 0, 0);
    }
  };

  // ---- rounds of the current item X, the next (Y) and the one after (Z), -1
  // when absent; the fields of X and Y the steps read; windows by item count
  int kx = find_item(0);
  if (kx < 0) return;
  int ky = find_item(kx + 1);
  int kz = ky < 0 ? -1 : find_item(ky + 1);
  int x_hk, x_lk, x_nt, y_hk = 0, y_lk = 0, y_nt = 0;
  int nitem = 0;                // items begun; X's window is nitem % 3
  int wbase = 0;                // first block id in X's window
  int kt = 0;                   // X's tile at this step
  auto win_of = [&](int ahead) __attribute__((always_inline)) { return (nitem + ahead) % 3; };
  // per item, so that a step does no division: X's and Y's windows (offsets
  // into win; indexed from win itself, so that the compiler sees these reads
  // never touch the K/V buffers that copies in flight write) and KV-head
  // offsets in the pool (16-byte units)
  int x_win = 0, y_win = kWin;
  int x_hoff = 0, y_hoff = 0;
  int dma_k = -1;               // round whose window is to be loaded in the next step
  // a window's ids in flight: loaded into registers in one step, written to LDS
  // at the start of the next (or at an item switch); plain stores, so that the
  // compiler sees exactly which LDS they write (an LDS copy in flight into the
  // windows would make every fragment read of the step wait for it)
  int idv[kWin / kPrefillThreads];
  int idv_dst = -1;

  // per-lane and per-wave state of X
  int lim, wave_last, wave_lim_min;
  uint4 qf[kKS];
  f32x16_t o[kDB];
  float m, lsum;
  // make the item of round k current: its fields, this lane's mask limit, Q rows
  auto begin_item = [&](int k) __attribute__((always_inline)) {
    const Item it = item_info(int(rank_at(k)));
    x_hk = it.hk;
    x_lk = it.Lk;
    x_nt = it.nt;
    x_hoff = it.hk * slab16;
    x_win = win_of(0) * kWin;
    y_win = win_of(1) * kWin;
    const int qrow = it.row0 + col % kBM;
    const int last = it.Lk - it.Lq + qrow;
    lim = last < it.Lk - 1 ? last : it.Lk - 1;
    const int rr = qrow < it.Lq - 1 ? qrow : it.Lq - 1;   // rows past Lq are not written
    const int needed = it.Lk - it.Lq + rr < it.Lk - 1 ? it.Lk - it.Lq + rr : it.Lk - 1;
    wave_last = __builtin_amdgcn_readfirstlane(int(wave_max(float(needed))));
    wave_lim_min = __builtin_amdgcn_readfirstlane(int(-wave_max(-float(lim))));
    const uint4* qp = reinterpret_cast<const uint4*>(
        a.q + ((long long)(it.q0 + rr) * a.num_q_heads + it.hk * kG + col / kBM) * kD);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qf[ks] = qp[ks * 2 + half];
    m = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  };
  auto next_fields = [&]() __attribute__((always_inline)) {
    if (ky >= 0) {
      const Item it = item_info(int(rank_at(ky)));
      y_hk = it.hk;
      y_lk = it.Lk;
      y_nt = it.nt;
      y_hoff = it.hk * slab16;
    }
  };

  auto window_load = [&](int k, int wi) __attribute__((always_inline)) {
    const Item it = item_info(int(rank_at(k)));
    const int* row = a.block_tables + (long long)it.s * a.max_blocks_per_seq;
    const int nblk = item_blocks(it.nt, it.Lk);
#pragma unroll
    for (int j = 0; j < kWin / kPrefillThreads; ++j) {
      const int i = j * kPrefillThreads + tid;
      idv[j] = row[i < nblk ? i : nblk - 1];
    }
    idv_dst = wi * kWin;
  };
  auto window_store = [&]() __attribute__((always_inline)) {
    if (idv_dst >= 0) {
#pragma unroll
      for (int j = 0; j < kWin / kPrefillThreads; ++j) win[idv_dst + j * kPrefillThreads + tid] = idv[j];
      idv_dst = -1;
    }
  };

  // ---- copies: the pool's rows straight into LDS (buffer_load ... lds through
  // a descriptor over the block, 16 bytes per lane); a tile lies in one block, keys
  // past Lk read slots of that block (in bounds; masked, their V zeroed).
  // Offsets (16-byte units) of tile t of KV head hk inside a block: K rows, V rows
  auto k_off = [&](int hoff, int t) __attribute__((always_inline)) { return hoff + ((t * kBN) & bmask); };
  auto v_off = [&](int hoff, int t) __attribute__((always_inline)) { return hoff + (((t * kBN) & bmask) >> 3) * kD; };
  auto issue_k = [&](int off, int blk, uint4 (*ks)[kBN]) __attribute__((always_inline)) {
#if PA_PREFILL_COPY_BUFFER
    // a descriptor over the block (every KV head's slab; off holds the head's)
    const auto r = copy_rsrc(kbase + (long long)blk * blk16, blk16 * 16);
#pragma unroll
    for (int u = 0; u < kKW; ++u) {
      const int c = w * kKW + u;
      buffer_row_to_lds(r, (off + (c << bshift)) * 16, lane * 16, &ks[c][0]);
    }
#else
    const uint4* ksrc = kbase + ((long long)blk * blk16 + off) + lane;
#pragma unroll
    for (int u = 0; u < kKW; ++u) {
      const int c = w * kKW + u;
      load_row_to_lds(ksrc + (c << bshift), &ks[c][0]);
    }
#endif
  };
  auto issue_v = [&](int off, int blk, uint4 (*vs)[kD]) __attribute__((always_inline)) {
#if PA_PREFILL_COPY_BUFFER
    const auto r = copy_rsrc(vbase + (long long)blk * blk16, blk16 * 16);
#pragma unroll
    for (int u = 0; u < kVW; ++u) {
      const int e = w * kVW + u;
      const int j = e / (kD / 64), dh = e % (kD / 64);
      buffer_row_to_lds(r, (off + j * kD + dh * 64) * 16, lane * 16, &vs[j][dh * 64]);
    }
#else
    const uint4* vb = vbase + ((long long)blk * blk16 + off) + lane;
#pragma unroll
    for (int u = 0; u < kVW; ++u) {
      const int e = w * kVW + u;
      const int j = e / (kD / 64), dh = e % (kD / 64);
      load_row_to_lds(vb + j * kD + dh * 64, &vs[j][dh * 64]);
    }
#endif
  };
  // once a V tile with `valid` keys before the end of its item's context has
  // landed in vs (after a barrier), zero the V values of the keys past it: their
  // weights are 0, but a stale or NaN value would still poison 0 * v
  auto fix_tail = [&](int valid, uint4 (*vs)[kD]) __attribute__((always_inline)) {
    if (valid >= kBN) return;
    for (int e = tid; e < (kBN / 8) * kD; e += kPrefillThreads) {
      const int j = e / kD, d = e % kD;
      const int nv = valid - j * 8;
      if (nv < 8) {
        uint4 v = vs[j][d];
        v.x &= (0 < nv ? 0x0000ffffu : 0u) | (1 < nv ? 0xffff0000u : 0u);
        v.y &= (2 < nv ? 0x0000ffffu : 0u) | (3 < nv ? 0xffff0000u : 0u);
        v.z &= (4 < nv ? 0x0000ffffu : 0u) | (5 < nv ? 0xffff0000u : 0u);
        v.w &= (6 < nv ? 0x0000ffffu : 0u) | (7 < nv ? 0xffff0000u : 0u);
        vs[j][d] = v;
      }
    }
    __syncthreads();
  };
  // move X's window so that it starts at block `first` (every thread; between
  // barriers; only for items longer than a window)
  auto refill = [&](int first) __attribute__((always_inline)) {
    __syncthreads();
    const Item it = item_info(int(rank_at(kx)));
    const int* row = a.block_tables + (long long)it.s * a.max_blocks_per_seq;
    const int nblk = item_blocks(it.nt, it.Lk);
    const int xw = win_of(0) * kWin;
    for (int i = tid; i < kWin && first + i < nblk; i += kPrefillThreads) win[xw + i] = row[first + i];
    wbase = first;
    __syncthreads();
  };

  // ---- the copies of a step, planned one step ahead: the offset of the tile
  // inside its block (-1: no copy) and the block id, read from LDS then and kept
  // raw in a VGPR so that the read's latency is not waited for. cv_valid: keys
  // of the V tile before the end of its item's context.
  int ck_off, cv_off, cv_valid;
  int ck_id, cv_id;
  // plan the step at X's tile t0 (Y follows when ky >= 0). Common case: both
  // copies read X (one branch); the last two steps of an item also read Y.
  auto plan = [&](int t0) __attribute__((always_inline)) {
    const int tk = t0 + 2, tv = t0 + 1, n = x_nt;
    const int bk = (tk * kBN) >> bshift, bv = (tv * kBN) >> bshift;
    if (__builtin_expect(tk < n, 1)) {
      if (__builtin_expect(bk - wbase >= kWin, 0)) refill(bv);
      ck_off = k_off(x_hoff, tk);
      ck_id = win[x_win + bk - wbase];
      cv_off = v_off(x_hoff, tv);
      cv_valid = x_lk - tv * kBN;
      cv_id = win[x_win + bv - wbase];
      return;
    }
    ck_off = cv_off = -1;
    cv_valid = kBN;
    if (ky >= 0 && tk == n) {
      ck_off = k_off(y_hoff, 0);
      ck_id = win[y_win];
    } else if (ky >= 0 && tk == n + 1 && y_nt >= 2) {
      ck_off = k_off(y_hoff, 1);
      ck_id = win[y_win + (kBN >> bshift)];
    }
    if (tv < n) {
      cv_off = v_off(x_hoff, tv);
      cv_valid = x_lk - tv * kBN;
      cv_id = win[x_win + bv - wbase];
    } else if (ky >= 0) {
      cv_off = v_off(y_hoff, 0);
      cv_valid = y_lk;
      cv_id = win[y_win];
    }
  };

  // ---- the tile arithmetic (as in the one-item kernel)
  auto qk_tile = [&](const uint4 (*kc)[kBN], f32x16_t (&sacc)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[mb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kc[ks * 2 + half][mb * 32 + l32]),
                                                           as_bf16x8(qf[ks]), sacc[mb], 0, 0, 0);
  };
  auto softmax_max = [&](f32x16_t (&sacc)[2]) __attribute__((always_inline)) {
    const int key0 = kt * kBN;
    if (key0 + kBN - 1 > wave_lim_min) {   // some column masks keys here
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + mb * 32 + (i / 4) * 8 + half * 4 + (i % 4);
          if (key > lim) sacc[mb][i] = -INFINITY;
        }
    }
    float smax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) smax = max3f(smax, sacc[mb][i], sacc[mb][i + 1]);
    smax = pair_max(smax);
    const float mt = smax * sc;
    const bool grow = mt > m + 8.f;
    if (__any(grow)) {
      const float mn = grow ? mt : m;
      const float alpha = grow ? fast_exp2(m - mn) : 1.f;   // m = -inf: no key seen yet
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m = mn;
    }
  };
  uint4 pf[4];
  auto softmax_exp = [&](f32x16_t (&sacc)[2]) __attribute__((always_inline)) {
    const float mneg = m == -INFINITY ? 0.f : -m;
    uint32_t packed[2][8];
    float ps = lsum;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        f32x2_t pp;
        pp.x = fast_exp2(fmaf(sacc[mb][i], sc, mneg));
        pp.y = fast_exp2(fmaf(sacc[mb][i + 1], sc, mneg));
        const bf16x2_t pk = __builtin_convertvector(pp, bf16x2_t);
        ps = __builtin_amdgcn_fdot2_f32_bf16(pk, kOnesBf16x2, ps, false);
        packed[mb][i / 2] = __builtin_bit_cast(uint32_t, pk);
      }
    lsum = ps;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const auto r0 = __builtin_amdgcn_permlane32_swap(packed[mb][4 * j], packed[mb][4 * j + 2], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(packed[mb][4 * j + 1], packed[mb][4 * j + 3], false, false);
        pf[2 * mb + j] = make_uint4(r0[0], r1[0], r0[1], r1[1]);
      }
  };
  auto pv_tile = [&](const uint4 (*vc)[kD]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vc[2 * t + half][db * 32 + l32]),
                                                        as_bf16x8(pf[t]), o[db], 0, 0, 0);
  };
  // normalise and write X's rows of this lane
  auto write_out = [&]() __attribute__((always_inline)) {
    uint16_t* op = out_row(item_info(int(rank_at(kx))));
    const float L = pair_sum(lsum);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (op) {
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + g4 * 8 + half * 4;
          const f32x2_t lo = {o[db][4 * g4 + 0] * inv, o[db][4 * g4 + 1] * inv};
          const f32x2_t hi = {o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv};
          *reinterpret_cast<uint2*>(op + d) =
              make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t)),
                         __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t)));
        }
    }
  };

  // ---- one step at X's tile kt: copies planned by the previous step; the
  // softmax and PV of tile kt with the QK^T of tile kt+1 interleaved (on X's
  // last tile that QK^T reads whatever K buffer is there and its scores are
  // dropped: one code path for every step keeps the registers of the
  // one-item kernel). After the barrier of X's last step: X's output, then Y
  // becomes X, its Q rows are loaded and its first QK^T runs.
  // Returns false when the workgroup has no item left.
  f32x16_t s_a[2], s_b[2];
  auto step = [&](const uint4 (*k_next)[kBN], const uint4 (*v_cur)[kD], uint4 (*k_dst)[kBN],
                  uint4 (*v_dst)[kD], uint4 (*k_alt)[kBN], f32x16_t (&s_cur)[2], f32x16_t (&s_next)[2]) __attribute__((always_inline)) {
    // this step's copies (planned by the previous step); the next step's are
    // planned first, while no copy is in flight, so that the window reads wait
    // for nothing
    const int koff = ck_off, voff = cv_off, tail_valid = cv_off >= 0 ? cv_valid : kBN;
    const int kid = __builtin_amdgcn_readfirstlane(ck_id), vid = __builtin_amdgcn_readfirstlane(cv_id);
    const bool last = kt + 1 == x_nt;
    window_store();
    if (__builtin_expect(!last, 1)) plan(kt + 1);
    if (__builtin_expect(koff >= 0, 1)) issue_k(koff, kid, k_dst);
    if (__builtin_expect(voff >= 0, 1)) issue_v(voff, vid, v_dst);
    // the window of the item after next: its ids land by this step's barrier
    if (__builtin_expect(dma_k >= 0, 0)) {
      window_load(dma_k, win_of(2));
      dma_k = -1;
    }
    if (__builtin_expect(kt * kBN <= wave_last, 1)) {
      softmax_max(s_cur);
      // the two waves sharing a SIMD come from different workgroups; while this
      // one issues MFMAs it takes issue priority, so that the matrix pipe stays
      // fed when both are ready
      __builtin_amdgcn_s_setprio(1);
      qk_tile(k_next, s_next);
      softmax_exp(s_cur);
      constexpr int kQkMfma = 2 * kKS, kQkReads = 2 * kKS, kLead = PA_PREFILL_STEP_LEAD;
      __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
      for (int i = 0; i < kQkMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 96 / kQkMfma, 0);
        if (i < kQkReads - kLead) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      pv_tile(v_cur);
      constexpr int kPvReads = 4 * kDB;
      __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
      for (int i = 0; i < kPvReads - kLead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kLead, 0);
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
    if (__builtin_expect(tail_valid < kBN, 0)) fix_tail(tail_valid, v_dst);
    if (__builtin_expect(!last, 1)) {
      ++kt;
      return true;
    }
    write_out();
    if (ky < 0) return false;
    // Y becomes X, Z becomes Y; the window X used takes the item after Z
    const bool one_tile = x_nt == 1;
    kx = ky;
    ky = kz;
    kz = kz < 0 ? -1 : find_item(kz + 1);
    ++nitem;
    wbase = 0;
    kt = 0;
    begin_item(kx);
    next_fields();
    window_store();
    // after a one-tile item no step has copied this item's first K tile yet
    if (one_tile) issue_k(k_off(x_hoff, 0), __builtin_amdgcn_readfirstlane(win[x_win]), k_alt);
    // each wave copies a quarter of a tile's rows and writes part of a window:
    // all wait for all
    __syncthreads();
    plan(0);
    dma_k = kz;                    // copied by the next step
    if (0 <= wave_last) qk_tile(k_next, s_next);   // K of X's first tile sits in k_next
    __syncthreads();               // every wave is done with that K before it is copied over
    return true;
  };

  // ---- first item: windows of X and Y, then X's first tiles and Q rows
  window_dma(kx, win_of(0));
  if (ky >= 0) window_dma(ky, win_of(1));
  __syncthreads();
  begin_item(kx);
  next_fields();
  plan(0);
  issue_k(k_off(x_hoff, 0), __builtin_amdgcn_readfirstlane(win[x_win]), k_a);
  issue_v(v_off(x_hoff, 0), __builtin_amdgcn_readfirstlane(win[x_win]), v_a);
  if (x_nt >= 2) issue_k(k_off(x_hoff, 1), __builtin_amdgcn_readfirstlane(win[x_win + (kBN >> bshift)]), k_b);
  dma_k = kz;                      // copied by the first step
  __syncthreads();
  fix_tail(x_lk, v_a);
  if (0 <= wave_last) qk_tile(k_a, s_a);
  __syncthreads();
  // position parity picks the buffers: K(p) in k_a / k_b and V(p) in v_a / v_b
  // by p mod 2, p counting tiles over the workgroup's items
  for (;;) {
    if (!step(k_b, v_a, k_a, v_b, k_b, s_a, s_b)) break;
    if (!step(k_a, v_b, k_b, v_a, k_a, s_b, s_a)) break;
  }
}

constexpr int kNBLaunch = PA_PREFILL_NB;

template <int kD, bool kFp8, bool kBig, bool kPacked = false>
static bool launch_prefill_gb(int G, const PrefillArgs& a, unsigned grid, hipStream_t stream) {
  switch (G) {
    case 1: prefill_kernel<kD, 1, kNBLaunch, kFp8, kBig, kPacked><<<grid, kPrefillThreads, 0, stream>>>(a); return true;
    case 2: prefill_kernel<kD, 2, kNBLaunch, kFp8, kBig, kPacked><<<grid, kPrefillThreads, 0, stream>>>(a); return true;
    case 4: prefill_kernel<kD, 4, kNBLaunch, kFp8, kBig, kPacked><<<grid, kPrefillThreads, 0, stream>>>(a); return true;
    case 8: prefill_kernel<kD, 8, kNBLaunch, kFp8, kBig, kPacked><<<grid, kPrefillThreads, 0, stream>>>(a); return true;
    default: return false;
  }
}

template <int kD, bool kFp8>
static bool launch_prefill_g(int G, const PrefillArgs& a, unsigned grid, hipStream_t stream) {
  if (!a.block_tables) return !kFp8 && launch_prefill_gb<kD, false, false, true>(G, a, grid, stream);
  return a.block_size >= kBN ? launch_prefill_gb<kD, kFp8, true>(G, a, grid, stream)
                             : launch_prefill_gb<kD, kFp8, false>(G, a, grid, stream);
}

template <int kD>
static bool launch_prefill_persist(int G, const PrefillArgs& a, int num_items, unsigned grid, hipStream_t stream) {
  switch (G) {
    case 1: prefill_persist_kernel<kD, 1><<<grid, kPrefillThreads, 0, stream>>>(a, num_items); return true;
    case 2: prefill_persist_kernel<kD, 2><<<grid, kPrefillThreads, 0, stream>>>(a, num_items); return true;
    case 4: prefill_persist_kernel<kD, 4><<<grid, kPrefillThreads, 0, stream>>>(a, num_items); return true;
    case 8: prefill_persist_kernel<kD, 8><<<grid, kPrefillThreads, 0, stream>>>(a, num_items); return true;
    default: return false;
  }
}

// resident workgroups of a persistent prefill launch: 0 = two per CU (what the
// kernel's registers and LDS allow), > 0 = that many, < 0 = no persistent
// launch (one workgroup per work item)
static int g_prefill_slots = 0;

void set_prefill_slots(int n) { g_prefill_slots = n; }

// compute units of the current device (looked up once per device)
static int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

hipError_t launch_prefill(const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                          const int32_t* cu_q, const int32_t* cu_k, const int32_t* block_tables,
                          int max_blocks_per_seq, int num_seqs, int num_q_heads,
                          int max_seqlen_q, int max_seqlen_k, float scale, uint16_t* out,
                          const PoolDims& pool, const float* k_scale, const float* v_scale,
                          hipStream_t stream) {
  const int G = num_q_heads / pool.num_kv_heads;
  const int bm = kPrefillWaves * 32 * kNBLaunch / G;
  PrefillArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.block_tables = block_tables;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.out = out;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool.num_kv_heads;
  a.block_size = pool.block_size;
  a.block_shift = block_tables ? __builtin_ctz(unsigned(pool.block_size)) : 0;
  a.max_seqlen_q = max_seqlen_q;
  a.cap_k = max_seqlen_k;
  a.num_qblocks = (max_seqlen_q + bm - 1) / bm;
  a.scale_log2 = scale * kLog2e;
  const long long items = (long long)num_seqs * a.num_qblocks * pool.num_kv_heads;
  const unsigned grid = unsigned(items);
  if (grid == 0) return hipSuccess;
  bool ok;
  // bf16 pool, blocks of at least one tile: the persistent kernel
  if (kNBLaunch == 1 && block_tables && !pool.fp8 && pool.block_size >= kBN && num_seqs <= kSortMax &&
      g_prefill_slots >= 0 && items <= 0x7fffffffLL) {
    const int slots = g_prefill_slots > 0 ? g_prefill_slots : 2 * device_cus();
    if (slots > 0) {
      const unsigned pg = items < slots ? unsigned(items) : unsigned(slots);
      ok = pool.head_dim == 64 ? launch_prefill_persist<64>(G, a, int(items), pg, stream)
                               : launch_prefill_persist<128>(G, a, int(items), pg, stream);
      if (!ok) return hipErrorInvalidValue;
      return hipGetLastError();
    }
  }
  if (pool.head_dim == 64)
    ok = pool.fp8 ? launch_prefill_g<64, true>(G, a, grid, stream) : launch_prefill_g<64, false>(G, a, grid, stream);
  else
    ok = pool.fp8 ? launch_prefill_g<128, true>(G, a, grid, stream) : launch_prefill_g<128, false>(G, a, grid, stream);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
