// Residual add fused with RMSNorm ("nano-vllm-lite：深入理解LLM推理机制的教育级开源项目",
// 核心技术改进 §1 CUDA融合内核：Add+RMSNorm): one pass over a row reads x and the
// residual, writes the new residual h = x + r and y = h * w / sqrt(mean(h^2) + eps);
// the sum never goes back to memory before it is normalised.
//
// HBM-bound: per row 2·H·2 bytes read (x, r) and 2·H·2 written (y, h); the weight
// vector is re-read by every row from L2. A row is spread over kL lanes (8..64
// lanes of one wave, or 2..16 waves of one workgroup for long rows); each lane
// holds kV 16-byte vectors of x and r in registers, so the row is read once and
// its mean square needs one reduction over the kL lanes.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

// Workgroup size for rows of kL lanes: 256 threads, or one row per workgroup
// for rows wider than that.
constexpr int norm_threads(int kL) { return kL > 256 ? kL : 256; }

struct NormArgs {
  const uint16_t* x;
  const uint16_t* r;    // nullptr: plain RMSNorm (h = x)
  const uint16_t* w;
  uint16_t* out;
  uint16_t* r_out;
  int num_tokens;
  int hidden;
  float eps;
};

// Sum over the kL lanes (kL / 64 = 2..16 waves) that share a row.
template <int kL>
__device__ __forceinline__ float sum_lanes_multiwave(float v, float* red) {
  constexpr int kWavesPerRow = kL / kWave;
  v = wave_sum(v);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if ((threadIdx.x % kWave) == 0) red[wave] = v;
  __syncthreads();
  const int first = wave - wave % kWavesPerRow;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kWavesPerRow; ++k) s += red[first + k];
  return s;
}

template <int kL, int kV, bool kRes>
__global__ void __launch_bounds__(norm_threads(kL)) add_rmsnorm_kernel(NormArgs a) {
  constexpr int kThreads = norm_threads(kL);
  constexpr int kRows = kThreads / kL;       // rows per workgroup
  __shared__ float red[kThreads / kWave];
  const int tid = threadIdx.x;
  const int l = tid % kL;
  const long long row = (long long)blockIdx.x * kRows + tid / kL;
  const int nvec = a.hidden >> 3;            // 16-byte vectors per row
  const bool live = row < a.num_tokens;
  const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(a.x) + row * nvec;
  const u32x4_t* rp = reinterpret_cast<const u32x4_t*>(a.r) + row * nvec;

  // Every load of the row is issued before any store: out / r_out may be the
  // same buffers as x / r (in place), each element read and written by one lane.
  u32x4_t xv[kV], rv[kV];
#pragma unroll
  for (int j = 0; j < kV; ++j) {
    const int i = l + j * kL;
    const bool ok = live && i < nvec;
    xv[j] = ok ? __builtin_nontemporal_load(xp + i) : u32x4_t{0, 0, 0, 0};
    if constexpr (kRes) rv[j] = ok ? __builtin_nontemporal_load(rp + i) : u32x4_t{0, 0, 0, 0};
  }

  float h[kV][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kV; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float lo = bf16_lo(xv[j][e]), hi = bf16_hi(xv[j][e]);
      if constexpr (kRes) {
        lo += bf16_lo(rv[j][e]);
        hi += bf16_hi(rv[j][e]);
      }
      h[j][2 * e] = lo;
      h[j][2 * e + 1] = hi;
      ss = __builtin_fmaf(lo, lo, ss);
      ss = __builtin_fmaf(hi, hi, ss);
    }
  }

  if constexpr (kRes) {
    // the float32 sum of two bf16 values rounds to the same bf16 as their exact sum
    u32x4_t* rop = reinterpret_cast<u32x4_t*>(a.r_out) + row * nvec;
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const int i = l + j * kL;
      if (live && i < nvec) {
        u32x4_t pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = f32_to_bf16(h[j][2 * e]) | (f32_to_bf16(h[j][2 * e + 1]) << 16);
        rop[i] = pk;
      }
    }
  }

  if constexpr (kL > kWave) {
    ss = sum_lanes_multiwave<kL>(ss, red);
  } else {
#pragma unroll
    for (int m = kL / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, kL);
  }
  const float inv = 1.0f / sqrtf(ss / float(a.hidden) + a.eps);

  u32x4_t* op = reinterpret_cast<u32x4_t*>(a.out) + row * nvec;
  const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(a.w);
#pragma unroll
  for (int j = 0; j < kV; ++j) {
    const int i = l + j * kL;
    if (live && i < nvec) {
      const u32x4_t wv = wp[i];
      u32x4_t pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y0 = (h[j][2 * e] * inv) * bf16_lo(wv[e]);
        const float y1 = (h[j][2 * e + 1] * inv) * bf16_hi(wv[e]);
        pk[e] = f32_to_bf16(y0) | (f32_to_bf16(y1) << 16);
      }
      op[i] = pk;
    }
  }
}

template <int kL, int kV>
hipError_t launch_norm(const NormArgs& a, hipStream_t stream) {
  constexpr int kThreads = norm_threads(kL);
  constexpr int kRows = kThreads / kL;
  const unsigned grid = unsigned((a.num_tokens + kRows - 1) / kRows);
  if (a.r)
    add_rmsnorm_kernel<kL, kV, true><<<grid, kThreads, 0, stream>>>(a);
  else
    add_rmsnorm_kernel<kL, kV, false><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

// One 16-byte vector of x and of r per lane (the most loads in flight per byte
// of registers): a row gets the next power of two >= hidden/8 lanes, at least
// 8, at most 512; longer rows take 2 vectors per lane on 512 or 1024 lanes.
// Measured on MI355X with T rows x H (TB/s, 1 vs 2-4 vectors per lane):
// 4344 x 4096 5.34 vs 4.53-5.25, 4344 x 1024 4.64 vs 3.8-4.4, 139008 x 128
// 5.26 vs 5.02.
hipError_t launch_add_rmsnorm(const uint16_t* x, const uint16_t* r, const uint16_t* w, uint16_t* out,
                              uint16_t* r_out, int num_tokens, int hidden, float eps, hipStream_t stream) {
  NormArgs a{x, r, w, out, r_out, num_tokens, hidden, eps};
  const int nvec = hidden / 8;
#if defined(PA_NORM_FORCE_L) && defined(PA_NORM_FORCE_V)
  // tuning builds: one fixed shape for every row length it can hold
  if (nvec <= PA_NORM_FORCE_L * PA_NORM_FORCE_V) return launch_norm<PA_NORM_FORCE_L, PA_NORM_FORCE_V>(a, stream);
#endif
  if (nvec <= 8) return launch_norm<8, 1>(a, stream);
  if (nvec <= 16) return launch_norm<16, 1>(a, stream);
  if (nvec <= 32) return launch_norm<32, 1>(a, stream);
  if (nvec <= 64) return launch_norm<64, 1>(a, stream);
  if (nvec <= 128) return launch_norm<128, 1>(a, stream);
  if (nvec <= 256) return launch_norm<256, 1>(a, stream);
  if (nvec <= 512) return launch_norm<512, 1>(a, stream);
  if (nvec <= 1024) return launch_norm<512, 2>(a, stream);
  return launch_norm<1024, 2>(a, stream);
}

}  // namespace pa
