// Device helpers shared by the HIP kernels of libpa (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 += a.lo*b.lo + a.hi*b.hi with bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two e4m3 bytes (byte pair `hi_word` of a dword) -> two bf16 packed in a dword.
// The conversion is exact: every e4m3 value is a bf16 value.
template <bool kHiWord>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t packed) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, kHiWord));
}

// 16-byte load marked non-temporal (streamed, read once).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               kCtrl, 0xf, 0xf, false));
}

// Reductions over the 64 lanes of a wave; every lane receives the result.
// Inside each row of 16 lanes: quad xor-1, quad xor-2, rotate by 4, rotate by 8;
// the four row results are then combined through lanes 0, 16, 32 and 48.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));    // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f32<0x4E>(x));    // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f32<0x124>(x));   // row_ror:4
  x = fmaxf(x, dpp_f32<0x128>(x));   // row_ror:8
  float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x124>(x);
  x += dpp_f32<0x128>(x);
  float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return (a + b) + (c + d);
}

// OCP e4m3fn code nearest to x (ties to even), |x| > 448 saturated to 448.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float ax = __builtin_fabsf(x);
  uint32_t code;
  if (!(ax == ax)) return 0x7fu | sign;
  if (ax > 448.0f) {
    code = 0x7eu;
  } else if (ax < 0.015625f) {
    // below 2^-6 the codes are the multiples of 2^-9; ax * 512 is exact
    code = uint32_t(__builtin_rintf(ax * 512.0f));
  } else {
    // keep 3 mantissa bits with round-to-nearest-even at bit 20, then move the
    // exponent from bias 127 to bias 7
    uint32_t a = __float_as_uint(ax);
    a += 0x7ffffu + ((a >> 20) & 1u);
    code = (a >> 20) - (120u << 3);
  }
  return code | sign;
}

}  // namespace pa
