// lca_device.h -- device-side helpers shared by the gfx950 kernels:
// storage codecs (FP8 E4M3 with per-64 scale, MXFP4 E2M1/E8M0, bf16), the
// order-preserving map from float64 scores to uint64 keys, and wave-level
// reductions.  gfx950 only (64-lane wavefronts).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lca_internal.h"

namespace lca {

// byte sizes of carved workspace regions are rounded up to 256
__host__ __device__ static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }


constexpr int WAVE = 64;

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Round-to-nearest-even of a finite fp32 value onto bfloat16.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------- FP8 -----
// OCP E4M3 (bias 7, max 448, S.1111.111 = NaN), exact decode.  gfx950's
// hardware conversion decodes OCP E4M3 (checked by the codec tests).
__device__ __forceinline__ float2 fp8x2_to_f32(uint32_t packed16) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8(packed16, false);
  return make_float2(v[0], v[1]);
}

// Round-to-nearest-even onto E4M3 with saturation at +-448, from a finite
// fp32 value.  Works on the binary exponent and the 3 kept mantissa bits.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  float a = fabsf(y);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {               // below 2^-6: subnormal grid 2^-9
    code = (uint32_t)rintf(a * 512.0f);     // 0..8 (8 is the smallest normal)
  } else {
    int e = ilogbf(a);                      // -6..8
    float mant = ldexpf(a, -e);             // [1, 2), exact
    uint32_t r = (uint32_t)rintf((mant - 1.0f) * 8.0f);   // 0..8, RNE
    if (r == 8u) { r = 0u; e += 1; }
    code = ((uint32_t)(e + 7) << 3) | r;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | sign;
}

// ---------------------------------------------------------------- MXFP4 ---
// Shared exponent of a 32-element block: floor(log2 amax) - 2 clamped to the
// E8M0 range; amax == 0 gives -127.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (amax == 0.0f) return -127;
  int e = ilogbf(amax) - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Round-to-nearest-even onto E2M1 magnitudes {0,.5,1,1.5,2,3,4,6}, saturating,
// keeping the sign bit of the input.
__device__ __forceinline__ uint32_t f32_to_e2m1(float y) {
  float a = fabsf(y);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return c | ((__float_as_uint(y) >> 28) & 8u);
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t m = c & 7u;
  float v = (m < 2u) ? 0.5f * (float)m : (float)(1u << ((m >> 1) - 1u)) * (1.0f + 0.5f * (float)(m & 1u));
  return (c & 8u) ? -v : v;
}

// ------------------------------------------------------- score keys -------
// Order-preserving map from a float64 score to uint64 (larger key = larger
// score).  -0.0 is folded onto +0.0 so equal scores get equal keys.  Key 0 is
// below every real score and marks "no entry".
__device__ __forceinline__ uint64_t score_key(double s) {
  s = s + 0.0;
  uint64_t b = (uint64_t)__double_as_longlong(s);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ double key_score(uint64_t k) {
  uint64_t b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)b);
}

// --------------------------------------------------------- wave utils -----
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, o, WAVE);
  hi = __shfl_xor(hi, o, WAVE);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t t = shfl_xor_u64(v, o);
    v = t > v ? t : v;
  }
  return v;
}

// ------------------------------------------------ DPP wavefront primitives
// Row (16-lane) steps use DPP permutes, which run at VALU latency; the four
// row results are then combined through v_readlane.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_QP_1032 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int DPP_QP_2301 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118;

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// max over the wavefront, returned to every lane (uniform)
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
  auto step = [](uint64_t x, uint32_t lo, uint32_t hi) {
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    return y > x ? y : x;
  };
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  v = step(v, dpp_u32<DPP_QP_1032>(lo, lo), dpp_u32<DPP_QP_1032>(hi, hi));
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  v = step(v, dpp_u32<DPP_QP_2301>(lo, lo), dpp_u32<DPP_QP_2301>(hi, hi));
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  v = step(v, dpp_u32<DPP_ROW_HALF_MIRROR>(lo, lo), dpp_u32<DPP_ROW_HALF_MIRROR>(hi, hi));
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  v = step(v, dpp_u32<DPP_ROW_MIRROR>(lo, lo), dpp_u32<DPP_ROW_MIRROR>(hi, hi));
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t y = ((uint64_t)readlane_u32(hi, 16 * r + 15) << 32) | readlane_u32(lo, 16 * r + 15);
    m = y > m ? y : m;
  }
  return m;
}

__device__ __forceinline__ uint64_t wave_min_u64_dpp(uint64_t v) {
  auto step = [](uint64_t x, uint32_t lo, uint32_t hi) {
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    return y < x ? y : x;
  };
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  v = step(v, dpp_u32<DPP_QP_1032>(lo, lo), dpp_u32<DPP_QP_1032>(hi, hi));
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  v = step(v, dpp_u32<DPP_QP_2301>(lo, lo), dpp_u32<DPP_QP_2301>(hi, hi));
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  v = step(v, dpp_u32<DPP_ROW_HALF_MIRROR>(lo, lo), dpp_u32<DPP_ROW_HALF_MIRROR>(hi, hi));
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  v = step(v, dpp_u32<DPP_ROW_MIRROR>(lo, lo), dpp_u32<DPP_ROW_MIRROR>(hi, hi));
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  uint64_t m = ~0ull;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t y = ((uint64_t)readlane_u32(hi, 16 * r + 15) << 32) | readlane_u32(lo, 16 * r + 15);
    m = y < m ? y : m;
  }
  return m;
}

// inclusive prefix sum over the wavefront (lane order)
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  const int lane = threadIdx.x & 63;
  uint32_t x = (uint32_t)v;
  x += dpp_u32<DPP_ROW_SHR1>(0u, x);
  x += dpp_u32<DPP_ROW_SHR2>(0u, x);
  x += dpp_u32<DPP_ROW_SHR4>(0u, x);
  x += dpp_u32<DPP_ROW_SHR8>(0u, x);
  const uint32_t r0 = readlane_u32(x, 15), r1 = readlane_u32(x, 31), r2 = readlane_u32(x, 47);
  const int row = lane >> 4;
  x += (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
  return (int)x;
}

// Number of set lanes strictly below this lane in a 64-bit ballot.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  const int lane = threadIdx.x & 63;
  return __popcll(mask & ((1ull << lane) - 1ull));
}

}  // namespace lca
