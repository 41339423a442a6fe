// compress.hip -- softmax-gated pooling with positional bias, fused with the
// cache encoders (FP8 E4M3 + per-64 fp32 scale, MXFP4, bf16, fp32).
//
// [release notes (agentlenshq.com), 壓縮稀疏注意力 (CSA): KV compressed 4x along
//  the sequence by softmax-gated pooling with a learned positional bias;
//  重度壓縮注意力 (HCA): the same at 128x; 架構實現: most KV entries in FP8, the
//  indexer in FP4.]
//
// One workgroup pools one block of m raw tokens: D threads (one per channel),
// the m gate weights are formed once in LDS, each thread accumulates its
// channel over the m tokens in fp32 (coalesced row reads), and the encoder
// runs on the pooled row while it is still in registers: a wavefront is
// exactly one 64-channel FP8 scale group, a half wavefront one 32-channel MX
// block.  The kernel is HBM-bound (every raw token read once).
#include "lca_device.h"

namespace lca {

template <int XDT, int ODT, int D>
__global__ __launch_bounds__(D) void pool_encode_kernel(CompressArgs a) {
  const int b = blockIdx.y;
  const int i = blockIdx.x;
  if (i >= a.nblk[b]) return;
  const int tid = threadIdx.x;
  const int m = a.m;
  const int64_t tok0 = (int64_t)a.x_tok0[b] + (int64_t)i * m;

  __shared__ float wgt[1024];
  __shared__ float red[2][D / WAVE];

  // gate logits + positional bias, block max
  const float* g = a.gate + (int64_t)b * a.x_rows + tok0;
  float mx = -INFINITY;
  for (int u = tid; u < m; u += D) {
    float v = g[u] + a.bias[u];
    wgt[u] = v;
    mx = fmaxf(mx, v);
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[0][tid >> 6] = mx;
  __syncthreads();
  mx = red[0][0];
#pragma unroll
  for (int w = 1; w < D / WAVE; ++w) mx = fmaxf(mx, red[0][w]);
  float z = 0.0f;
  for (int u = tid; u < m; u += D) {
    const float e = expf(wgt[u] - mx);
    wgt[u] = e;
    z += e;
  }
  z = wave_sum(z);
  if ((tid & 63) == 0) red[1][tid >> 6] = z;
  __syncthreads();
  z = red[1][0];
#pragma unroll
  for (int w = 1; w < D / WAVE; ++w) z += red[1][w];
  const float inv_z = 1.0f / z;

  // pooled channel tid
  float c = 0.0f;
  if (XDT == DT_F32) {
    const float* x = (const float*)a.x + ((int64_t)b * a.x_rows + tok0) * D + tid;
    for (int u = 0; u < m; ++u) c = fmaf(wgt[u] * inv_z, x[(int64_t)u * D], c);
  } else {
    const uint16_t* x = (const uint16_t*)a.x + ((int64_t)b * a.x_rows + tok0) * D + tid;
    for (int u = 0; u < m; ++u) c = fmaf(wgt[u] * inv_z, bf16_to_f32(x[(int64_t)u * D]), c);
  }
  if (m == 1) {
    // exact copy (weight is 1): keep the input bits
    if (XDT == DT_F32) c = ((const float*)a.x)[((int64_t)b * a.x_rows + tok0) * D + tid];
    else c = bf16_to_f32(((const uint16_t*)a.x)[((int64_t)b * a.x_rows + tok0) * D + tid]);
  }

  const int64_t row = (int64_t)b * a.dst_rows + a.dst_row0[b] + i;
  if (a.pooled) a.pooled[((int64_t)b * a.nblk_max + i) * D + tid] = c;

  if (ODT == DT_F32) {
    ((float*)a.dst)[row * D + tid] = c;
  } else if (ODT == DT_BF16) {
    ((uint16_t*)a.dst)[row * D + tid] = f32_to_bf16(c);
  } else if (ODT == DT_FP8) {
    float amax = wave_max(fabsf(c));          // one wavefront = one 64-channel group
    float s = 1.0f;
    if (amax != 0.0f) {
      s = amax / 448.0f;
      if (s == 0.0f) s = __uint_as_float(1u);  // 2^-149
    }
    ((uint8_t*)a.dst)[row * D + tid] = (uint8_t)f32_to_e4m3(c / s);
    if ((tid & 63) == 0) ((float*)a.dst_scale)[row * (D / 64) + (tid >> 6)] = s;
  } else {  // MXFP4
    float amax = fabsf(c);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, WAVE));
    const int X = mx_shared_exp(amax);
    const uint32_t code = f32_to_e2m1(ldexpf(c, -X));
    const uint32_t hi = __shfl_down(code, 1, WAVE);
    if ((tid & 1) == 0) ((uint8_t*)a.dst)[row * (D / 2) + (tid >> 1)] = (uint8_t)(code | (hi << 4));
    if ((tid & 31) == 0) ((uint8_t*)a.dst_scale)[row * (D / 32) + (tid >> 5)] = (uint8_t)(X + 127);
  }
}

template <int XDT, int ODT>
static hipError_t launch_d(const CompressArgs& a, hipStream_t s) {
  dim3 grid(a.nblk_max, a.B);
  if (a.D == 64) hipLaunchKernelGGL((pool_encode_kernel<XDT, ODT, 64>), grid, dim3(64), 0, s, a);
  else hipLaunchKernelGGL((pool_encode_kernel<XDT, ODT, 128>), grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

template <int XDT>
static hipError_t launch_o(const CompressArgs& a, hipStream_t s) {
  switch (a.dst_dt) {
    case DT_F32: return launch_d<XDT, DT_F32>(a, s);
    case DT_BF16: return launch_d<XDT, DT_BF16>(a, s);
    case DT_FP8: return launch_d<XDT, DT_FP8>(a, s);
    default: return launch_d<XDT, DT_MXFP4>(a, s);
  }
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (a.nblk_max == 0 || a.B == 0) return hipSuccess;
  return a.x_dt == DT_F32 ? launch_o<DT_F32>(a, s) : launch_o<DT_BF16>(a, s);
}

}  // namespace lca
