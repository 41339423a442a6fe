// compress_body.h -- the body of one compress block (softmax-gated pooling of
// m raw tokens fused with the cache encoder), shared by the compress kernels
// and the fused decode-step kernel.  The method and its sources are
// described in compress.hip.
#pragma once
#include "lca_device.h"

namespace lca {

// 256 threads per block.  For the pooling sum, thread t reads 16-byte pieces
// (8 bf16 or 4 fp32 channels) of the tokens of its token group: chunk
// t % NCK of a row, tokens t / NCK, t / NCK + G, ...; all of a thread's token
// loads of a batch are issued before the gate softmax.  The G group partials
// are then added in LDS in group order, and thread d < D encodes channel d.
constexpr int PE_THREADS = 256;

struct PeShared {
  float wgt[1024];                              // gate weights of the block
  float red[2][PE_THREADS / WAVE];
  __align__(16) float part[2048];               // [G][D] group partials
  __align__(16) float part2[2048];              // per-channel gates: [G][D] softmax sums
};

template <int ODT, int D>
__device__ __forceinline__ void encode_row(const CompressArgs& a, int b, int i, float c);

// Whether block i of sequence b lies inside the buffers the call describes:
// the tokens it reads (its span less the overlap rows a sequence's first
// block skips) within [0, x_rows), its output row within [0, dst_rows).  A
// block outside them (device-resident x_tok0 / dst_row0 out of range) is
// skipped: nothing is read or written for it.
__device__ __forceinline__ bool block_in_range(const CompressArgs& a, int b, int i) {
  const int64_t tok0 = (int64_t)a.x_tok0[b] + (int64_t)i * a.m;
  const int64_t row = (int64_t)a.dst_row0[b] + i;
  const int skip = (a.overlap > 0 && row == 0) ? a.overlap : 0;
  return tok0 + skip >= 0 && tok0 + a.m + a.overlap <= a.x_rows && row >= 0 && row < a.dst_rows;
}

// Per-channel gates (gate [B][x_rows][D], bias [m + overlap][D]): one softmax
// per channel over the block's span.  Thread t handles CPL channels of the
// tokens of its group, as in pool_encode_block; pass 1 finds each channel's
// maximum logit (group maxima reduced in LDS), pass 2 accumulates exp-weighted
// sums and the softmax denominators, reduced in LDS in group order.
template <int XDT, int ODT, int D>
__device__ __forceinline__ void pool_encode_block_pc(const CompressArgs& a, int b, int i, PeShared& S) {
  constexpr int CPL = XDT == DT_F32 ? 4 : 8;
  constexpr int NCK = D / CPL;
  constexpr int G = PE_THREADS / NCK;
  static_assert(G * D <= 2048, "group partials fit");
  if (i >= a.nblk[b] || !block_in_range(a, b, i)) return;
  const int64_t tok0 = (int64_t)a.x_tok0[b] + (int64_t)i * a.m;
  const int span = a.m + a.overlap;
  const int skip = (a.overlap > 0 && a.dst_row0[b] + i == 0) ? a.overlap : 0;
  const int tid = threadIdx.x;
  const int ck = tid % NCK, grp = tid / NCK;
  float (*part)[D] = (float (*)[D])S.part;
  float (*part2)[D] = (float (*)[D])S.part2;
  const float* grow = a.gate + ((int64_t)b * a.x_rows + tok0) * D + ck * CPL;
  const float* brow = a.bias + ck * CPL;
  auto logits = [&](int u, float* v) {
    const float4* gp = (const float4*)(grow + (int64_t)u * D);
    const float4* bp = (const float4*)(brow + (int64_t)u * D);
#pragma unroll
    for (int h = 0; h < CPL / 4; ++h) {
      const float4 g4 = gp[h], b4 = bp[h];
      v[4 * h] = g4.x + b4.x; v[4 * h + 1] = g4.y + b4.y; v[4 * h + 2] = g4.z + b4.z; v[4 * h + 3] = g4.w + b4.w;
    }
  };
  float mx[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) mx[c] = -INFINITY;
  for (int u = skip + grp; u < span; u += G) {
    float v[CPL];
    logits(u, v);
#pragma unroll
    for (int c = 0; c < CPL; ++c) mx[c] = fmaxf(mx[c], v[c]);
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) part[grp][ck * CPL + c] = mx[c];
  __syncthreads();
  if (tid < D) {
    float m0 = part[0][tid];
#pragma unroll
    for (int q = 1; q < G; ++q) m0 = fmaxf(m0, part[q][tid]);
    S.wgt[tid] = m0;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CPL; ++c) mx[c] = S.wgt[ck * CPL + c];
  float acc[CPL], zc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = zc[c] = 0.f;
  const char* xrow = (const char*)a.x + (((int64_t)b * a.x_rows + tok0) * D + ck * CPL) * (XDT == DT_F32 ? 4 : 2);
  const int64_t rstride = (int64_t)D * (XDT == DT_F32 ? 4 : 2);
  for (int u = skip + grp; u < span; u += G) {
    float v[CPL], xf[CPL];
    logits(u, v);
    const int4 xv = *(const int4*)(xrow + u * rstride);
    if (XDT == DT_F32) {
      xf[0] = __int_as_float(xv.x); xf[1] = __int_as_float(xv.y);
      xf[2] = __int_as_float(xv.z); xf[3] = __int_as_float(xv.w);
    } else {
      const uint32_t q[4] = {(uint32_t)xv.x, (uint32_t)xv.y, (uint32_t)xv.z, (uint32_t)xv.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xf[2 * k] = __uint_as_float(q[k] << 16);
        xf[2 * k + 1] = __uint_as_float(q[k] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float e = expf(v[c] - mx[c]);
      zc[c] += e;
      acc[c] = fmaf(e, xf[c], acc[c]);
    }
  }
  __syncthreads();                              // part is re-used
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    part[grp][ck * CPL + c] = acc[c];
    part2[grp][ck * CPL + c] = zc[c];
  }
  __syncthreads();
  if (tid >= D) return;
  float c = 0.f, z = 0.f;
#pragma unroll
  for (int q = 0; q < G; ++q) {
    c += part[q][tid];
    z += part2[q][tid];
  }
  encode_row<ODT, D>(a, b, i, c / z);
}

// Block i of sequence b of one compress call.
template <int XDT, int ODT, int D>
__device__ __forceinline__ void pool_encode_block(const CompressArgs& a, int b, int i, PeShared& S) {
  constexpr int CPL = XDT == DT_F32 ? 4 : 8;    // channels per 16-byte piece
  constexpr int NCK = D / CPL;                  // pieces per token row
  constexpr int G = PE_THREADS / NCK;           // token groups
  constexpr int TB = 16;                        // token loads in flight per thread and batch
  static_assert(G * D <= 2048, "group partials fit");
  if (a.gate_pc) {
    pool_encode_block_pc<XDT, ODT, D>(a, b, i, S);
    return;
  }
  const int nblk = a.nblk[b];
  const int64_t tok0 = (int64_t)a.x_tok0[b] + (int64_t)i * a.m;
  if (i >= nblk || !block_in_range(a, b, i)) return;
  const int tid = threadIdx.x;
  const int ck = tid % NCK, grp = tid / NCK;
  const int m = a.m + a.overlap;                 // tokens of the block's span
  // the first block of a sequence has no tokens before it: its overlap rows
  // are neither read nor weighted
  const int skip = (a.overlap > 0 && a.dst_row0[b] + i == 0) ? a.overlap : 0;

  float* wgt = S.wgt;
  auto& red = S.red;
  float (*part)[D] = (float (*)[D])S.part;

  const char* xrow = (const char*)a.x + (((int64_t)b * a.x_rows + tok0) * D + ck * CPL) * (XDT == DT_F32 ? 4 : 2);
  const int64_t rstride = (int64_t)D * (XDT == DT_F32 ? 4 : 2);
  int4 xv[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const int u = grp + t * G;
    xv[t] = u >= skip && u < m ? *(const int4*)(xrow + u * rstride) : make_int4(0, 0, 0, 0);
  }

  // gate logits + positional bias, block max and sum
  const float* gp = a.gate + (int64_t)b * a.x_rows + tok0;
  float mx = -INFINITY;
  for (int u = tid; u < m; u += PE_THREADS) {
    const float v = u >= skip ? gp[u] + a.bias[u] : -INFINITY;
    wgt[u] = v;
    mx = fmaxf(mx, v);
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[0][tid >> 6] = mx;
  __syncthreads();
  mx = red[0][0];
#pragma unroll
  for (int w = 1; w < PE_THREADS / WAVE; ++w) mx = fmaxf(mx, red[0][w]);
  float z = 0.0f;
  for (int u = tid; u < m; u += PE_THREADS) {
    const float e = u >= skip ? expf(wgt[u] - mx) : 0.0f;
    wgt[u] = e;
    z += e;
  }
  z = wave_sum(z);
  if ((tid & 63) == 0) red[1][tid >> 6] = z;
  __syncthreads();
  z = red[1][0];
#pragma unroll
  for (int w = 1; w < PE_THREADS / WAVE; ++w) z += red[1][w];
  const float inv_z = 1.0f / z;

  // this group's share of CPL channels, its tokens in increasing order
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  auto add = [&](const int4& v, float w) {
    if (XDT == DT_F32) {
      acc[0] = fmaf(w, __int_as_float(v.x), acc[0]);
      acc[1] = fmaf(w, __int_as_float(v.y), acc[1]);
      acc[2] = fmaf(w, __int_as_float(v.z), acc[2]);
      acc[3] = fmaf(w, __int_as_float(v.w), acc[3]);
    } else {
      const uint32_t q[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] = fmaf(w, __uint_as_float(q[k] << 16), acc[2 * k]);
        acc[2 * k + 1] = fmaf(w, __uint_as_float(q[k] & 0xFFFF0000u), acc[2 * k + 1]);
      }
    }
  };
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const int u = grp + t * G;
    if (u >= skip && u < m) add(xv[t], wgt[u] * inv_z);
  }
  for (int t0 = TB; grp + t0 * G < m; t0 += TB) {
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int u = grp + (t0 + t) * G;
      xv[t] = u >= skip && u < m ? *(const int4*)(xrow + u * rstride) : make_int4(0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int u = grp + (t0 + t) * G;
      if (u >= skip && u < m) add(xv[t], wgt[u] * inv_z);
    }
  }
  if (m == 1) {
    // exact copy (weight is 1): keep the input bits
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    add(xv[0], 1.0f);
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) part[grp][ck * CPL + c] = acc[c];
  __syncthreads();
  if (tid >= D) return;
  float c = 0.f;
#pragma unroll
  for (int q = 0; q < G; ++q) c += part[q][tid];
  if (m == 1) c = part[0][tid];
  encode_row<ODT, D>(a, b, i, c);
}

// Thread tid < D writes channel tid of block i's pooled row c in the output
// encoding (the FP8 and MXFP4 scale groups are whole wavefronts).
template <int ODT, int D>
__device__ __forceinline__ void encode_row(const CompressArgs& a, int b, int i, float c) {
  const int tid = threadIdx.x;
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

}  // namespace lca
