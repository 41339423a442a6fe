// attend.hip -- shared-KV (MQA) attention over compressed entries, a window of
// raw tokens and a per-head sink, with split-KV partials and an LSE merge.
//
// [wiki (chenshi221), 关键技术方法 › 架构创新: CSA = top-k sparse selection + MQA,
//  HCA = dense attention over heavily compressed entries, both with a
//  sliding-window branch and an attention sink; release notes
//  (agentlenshq.com), 壓縮稀疏注意力 (CSA) / 重度壓縮注意力 (HCA): the window
//  covers recent uncompressed tokens; 架構實現: entries stored in FP8.]
//
// For query row r and head h, the attended list is the selected entries (CSA)
// or entries 0..n_elig-1 (HCA), followed by the window tokens.  One vector
// per item is both key and value.  The sink logit joins the softmax
// denominator only, unscaled.  A workgroup processes one (row, split) pair:
// one contiguous range of the list for all heads, and either writes the final
// row (one split) or an unnormalised partial (running max m, sum l, weighted
// sum o) that the merge kernel combines in split order together with the sink.
#include "lca_device.h"

namespace lca {

constexpr int ATT_THREADS = 256;
constexpr int ATT_SPLIT = 256;     // list items per split
constexpr int ATT_TE = 32;         // items per LDS tile (VALU path)

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Number of splits per row; a single split when there are enough rows to fill
// the GPU on their own.
static int att_splits(int64_t R, int64_t n_kv_max, int64_t W_buf) {
  if (R >= 256) return 1;
  const int64_t L = n_kv_max + W_buf;
  const int64_t s = (L + ATT_SPLIT - 1) / ATT_SPLIT;
  return (int)(s < 1 ? 1 : s);
}

size_t attend_ws_bytes(int B, int Tq, int Hq, int D, int64_t n_kv_max, int64_t W_buf) {
  const int64_t R = (int64_t)B * Tq;
  const int S = att_splits(R, n_kv_max, W_buf);
  if (S == 1) return 0;
  return align256(sizeof(float) * R * S * Hq * 2) + align256(sizeof(float) * R * S * Hq * D);
}

// Item p of row r's list: returns the source pointer class and row, or -1.
struct ListItem {
  int kind;      // 0 entry, 1 window token, -1 skip
  int64_t row;   // row in kv ([B][N_cap]) or win ([B][W_buf])
};

__device__ __forceinline__ ListItem list_item(const AttendArgs& A, int b, int r, int p, int nkv) {
  ListItem it;
  if (p < nkv) {
    int64_t j = A.sparse ? (int64_t)A.idx[(int64_t)r * A.k + p] : (int64_t)p;
    if (j < 0 || j >= A.N_cap) { it.kind = -1; it.row = 0; return it; }
    it.kind = 0;
    it.row = (int64_t)b * A.N_cap + j;
  } else {
    it.kind = 1;
    it.row = (int64_t)b * A.W_buf + A.win_begin[r] + (p - nkv);
  }
  return it;
}

template <int KVDT>
__device__ __forceinline__ float kv_elem(const AttendArgs& A, int64_t row, int d) {
  if (KVDT == DT_F32) return ((const float*)A.kv)[row * A.D + d];
  if (KVDT == DT_BF16) return bf16_to_f32(((const uint16_t*)A.kv)[row * A.D + d]);
  const uint8_t c = ((const uint8_t*)A.kv)[row * A.D + d];
  const float2 v = fp8x2_to_f32((uint32_t)c);
  return v.x * A.kv_scale[row * (A.D / 64) + d / 64];
}

template <int WDT>
__device__ __forceinline__ float win_elem(const AttendArgs& A, int64_t row, int d) {
  if (WDT == DT_F32) return ((const float*)A.win)[row * A.D + d];
  return bf16_to_f32(((const uint16_t*)A.win)[row * A.D + d]);
}

template <int QDT>
__device__ __forceinline__ float q_elem(const AttendArgs& A, int64_t i) {
  if (QDT == DT_F32) return ((const float*)A.q)[i];
  return bf16_to_f32(((const uint16_t*)A.q)[i]);
}

__device__ __forceinline__ void store_out(const AttendArgs& A, int64_t i, float v) {
  if (A.out_dt == DT_F32) ((float*)A.out)[i] = v;
  else ((uint16_t*)A.out)[i] = f32_to_bf16(v);
}

// ------------------------------------------------------------------------
// fp32 VALU kernel (any storage types; used for F32 inputs).
// ------------------------------------------------------------------------
template <int QDT, int KVDT, int WDT, int HQ>
__global__ __launch_bounds__(ATT_THREADS) void attend_valu_kernel(AttendArgs A, int S, float* part_ml, float* part_o) {
  constexpr int D = 128;
  constexpr int TPH = ATT_THREADS / HQ;      // threads per head
  constexpr int DPT = D / TPH;               // output dims per thread
  const int split = blockIdx.x, r = blockIdx.y;
  const int b = r / A.Tq;
  const int tid = threadIdx.x;
  const int nkv = A.sparse ? A.k : A.n_elig[r];
  const int L = nkv + A.win_len[r];
  const int p0 = split * ATT_SPLIT;
  const int p1 = min(L, p0 + (S == 1 ? L : ATT_SPLIT));

  __shared__ float qs[HQ][D];
  __shared__ float kvs[ATT_TE][D + 1];
  __shared__ float lg[HQ][ATT_TE + 1];
  __shared__ float mrun[HQ], lrun[HQ], alpha[HQ];
  __shared__ int valid[ATT_TE];

  for (int i = tid; i < HQ * D; i += ATT_THREADS) qs[i / D][i % D] = q_elem<QDT>(A, (int64_t)r * HQ * D + i) * A.scale;
  if (tid < HQ) { mrun[tid] = -INFINITY; lrun[tid] = 0.f; }
  const int h = tid / TPH, d0 = (tid % TPH) * DPT;
  float acc[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) acc[i] = 0.f;
  __syncthreads();

  for (int t0 = p0; t0 < p1; t0 += ATT_TE) {
    // stage a tile of items as fp32
    for (int i = tid; i < ATT_TE * D; i += ATT_THREADS) {
      const int e = i / D, d = i % D;
      const int p = t0 + e;
      float v = 0.f;
      int ok = 0;
      if (p < p1) {
        const ListItem it = list_item(A, b, r, p, nkv);
        if (it.kind == 0) { v = kv_elem<KVDT>(A, it.row, d); ok = 1; }
        else if (it.kind == 1) { v = win_elem<WDT>(A, it.row, d); ok = 1; }
      }
      kvs[e][d] = v;
      if (d == 0) valid[e] = ok;
    }
    __syncthreads();
    // logits
    for (int i = tid; i < HQ * ATT_TE; i += ATT_THREADS) {
      const int hh = i / ATT_TE, e = i % ATT_TE;
      float s = 0.f;
      for (int d = 0; d < D; ++d) s = fmaf(qs[hh][d], kvs[e][d], s);
      lg[hh][e] = valid[e] ? s : -INFINITY;
    }
    __syncthreads();
    // online softmax per head
    if (tid < HQ) {
      float mt = mrun[tid];
      for (int e = 0; e < ATT_TE; ++e) mt = fmaxf(mt, lg[tid][e]);
      const float a = (mt == -INFINITY) ? 1.f : expf(mrun[tid] - mt);
      float ls = lrun[tid] * a;
      for (int e = 0; e < ATT_TE; ++e) {
        const float pe = (lg[tid][e] == -INFINITY) ? 0.f : expf(lg[tid][e] - mt);
        lg[tid][e] = pe;
        ls += pe;
      }
      mrun[tid] = mt; lrun[tid] = ls; alpha[tid] = a;
    }
    __syncthreads();
    const float a = alpha[h];
#pragma unroll
    for (int i = 0; i < DPT; ++i) acc[i] *= a;
    for (int e = 0; e < ATT_TE; ++e) {
      const float pe = lg[h][e];
#pragma unroll
      for (int i = 0; i < DPT; ++i) acc[i] = fmaf(pe, kvs[e][d0 + i], acc[i]);
    }
    __syncthreads();
  }

  if (S == 1) {
    // final: add the sink and normalise
    const float sk = A.sink[h];
    const float m = mrun[h];
    const float M = fmaxf(m, sk);
    const float em = (m == -INFINITY) ? 0.f : expf(m - M);
    const float Z = expf(sk - M) + lrun[h] * em;
    const float f = em / Z;
#pragma unroll
    for (int i = 0; i < DPT; ++i) store_out(A, ((int64_t)r * HQ + h) * D + d0 + i, acc[i] * f);
    if (A.lse && tid % TPH == 0) A.lse[(int64_t)r * HQ + h] = M + logf(Z);
  } else {
    const int64_t base = ((int64_t)r * S + split) * HQ + h;
#pragma unroll
    for (int i = 0; i < DPT; ++i) part_o[base * D + d0 + i] = acc[i];
    if (tid % TPH == 0) { part_ml[base * 2] = mrun[h]; part_ml[base * 2 + 1] = lrun[h]; }
  }
}

// ------------------------------------------------------------------------
// merge: combine the split partials of one row in split order with the sink
// ------------------------------------------------------------------------
__global__ __launch_bounds__(128) void attend_merge_kernel(AttendArgs A, int S, const float* part_ml,
                                                           const float* part_o) {
  const int r = blockIdx.x / A.Hq, h = blockIdx.x % A.Hq;
  const int d = threadIdx.x;
  const float sk = A.sink[h];
  float M = sk;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part_ml[(((int64_t)r * S + s) * A.Hq + h) * 2]);
  float Z = expf(sk - M), o = 0.f;
  for (int s = 0; s < S; ++s) {
    const int64_t base = ((int64_t)r * S + s) * A.Hq + h;
    const float m = part_ml[base * 2];
    if (m == -INFINITY) continue;
    const float e = expf(m - M);
    Z += part_ml[base * 2 + 1] * e;
    o = fmaf(part_o[base * A.D + d], e, o);
  }
  store_out(A, ((int64_t)r * A.Hq + h) * A.D + d, o / Z);
  if (A.lse && d == 0) A.lse[(int64_t)r * A.Hq + h] = M + logf(Z);
}

// ------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------
template <int QDT, int KVDT, int WDT>
static hipError_t launch_h(const AttendArgs& a, hipStream_t s, int S, float* ml, float* po) {
  dim3 grid(S, (unsigned)(a.B * a.Tq));
  switch (a.Hq) {
    case 16: hipLaunchKernelGGL((attend_valu_kernel<QDT, KVDT, WDT, 16>), grid, dim3(ATT_THREADS), 0, s, a, S, ml, po); break;
    case 32: hipLaunchKernelGGL((attend_valu_kernel<QDT, KVDT, WDT, 32>), grid, dim3(ATT_THREADS), 0, s, a, S, ml, po); break;
    default: hipLaunchKernelGGL((attend_valu_kernel<QDT, KVDT, WDT, 64>), grid, dim3(ATT_THREADS), 0, s, a, S, ml, po); break;
  }
  return hipGetLastError();
}

template <int QDT, int KVDT>
static hipError_t launch_w(const AttendArgs& a, hipStream_t s, int S, float* ml, float* po) {
  return a.win_dt == DT_F32 ? launch_h<QDT, KVDT, DT_F32>(a, s, S, ml, po) : launch_h<QDT, KVDT, DT_BF16>(a, s, S, ml, po);
}

template <int QDT>
static hipError_t launch_kv(const AttendArgs& a, hipStream_t s, int S, float* ml, float* po) {
  switch (a.kv_dt) {
    case DT_F32: return launch_w<QDT, DT_F32>(a, s, S, ml, po);
    case DT_BF16: return launch_w<QDT, DT_BF16>(a, s, S, ml, po);
    default: return launch_w<QDT, DT_FP8>(a, s, S, ml, po);
  }
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  const int64_t R = (int64_t)a.B * a.Tq;
  if (R == 0) return hipSuccess;
  const int64_t nkv = a.sparse ? a.k : a.N_cap;
  const int S = att_splits(R, nkv, a.W_buf);
  float* ml = nullptr;
  float* po = nullptr;
  if (S > 1) {
    ml = (float*)a.ws;
    po = (float*)((char*)a.ws + align256(sizeof(float) * R * S * a.Hq * 2));
  }
  hipError_t e = a.q_dt == DT_F32 ? launch_kv<DT_F32>(a, s, S, ml, po) : launch_kv<DT_BF16>(a, s, S, ml, po);
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3((unsigned)(R * a.Hq)), dim3(128), 0, s, a, S, ml, po);
  return hipGetLastError();
}

}  // namespace lca
