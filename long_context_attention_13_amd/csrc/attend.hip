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
#include "attend_mfma.h"

namespace lca {

constexpr int ATT_THREADS = 256;
constexpr int ATT_TE = 32;         // items per LDS tile (VALU path)

size_t attend_ws_bytes(int B, int Tq, int Hq, int D, int64_t n_kv_max, int64_t W_buf) {
  const int64_t R = (int64_t)B * Tq;
  const Plan P = att_plan(R, n_kv_max, W_buf);
  if (P.S == 1) return 0;
  return align256(sizeof(float) * R * P.S * Hq * 2) + align256(sizeof(float) * R * P.S * Hq * D);
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
__device__ __forceinline__ float kv_elem(const void* kv, const float* kv_scale, int64_t row, int D, int d) {
  if (KVDT == DT_F32) return ((const float*)kv)[row * D + d];
  if (KVDT == DT_BF16) return bf16_to_f32(((const uint16_t*)kv)[row * D + d]);
  const uint8_t c = ((const uint8_t*)kv)[row * D + d];
  const float2 v = fp8x2_to_f32((uint32_t)c);
  return v.x * kv_scale[row * (D / 64) + d / 64];
}

template <int WDT>
__device__ __forceinline__ float win_elem(const void* win, int64_t row, int D, int d) {
  if (WDT == DT_F32) return ((const float*)win)[row * D + d];
  return bf16_to_f32(((const uint16_t*)win)[row * D + d]);
}

template <int QDT>
__device__ __forceinline__ float q_elem(const AttendArgs& A, int64_t i) {
  if (QDT == DT_F32) return ((const float*)A.q)[i];
  return bf16_to_f32(((const uint16_t*)A.q)[i]);
}

// ------------------------------------------------------------------------
// fp32 VALU kernel (any storage types; used for F32 inputs and for separate
// values: the value tile is staged beside the key tile).
// ------------------------------------------------------------------------
template <int QDT, int KVDT, int WDT, int HQ>
__global__ __launch_bounds__(ATT_THREADS) void attend_valu_kernel(AttendArgs A, int S, int split_items, float* part_ml,
                                                                   float* part_o) {
  constexpr int D = 128;
  constexpr int TPH = ATT_THREADS / HQ;      // threads per head
  constexpr int DPT = D / TPH;               // output dims per thread
  const int split = blockIdx.x, r = blockIdx.y;
  const int b = r / A.Tq;
  const int tid = threadIdx.x;
  const int nkv = A.sparse ? A.k : A.n_elig[r];
  const int L = nkv + A.win_len[r];
  const int p0 = split * split_items;
  const int p1 = S == 1 ? L : min(L, p0 + split_items);
  if (S > 1 && p0 >= L) return;             // an empty split: the merge does not read it

  __shared__ float qs[HQ][D];
  __shared__ float kvs[ATT_TE][D + 1];
  __shared__ float vls[ATT_TE][D + 1];          // values, when they are separate
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
      float v = 0.f, vv = 0.f;
      int ok = 0;
      if (p < p1) {
        const ListItem it = list_item(A, b, r, p, nkv);
        if (it.kind == 0) {
          v = kv_elem<KVDT>(A.kv, A.kv_scale, it.row, D, d);
          if (A.v) vv = kv_elem<KVDT>(A.v, A.v_scale, it.row, D, d);
          ok = 1;
        } else if (it.kind == 1) {
          v = win_elem<WDT>(A.win, it.row, D, d);
          if (A.v) vv = win_elem<WDT>(A.win_v, it.row, D, d);
          ok = 1;
        }
      }
      kvs[e][d] = v;
      if (A.v) vls[e][d] = vv;
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
    float (*vals)[D + 1] = A.v ? vls : kvs;
    for (int e = 0; e < ATT_TE; ++e) {
      const float pe = lg[h][e];
#pragma unroll
      for (int i = 0; i < DPT; ++i) acc[i] = fmaf(pe, vals[e][d0 + i], acc[i]);
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
    if (tid % TPH == 0) {
      // partial maxima in base 2, as the matrix-core kernel writes them
      part_ml[base * 2] = mrun[h] == -INFINITY ? -INFINITY : mrun[h] * LOG2E;
      part_ml[base * 2 + 1] = lrun[h];
    }
  }
}

// ------------------------------------------------------------------------
// bf16 matrix-core kernel: bf16 queries, bf16 or FP8 items, bf16 window.
//
// Each wavefront owns 16 heads; the workgroup's waves share one LDS copy of
// each 64-item tile.  Per tile:
//   S^T = K Q^T      16x16x32 bf16 MFMA, items x heads (K from LDS, Q^T in
//                    registers).  FP8 items are staged as their exact bf16
//                    codes; the two per-64 scales multiply the fp32 partial
//                    dot products of dims 0-63 and 64-127.
//   online softmax   per head = per lane column; the max over a tile's items
//                    is one in-lane max plus two cross-lane steps.
//   O^T += V^T P^T   16x16x32 bf16 MFMA, dims x heads.  The B operand is the
//                    softmax numerator straight from the S^T accumulator
//                    layout (items taken in a permuted order that the V^T
//                    reads follow), with the FP8 scales folded in.
// The next tile's items are fetched into registers while the current one is
// computed.
template <int KVDT, int HQ, int QB>
__global__ __launch_bounds__(HQ * 4 * QB, HQ * 4 * QB == 256 ? 2 : 1) void attend_mfma_kernel(
    AttendArgs A, int S, int split_items, float* part_ml, float* part_o) {
  __shared__ MtShared<QB> sm;
  attend_mfma_body<KVDT, HQ, QB>(A, S, split_items, part_ml, part_o, blockIdx.x, blockIdx.y, sm);
}

__global__ __launch_bounds__(128) void attend_merge_kernel(AttendArgs A, int S, int split_items, const float* part_ml,
                                                           const float* part_o) {
  __shared__ MgShared sm;
  attend_merge_body(A, S, split_items, part_ml, part_o, blockIdx.x, sm);
}

// Several attention calls in one launch: block x of the grid is block
// x - blk0[j] of job j, i.e. split (x - blk0[j]) % S[j] of row (x - blk0[j]) / S[j].
template <int KVDT, int HQ>
__global__ __launch_bounds__(HQ * 4, HQ * 4 == 256 ? 2 : 1) void attend_mfma_batch_kernel(AttendBatch bt) {
  __shared__ MtShared<1> sm;
  int j = 0;
  while (j + 1 < bt.njobs && (int)blockIdx.x >= bt.blk0[j + 1]) ++j;
  const int local = (int)blockIdx.x - bt.blk0[j];
  const int S = bt.S[j];
  attend_mfma_body<KVDT, HQ, 1>(bt.job[j], S, bt.items[j], bt.ml[j], bt.po[j], local % S, local / S, sm);
}

__global__ __launch_bounds__(128) void attend_merge_batch_kernel(AttendBatch bt) {
  __shared__ MgShared sm;
  int j = 0;
  while (j + 1 < bt.njobs && (int)blockIdx.x >= bt.mblk0[j + 1]) ++j;
  attend_merge_body(bt.job[j], bt.S[j], bt.items[j], bt.ml[j], bt.po[j], (int)blockIdx.x - bt.mblk0[j], sm);
}

// ------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------
template <int QDT, int KVDT, int WDT>
static hipError_t launch_h(const AttendArgs& a, hipStream_t s, Plan P, float* ml, float* po) {
  dim3 grid(P.S, (unsigned)(a.B * a.Tq));
  switch (a.Hq) {
    case 16: hipLaunchKernelGGL((attend_valu_kernel<QDT, KVDT, WDT, 16>), grid, dim3(ATT_THREADS), 0, s, a, P.S, P.items, ml, po); break;
    case 32: hipLaunchKernelGGL((attend_valu_kernel<QDT, KVDT, WDT, 32>), grid, dim3(ATT_THREADS), 0, s, a, P.S, P.items, ml, po); break;
    default: hipLaunchKernelGGL((attend_valu_kernel<QDT, KVDT, WDT, 64>), grid, dim3(ATT_THREADS), 0, s, a, P.S, P.items, ml, po); break;
  }
  return hipGetLastError();
}

template <int QDT, int KVDT>
static hipError_t launch_w(const AttendArgs& a, hipStream_t s, Plan P, float* ml, float* po) {
  return a.win_dt == DT_F32 ? launch_h<QDT, KVDT, DT_F32>(a, s, P, ml, po) : launch_h<QDT, KVDT, DT_BF16>(a, s, P, ml, po);
}

template <int QDT>
static hipError_t launch_kv(const AttendArgs& a, hipStream_t s, Plan P, float* ml, float* po) {
  switch (a.kv_dt) {
    case DT_F32: return launch_w<QDT, DT_F32>(a, s, P, ml, po);
    case DT_BF16: return launch_w<QDT, DT_BF16>(a, s, P, ml, po);
    default: return launch_w<QDT, DT_FP8>(a, s, P, ml, po);
  }
}

template <int KVDT, int HQ>
static void launch_mfma_h(const AttendArgs& a, hipStream_t s, Plan P, float* ml, float* po) {
  constexpr int QB = att_qb<HQ>();
  if (!a.sparse && P.S == 1 && a.Tq >= 2 * QB) {
    if (attend_dense_wide_applies(a)) {
      (void)launch_attend_dense_wide(a, s);   // the caller reads hipGetLastError
      return;
    }
    dim3 grid(1, (unsigned)(a.B * ((a.Tq + QB - 1) / QB)));
    hipLaunchKernelGGL((attend_mfma_kernel<KVDT, HQ, QB>), grid, dim3(HQ * 4 * QB), 0, s, a, 1, P.items, ml, po);
  } else if (a.sparse && P.S == 1 && attend_sparse_wide_applies(a)) {
    (void)launch_attend_sparse_wide(a, s);   // the caller reads hipGetLastError
  } else {
    dim3 grid(P.S, (unsigned)(a.B * a.Tq));
    hipLaunchKernelGGL((attend_mfma_kernel<KVDT, HQ, 1>), grid, dim3(HQ * 4), 0, s, a, P.S, P.items, ml, po);
  }
}

template <int KVDT>
static hipError_t launch_mfma(const AttendArgs& a, hipStream_t s, Plan P, float* ml, float* po) {
  switch (a.Hq) {
    case 16: launch_mfma_h<KVDT, 16>(a, s, P, ml, po); break;
    case 32: launch_mfma_h<KVDT, 32>(a, s, P, ml, po); break;
    default: launch_mfma_h<KVDT, 64>(a, s, P, ml, po); break;
  }
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  const int64_t R = (int64_t)a.B * a.Tq;
  if (R == 0) return hipSuccess;
  const int64_t nkv = a.sparse ? a.k : a.N_cap;
  const Plan P = att_plan(R, nkv, a.W_buf);
  float* ml = nullptr;
  float* po = nullptr;
  if (P.S > 1) {
    ml = (float*)a.ws;
    po = (float*)((char*)a.ws + align256(sizeof(float) * R * P.S * a.Hq * 2));
  }
  hipError_t e;
  const bool mfma = a.q_dt == DT_BF16 && a.win_dt == DT_BF16 && (a.kv_dt == DT_BF16 || a.kv_dt == DT_FP8) && !a.v;
  if (mfma) e = a.kv_dt == DT_FP8 ? launch_mfma<DT_FP8>(a, s, P, ml, po) : launch_mfma<DT_BF16>(a, s, P, ml, po);
  else e = a.q_dt == DT_F32 ? launch_kv<DT_F32>(a, s, P, ml, po) : launch_kv<DT_BF16>(a, s, P, ml, po);
  if (e != hipSuccess || P.S == 1) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3((unsigned)(R * a.Hq)), dim3(128), 0, s, a, P.S, P.items, ml, po);
  return hipGetLastError();
}

// A call the batch launcher can take: the bf16-MFMA path in its one-row,
// split layout (not a prefill-shaped call -- many rows, no split -- which
// the single call runs with the grouped dense layout or the wide kernels).
bool attend_batchable(const AttendArgs& a) {
  const bool mfma = a.q_dt == DT_BF16 && a.win_dt == DT_BF16 && (a.kv_dt == DT_BF16 || a.kv_dt == DT_FP8) && !a.v;
  if (!mfma) return false;
  const int64_t R = (int64_t)a.B * a.Tq;
  const Plan P = att_plan(R, a.sparse ? a.k : a.N_cap, a.W_buf);
  const int qb = a.Hq == 16 ? att_qb<16>() : a.Hq == 32 ? att_qb<32>() : att_qb<64>();
  if (a.sparse) return !(P.S == 1 && attend_sparse_wide_applies(a));
  return !(P.S == 1 && a.Tq >= 2 * qb);
}

void attend_batch_plan(AttendBatch& bt) {
  int nb = 0, nm = 0;
  for (int j = 0; j < bt.njobs; ++j) {
    const AttendArgs& a = bt.job[j];
    const int64_t R = (int64_t)a.B * a.Tq;
    const Plan P = att_plan(R, a.sparse ? a.k : a.N_cap, a.W_buf);
    bt.S[j] = P.S;
    bt.items[j] = P.items;
    bt.ml[j] = P.S > 1 ? (float*)a.ws : nullptr;
    bt.po[j] = P.S > 1 ? (float*)((char*)a.ws + align256(sizeof(float) * R * P.S * a.Hq * 2)) : nullptr;
    bt.blk0[j] = nb;
    bt.mblk0[j] = nm;
    nb += (int)(R * P.S);
    nm += P.S > 1 ? (int)(R * a.Hq) : 0;
  }
  bt.blk0[bt.njobs] = nb;
  bt.mblk0[bt.njobs] = nm;
}

hipError_t launch_attend_batch_mfma(const AttendBatch& bt, hipStream_t s) {
  const int nb = bt.blk0[bt.njobs];
  if (nb == 0) return hipSuccess;
  const bool fp8 = bt.job[0].kv_dt == DT_FP8;
  switch (bt.job[0].Hq) {
    case 16:
      if (fp8) hipLaunchKernelGGL((attend_mfma_batch_kernel<DT_FP8, 16>), dim3(nb), dim3(64), 0, s, bt);
      else hipLaunchKernelGGL((attend_mfma_batch_kernel<DT_BF16, 16>), dim3(nb), dim3(64), 0, s, bt);
      break;
    case 32:
      if (fp8) hipLaunchKernelGGL((attend_mfma_batch_kernel<DT_FP8, 32>), dim3(nb), dim3(128), 0, s, bt);
      else hipLaunchKernelGGL((attend_mfma_batch_kernel<DT_BF16, 32>), dim3(nb), dim3(128), 0, s, bt);
      break;
    default:
      if (fp8) hipLaunchKernelGGL((attend_mfma_batch_kernel<DT_FP8, 64>), dim3(nb), dim3(256), 0, s, bt);
      else hipLaunchKernelGGL((attend_mfma_batch_kernel<DT_BF16, 64>), dim3(nb), dim3(256), 0, s, bt);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_attend_batch_merge(const AttendBatch& bt, hipStream_t s) {
  const int nm = bt.mblk0[bt.njobs];
  if (nm == 0) return hipSuccess;
  hipLaunchKernelGGL(attend_merge_batch_kernel, dim3(nm), dim3(128), 0, s, bt);
  return hipGetLastError();
}

hipError_t launch_attend_batch(const AttendBatch& in, hipStream_t s) {
  AttendBatch bt = in;
  attend_batch_plan(bt);
  const hipError_t e = launch_attend_batch_mfma(bt, s);
  if (e != hipSuccess) return e;
  return launch_attend_batch_merge(bt, s);
}

}  // namespace lca
