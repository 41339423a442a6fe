// index.hip -- lightning indexer scoring and exact top-k selection on gfx950.
//
// [release notes (agentlenshq.com), 壓縮稀疏注意力 (CSA): the lightning indexer
//  scores compressed blocks with ReLU-scored multi-head dot products in FP4
//  and keeps the top-k per query; wiki (chenshi221), 基础设施: MXFP4 on the
//  indexer QK path.]
//
// Score of entry j for query row r:  s_j = sum_h w_h * max(0, <q_h, k_j>),
// evaluated so that it equals the float64 left-to-right evaluation exactly:
//   * MXFP4: one scaled FP4 MFMA (16x16x128) gives the per-head dot products
//     of 16 keys.  E2M1 products are multiples of 1/4 below 36, so a 32-element
//     block sum is an integer multiple of 2^(e-2) below 2^(e+11); with at most
//     four blocks whose scale exponents differ by <= 9 every partial sum fits
//     in 24 bits and the fp32 result is exact, whatever the internal order.
//     Keys outside that envelope take an exact float64 path.
//   * F32: float64 FMA chain over the elements (fp32 products are exact in
//     float64, so fma == add of the rounded product).
//   * head combine: float64 multiply then add, in head order.
// Selection orders by (s desc, j asc).  Scores map to uint64 keys that order
// like the doubles.
//
// Two kernels:
//   chunk kernel  one wavefront scores CH = 64*KPL consecutive entries for one
//                 or two query rows (rows 0-7 / 8-15 of the MFMA A operand),
//                 keeps each lane's best key, sorts the 64 lane maxima with a
//                 wavefront bitonic network, and emits every entry whose key
//                 reaches the r-th lane maximum (r from the expected number
//                 of top-k entries in a chunk), plus the largest key it did
//                 NOT emit.  This streams the MXFP4 key cache once.
//   select kernel one 1024-thread workgroup per query row runs an exact radix
//                 select over the candidates, then certifies: if any chunk's
//                 largest excluded key could rank inside the result (or a
//                 chunk overflowed), the row is redone from scratch by
//                 re-scoring every entry in streamed passes.  Rows with few
//                 entries are always done that way.  Output in ascending index
//                 order through an LDS bitmap.
#include "attend_mfma.h"
#include "index_chunk.h"
#include "index_select.h"

namespace lca {

template <int DT, int KPL, int HP, int NQ>
__global__ __launch_bounds__(256) void index_chunk_kernel(IndexArgs A, IdxWs W, int NCH, int groups_per_b) {
  __shared__ ChunkShared<NQ> sm;
  index_chunk_body<DT, KPL, HP, NQ>(A, W, NCH, groups_per_b, blockIdx.x, blockIdx.y, sm);
}

template <int DT, int HP>
__global__ __launch_bounds__(SEL_THREADS) void index_select_kernel(IndexArgs A, IdxWs W, int NCH, int CH) {
  extern __shared__ __align__(16) char smem[];
  index_select_body<DT, HP>(A, W, NCH, CH, blockIdx.x, smem);
}

// The selection of the decode step with the merge of the dense attention
// jobs' split partials in the same launch (they are complete once the scan
// launch is, and the selection occupies one workgroup per row): blocks
// [0, B*Tq) select a row each; each later block merges SEL_THREADS / 128
// (row, head) units, 128 threads per unit.
template <int DT, int HP>
__global__ __launch_bounds__(SEL_THREADS) void index_select_merge_kernel(IndexArgs A, IdxWs W, int NCH, int CH,
                                                                         AttendBatch mb) {
  extern __shared__ __align__(16) char smem[];
  const int nsel = A.B * A.Tq;
  if ((int)blockIdx.x < nsel) {
    index_select_body<DT, HP>(A, W, NCH, CH, blockIdx.x, smem);
    return;
  }
  constexpr int UPB = SEL_THREADS / 128;
  const int units = mb.mblk0[mb.njobs];
  const int g = threadIdx.x >> 7;
  int u = ((int)blockIdx.x - nsel) * UPB + g;
  const bool real = u < units;
  if (!real) u = units - 1;               // takes part in the barriers only
  int j = 0;
  while (j + 1 < mb.njobs && u >= mb.mblk0[j + 1]) ++j;
  MgShared& sm = ((MgShared*)smem)[g];
  attend_merge_body<true, 16, 16>(mb.job[j], mb.S[j], mb.items[j], mb.ml[j], mb.po[j], u - mb.mblk0[j], sm, real);
}

// ------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------
size_t index_ws_bytes(int B, int Tq, int H, int d, int64_t N_cap, int k, int dt) {
  IndexArgs a{};
  a.B = B; a.Tq = Tq; a.H = H; a.d = d; a.N_cap = N_cap; a.k = k; a.dt = dt;
  if (index_prefill_applies(a)) return index_prefill_ws_bytes(B, Tq, N_cap, k);
  const int kpl = choose_kpl(a, nq_of(dt, H, Tq));
  const int64_t NCH = (N_cap + 64 * kpl - 1) / (64 * kpl);
  return carve_bytes((int64_t)B * Tq, NCH > 0 ? NCH : 1);
}

template <int DT, int KPL, int HP, int NQ>
static hipError_t launch_t(const IndexArgs& a, hipStream_t s) {
  const int CH = 64 * KPL;
  const int64_t NCH = (a.N_cap + CH - 1) / CH;
  IdxWs W = carve(a.ws, (int64_t)a.B * a.Tq, NCH > 0 ? NCH : 1);
  const int gpb = (a.Tq + NQ - 1) / NQ;
  if (a.N_cap > NDIRECT) {
    dim3 grid((unsigned)NCH, (unsigned)(a.B * gpb));
    hipLaunchKernelGGL((index_chunk_kernel<DT, KPL, HP, NQ>), grid, dim3(256), 0, s, a, W, (int)NCH, gpb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t smem = select_smem(DT, a.H, a.d);
  hipLaunchKernelGGL((index_select_kernel<DT, HP>), dim3((unsigned)(a.B * a.Tq)), dim3(SEL_THREADS), smem, s, a, W,
                     (int)NCH, CH);
  return hipGetLastError();
}

template <int DT, int HP, int NQ>
static hipError_t launch_k(const IndexArgs& a, hipStream_t s) {
  switch (choose_kpl(a, NQ)) {
    case 32: return launch_t<DT, 32, HP, NQ>(a, s);
    case 16: return launch_t<DT, 16, HP, NQ>(a, s);
    default: return launch_t<DT, 4, HP, NQ>(a, s);
  }
}

// The decode chunk path of an MXFP4 indexer with at most 8 heads, whose scan
// a fused launch can run (the select then runs on its own).
bool index_scan_fusable(const IndexArgs& a) {
  return (int64_t)a.B * a.Tq > 0 && !index_prefill_applies(a) && a.dt == DT_MXFP4 && a.H <= 8 && a.N_cap > NDIRECT;
}

hipError_t launch_index_select_merge(const IndexArgs& a, const ScanPlan& p, const AttendBatch& mb, hipStream_t s) {
  constexpr int UPB = SEL_THREADS / 128;
  static_assert(UPB * sizeof(MgShared) <= sizeof(SelShared) + 12 * (size_t)CMAX, "merge units fit the LDS");
  const int units = mb.mblk0[mb.njobs];
  const size_t smem = select_smem(DT_MXFP4, a.H, a.d);
  const unsigned nb = (unsigned)(a.B * a.Tq + (units + UPB - 1) / UPB);
  hipLaunchKernelGGL((index_select_merge_kernel<DT_MXFP4, 8>), dim3(nb), dim3(SEL_THREADS), smem, s, a, p.W, p.NCH,
                     p.CH, mb);
  return hipGetLastError();
}

hipError_t launch_index_select(const IndexArgs& a, const ScanPlan& p, hipStream_t s) {
  const size_t smem = select_smem(DT_MXFP4, a.H, a.d);
  hipLaunchKernelGGL((index_select_kernel<DT_MXFP4, 8>), dim3((unsigned)(a.B * a.Tq)), dim3(SEL_THREADS), smem, s, a,
                     p.W, p.NCH, p.CH);
  return hipGetLastError();
}

hipError_t launch_index(const IndexArgs& a, hipStream_t s) {
  if ((int64_t)a.B * a.Tq == 0) return hipSuccess;
  if (index_prefill_applies(a)) return launch_index_prefill(a, s);
  const int nq = nq_of(a.dt, a.H, a.Tq);
  if (a.dt == DT_MXFP4) {
    if (a.H <= 8) return nq == 2 ? launch_k<DT_MXFP4, 8, 2>(a, s) : launch_k<DT_MXFP4, 8, 1>(a, s);
    return launch_k<DT_MXFP4, 16, 1>(a, s);
  }
  return launch_k<DT_F32, 16, 1>(a, s);
}

}  // namespace lca
