// step.hip -- one decode step of the layer pair with fewer dependent
// launches: the compress jobs in one launch, the indexer's scan and the dense
// (HCA) attention splits in one launch (they do not depend on each other),
// the indexer's select with the merge of the dense jobs' splits beside it,
// the sparse (CSA) attention splits, and the merge of the sparse jobs'
// splits.  Each part runs the kernel body of its own call
// (compress.hip, index_chunk.h, attend_mfma.h), so the results are the same
// bytes as lca_compress_batch, lca_lightning_index_topk and lca_attend_batch
// issued in that order.
//
// [release notes (agentlenshq.com), 壓縮稀疏注意力 (CSA) / 重度壓縮注意力 (HCA):
//  the HCA branch attends over every compressed entry and needs no selection,
//  only the CSA branch waits for the indexer's top-k.]
#include "attend_mfma.h"
#include "index_chunk.h"

namespace lca {

// Blocks [0, nscan) are the indexer scan (chunk bid % NCH of row group
// bid / NCH); the rest are the splits of the dense attention jobs in `bt`.
// Three workgroups per CU (168 VGPRs; the LDS union, 44.8 KB, also fits three):
// a scan that fills two workgroups per CU leaves the third to the attention.
template <int KPL, int NQ, int KVDT>
__global__ __launch_bounds__(256, 3) void step_scan_attend_kernel(IndexArgs A, IdxWs W, int NCH, int gpb, int nscan,
                                                                  AttendBatch bt) {
  __shared__ union {
    ChunkShared<NQ> ch;
    MtShared<1> at;
  } sm;
  const int bid = blockIdx.x;
  if (bid < nscan) {
    index_chunk_body<DT_MXFP4, KPL, 8, NQ>(A, W, NCH, gpb, bid % NCH, bid / NCH, sm.ch);
    return;
  }
  const int x = bid - nscan;
  int j = 0;
  while (j + 1 < bt.njobs && x >= bt.blk0[j + 1]) ++j;
  const int local = x - bt.blk0[j];
  const int S = bt.S[j];
  attend_mfma_body<KVDT, 64, 1>(bt.job[j], S, bt.items[j], bt.ml[j], bt.po[j], local % S, local / S, sm.at);
}

template <int KPL, int NQ, int KVDT>
static void launch_fused(const IndexArgs& ia, const ScanPlan& p, const AttendBatch& dense, hipStream_t s) {
  const int nscan = p.NCH * ia.B * p.gpb;
  const int nb = nscan + dense.blk0[dense.njobs];
  hipLaunchKernelGGL((step_scan_attend_kernel<KPL, NQ, KVDT>), dim3((unsigned)nb), dim3(256), 0, s, ia, p.W, p.NCH,
                     p.gpb, nscan, dense);
}

template <int NQ, int KVDT>
static void launch_fused_k(const IndexArgs& ia, const ScanPlan& p, const AttendBatch& dense, hipStream_t s) {
  switch (p.kpl) {
    case 32: launch_fused<32, NQ, KVDT>(ia, p, dense, s); break;
    case 16: launch_fused<16, NQ, KVDT>(ia, p, dense, s); break;
    default: launch_fused<4, NQ, KVDT>(ia, p, dense, s); break;
  }
}

// The jobs of `all` selected by `want`, with their plans and block offsets
// of their own.
static AttendBatch sub_batch(const AttendBatch& all, bool dense) {
  AttendBatch sub{};
  int nb = 0, nm = 0;
  for (int j = 0; j < all.njobs; ++j) {
    if ((all.job[j].sparse == 0) != dense) continue;
    const int i = sub.njobs++;
    sub.job[i] = all.job[j];
    sub.S[i] = all.S[j];
    sub.items[i] = all.items[j];
    sub.ml[i] = all.ml[j];
    sub.po[i] = all.po[j];
    sub.blk0[i] = nb;
    sub.mblk0[i] = nm;
    nb += all.blk0[j + 1] - all.blk0[j];
    nm += all.mblk0[j + 1] - all.mblk0[j];
  }
  sub.blk0[sub.njobs] = nb;
  sub.mblk0[sub.njobs] = nm;
  return sub;
}

hipError_t launch_decode_step(const AppendBatch* app, const AppendMap* mp, const CompressBatch& cb,
                              const IndexArgs& ia, const AttendBatch& ab, hipStream_t s) {
  hipError_t e;
  if (app != nullptr) {
    e = launch_append_compress(*app, *mp, cb, s);
    if (e != hipSuccess) return e;
  } else if (cb.njobs > 0) {
    e = launch_compress_batch(cb, s);
    if (e != hipSuccess) return e;
  }
  AttendBatch all = ab;
  attend_batch_plan(all);
  const AttendBatch dense = sub_batch(all, true);
  const bool fuse = ab.njobs > 0 && dense.blk0[dense.njobs] > 0 && index_scan_fusable(ia) && all.job[0].Hq == 64;
  if (!fuse) {
    e = launch_index(ia, s);
    if (e != hipSuccess) return e;
    if (ab.njobs == 0) return hipSuccess;
    e = launch_attend_batch_mfma(all, s);
    if (e != hipSuccess) return e;
    return launch_attend_batch_merge(all, s);
  }
  const ScanPlan p = index_scan_plan(ia);
  const bool fp8 = all.job[0].kv_dt == DT_FP8;
  if (p.nq == 2) {
    if (fp8) launch_fused_k<2, DT_FP8>(ia, p, dense, s);
    else launch_fused_k<2, DT_BF16>(ia, p, dense, s);
  } else {
    if (fp8) launch_fused_k<1, DT_FP8>(ia, p, dense, s);
    else launch_fused_k<1, DT_BF16>(ia, p, dense, s);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the dense jobs' partials are complete: their merge runs beside the select
  e = launch_index_select_merge(ia, p, dense, s);
  if (e != hipSuccess) return e;
  const AttendBatch sparse = sub_batch(all, false);
  if (sparse.njobs > 0) {
    e = launch_attend_batch_mfma(sparse, s);
    if (e != hipSuccess) return e;
  }
  return launch_attend_batch_merge(sparse, s);
}

}  // namespace lca
