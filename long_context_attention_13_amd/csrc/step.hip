// step.hip -- one decode step of the layer pair with fewer dependent
// launches: the compress jobs, the indexer's scan and the dense (HCA)
// attention splits in one launch (nothing in it waits for another part: the
// scan and attention workgroups that read a row the step compresses compute
// that row themselves),
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
#include "compress_body.h"
#include "index_chunk.h"

namespace lca {

// The compress jobs can join the scan launch when nothing in it waits for
// them: the compress workgroups write the caches, and the scan workgroup
// whose chunk holds a sequence's new key row (or the attention split whose
// range holds its new entry) computes that row itself from the raw tokens
// with the same code, so it reads the bytes the compress job writes.
struct StepFold {
  int ncomp;                          // compress workgroups at the front of the grid (0: none)
  int bmax;                           // workgroups per compress job
  int key;                            // the compress job writing the indexer keys (-1: none)
  int ent[MAX_ATTEND_JOBS];           // per dense job: the compress job writing its entries (-1: none)
};

// Row 0 of `code` / `scale` (any address space) = the row compress job k
// writes for sequence b (its block 0; bf16 tokens, width 128).
template <int ODT>
__device__ __forceinline__ void fresh_row(const CompressArgs& k, int b, void* code, void* scale, int64_t* zero,
                                          PeShared& pe) {
  CompressArgs a = k;
  a.x = (const char*)k.x + (int64_t)b * k.x_rows * 128 * 2;
  a.gate = k.gate + (int64_t)b * k.x_rows * (k.gate_pc ? 128 : 1);
  a.x_tok0 = k.x_tok0 + b;
  a.nblk = k.nblk + b;
  a.dst_row0 = zero;
  a.dst = code;
  a.dst_scale = scale;
  a.dst_rows = 1;
  a.pooled = nullptr;
  a.B = 1;
  a.nblk_max = 1;
  pool_encode_block<DT_BF16, ODT, 128>(a, 0, 0, pe);
}

// After the compress blocks come the splits of the dense attention jobs in
// `bt`, then the nscan blocks of the indexer scan (chunk i % NCH of row group
// i / NCH for scan block i): the splits are dispatched first, so their
// gathers and partial writes start ahead of the scan's stream instead of
// trailing it (about 1 us less per step at the 1M layer pair).
// Three workgroups per CU with 2048-key chunks (the long contexts: 168
// VGPRs; the LDS union, 44.8 KB, also fits three): a scan that fills two
// workgroups per CU leaves the third to the attention.  The smaller chunks
// need more registers and take two.
// With fd.ncomp > 0 the first fd.ncomp blocks are the compress jobs (job
// bid / bmax, sequence bid % bmax), in front of the scan and attention blocks.
template <int KPL, int NQ, int KVDT>
__global__ __launch_bounds__(256, KPL == 32 ? 3 : 2) void step_scan_attend_kernel(IndexArgs A, IdxWs W, int NCH, int gpb, int nscan,
                                                                  AttendBatch bt, CompressBatch cb, StepFold fd) {
  __shared__ union {
    ChunkShared<NQ> ch;
    MtShared<1> at;
    PeShared pe;
  } sm;
  __shared__ __align__(16) uint8_t fresh[256 + 16];
  __shared__ int64_t zero;
  int bid = blockIdx.x;
  if (bid < fd.ncomp) {
    const CompressArgs& a = cb.job[bid / fd.bmax];
    const int b = bid % fd.bmax;
    if (b >= a.B) return;
    switch (a.dst_dt) {
      case DT_F32: pool_encode_block<DT_BF16, DT_F32, 128>(a, b, 0, sm.pe); break;
      case DT_BF16: pool_encode_block<DT_BF16, DT_BF16, 128>(a, b, 0, sm.pe); break;
      case DT_FP8: pool_encode_block<DT_BF16, DT_FP8, 128>(a, b, 0, sm.pe); break;
      default: pool_encode_block<DT_BF16, DT_MXFP4, 128>(a, b, 0, sm.pe); break;
    }
    return;
  }
  bid -= fd.ncomp;
  const int ndense = bt.blk0[bt.njobs];
  bid = bid < ndense ? bid + nscan : bid - ndense;     // [0, nscan): scan; then the splits
  if (threadIdx.x == 0) zero = 0;
  __syncthreads();
  if (bid < nscan) {
    const int c = bid % NCH, g = bid / NCH;
    FreshKey F{-1, fresh, fresh + 64};
    if (fd.key >= 0) {
      const CompressArgs& k = cb.job[fd.key];
      const int b = g / gpb;
      const int jn = k.nblk[b] > 0 ? (int)k.dst_row0[b] : -1;
      if (jn >= c * 64 * KPL && jn < (c + 1) * 64 * KPL) {     // uniform over the workgroup
        fresh_row<DT_MXFP4>(k, b, fresh, fresh + 64, &zero, sm.pe);
        __syncthreads();
        F.j = jn;
      }
    }
    index_chunk_body<DT_MXFP4, KPL, 8, NQ>(A, W, NCH, gpb, c, g, sm.ch, F);
    return;
  }
  const int x = bid - nscan;
  int j = 0;
  while (j + 1 < bt.njobs && x >= bt.blk0[j + 1]) ++j;
  const int local = x - bt.blk0[j];
  const int S = bt.S[j];
  FreshEnt fe{-1, fresh, (const float*)(fresh + 128)};
  if (fd.ent[j] >= 0) {
    const CompressArgs& k = cb.job[fd.ent[j]];
    const AttendArgs& aj = bt.job[j];
    const int r = local / S, b = r / aj.Tq;
    const int en = k.nblk[b] > 0 ? (int)k.dst_row0[b] : -1;
    const int p0 = (local % S) * bt.items[j];
    if (en >= p0 && en < p0 + bt.items[j] && en < att_nelig(aj, r)) {   // uniform over the workgroup
      fresh_row<KVDT>(k, b, fresh, fresh + 128, &zero, sm.pe);
      __syncthreads();
      fe.j = en;
    }
  }
  attend_mfma_body<KVDT, 64, 1>(bt.job[j], S, bt.items[j], bt.ml[j], bt.po[j], local % S, local / S, sm.at, fe);
}

template <int KPL, int NQ, int KVDT>
static void launch_fused(const IndexArgs& ia, const ScanPlan& p, const AttendBatch& dense, const CompressBatch& cb,
                         const StepFold& fd, hipStream_t s) {
  const int nscan = p.NCH * ia.B * p.gpb;
  const int nb = fd.ncomp + nscan + dense.blk0[dense.njobs];
  hipLaunchKernelGGL((step_scan_attend_kernel<KPL, NQ, KVDT>), dim3((unsigned)nb), dim3(256), 0, s, ia, p.W, p.NCH,
                     p.gpb, nscan, dense, cb, fd);
}

template <int NQ, int KVDT>
static void launch_fused_k(const IndexArgs& ia, const ScanPlan& p, const AttendBatch& dense, const CompressBatch& cb,
                           const StepFold& fd, hipStream_t s) {
  switch (p.kpl) {
    case 32: launch_fused<32, NQ, KVDT>(ia, p, dense, cb, fd, s); break;
    case 16: launch_fused<16, NQ, KVDT>(ia, p, dense, cb, fd, s); break;
    default: launch_fused<4, NQ, KVDT>(ia, p, dense, cb, fd, s); break;
  }
}

static StepFold no_fold() {
  StepFold fd{};
  fd.key = -1;
  for (int j = 0; j < MAX_ATTEND_JOBS; ++j) fd.ent[j] = -1;
  return fd;
}

// Byte ranges of the buffers the fused launch touches, for the aliasing
// checks of plan_fold (a null pointer is an empty range).
struct Span {
  const char* lo;
  const char* hi;
};
static Span span(const void* p, int64_t bytes) {
  const char* c = (const char*)p;
  return p ? Span{c, c + bytes} : Span{nullptr, nullptr};
}
static bool overlap(const Span& a, const Span& b) { return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi; }
static bool same(const Span& a, const Span& b) { return a.lo == b.lo && a.hi == b.hi; }
static int64_t row_bytes(int dt, int D) { return dt == DT_F32 ? 4 * D : dt == DT_BF16 ? 2 * D : dt == DT_FP8 ? D : D / 2; }
static int64_t scale_row_bytes(int dt, int D) { return dt == DT_FP8 ? D / 64 * 4 : dt == DT_MXFP4 ? D / 32 : 0; }

// Which compress jobs the scan launch can take (see StepFold); ncomp = 0 when
// they cannot all be taken (they then run in a launch of their own first).
// Nothing in the fused launch may read what a compress job writes, except the
// indexer keys (written as exactly the key cache: same rows, same layout) and
// a dense job's entries (exactly that job's cache), whose new rows the readers
// compute themselves; and no compress job may read what the launch writes.
static StepFold plan_fold(const CompressBatch& cb, const IndexArgs& ia, const AttendBatch& dense) {
  StepFold fd = no_fold();
  const int64_t R = (int64_t)ia.B * ia.Tq;
  const Span ki = span(ia.ki, ia.B * ia.N_cap * ia.d / 2), kis = span(ia.ki_scale, ia.B * ia.N_cap * ia.d / 32);
  // what the scan reads (besides the keys) and writes
  const Span scan_in[] = {span(ia.qi, R * ia.H * ia.d / 2), span(ia.qi_scale, R * ia.H * ia.d / 32),
                          span(ia.w, R * ia.H * 4), span(ia.n_elig, R * 4)};
  const Span scan_out = span(ia.ws, (int64_t)ia.ws_bytes);
  int bmax = 0;
  for (int c = 0; c < cb.njobs; ++c) {
    const CompressArgs& k = cb.job[c];
    if (k.B == 0) continue;
    if (k.nblk_max != 1 || k.overlap != 0 || k.x_dt != DT_BF16 || k.D != 128) return no_fold();
    bmax = k.B > bmax ? k.B : bmax;
    const Span dst = span(k.dst, k.B * k.dst_rows * row_bytes(k.dst_dt, k.D));
    const Span dsc = span(k.dst_scale, k.B * k.dst_rows * scale_row_bytes(k.dst_dt, k.D));
    const Span pooled = span(k.pooled, (int64_t)k.B * k.nblk_max * k.D * 4);
    const Span outs[] = {dst, dsc, pooled};
    const Span ins[] = {span(k.x, k.B * k.x_rows * k.D * 2), span(k.gate, k.B * k.x_rows * (k.gate_pc ? k.D : 1) * 4),
                        span(k.bias, (int64_t)(k.m + k.overlap) * (k.gate_pc ? k.D : 1) * 4),
                        span(k.x_tok0, k.B * 4), span(k.nblk, k.B * 4), span(k.dst_row0, k.B * 8)};
    for (const Span& in : ins)
      if (overlap(in, scan_out)) return no_fold();
    for (const Span& o : outs)
      for (const Span& r : scan_in)
        if (overlap(o, r) || overlap(o, scan_out)) return no_fold();
    // the indexer keys: written exactly as the key cache, or not at all
    if (overlap(dst, ki) || overlap(dst, kis) || overlap(dsc, ki) || overlap(dsc, kis) || overlap(pooled, ki) ||
        overlap(pooled, kis)) {
      if (!same(dst, ki) || !same(dsc, kis) || k.dst_dt != DT_MXFP4 || ia.dt != DT_MXFP4 || ia.d != 128 ||
          k.B != ia.B || k.dst_rows != ia.N_cap || fd.key >= 0)
        return no_fold();
      fd.key = c;
    }
    for (int j = 0; j < dense.njobs; ++j) {
      const AttendArgs& a = dense.job[j];
      const int64_t Ra = (int64_t)a.B * a.Tq;
      const Span kv = span(a.kv, a.B * a.N_cap * row_bytes(a.kv_dt, a.D));
      const Span kvs = span(a.kv_scale, a.B * a.N_cap * scale_row_bytes(a.kv_dt, a.D));
      const Span a_in[] = {span(a.q, Ra * a.Hq * a.D * 2), span(a.win, a.B * a.W_buf * a.D * 2),
                           span(a.win_begin, Ra * 4), span(a.win_len, Ra * 4), span(a.sink, (int64_t)a.Hq * 4),
                           span(a.n_elig, Ra * 4)};
      const Span a_out[] = {span(a.ws, (int64_t)a.ws_bytes), span(a.out, Ra * a.Hq * a.D * (a.out_dt == DT_F32 ? 4 : 2)),
                            span(a.lse, Ra * a.Hq * 4)};
      for (const Span& in : ins)
        for (const Span& w : a_out)
          if (overlap(in, w)) return no_fold();
      for (const Span& o : outs) {
        for (const Span& r : a_in)
          if (overlap(o, r)) return no_fold();
        for (const Span& w : a_out)
          if (overlap(o, w)) return no_fold();
      }
      if (overlap(dst, kv) || overlap(dst, kvs) || overlap(dsc, kv) || overlap(dsc, kvs) || overlap(pooled, kv) ||
          overlap(pooled, kvs)) {
        if (!same(dst, kv) || !same(dsc, kvs) || k.dst_dt != a.kv_dt || k.B != a.B || k.dst_rows != a.N_cap ||
            fd.ent[j] >= 0)
          return no_fold();
        fd.ent[j] = c;
      }
    }
  }
  fd.bmax = bmax;
  fd.ncomp = cb.njobs * bmax;
  return fd;
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

static bool compress_work(const CompressBatch& cb) {
  for (int c = 0; c < cb.njobs; ++c)
    if (cb.job[c].B > 0 && cb.job[c].nblk_max > 0) return true;
  return false;
}

hipError_t log_start(LaunchLog* lg, hipStream_t s) {
  if (lg == nullptr) return hipSuccess;
  lg->n = 0;
  return lg->cap > 0 ? hipEventRecord(lg->ev[0], s) : hipSuccess;
}

hipError_t log_launch(LaunchLog* lg, hipStream_t s, const char* name) {
  if (lg == nullptr || lg->n + 1 >= lg->cap) return hipSuccess;
  if (lg->names) lg->names[lg->n] = name;
  lg->n++;
  return hipEventRecord(lg->ev[lg->n], s);
}

hipError_t launch_decode_step(const AppendBatch* app, const AppendMap* mp, const CompressBatch& cb,
                              const IndexArgs& ia, const AttendBatch& ab, hipStream_t s, LaunchLog* lg) {
  hipError_t e = log_start(lg, s);
  if (e != hipSuccess) return e;
  AttendBatch all = ab;
  attend_batch_plan(all);
  const AttendBatch dense = sub_batch(all, true);
  const bool fuse = ab.njobs > 0 && dense.blk0[dense.njobs] > 0 && index_scan_fusable(ia) && all.job[0].Hq == 64;
  // the compress jobs join the scan launch when they can (the appends, if
  // any, then run in a launch of their own first); otherwise they run first,
  // with the appends in the same launch
  const StepFold fd = fuse ? plan_fold(cb, ia, dense) : no_fold();
  if (app != nullptr && fd.ncomp > 0) {
    e = launch_decode_append(*app, s);
    if (e == hipSuccess) e = log_launch(lg, s, "decode_append_kernel");
    if (e != hipSuccess) return e;
  } else if (app != nullptr) {
    e = launch_append_compress(*app, *mp, cb, s);
    if (e == hipSuccess) e = log_launch(lg, s, "append_compress_kernel");
    if (e != hipSuccess) return e;
  } else if (cb.njobs > 0 && fd.ncomp == 0) {
    e = launch_compress_batch(cb, s);
    if (e == hipSuccess && compress_work(cb)) e = log_launch(lg, s, "pool_encode_batch_kernel");
    if (e != hipSuccess) return e;
  }
  if (!fuse) {
    e = launch_index(ia, s);
    if (e == hipSuccess && (int64_t)ia.B * ia.Tq > 0) e = log_launch(lg, s, "index_chunk_kernel + index_select_kernel");
    if (e != hipSuccess) return e;
    if (ab.njobs == 0) return hipSuccess;
    e = launch_attend_batch_mfma(all, s);
    if (e == hipSuccess && all.blk0[all.njobs] > 0) e = log_launch(lg, s, "attend_mfma_batch_kernel");
    if (e != hipSuccess) return e;
    e = launch_attend_batch_merge(all, s);
    if (e == hipSuccess && all.mblk0[all.njobs] > 0) e = log_launch(lg, s, "attend_merge_batch_kernel");
    return e;
  }
  const ScanPlan p = index_scan_plan(ia);
  const bool fp8 = all.job[0].kv_dt == DT_FP8;
  if (p.nq == 2) {
    if (fp8) launch_fused_k<2, DT_FP8>(ia, p, dense, cb, fd, s);
    else launch_fused_k<2, DT_BF16>(ia, p, dense, cb, fd, s);
  } else {
    if (fp8) launch_fused_k<1, DT_FP8>(ia, p, dense, cb, fd, s);
    else launch_fused_k<1, DT_BF16>(ia, p, dense, cb, fd, s);
  }
  e = hipGetLastError();
  if (e == hipSuccess) e = log_launch(lg, s, "step_scan_attend_kernel");
  if (e != hipSuccess) return e;
  // the dense jobs' partials are complete: their merge runs beside the select
  e = launch_index_select_merge(ia, p, dense, s);
  if (e == hipSuccess) e = log_launch(lg, s, "index_select_merge_kernel");
  if (e != hipSuccess) return e;
  const AttendBatch sparse = sub_batch(all, false);
  if (sparse.njobs > 0) {
    e = launch_attend_batch_mfma(sparse, s);
    if (e == hipSuccess && sparse.blk0[sparse.njobs] > 0) e = log_launch(lg, s, "attend_mfma_batch_kernel");
    if (e != hipSuccess) return e;
  }
  e = launch_attend_batch_merge(sparse, s);
  if (e == hipSuccess && sparse.mblk0[sparse.njobs] > 0) e = log_launch(lg, s, "attend_merge_batch_kernel");
  return e;
}

}  // namespace lca
