// abi.cpp -- the extern "C" entry points declared in include/lca.h: argument
// validation (before anything is enqueued), workspace checks, launch
// configuration and error reporting.  No HIP call is made before validation
// succeeds, so loading the library and validating arguments need no GPU.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/lca.h"
#include "lca_internal.h"

namespace {

thread_local char g_err[512] = "";

lca_status fail(lca_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

lca_status ok() {
  g_err[0] = '\0';
  return LCA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

#define REQ(cond, st, ...) \
  do {                      \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define PTR(p) REQ((p) != nullptr && aligned16(p), LCA_EINVAL, "%s must be a non-null 16-byte aligned pointer", #p)

lca_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LCA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Validation of one compress call; on success *out holds the launch
// arguments (B = 0 when there is nothing to do).
lca_status compress_check(const char* name, int mmax, const void* x, lca_dtype x_dt, int64_t x_rows,
                          const float* gate, const float* pos_bias, int32_t m, const int32_t* x_tok0,
                          const int32_t* nblk, const int64_t* dst_row0, int32_t B, int32_t nblk_max,
                          int32_t D, void* dst, lca_dtype dst_dt, void* dst_scale, int64_t dst_rows,
                          float* pooled, int32_t gate_pc, int32_t overlap, lca::CompressArgs* out) {
  *out = lca::CompressArgs{};
  REQ(B >= 0 && nblk_max >= 0, LCA_EINVAL, "%s: B and nblk_max must be >= 0", name);
  REQ(m >= 1 && m <= mmax, LCA_ENOTSUP, "%s: m=%d outside [1, %d]", name, m, mmax);
  REQ(gate_pc == 0 || gate_pc == 1, LCA_EINVAL, "%s: gate_pc=%d (0 or 1)", name, gate_pc);
  REQ(overlap >= 0 && overlap <= m && m + overlap <= 1024, LCA_EINVAL,
      "%s: overlap=%d outside [0, m] or m + overlap > 1024", name, overlap);
  REQ(D == 64 || D == 128, LCA_ENOTSUP, "%s: D=%d (supported: 64, 128)", name, D);
  REQ(x_dt == LCA_F32 || x_dt == LCA_BF16, LCA_ENOTSUP, "%s: x_dt must be F32 or BF16", name);
  REQ(dst_dt >= LCA_F32 && dst_dt <= LCA_MXFP4, LCA_ENOTSUP, "%s: unknown dst_dt %d", name, (int)dst_dt);
  REQ(x_rows >= 0 && dst_rows >= 0, LCA_EINVAL, "%s: x_rows and dst_rows must be >= 0", name);
  REQ(B <= 65535, LCA_ENOTSUP, "%s: B=%d exceeds 65535", name, B);
  REQ((int64_t)nblk_max * m + overlap <= x_rows, LCA_EINVAL, "%s: nblk_max*m + overlap=%lld exceeds x_rows=%lld",
      name, (long long)nblk_max * m + overlap, (long long)x_rows);
  REQ(nblk_max <= dst_rows, LCA_EINVAL, "%s: nblk_max=%d exceeds dst_rows=%lld", name, nblk_max,
      (long long)dst_rows);
  out->x_dt = (int)x_dt; out->D = D;
  if (B == 0 || nblk_max == 0) return ok();
  PTR(x); PTR(gate); PTR(pos_bias); PTR(x_tok0); PTR(nblk); PTR(dst_row0); PTR(dst);
  if (dst_dt == LCA_FP8E4M3 || dst_dt == LCA_MXFP4) {
    PTR(dst_scale);
  } else {
    REQ(dst_scale == nullptr, LCA_EINVAL, "%s: dst_scale must be NULL for F32/BF16 output", name);
  }
  if (pooled) REQ(aligned16(pooled), LCA_EINVAL, "%s: pooled must be 16-byte aligned", name);
  *out = lca::CompressArgs{x, (int)x_dt, x_rows, gate, pos_bias, m, x_tok0, nblk, dst_row0,
                           B, nblk_max, D, dst, (int)dst_dt, dst_scale, dst_rows, pooled, gate_pc, overlap};
  return ok();
}

lca_status compress_common(const char* name, int mmax, const void* x, lca_dtype x_dt, int64_t x_rows,
                           const float* gate, const float* pos_bias, int32_t m, const int32_t* x_tok0,
                           const int32_t* nblk, const int64_t* dst_row0, int32_t B, int32_t nblk_max,
                           int32_t D, void* dst, lca_dtype dst_dt, void* dst_scale, int64_t dst_rows,
                           float* pooled, void* stream) {
  lca::CompressArgs a;
  const lca_status st = compress_check(name, mmax, x, x_dt, x_rows, gate, pos_bias, m, x_tok0, nblk, dst_row0, B,
                                       nblk_max, D, dst, dst_dt, dst_scale, dst_rows, pooled, 0, 0, &a);
  if (st != LCA_OK || a.B == 0) return st;
  return hip_status(lca::launch_compress(a, (hipStream_t)stream), name);
}

// Validation of one attention call; on success *out holds the launch
// arguments (B*Tq = 0 when there is nothing to do).
lca_status attend_check(const char* name, int sparse, const void* q, lca_dtype q_dt, const void* kv, lca_dtype kv_dt,
                        const float* kv_scale, int64_t N_cap, const int32_t* idx, int32_t k,
                        const int32_t* n_elig, const void* win, lca_dtype win_dt, int64_t W_buf,
                        const int32_t* win_begin, const int32_t* win_len, const float* sink, float scale,
                        int32_t B, int32_t Tq, int32_t Hq, int32_t D, void* out, lca_dtype out_dt, float* lse,
                        void* ws, size_t ws_bytes, lca::AttendArgs* outa) {
  *outa = lca::AttendArgs{};
  outa->q_dt = (int)q_dt; outa->kv_dt = (int)kv_dt; outa->win_dt = (int)win_dt; outa->Hq = Hq; outa->D = D;
  REQ(B >= 0 && Tq >= 0, LCA_EINVAL, "%s: B and Tq must be >= 0", name);
  REQ(D == 128, LCA_ENOTSUP, "%s: D=%d (supported: 128)", name, D);
  REQ(Hq == 16 || Hq == 32 || Hq == 64, LCA_ENOTSUP, "%s: Hq=%d (supported: 16, 32, 64)", name, Hq);
  REQ(q_dt == LCA_F32 || q_dt == LCA_BF16, LCA_ENOTSUP, "%s: q_dt must be F32 or BF16", name);
  REQ(kv_dt == LCA_F32 || kv_dt == LCA_BF16 || kv_dt == LCA_FP8E4M3, LCA_ENOTSUP,
      "%s: kv_dt must be F32, BF16 or FP8E4M3", name);
  REQ(win_dt == LCA_F32 || win_dt == LCA_BF16, LCA_ENOTSUP, "%s: win_dt must be F32 or BF16", name);
  REQ(out_dt == LCA_F32 || out_dt == LCA_BF16, LCA_ENOTSUP, "%s: out_dt must be F32 or BF16", name);
  REQ(N_cap >= 0 && N_cap < (1ll << 31), LCA_EINVAL, "%s: N_cap out of range", name);
  REQ(W_buf >= 0 && W_buf < (1ll << 31), LCA_EINVAL, "%s: W_buf out of range", name);
  REQ(scale == scale, LCA_EINVAL, "%s: scale is NaN", name);
  REQ(Tq <= 65535 * 1024 && (int64_t)B * Tq < (1ll << 31), LCA_ENOTSUP, "%s: too many query rows", name);
  if (sparse) REQ(k >= 0 && k <= 2048, LCA_EINVAL, "%s: k=%d outside [0, 2048]", name, k);
  if ((int64_t)B * Tq == 0) return ok();
  PTR(q); PTR(win); PTR(win_begin); PTR(win_len); PTR(sink); PTR(out);
  if (N_cap > 0) PTR(kv);
  if (kv_dt == LCA_FP8E4M3 && N_cap > 0) PTR(kv_scale);
  if (kv_dt != LCA_FP8E4M3) REQ(kv_scale == nullptr, LCA_EINVAL, "%s: kv_scale must be NULL unless FP8", name);
  if (lse) REQ(aligned16(lse), LCA_EINVAL, "%s: lse must be 16-byte aligned", name);
  const size_t need = lca::attend_ws_bytes(B, Tq, Hq, D, sparse ? k : N_cap, W_buf);
  if (need > 0) {
    REQ(ws != nullptr && aligned16(ws), LCA_EWORKSPACE, "%s: workspace of %zu bytes required", name, need);
    REQ(ws_bytes >= need, LCA_EWORKSPACE, "%s: workspace too small (%zu < %zu)", name, ws_bytes, need);
  }
  lca::AttendArgs& a = *outa;
  a.q = q; a.q_dt = (int)q_dt; a.kv = kv; a.kv_dt = (int)kv_dt; a.kv_scale = kv_scale; a.N_cap = N_cap;
  a.sparse = sparse; a.idx = idx; a.k = k; a.n_elig = n_elig; a.win = win; a.win_dt = (int)win_dt; a.W_buf = W_buf;
  a.win_begin = win_begin; a.win_len = win_len; a.sink = sink; a.scale = scale;
  a.B = B; a.Tq = Tq; a.Hq = Hq; a.D = D; a.out = out; a.out_dt = (int)out_dt; a.lse = lse;
  a.ws = ws; a.ws_bytes = ws_bytes;
  return ok();
}

lca_status attend_common(const char* name, int sparse, const void* q, lca_dtype q_dt, const void* kv, lca_dtype kv_dt,
                         const float* kv_scale, int64_t N_cap, const int32_t* idx, int32_t k,
                         const int32_t* n_elig, const void* win, lca_dtype win_dt, int64_t W_buf,
                         const int32_t* win_begin, const int32_t* win_len, const float* sink, float scale,
                         int32_t B, int32_t Tq, int32_t Hq, int32_t D, void* out, lca_dtype out_dt, float* lse,
                         void* ws, size_t ws_bytes, void* stream) {
  lca::AttendArgs a;
  const lca_status st = attend_check(name, sparse, q, q_dt, kv, kv_dt, kv_scale, N_cap, idx, k, n_elig, win, win_dt,
                                     W_buf, win_begin, win_len, sink, scale, B, Tq, Hq, D, out, out_dt, lse, ws,
                                     ws_bytes, &a);
  if (st != LCA_OK || (int64_t)a.B * a.Tq == 0) return st;
  return hip_status(lca::launch_attend(a, (hipStream_t)stream), name);
}

}  // namespace

extern "C" {

int32_t lca_abi_version(void) { return LCA_ABI_VERSION; }

const char* lca_last_error(void) { return g_err; }

lca_status lca_csa_compress(const void* x, lca_dtype x_dt, int64_t x_rows, const float* gate,
                            const float* pos_bias, int32_t m, const int32_t* x_tok0, const int32_t* nblk,
                            const int64_t* dst_row0, int32_t B, int32_t nblk_max, int32_t D, void* dst,
                            lca_dtype dst_dt, void* dst_scale, int64_t dst_rows, float* pooled, void* stream) {
  return compress_common("lca_csa_compress", 64, x, x_dt, x_rows, gate, pos_bias, m, x_tok0, nblk, dst_row0, B,
                         nblk_max, D, dst, dst_dt, dst_scale, dst_rows, pooled, stream);
}

lca_status lca_hca_compress(const void* x, lca_dtype x_dt, int64_t x_rows, const float* gate,
                            const float* pos_bias, int32_t m, const int32_t* x_tok0, const int32_t* nblk,
                            const int64_t* dst_row0, int32_t B, int32_t nblk_max, int32_t D, void* dst,
                            lca_dtype dst_dt, void* dst_scale, int64_t dst_rows, float* pooled, void* stream) {
  return compress_common("lca_hca_compress", 1024, x, x_dt, x_rows, gate, pos_bias, m, x_tok0, nblk, dst_row0,
                         B, nblk_max, D, dst, dst_dt, dst_scale, dst_rows, pooled, stream);
}

}  // extern "C"

namespace {

lca_status compress_batch_check(const char* who, const lca_compress_job* jobs, int32_t njobs, int min_jobs,
                                lca::CompressBatch* out) {
  REQ(njobs >= min_jobs && njobs <= LCA_MAX_COMPRESS_JOBS, LCA_EINVAL, "%s: njobs=%d outside [%d, %d]", who, njobs,
      min_jobs, LCA_MAX_COMPRESS_JOBS);
  REQ(njobs == 0 || jobs != nullptr, LCA_EINVAL, "%s: jobs is NULL", who);
  static_assert(LCA_MAX_COMPRESS_JOBS == lca::MAX_COMPRESS_JOBS, "job limits agree");
  lca::CompressBatch& bt = *out;
  bt = lca::CompressBatch{};
  bt.njobs = njobs;
  for (int j = 0; j < njobs; ++j) {
    const lca_compress_job& J = jobs[j];
    char name[96];
    snprintf(name, sizeof(name), "%s: compress job %d", who, j);
    const lca_status st = compress_check(name, 1024, J.x, J.x_dt, J.x_rows, J.gate, J.pos_bias, J.m, J.x_tok0, J.nblk,
                                         J.dst_row0, J.B, J.nblk_max, J.D, J.dst, J.dst_dt, J.dst_scale, J.dst_rows,
                                         J.pooled, J.gate_pc, J.overlap, &bt.job[j]);
    if (st != LCA_OK) return st;
    REQ(J.x_dt == jobs[0].x_dt && J.D == jobs[0].D, LCA_ENOTSUP, "%s: x_dt/D differ from job 0", name);
  }
  return ok();
}

}  // namespace

extern "C" {

lca_status lca_compress_batch(const lca_compress_job* jobs, int32_t njobs, void* stream) {
  lca::CompressBatch bt;
  const lca_status st = compress_batch_check("lca_compress_batch", jobs, njobs, 1, &bt);
  if (st != LCA_OK) return st;
  return hip_status(lca::launch_compress_batch(bt, (hipStream_t)stream), "lca_compress_batch");
}

size_t lca_index_topk_ws(int32_t B, int32_t Tq, int32_t H_I, int32_t d_I, int64_t N_cap, int32_t k) {
  if (B <= 0 || Tq <= 0 || N_cap < 0) return 0;
  return lca::index_ws_bytes(B, Tq, H_I, d_I, N_cap, k, lca::DT_MXFP4 /* same layout for both types */);
}

}  // extern "C"

namespace {

// Validation of one indexer call; on success *out holds the launch arguments
// (B*Tq = 0 when there is nothing to do).
lca_status index_check(const char* name, const void* qi, lca_dtype qi_dt, const uint8_t* qi_scale, const float* w,
                       const void* ki, lca_dtype ki_dt, const uint8_t* ki_scale, const int32_t* n_elig, int32_t B,
                       int32_t Tq, int32_t H_I, int32_t d_I, int64_t N_cap, int32_t k, int32_t* idx_out,
                       double* score_out, void* ws, size_t ws_bytes, lca::IndexArgs* out) {
  *out = lca::IndexArgs{};
  REQ(B >= 0 && Tq >= 0, LCA_EINVAL, "%s: B and Tq must be >= 0", name);
  REQ(k >= 1 && k <= 2048, LCA_EINVAL, "%s: k=%d outside [1, 2048]", name, k);
  REQ(N_cap >= 0 && N_cap < (1ll << 31), LCA_EINVAL, "%s: N_cap out of range", name);
  REQ(qi_dt == ki_dt, LCA_ENOTSUP, "%s: qi_dt and ki_dt must match", name);
  if (qi_dt == LCA_MXFP4) {
    REQ(H_I >= 1 && H_I <= 16, LCA_ENOTSUP, "%s: MXFP4 needs 1 <= H_I <= 16 (got %d)", name, H_I);
    REQ(d_I == 64 || d_I == 128, LCA_ENOTSUP, "%s: MXFP4 needs d_I in {64, 128} (got %d)", name, d_I);
  } else if (qi_dt == LCA_F32) {
    REQ(H_I >= 1 && H_I <= 16, LCA_ENOTSUP, "%s: F32 needs 1 <= H_I <= 16 (got %d)", name, H_I);
    REQ(d_I == 32 || d_I == 64 || d_I == 128, LCA_ENOTSUP, "%s: F32 needs d_I in {32, 64, 128}", name);
  } else {
    return fail(LCA_ENOTSUP, "%s: qi_dt must be F32 or MXFP4", name);
  }
  {
    const int nq = (qi_dt == LCA_MXFP4 && H_I <= 8 && Tq > 1) ? 2 : 1;   // query rows per wavefront
    REQ((int64_t)B * ((Tq + nq - 1) / nq) <= 65535, LCA_ENOTSUP, "%s: too many query rows", name);
  }
  if ((int64_t)B * Tq == 0) return ok();
  PTR(qi); PTR(w); PTR(n_elig); PTR(idx_out);
  if (N_cap > 0) PTR(ki);
  if (qi_dt == LCA_MXFP4) {
    PTR(qi_scale);
    if (N_cap > 0) PTR(ki_scale);
  } else {
    REQ(qi_scale == nullptr && ki_scale == nullptr, LCA_EINVAL, "%s: scales must be NULL for F32", name);
  }
  if (score_out) REQ(aligned16(score_out), LCA_EINVAL, "%s: score_out must be 16-byte aligned", name);
  const size_t need = lca_index_topk_ws(B, Tq, H_I, d_I, N_cap, k);
  REQ(ws != nullptr && aligned16(ws), LCA_EWORKSPACE, "%s: workspace of %zu bytes required", name, need);
  REQ(ws_bytes >= need, LCA_EWORKSPACE, "%s: workspace too small (%zu < %zu)", name, ws_bytes, need);
  lca::IndexArgs& a = *out;
  a.qi = qi; a.dt = (int)qi_dt; a.qi_scale = qi_scale; a.w = w; a.ki = ki; a.ki_scale = ki_scale;
  a.n_elig = n_elig; a.B = B; a.Tq = Tq; a.H = H_I; a.d = d_I; a.N_cap = N_cap; a.k = k;
  a.idx_out = idx_out; a.score_out = score_out; a.ws = ws; a.ws_bytes = ws_bytes;
  return ok();
}

}  // namespace

extern "C" {

lca_status lca_lightning_index_topk(const void* qi, lca_dtype qi_dt, const uint8_t* qi_scale, const float* w,
                                    const void* ki, lca_dtype ki_dt, const uint8_t* ki_scale,
                                    const int32_t* n_elig, int32_t B, int32_t Tq, int32_t H_I, int32_t d_I,
                                    int64_t N_cap, int32_t k, int32_t* idx_out, double* score_out, void* ws,
                                    size_t ws_bytes, void* stream) {
  lca::IndexArgs a;
  const lca_status st = index_check("lca_lightning_index_topk", qi, qi_dt, qi_scale, w, ki, ki_dt, ki_scale, n_elig,
                                    B, Tq, H_I, d_I, N_cap, k, idx_out, score_out, ws, ws_bytes, &a);
  if (st != LCA_OK || (int64_t)a.B * a.Tq == 0) return st;
  return hip_status(lca::launch_index(a, (hipStream_t)stream), "lca_lightning_index_topk");
}

}  // extern "C"

namespace {

lca_status attend_batch_check(const char* who, const lca_attend_job* jobs, int32_t njobs, int min_jobs,
                              lca::AttendBatch* out) {
  REQ(njobs >= min_jobs && njobs <= LCA_MAX_ATTEND_JOBS, LCA_EINVAL, "%s: njobs=%d outside [%d, %d]", who, njobs,
      min_jobs, LCA_MAX_ATTEND_JOBS);
  REQ(njobs == 0 || jobs != nullptr, LCA_EINVAL, "%s: jobs is NULL", who);
  static_assert(LCA_MAX_ATTEND_JOBS == lca::MAX_ATTEND_JOBS, "job limits agree");
  lca::AttendBatch& bt = *out;
  bt = lca::AttendBatch{};
  bt.njobs = njobs;
  for (int j = 0; j < njobs; ++j) {
    const lca_attend_job& J = jobs[j];
    char name[96];
    snprintf(name, sizeof(name), "%s: attention job %d", who, j);
    REQ(J.sparse == 0 || J.sparse == 1, LCA_EINVAL, "%s: sparse must be 0 or 1", name);
    const bool rows = (int64_t)J.B * J.Tq > 0;
    if (J.sparse) {
      REQ(!rows || J.k <= 0 || (J.idx != nullptr && aligned16(J.idx)), LCA_EINVAL,
          "%s: idx must be a non-null 16-byte aligned pointer", name);
    } else {
      REQ(!rows || (J.n_elig != nullptr && aligned16(J.n_elig)), LCA_EINVAL,
          "%s: n_elig must be a non-null 16-byte aligned pointer", name);
    }
    const lca_status st = attend_check(name, J.sparse, J.q, J.q_dt, J.kv, J.kv_dt, J.kv_scale, J.N_cap,
                                       J.sparse ? J.idx : nullptr, J.sparse ? J.k : 0, J.sparse ? nullptr : J.n_elig,
                                       J.win, J.win_dt, J.W_buf, J.win_begin, J.win_len, J.sink, J.scale, J.B, J.Tq,
                                       J.Hq, J.D, J.out, J.out_dt, J.lse, J.ws, J.ws_bytes, &bt.job[j]);
    if (st != LCA_OK) return st;
    lca::AttendArgs& a = bt.job[j];
    if ((int64_t)J.B * J.Tq == 0) {
      // nothing to do for this job: keep a launchable descriptor with no rows
      a.B = 0; a.Tq = 0; a.sparse = 1; a.k = 0; a.Hq = J.Hq; a.D = J.D;
    }
    REQ(J.q_dt == LCA_BF16 && J.win_dt == LCA_BF16 && (J.kv_dt == LCA_BF16 || J.kv_dt == LCA_FP8E4M3), LCA_ENOTSUP,
        "%s: batched attention takes bf16 queries and windows and bf16 or FP8 entries", name);
    REQ(J.kv_dt == jobs[0].kv_dt && J.Hq == jobs[0].Hq, LCA_ENOTSUP, "%s: kv_dt/Hq differ from job 0", name);
    REQ((int64_t)J.B * J.Tq == 0 || lca::attend_batchable(a), LCA_ENOTSUP,
        "%s: prefill-shaped calls (many query rows, no split) are not batched; use the single call", name);
  }
  return ok();
}

// The dense attention jobs of a decode step run beside the indexer's scan,
// so none may write memory that the indexer writes: its output, scores and
// workspace against each dense job's output, lse and workspace (the bytes the
// kernels touch: the needed workspace sizes, not the declared ones).
struct Span {
  uintptr_t a, n;
};
bool spans_overlap(Span x, Span y) { return x.n > 0 && y.n > 0 && x.a < y.a + y.n && y.a < x.a + x.n; }

lca_status step_disjoint_check(const char* name, const lca::IndexArgs& ia, const lca::AttendBatch& ab) {
  const int64_t R = (int64_t)ia.B * ia.Tq;
  if (R == 0) return ok();
  const Span iw[3] = {{(uintptr_t)ia.idx_out, (uintptr_t)(R * ia.k * 4)},
                      {(uintptr_t)ia.score_out, ia.score_out ? (uintptr_t)(R * ia.k * 8) : 0},
                      {(uintptr_t)ia.ws, lca::index_ws_bytes(ia.B, ia.Tq, ia.H, ia.d, ia.N_cap, ia.k, ia.dt)}};
  for (int j = 0; j < ab.njobs; ++j) {
    const lca::AttendArgs& a = ab.job[j];
    const int64_t Ra = (int64_t)a.B * a.Tq;
    if (a.sparse || Ra == 0) continue;
    const Span aw[3] = {{(uintptr_t)a.out, (uintptr_t)(Ra * a.Hq * a.D * (a.out_dt == lca::DT_F32 ? 4 : 2))},
                        {(uintptr_t)a.lse, a.lse ? (uintptr_t)(Ra * a.Hq * 4) : 0},
                        {(uintptr_t)a.ws, lca::attend_ws_bytes(a.B, a.Tq, a.Hq, a.D, a.N_cap, a.W_buf)}};
    for (const Span& x : aw)
      for (const Span& y : iw)
        REQ(!spans_overlap(x, y), LCA_EINVAL,
            "%s: dense attention job %d writes memory that the index job writes (they run concurrently)", name, j);
  }
  return ok();
}

}  // namespace

extern "C" {

lca_status lca_attend_batch(const lca_attend_job* jobs, int32_t njobs, void* stream) {
  lca::AttendBatch bt;
  const lca_status st = attend_batch_check("lca_attend_batch", jobs, njobs, 1, &bt);
  if (st != LCA_OK) return st;
  return hip_status(lca::launch_attend_batch(bt, (hipStream_t)stream), "lca_attend_batch");
}

lca_status lca_decode_step(const lca_compress_job* cjobs, int32_t ncjobs, const lca_index_job* ijob,
                           const lca_attend_job* ajobs, int32_t najobs, void* stream) {
  const char* name = "lca_decode_step";
  lca::CompressBatch cb;
  lca_status st = compress_batch_check(name, cjobs, ncjobs, 0, &cb);
  if (st != LCA_OK) return st;
  lca::IndexArgs ia{};                 // no index job: B = 0
  if (ijob != nullptr) {
    const lca_index_job& I = *ijob;
    st = index_check("lca_decode_step: index job", I.qi, I.qi_dt, I.qi_scale, I.w, I.ki, I.ki_dt, I.ki_scale,
                     I.n_elig, I.B, I.Tq, I.H_I, I.d_I, I.N_cap, I.k, I.idx_out, I.score_out, I.ws, I.ws_bytes, &ia);
    if (st != LCA_OK) return st;
  }
  lca::AttendBatch ab;
  st = attend_batch_check(name, ajobs, najobs, 0, &ab);
  if (st != LCA_OK) return st;
  st = step_disjoint_check(name, ia, ab);
  if (st != LCA_OK) return st;
  return hip_status(lca::launch_decode_step(nullptr, nullptr, cb, ia, ab, (hipStream_t)stream), name);
}

lca_status lca_decode_step_noalloc(const lca_compress_job* cjobs, int32_t ncjobs, const lca_index_job* ijob,
                                   const lca_attend_job* ajobs, int32_t najobs, void* stream) {
  const char* name = "lca_decode_step_noalloc";
  static_assert(LCA_NOALLOC_SCRATCH_BYTES == lca::NOALLOC_SCRATCH_BYTES, "scratch sizes agree");
  REQ(najobs >= 0 && najobs <= LCA_MAX_ATTEND_JOBS, LCA_EINVAL, "%s: njobs=%d outside [0, %d]", name, najobs,
      LCA_MAX_ATTEND_JOBS);
  REQ(najobs == 0 || ajobs != nullptr, LCA_EINVAL, "%s: jobs is NULL", name);
  // the workspaces, one after another in the scratch (256-byte aligned)
  lca_index_job I{};
  lca_attend_job A[LCA_MAX_ATTEND_JOBS];
  size_t off[1 + LCA_MAX_ATTEND_JOBS] = {}, need = 0;
  if (ijob != nullptr) {
    I = *ijob;
    I.ws_bytes = (I.B > 0 && I.Tq > 0) ? lca_index_topk_ws(I.B, I.Tq, I.H_I, I.d_I, I.N_cap, I.k) : 0;
    off[0] = need;
    need += round256(I.ws_bytes);
  }
  for (int j = 0; j < najobs; ++j) {
    A[j] = ajobs[j];
    const bool rows = (int64_t)A[j].B * A[j].Tq > 0 && A[j].B > 0 && A[j].Tq > 0;
    A[j].ws_bytes = rows ? lca_attend_ws(A[j].B, A[j].Tq, A[j].Hq, A[j].D, A[j].sparse ? A[j].k : A[j].N_cap,
                                         A[j].W_buf)
                         : 0;
    off[1 + j] = need;
    need += round256(A[j].ws_bytes);
  }
  REQ(need <= LCA_NOALLOC_SCRATCH_BYTES, LCA_EWORKSPACE,
      "%s: the step needs %zu bytes of scratch; the library holds %zu per device (use lca_decode_step with "
      "caller workspaces)", name, need, (size_t)LCA_NOALLOC_SCRATCH_BYTES);
  // validation with stand-in workspace addresses: nothing touches the GPU
  // before every job is valid
  const uintptr_t standin = (uintptr_t)1 << 12;
  I.ws = (void*)(standin + off[0]);
  for (int j = 0; j < najobs; ++j) A[j].ws = (void*)(standin + off[1 + j]);
  lca::CompressBatch cb;
  lca_status st = compress_batch_check(name, cjobs, ncjobs, 0, &cb);
  if (st != LCA_OK) return st;
  lca::IndexArgs ia{};
  if (ijob != nullptr) {
    st = index_check("lca_decode_step_noalloc: index job", I.qi, I.qi_dt, I.qi_scale, I.w, I.ki, I.ki_dt, I.ki_scale,
                     I.n_elig, I.B, I.Tq, I.H_I, I.d_I, I.N_cap, I.k, I.idx_out, I.score_out, I.ws, I.ws_bytes, &ia);
    if (st != LCA_OK) return st;
  }
  lca::AttendBatch ab;
  st = attend_batch_check(name, A, najobs, 0, &ab);
  if (st != LCA_OK) return st;
  st = step_disjoint_check(name, ia, ab);
  if (st != LCA_OK) return st;
  // the current device's scratch (when a workspace is needed at all)
  if (need > 0) {
    void* base = nullptr;
    st = hip_status(lca::noalloc_scratch(&base), name);
    if (st != LCA_OK) return st;
    if (ijob != nullptr) ia.ws = (char*)base + off[0];
    for (int j = 0; j < najobs; ++j) ab.job[j].ws = (char*)base + off[1 + j];
  }
  return hip_status(lca::launch_decode_step(nullptr, nullptr, cb, ia, ab, (hipStream_t)stream), name);
}

lca_status lca_decode_step_events(const lca_compress_job* cjobs, int32_t ncjobs, const lca_index_job* ijob,
                                  const lca_attend_job* ajobs, int32_t najobs, void* const* events, int32_t nevents,
                                  const char** names, int32_t* nlaunch, void* stream) {
  const char* name = "lca_decode_step_events";
  REQ(events != nullptr && nevents >= LCA_MAX_STEP_LAUNCHES + 1, LCA_EINVAL,
      "%s: events must hold at least %d event handles", name, LCA_MAX_STEP_LAUNCHES + 1);
  REQ(nlaunch != nullptr, LCA_EINVAL, "%s: nlaunch is NULL", name);
  for (int i = 0; i <= LCA_MAX_STEP_LAUNCHES; ++i)
    REQ(events[i] != nullptr, LCA_EINVAL, "%s: events[%d] is NULL", name, i);
  lca::CompressBatch cb;
  lca_status st = compress_batch_check(name, cjobs, ncjobs, 0, &cb);
  if (st != LCA_OK) return st;
  lca::IndexArgs ia{};
  if (ijob != nullptr) {
    const lca_index_job& I = *ijob;
    st = index_check("lca_decode_step_events: index job", I.qi, I.qi_dt, I.qi_scale, I.w, I.ki, I.ki_dt, I.ki_scale,
                     I.n_elig, I.B, I.Tq, I.H_I, I.d_I, I.N_cap, I.k, I.idx_out, I.score_out, I.ws, I.ws_bytes, &ia);
    if (st != LCA_OK) return st;
  }
  lca::AttendBatch ab;
  st = attend_batch_check(name, ajobs, najobs, 0, &ab);
  if (st != LCA_OK) return st;
  st = step_disjoint_check(name, ia, ab);
  if (st != LCA_OK) return st;
  lca::LaunchLog lg{(hipEvent_t*)events, LCA_MAX_STEP_LAUNCHES + 1, 0, names};
  st = hip_status(lca::launch_decode_step(nullptr, nullptr, cb, ia, ab, (hipStream_t)stream, &lg), name);
  *nlaunch = lg.n;
  return st;
}

}  // extern "C"

namespace {

lca_status append_batch_check(const char* who, const lca_append_job* jobs, int32_t njobs, int min_jobs,
                              lca::AppendBatch* out) {
  REQ(njobs >= min_jobs && njobs <= LCA_MAX_APPEND_JOBS, LCA_EINVAL, "%s: njobs=%d outside [%d, %d]", who, njobs,
      min_jobs, LCA_MAX_APPEND_JOBS);
  REQ(njobs == 0 || jobs != nullptr, LCA_EINVAL, "%s: jobs is NULL", who);
  static_assert(LCA_MAX_APPEND_JOBS == lca::MAX_APPEND_JOBS, "job limits agree");
  lca::AppendBatch& bt = *out;
  bt = lca::AppendBatch{};
  bt.njobs = njobs;
  for (int j = 0; j < njobs; ++j) {
    const lca_append_job& J = jobs[j];
    char name[96];
    snprintf(name, sizeof(name), "%s: append job %d", who, j);
    REQ(J.B >= 0 && J.B <= (1 << 20), LCA_EINVAL, "%s: B=%d out of range", name, J.B);
    REQ(J.D == 64 || J.D == 128, LCA_ENOTSUP, "%s: D=%d (64 or 128)", name, J.D);
    REQ(J.x_dt == LCA_BF16 || J.x_dt == LCA_F32, LCA_ENOTSUP, "%s: x_dt must be bf16 or f32", name);
    REQ(J.m >= 0 && J.m <= 1024, LCA_EINVAL, "%s: m=%d outside [0, 1024]", name, J.m);
    REQ(J.W >= 0, LCA_EINVAL, "%s: W=%d negative", name, J.W);
    REQ(J.overlap >= 0 && J.overlap <= J.m, LCA_EINVAL, "%s: overlap=%d outside [0, m]", name, J.overlap);
    REQ(J.gate_pc == 0 || J.gate_pc == 1, LCA_EINVAL, "%s: gate_pc=%d (0 or 1)", name, J.gate_pc);
    REQ(J.R >= 1 && J.R >= J.m + J.overlap && J.R >= J.W && J.R < (1ll << 30), LCA_EINVAL,
        "%s: R=%lld must be >= max(1, m + overlap, W)", name, (long long)J.R);
    REQ((J.g_new == nullptr) == (J.gring == nullptr), LCA_EINVAL, "%s: g_new and gring go together", name);
    REQ((J.win_begin == nullptr) == (J.win_len == nullptr), LCA_EINVAL, "%s: win_begin and win_len go together",
        name);
    if (J.B > 0) {
      REQ(J.x_new != nullptr && aligned16(J.x_new), LCA_EINVAL, "%s: x_new must be a non-null 16-byte aligned pointer",
          name);
      REQ(J.ring != nullptr && aligned16(J.ring), LCA_EINVAL, "%s: ring must be a non-null 16-byte aligned pointer",
          name);
      REQ(J.len != nullptr, LCA_EINVAL, "%s: len is NULL", name);
    }
    lca::AppendArgs& a = bt.job[j];
    a.x_new = J.x_new; a.x_dt = (int)J.x_dt; a.g_new = J.g_new; a.ring = J.ring; a.gring = J.gring; a.R = J.R;
    a.len = J.len; a.m = J.m; a.W = J.W; a.x_tok0 = J.x_tok0; a.nblk = J.nblk; a.dst_row0 = J.dst_row0;
    a.n_elig = J.n_elig; a.win_begin = J.win_begin; a.win_len = J.win_len; a.B = J.B; a.D = J.D;
    a.overlap = J.overlap; a.gate_pc = J.gate_pc;
  }
  return ok();
}

}  // namespace

extern "C" {

lca_status lca_decode_append(const lca_append_job* jobs, int32_t njobs, void* stream) {
  lca::AppendBatch bt;
  const lca_status st = append_batch_check("lca_decode_append", jobs, njobs, 1, &bt);
  if (st != LCA_OK) return st;
  return hip_status(lca::launch_decode_append(bt, (hipStream_t)stream), "lca_decode_append");
}

lca_status lca_decode_loop_step(const lca_append_job* app, int32_t napp, const lca_compress_job* cjobs,
                                int32_t ncjobs, const lca_index_job* ijob, const lca_attend_job* ajobs,
                                int32_t najobs, void* stream) {
  const char* name = "lca_decode_loop_step";
  lca::AppendBatch apb;
  lca_status st = append_batch_check(name, app, napp, 0, &apb);
  if (st != LCA_OK) return st;
  lca::CompressBatch cb;
  st = compress_batch_check(name, cjobs, ncjobs, 0, &cb);
  if (st != LCA_OK) return st;
  // pair every compress job that reads an append job's ring with that append
  lca::AppendMap mp{};
  bool used[LCA_MAX_APPEND_JOBS] = {};
  for (int j = 0; j < ncjobs; ++j) {
    const lca::CompressArgs& c = cb.job[j];
    mp.of[j] = -1;
    for (int a = 0; a < napp; ++a) {
      const lca::AppendArgs& A = apb.job[a];
      if (A.ring != c.x) continue;
      REQ(!used[a], LCA_EINVAL, "%s: compress jobs %d and another read the ring of append job %d", name, j, a);
      REQ(c.x_tok0 == A.x_tok0 && c.nblk == A.nblk && c.dst_row0 == A.dst_row0, LCA_EINVAL,
          "%s: compress job %d reads the ring of append job %d but not its x_tok0 / nblk / dst_row0", name, j, a);
      REQ(c.nblk_max == 1 && c.B == A.B && c.m == A.m && c.overlap == A.overlap && c.gate_pc == A.gate_pc &&
              c.x_rows == 2 * A.R &&
              c.x_dt == A.x_dt && c.D == A.D,
          LCA_EINVAL,
          "%s: compress job %d and append job %d disagree (nblk_max 1, B, m, overlap, gate_pc, x_rows = 2R, x_dt, D)", name,
          j, a);
      used[a] = true;
      mp.of[j] = a;
    }
  }
  for (int a = 0; a < napp; ++a)
    if (!used[a]) mp.extra[mp.nextra++] = a;
  lca::IndexArgs ia{};
  if (ijob != nullptr) {
    const lca_index_job& I = *ijob;
    st = index_check("lca_decode_loop_step: index job", I.qi, I.qi_dt, I.qi_scale, I.w, I.ki, I.ki_dt, I.ki_scale,
                     I.n_elig, I.B, I.Tq, I.H_I, I.d_I, I.N_cap, I.k, I.idx_out, I.score_out, I.ws, I.ws_bytes, &ia);
    if (st != LCA_OK) return st;
  }
  lca::AttendBatch ab;
  st = attend_batch_check(name, ajobs, najobs, 0, &ab);
  if (st != LCA_OK) return st;
  st = step_disjoint_check(name, ia, ab);
  if (st != LCA_OK) return st;
  return hip_status(lca::launch_decode_step(&apb, &mp, cb, ia, ab, (hipStream_t)stream), name);
}

size_t lca_attend_ws(int32_t B, int32_t Tq, int32_t Hq, int32_t D, int64_t n_kv_max, int64_t W_buf) {
  if (B <= 0 || Tq <= 0) return 0;
  return lca::attend_ws_bytes(B, Tq, Hq, D, n_kv_max, W_buf);
}

lca_status lca_sparse_mqa_attend(const void* q, lca_dtype q_dt, const void* kv, lca_dtype kv_dt,
                                 const float* kv_scale, int64_t N_cap, const int32_t* idx, int32_t k,
                                 const void* win, lca_dtype win_dt, int64_t W_buf, const int32_t* win_begin,
                                 const int32_t* win_len, const float* sink, float scale, int32_t B, int32_t Tq,
                                 int32_t Hq, int32_t D, void* out, lca_dtype out_dt, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
  const char* name = "lca_sparse_mqa_attend";
  if ((int64_t)B * Tq > 0 && k > 0) PTR(idx);
  REQ(k >= 0 && k <= 2048, LCA_EINVAL, "%s: k=%d outside [0, 2048]", name, k);
  return attend_common(name, 1, q, q_dt, kv, kv_dt, kv_scale, N_cap, idx, k, nullptr, win, win_dt,
                       W_buf, win_begin, win_len, sink, scale, B, Tq, Hq, D, out, out_dt, lse, ws, ws_bytes,
                       stream);
}

lca_status lca_attend_separate_v(int32_t sparse, const void* q, lca_dtype q_dt, const void* k, const void* v,
                                 lca_dtype kv_dt, const float* k_scale, const float* v_scale, int64_t N_cap,
                                 const int32_t* idx, int32_t kk, const int32_t* n_elig, const void* win_k,
                                 const void* win_v, lca_dtype win_dt, int64_t W_buf, const int32_t* win_begin,
                                 const int32_t* win_len, const float* sink, float scale, int32_t B, int32_t Tq,
                                 int32_t Hq, int32_t D, void* out, lca_dtype out_dt, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
  const char* name = "lca_attend_separate_v";
  REQ(sparse == 0 || sparse == 1, LCA_EINVAL, "%s: sparse must be 0 or 1", name);
  REQ(kk >= 0 && kk <= 2048, LCA_EINVAL, "%s: k=%d outside [0, 2048]", name, kk);
  const bool rows = (int64_t)B * Tq > 0;
  if (rows && sparse && kk > 0) PTR(idx);
  if (rows && !sparse) PTR(n_elig);
  lca::AttendArgs a;
  const lca_status st = attend_check(name, sparse, q, q_dt, k, kv_dt, k_scale, N_cap, idx, sparse ? kk : 0, n_elig,
                                     win_k, win_dt, W_buf, win_begin, win_len, sink, scale, B, Tq, Hq, D, out, out_dt,
                                     lse, ws, ws_bytes, &a);
  if (st != LCA_OK || !rows) return st;
  PTR(win_v);
  if (N_cap > 0) PTR(v);
  if (kv_dt == LCA_FP8E4M3 && N_cap > 0) PTR(v_scale);
  if (kv_dt != LCA_FP8E4M3) REQ(v_scale == nullptr, LCA_EINVAL, "%s: v_scale must be NULL unless FP8", name);
  a.v = N_cap > 0 ? v : win_v;          // non-null marks separate values
  a.v_scale = v_scale;
  a.win_v = win_v;
  return hip_status(lca::launch_attend(a, (hipStream_t)stream), name);
}

lca_status lca_window_attend(const void* q, lca_dtype q_dt, const void* win, lca_dtype win_dt, int64_t W_buf,
                             const int32_t* win_begin, const int32_t* win_len, const float* sink, float scale,
                             int32_t B, int32_t Tq, int32_t Hq, int32_t D, void* out, lca_dtype out_dt, float* lse,
                             void* ws, size_t ws_bytes, void* stream) {
  return attend_common("lca_window_attend", 1, q, q_dt, nullptr, LCA_BF16, nullptr, 0, nullptr, 0, nullptr, win,
                       win_dt, W_buf, win_begin, win_len, sink, scale, B, Tq, Hq, D, out, out_dt, lse, ws, ws_bytes,
                       stream);
}

lca_status lca_hca_attend(const void* q, lca_dtype q_dt, const void* kv, lca_dtype kv_dt, const float* kv_scale,
                          int64_t N_cap, const int32_t* n_elig, const void* win, lca_dtype win_dt, int64_t W_buf,
                          const int32_t* win_begin, const int32_t* win_len, const float* sink, float scale,
                          int32_t B, int32_t Tq, int32_t Hq, int32_t D, void* out, lca_dtype out_dt, float* lse,
                          void* ws, size_t ws_bytes, void* stream) {
  if ((int64_t)B * Tq > 0) PTR(n_elig);
  return attend_common("lca_hca_attend", 0, q, q_dt, kv, kv_dt, kv_scale, N_cap, nullptr, 0, n_elig, win, win_dt,
                       W_buf, win_begin, win_len, sink, scale, B, Tq, Hq, D, out, out_dt, lse, ws, ws_bytes,
                       stream);
}

}  // extern "C"
