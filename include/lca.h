/*
 * lca.h -- C ABI of the MI355X (gfx950) CSA/HCA hot-path library (liblca.so).
 *
 * The library implements DeepSeek-V4's hybrid compressed attention for decode
 * and chunked prefill:
 *   - compression of raw KV tokens by softmax-gated pooling with a learned
 *     positional bias, every m tokens into one entry (m = 4 for CSA, m' = 128
 *     for HCA);
 *   - the lightning indexer (ReLU-scored multi-head dot products on FP4) and
 *     top-k selection of compressed entries per query;
 *   - shared-KV (MQA) attention over the selected entries (CSA) or over all
 *     entries (HCA), plus a sliding window of recent raw tokens and a per-head
 *     attention sink.
 * Sources: "DeepSeek-V4 發佈說明：為 AI Agents 提供高效的 1M-Token 上下文"
 * (agentlenshq.com), sections 壓縮稀疏注意力 (CSA), 重度壓縮注意力 (HCA) and
 * 架構實現; "DeepSeek V4: Towards Highly Efficient Million-Token Context
 * Intelligence" (chenshi221.pages.dev wiki), section 关键技术方法 (架构创新,
 * 基础设施).
 *
 * Conventions (all entry points):
 *   - Every tensor pointer is a DEVICE pointer owned by the caller, at least
 *     16-byte aligned.  The library never allocates device memory and never
 *     synchronises; scratch space comes from a caller-provided workspace whose
 *     size the *_ws() queries return.
 *   - Every compute call is enqueued asynchronously on `stream` (a hipStream_t;
 *     NULL is the default stream) and keeps no state between calls.  Calls are
 *     thread-safe; calls that share a workspace must not overlap.
 *   - Layouts are row-major and dense; D (or d_I) is the innermost dimension.
 *     "[B][R][D]" means sequence b's row r starts at element (b*R + r)*D.
 *   - Storage types (lca_dtype):
 *       LCA_F32      float
 *       LCA_BF16     bfloat16 (uint16 bit patterns)
 *       LCA_FP8E4M3  OCP E4M3 bytes + one fp32 scale per 64 consecutive
 *                    elements of a row (decoded value = e4m3(code) * scale)
 *       LCA_MXFP4    OCP MX E2M1 nibbles, two per byte (element 2i in the low
 *                    nibble) + one E8M0 scale byte per 32 elements (decoded
 *                    value = e2m1(code) * 2^(byte - 127))
 *   - Host-side validation runs before anything is enqueued.  On any error the
 *     call returns a non-zero lca_status, enqueues nothing, and
 *     lca_last_error() returns a message (thread-local).  No exception crosses
 *     the ABI.  Loading the library and validating arguments need no GPU.
 *   - Values held in device index arrays (lengths, offsets, selected indices)
 *     cannot be checked on the host; the caller guarantees the ranges stated
 *     for each call.  Kernels clamp what they can (out-of-range selected
 *     indices are skipped) and never read outside the stated buffers when the
 *     ranges hold.
 *   - Inputs must be finite (no NaN/Inf, no FP8 NaN codes, no E8M0 0xFF).
 */
#ifndef LCA_H
#define LCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lca_status {
  LCA_OK = 0,
  LCA_EINVAL = 1,      /* null pointer, bad size or stride, misalignment, k out of range */
  LCA_ENOTSUP = 2,     /* unsupported dtype or shape combination */
  LCA_EHIP = 3,        /* a HIP runtime or launch error (message kept) */
  LCA_EWORKSPACE = 4   /* workspace pointer null or smaller than the *_ws() query */
} lca_status;

typedef enum lca_dtype {
  LCA_F32 = 0,
  LCA_BF16 = 1,
  LCA_FP8E4M3 = 2,
  LCA_MXFP4 = 3
} lca_dtype;

#define LCA_ABI_VERSION 3

/* Version of this ABI (LCA_ABI_VERSION). */
int32_t lca_abi_version(void);

/* Message describing the last failed call on this thread ("" if none). */
const char* lca_last_error(void);

/*
 * lca_csa_compress / lca_hca_compress -- softmax-gated pooling with positional
 * bias.  [release notes (agentlenshq.com), 壓縮稀疏注意力 (CSA): 4x along the
 * sequence; 重度壓縮注意力 (HCA): 128x.  wiki (chenshi221), 架构创新: every m
 * tokens become one entry.]
 *
 * For sequence b and block i < nblk[b], with tokens t = x_tok0[b] + i*m + u
 * (u = 0..m-1):
 *     a_u = gate[b][t] + pos_bias[u]
 *     w_u = exp(a_u - max a) / sum_u' exp(a_u' - max a)
 *     c   = sum_u w_u * x[b][t]            (accumulated in fp32)
 * c is written to row dst_row0[b] + i of sequence b in `dst`, encoded as
 * dst_dt (FP8: per-64 scale s = amax/448, codes RNE-saturated; MXFP4: per-32
 * shared exponent floor(log2 amax) - 2, E2M1 RNE-saturated; BF16: RNE).
 *   x        [B][x_rows][D]   x_dt in {F32, BF16}
 *   gate     [B][x_rows]      fp32, one logit per raw token
 *   pos_bias [m]              fp32
 *   x_tok0, nblk [B] int32; dst_row0 [B] int64 (device arrays), meant to
 *            satisfy 0 <= nblk[b] <= nblk_max, x_tok0[b] >= 0,
 *            x_tok0[b] + nblk[b]*m <= x_rows, 0 <= dst_row0[b],
 *            dst_row0[b] + nblk[b] <= dst_rows.  Blocks past nblk_max are not
 *            computed, and a block whose tokens or output row fall outside
 *            x / dst is skipped (nothing read or written for it).
 *   dst      [B][dst_rows][D] (MXFP4: [B][dst_rows][D/2] bytes)
 *   dst_scale FP8: float [B][dst_rows][D/64]; MXFP4: uint8 [B][dst_rows][D/32];
 *            must be NULL for F32/BF16.
 *   pooled   optional fp32 [B][nblk_max][D]: c before encoding (row i of
 *            sequence b), rows i >= nblk[b] untouched.
 * Supported: D in {64, 128}; csa_compress 1 <= m <= 64; hca_compress
 * 1 <= m <= 1024.  m = 1 with zero gate and bias is an exact copy (used to
 * encode raw values into a cache format).
 */
lca_status lca_csa_compress(const void* x, lca_dtype x_dt, int64_t x_rows, const float* gate,
                            const float* pos_bias, int32_t m, const int32_t* x_tok0,
                            const int32_t* nblk, const int64_t* dst_row0, int32_t B,
                            int32_t nblk_max, int32_t D, void* dst, lca_dtype dst_dt,
                            void* dst_scale, int64_t dst_rows, float* pooled, void* stream);

lca_status lca_hca_compress(const void* x, lca_dtype x_dt, int64_t x_rows, const float* gate,
                            const float* pos_bias, int32_t m, const int32_t* x_tok0,
                            const int32_t* nblk, const int64_t* dst_row0, int32_t B,
                            int32_t nblk_max, int32_t D, void* dst, lca_dtype dst_dt,
                            void* dst_scale, int64_t dst_rows, float* pooled, void* stream);

/*
 * lca_compress_batch -- several compress calls in one launch (for example the
 * CSA entry block, the indexer-key block and the HCA block of one decode
 * step).  Each job is the argument list of lca_csa_compress /
 * lca_hca_compress with the same meaning, layouts and caller guarantees, and
 * its result is bit-identical to that single call.  [Same passages as
 * lca_csa_compress.]
 *   jobs     host array of njobs descriptors, read during the call only;
 *            1 <= njobs <= LCA_MAX_COMPRESS_JOBS.
 * Each job is validated as a single call with 1 <= m <= 1024; all jobs must
 * share x_dt and D (LCA_ENOTSUP otherwise).  Jobs must not write overlapping
 * destination, scale or pooled rows (they run concurrently).  On any invalid
 * job nothing is enqueued and the message names the job.
 *
 * Two pooling variants, per job (both 0 = the single calls' pooling).  The
 * pages name softmax-gated pooling with a learned positional bias but give
 * neither the gate's shape nor whether blocks overlap:
 *   gate_pc = 1   one logit per token and channel: gate [B][x_rows][D] fp32,
 *                 pos_bias [m + overlap][D]; one softmax per channel:
 *                 c[d] = sum_u softmax_u(gate[b][t_u][d] + pos_bias[u][d]) x[b][t_u][d]
 *   overlap = o   (0 <= o <= m, m + o <= 1024) block i pools the m + o tokens
 *                 t_u = x_tok0[b] + i*m + u, u = 0 .. m+o-1: the o tokens
 *                 before the block and its m tokens (x_tok0 points o rows
 *                 before the first block's first token); pos_bias has m + o
 *                 rows.  For the first entry of a sequence (dst_row0[b] + i
 *                 == 0) the o leading tokens do not exist: they are neither
 *                 read nor weighted.  Caller guarantees
 *                 x_tok0[b] + nblk[b]*m + o <= x_rows.
 */
#define LCA_MAX_COMPRESS_JOBS 8
typedef struct lca_compress_job {
  const void* x; lca_dtype x_dt; int64_t x_rows;
  const float* gate; const float* pos_bias; int32_t m;
  const int32_t* x_tok0; const int32_t* nblk; const int64_t* dst_row0;
  int32_t B; int32_t nblk_max; int32_t D;
  void* dst; lca_dtype dst_dt; void* dst_scale; int64_t dst_rows;
  float* pooled;
  int32_t gate_pc; int32_t overlap;
} lca_compress_job;

lca_status lca_compress_batch(const lca_compress_job* jobs, int32_t njobs, void* stream);

/*
 * lca_lightning_index_topk -- lightning-indexer scores and top-k selection.
 * [release notes (agentlenshq.com), 壓縮稀疏注意力 (CSA): FP4, ReLU-scored
 * multi-head dot products pick the top-k compressed blocks per query; wiki
 * (chenshi221), 基础设施: MXFP4 on the indexer QK path.]
 *
 * Query row r = b*Tq + t scores entries j < n_elig[r] of sequence b:
 *     s_j = sum_{h<H_I} w[r][h] * max(0, sum_{i<d_I} qi[r][h][i] * ki[b][j][i])
 * with every per-head dot product and the head sum evaluated exactly as the
 * float64 sum left to right over i and then over h of the decoded values
 * (products formed, then added).  The selection orders entries by (s_j
 * descending, j ascending) and keeps the first min(k, n_elig[r]).
 *   qi     [B][Tq][H_I][d_I]   qi_dt in {F32, MXFP4}; qi_scale: E8M0
 *          [B][Tq][H_I][d_I/32] for MXFP4, NULL otherwise
 *   w      [B][Tq][H_I] fp32 head weights
 *   ki     [B][N_cap][d_I]     ki_dt == qi_dt; ki_scale E8M0 [B][N_cap][d_I/32]
 *   n_elig [B][Tq] int32 (device); the kernels clamp it to [0, N_cap]
 *   idx_out   [B][Tq][k] int32: the selected j in ascending order, -1 padded
 *   score_out optional [B][Tq][k] double: s_j of each idx_out entry (0 for -1)
 *   ws / ws_bytes: workspace of at least lca_index_topk_ws(...) bytes
 * Supported: 1 <= k <= 2048; MXFP4: H_I <= 16, d_I in {64, 128}; F32:
 * H_I <= 16, d_I in {32, 64, 128}; N_cap < 2^31.
 * Results are deterministic and independent of B and of the other rows.
 */
lca_status lca_lightning_index_topk(const void* qi, lca_dtype qi_dt, const uint8_t* qi_scale,
                                    const float* w, const void* ki, lca_dtype ki_dt,
                                    const uint8_t* ki_scale, const int32_t* n_elig, int32_t B,
                                    int32_t Tq, int32_t H_I, int32_t d_I, int64_t N_cap,
                                    int32_t k, int32_t* idx_out, double* score_out, void* ws,
                                    size_t ws_bytes, void* stream);

size_t lca_index_topk_ws(int32_t B, int32_t Tq, int32_t H_I, int32_t d_I, int64_t N_cap,
                         int32_t k);

/*
 * lca_sparse_mqa_attend -- CSA attention of each query over its selected
 * compressed entries, a window of raw tokens and a per-head sink.
 * [wiki (chenshi221), 架构创新: top-k sparse selection + MQA, sliding-window
 * branch and attention sink; release notes, 壓縮稀疏注意力 (CSA): the window
 * holds recent uncompressed tokens.]
 *
 * For query row r = b*Tq + t and head h (one vector per entry/token serves as
 * key and value, shared by all heads):
 *     l_j = scale * <q[r][h], kv[b][j]>     for j in idx[r] (entries != -1)
 *     l_u = scale * <q[r][h], win[b][u]>    for u in [win_begin[r], win_begin[r] + win_len[r])
 *     M   = max(sink[h], all l);  Z = exp(sink[h] - M) + sum exp(l - M)
 *     out[r][h] = (sum_j exp(l_j - M) kv[b][j] + sum_u exp(l_u - M) win[b][u]) / Z
 *     lse[r][h] = M + log Z
 * The sink logit is not multiplied by `scale` and has a zero value vector.
 *   q      [B][Tq][Hq][D]  q_dt in {F32, BF16}
 *   kv     [B][N_cap][D]   kv_dt in {F32, BF16, FP8E4M3}; kv_scale fp32
 *          [B][N_cap][D/64] for FP8, NULL otherwise
 *   idx    [B][Tq][k] int32 (device); entries < 0 or >= N_cap are skipped
 *   win    [B][W_buf][D]   win_dt in {F32, BF16}; win_begin/win_len [B][Tq]
 *          int32 (device), meant to satisfy 0 <= win_begin, 0 <= win_len,
 *          win_begin + win_len <= W_buf; the kernels clamp the begin to
 *          [0, W_buf - 1] and the length to [0, W_buf - begin], so no value
 *          reads outside `win`
 *   sink   [Hq] fp32
 *   out    [B][Tq][Hq][D]  out_dt in {F32, BF16}; lse optional fp32 [B][Tq][Hq]
 * Supported: D = 128; Hq in {16, 32, 64}; 0 <= k <= 2048.  F32 inputs are
 * computed in fp32; BF16/FP8 inputs use bf16 matrix cores with fp32
 * accumulation and softmax.
 */
lca_status lca_sparse_mqa_attend(const void* q, lca_dtype q_dt, const void* kv, lca_dtype kv_dt,
                                 const float* kv_scale, int64_t N_cap, const int32_t* idx,
                                 int32_t k, const void* win, lca_dtype win_dt, int64_t W_buf,
                                 const int32_t* win_begin, const int32_t* win_len,
                                 const float* sink, float scale, int32_t B, int32_t Tq,
                                 int32_t Hq, int32_t D, void* out, lca_dtype out_dt, float* lse,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * lca_hca_attend -- HCA attention: as lca_sparse_mqa_attend, but over every
 * eligible entry j < n_elig[r] of sequence b instead of a selected list.
 * [release notes (agentlenshq.com), 重度壓縮注意力 (HCA): the 128x compressed
 * sequence is short, so it is attended densely, plus a sliding window.]
 *   n_elig [B][Tq] int32 (device); the kernels clamp it to [0, N_cap].
 * Supported: as lca_sparse_mqa_attend.
 */
lca_status lca_hca_attend(const void* q, lca_dtype q_dt, const void* kv, lca_dtype kv_dt,
                          const float* kv_scale, int64_t N_cap, const int32_t* n_elig,
                          const void* win, lca_dtype win_dt, int64_t W_buf,
                          const int32_t* win_begin, const int32_t* win_len, const float* sink,
                          float scale, int32_t B, int32_t Tq, int32_t Hq, int32_t D, void* out,
                          lca_dtype out_dt, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * lca_attend_separate_v -- the attention of lca_sparse_mqa_attend (sparse = 1,
 * idx, k) or lca_hca_attend (sparse = 0, n_elig) with separate key and value
 * vectors: logits from k / win_k, weighted sums of v / win_v.  A variant: the
 * pages describe MQA over one compressed entry per block and leave open
 * whether one vector serves as key and value (the reading of the other calls)
 * [wiki (chenshi221), 架构创新: MQA over the selected compressed entries].
 *   k, v     [B][N_cap][D] of kv_dt; FP8: k_scale, v_scale fp32 [B][N_cap][D/64]
 *   win_k, win_v [B][W_buf][D] of win_dt
 * Other arguments, workspace and guarantees as lca_sparse_mqa_attend /
 * lca_hca_attend.  bf16 queries and windows with bf16 or FP8 entries run on
 * the matrix-core kernels (each tile's key and value rows staged separately;
 * with v = k the bytes of the shared-KV call); fp32 storage on the vector-ALU
 * kernel.
 */
lca_status lca_attend_separate_v(int32_t sparse, const void* q, lca_dtype q_dt, const void* k,
                                 const void* v, lca_dtype kv_dt, const float* k_scale,
                                 const float* v_scale, int64_t N_cap, const int32_t* idx, int32_t kk,
                                 const int32_t* n_elig, const void* win_k, const void* win_v,
                                 lca_dtype win_dt, int64_t W_buf, const int32_t* win_begin,
                                 const int32_t* win_len, const float* sink, float scale, int32_t B,
                                 int32_t Tq, int32_t Hq, int32_t D, void* out, lca_dtype out_dt,
                                 float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * lca_window_attend -- attention over the sliding window and the sink alone,
 * with no compressed entries: the attention of the multi-token-prediction
 * block that follows the 61 CSA/HCA layers of V4-Pro.  [release notes
 * (agentlenshq.com), 架構實現: the final MTP block of V4-Pro uses only
 * sliding-window attention.]  The softmax of lca_sparse_mqa_attend with an
 * empty selection (k = 0, no entry cache); arguments as there, workspace
 * lca_attend_ws(B, Tq, Hq, D, 0, W_buf).  In lca_attend_batch and
 * lca_decode_step the same job is sparse = 1, k = 0, kv = NULL, N_cap = 0.
 * Supported: D = 128; Hq in {16, 32, 64}.
 */
lca_status lca_window_attend(const void* q, lca_dtype q_dt, const void* win, lca_dtype win_dt,
                             int64_t W_buf, const int32_t* win_begin, const int32_t* win_len,
                             const float* sink, float scale, int32_t B, int32_t Tq, int32_t Hq,
                             int32_t D, void* out, lca_dtype out_dt, float* lse, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * lca_attend_batch -- several attention calls in one launch (one attention
 * launch and at most one merge launch for all jobs), for example the CSA and
 * HCA branches of one decode step.  Each job is the argument list of
 * lca_sparse_mqa_attend (sparse = 1: idx, k) or lca_hca_attend (sparse = 0:
 * n_elig) with the same meaning, layouts, workspace and caller guarantees,
 * and its result is bit-identical to that single call.  [Same passages as
 * the two single calls.]
 *   jobs     host array of njobs descriptors, read during the call only;
 *            1 <= njobs <= LCA_MAX_ATTEND_JOBS.
 * Each job is validated as its single call; in addition every job takes bf16
 * q and window and bf16 or FP8 entries, all jobs share kv_dt and Hq, and no
 * job may have the chunked-prefill shape (many query rows and no split: a
 * dense call with several rows per sequence, or a sparse call with bf16
 * entries and 64 heads, which the single call runs with kernels of their
 * own): LCA_ENOTSUP otherwise.  Jobs must not share output, lse or workspace
 * memory.  On any invalid job nothing is enqueued and the message names it.
 */
#define LCA_MAX_ATTEND_JOBS 4
typedef struct lca_attend_job {
  int32_t sparse;
  const void* q; lca_dtype q_dt;
  const void* kv; lca_dtype kv_dt; const float* kv_scale; int64_t N_cap;
  const int32_t* idx; int32_t k;
  const int32_t* n_elig;
  const void* win; lca_dtype win_dt; int64_t W_buf;
  const int32_t* win_begin; const int32_t* win_len;
  const float* sink; float scale;
  int32_t B; int32_t Tq; int32_t Hq; int32_t D;
  void* out; lca_dtype out_dt; float* lse;
  void* ws; size_t ws_bytes;
} lca_attend_job;

lca_status lca_attend_batch(const lca_attend_job* jobs, int32_t njobs, void* stream);

/*
 * lca_decode_step -- one decode step of the layer pair in one call:
 * lca_compress_batch(cjobs), then lca_lightning_index_topk(*ijob), then
 * lca_attend_batch(ajobs), with the results of those three calls issued in
 * that order (bit-identical), and with fewer dependent launches: the dense
 * attention jobs (sparse = 0) run beside the indexer's scan, since they read
 * nothing the indexer writes.  [release notes (agentlenshq.com), 壓縮稀疏注意力
 * (CSA) / 重度壓縮注意力 (HCA): only the CSA branch depends on the top-k.]
 *   cjobs    0 <= ncjobs <= LCA_MAX_COMPRESS_JOBS compress jobs (as lca_compress_batch)
 *   ijob     the indexer call's arguments (as lca_lightning_index_topk), or
 *            NULL for a step without an indexer (an HCA or window-only layer)
 *   ajobs    0 <= najobs <= LCA_MAX_ATTEND_JOBS attention jobs (as lca_attend_batch)
 * Each part is validated as its own call.  Dense attention jobs must not
 * read or write memory the indexer job writes (idx_out, score_out, its
 * workspace); a dense job whose output, lse or workspace overlaps those is
 * rejected with LCA_EINVAL; sparse jobs may read idx_out.  Host arrays are read during the
 * call only.  When every compress job has nblk_max = 1, overlap = 0, bf16
 * input and width 128, and no compress job writes any byte that the scan or
 * the dense jobs read or write -- except a job that writes exactly the
 * indexer's key cache (dst = ki, dst_scale = ki_scale, dst_rows = N_cap) or
 * exactly a dense job's entry cache (dst = kv, dst_scale = kv_scale,
 * dst_rows = N_cap) -- nor reads any byte they write, the compress jobs run
 * in the scan launch, and the scan and attention workgroups that read a new
 * row compute that row from the raw tokens themselves, with the same code
 * (same bytes).  Otherwise the compress jobs run in a launch of their own
 * first.  Either way the results are those of the three calls in order.
 */
/*
 * lca_decode_step_events -- lca_decode_step with HIP events recorded on
 * `stream` around its kernel launches, for measurement (same work, same
 * results).  events[0] is recorded before the first launch and events[i]
 * after launch i, so the elapsed time between events[i - 1] and events[i] is
 * the duration of launch i on the stream.  The step makes at most
 * LCA_MAX_STEP_LAUNCHES launches; their order follows lca_decode_step.
 *   events   host array of at least LCA_MAX_STEP_LAUNCHES + 1 hipEvent_t
 *            handles created by the caller (timing enabled to read times)
 *   names    NULL, or a host array of LCA_MAX_STEP_LAUNCHES pointers that
 *            receives, per launch, the name of its kernel (static strings)
 *   nlaunch  receives the number of launches made (events[0 .. *nlaunch] recorded)
 * Other arguments, validation and errors as lca_decode_step; LCA_EINVAL for a
 * NULL or short events array or a NULL nlaunch.  Not for use under stream
 * capture (events are recorded between the launches).
 */
#define LCA_MAX_STEP_LAUNCHES 8

typedef struct lca_index_job {
  const void* qi; lca_dtype qi_dt; const uint8_t* qi_scale; const float* w;
  const void* ki; lca_dtype ki_dt; const uint8_t* ki_scale; const int32_t* n_elig;
  int32_t B; int32_t Tq; int32_t H_I; int32_t d_I; int64_t N_cap; int32_t k;
  int32_t* idx_out; double* score_out; void* ws; size_t ws_bytes;
} lca_index_job;

lca_status lca_decode_step(const lca_compress_job* cjobs, int32_t ncjobs, const lca_index_job* ijob,
                           const lca_attend_job* ajobs, int32_t najobs, void* stream);

lca_status lca_decode_step_events(const lca_compress_job* cjobs, int32_t ncjobs, const lca_index_job* ijob,
                                  const lca_attend_job* ajobs, int32_t najobs, void* const* events, int32_t nevents,
                                  const char** names, int32_t* nlaunch, void* stream);

/*
 * lca_decode_step_noalloc -- lca_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same call, with every workspace taken from a
 * scratch array that the library holds in each GPU's memory
 * (LCA_NOALLOC_SCRATCH_BYTES per device, from the first call on that device
 * until the process ends) instead of from the jobs' ws / ws_bytes fields,
 * which are ignored.  Same results as lca_decode_step.  The call uses the
 * scratch of the current device (the stream must belong to it); it allocates
 * nothing.
 *   Errors: those of lca_decode_step; LCA_EWORKSPACE when the step's
 *   workspaces (the sizes lca_index_topk_ws and lca_attend_ws return, each
 *   rounded up to 256 bytes) exceed LCA_NOALLOC_SCRATCH_BYTES, before
 *   anything is enqueued.
 * Every call on one GPU uses that GPU's scratch, and the scratch keeps the
 * last call's contents: calls that overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller.  Nothing in the scratch
 * needs to start at zero (the kernels initialise what they read).
 */
#define LCA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

lca_status lca_decode_step_noalloc(const lca_compress_job* cjobs, int32_t ncjobs, const lca_index_job* ijob,
                                   const lca_attend_job* ajobs, int32_t najobs, void* stream);

/*
 * lca_decode_append -- the token append of a decode loop, for several raw-token
 * streams in one launch (for example a CSA layer's raw KV, its indexer's raw
 * keys and an HCA layer's raw KV): each sequence's new token goes into the
 * stream's ring, and the step's arguments for lca_decode_step are derived on
 * the device, so that one captured step can be replayed step after step.
 * [release notes (agentlenshq.com), 壓縮稀疏注意力 (CSA): the most recent
 * tokens stay uncompressed in a sliding window, and a block of m tokens
 * becomes one compressed entry once it is complete (m = 4 for CSA, 128 for
 * HCA).]
 * Ring: token t of sequence b is stored at rows t % R and t % R + R of
 * ring[b] ([B][2R][D]) and of gring[b] ([B][2R]), so that every run of at most
 * R consecutive tokens (a block being compressed, the window) is contiguous.
 *   x_new    [B][D] device, the new tokens (x_dt: bf16 or f32; the ring's type)
 *   g_new    [B] fp32 device, their gate logits, with gring; both NULL: no gate ring
 *            (gate_pc = 1: one logit per channel, g_new [B][D], gring [B][2R][D])
 *   len      [B] int64 device: tokens before the call; the call adds 1
 *   R        ring rows, >= max(1, m, W)
 *   m        compression block of the stream (0: not compressed)
 *   W        window of the stream's attention (0: no window outputs needed)
 * Outputs, for L = len + 1 tokens (device, each may be NULL):
 *   nblk[b] = 1 when L % m == 0 (a block completed), else 0
 *   x_tok0[b] = ring row of token L - m - overlap (the first token of the
 *            completed block's span; overlap 0 .. m as in the compress jobs,
 *            R >= m + overlap)
 *   dst_row0[b] = L / m - 1 (its cache row);  n_elig[b] = L / m
 *   win_begin[b], win_len[b]: ring rows of the last min(L, W) tokens
 * These are the x_tok0 / nblk / dst_row0 of a compress job with x = ring,
 * x_rows = 2R, gate = gring, nblk_max = 1, and the n_elig / win_begin /
 * win_len of an attention or indexer job with win = ring, W_buf = 2R, Tq = 1.
 * Jobs must not share len, rings or outputs.  Errors: LCA_EINVAL (null or
 * misaligned x_new/ring, null len, bad sizes), LCA_ENOTSUP (D not 64/128,
 * x_dt not bf16/f32).
 */
#define LCA_MAX_APPEND_JOBS 8
typedef struct lca_append_job {
  const void* x_new; lca_dtype x_dt; const float* g_new;
  void* ring; float* gring; int64_t R;
  int64_t* len; int32_t m; int32_t W;
  int32_t* x_tok0; int32_t* nblk; int64_t* dst_row0; int32_t* n_elig;
  int32_t* win_begin; int32_t* win_len;
  int32_t B; int32_t D;
  int32_t overlap; int32_t gate_pc;
} lca_append_job;

lca_status lca_decode_append(const lca_append_job* jobs, int32_t njobs, void* stream);

/*
 * lca_decode_loop_step -- one step of a decode loop in one call:
 * lca_decode_append(app) followed by lca_decode_step(cjobs, ijob, ajobs), with
 * the same results; the appends run inside the compress launch, or in a
 * launch of their own when the compress jobs join the scan launch (see
 * lca_decode_step).  [Sources as lca_decode_append and lca_decode_step.]
 * A compress job whose x is an append job's ring is that stream's block
 * compression: it must take x_tok0, nblk and dst_row0 from that append job,
 * have nblk_max = 1, the append job's B, m, x_dt and D, and x_rows = 2R; its
 * workgroup appends the token, then compresses.  Append jobs that no compress
 * job reads (for example a window-only stream) get workgroups of their own in
 * the same launch.  No two compress jobs may read one append job's ring, and
 * no compress job may read a ring through any other pointer.
 *   app      0 <= napp <= LCA_MAX_APPEND_JOBS append jobs (as lca_decode_append)
 *   cjobs, ijob (may be NULL), ajobs   as lca_decode_step
 * Errors: those of the two calls; LCA_EINVAL when a compress job breaks the
 * pairing rules above.
 */
lca_status lca_decode_loop_step(const lca_append_job* app, int32_t napp, const lca_compress_job* cjobs,
                                int32_t ncjobs, const lca_index_job* ijob, const lca_attend_job* ajobs,
                                int32_t najobs, void* stream);

/* Workspace bytes for the attention calls.  n_kv_max is k for
 * lca_sparse_mqa_attend and N_cap for lca_hca_attend; W_buf the window buffer
 * rows. */
size_t lca_attend_ws(int32_t B, int32_t Tq, int32_t Hq, int32_t D, int64_t n_kv_max,
                     int64_t W_buf);

#ifdef __cplusplus
}
#endif
#endif /* LCA_H */
