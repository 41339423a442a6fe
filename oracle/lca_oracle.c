/*
 * lca_oracle.c -- plain, slow, float64 CPU oracle for the CSA/HCA hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls anything in this directory, and this file shares no
 * code, table or constant generator with it.
 *
 * Sources (page title, section):
 *   [RN-CSA]  "DeepSeek-V4 發佈說明：為 AI Agents 提供高效的 1M-Token 上下文"
 *             (agentlenshq.com), section "壓縮稀疏注意力 (CSA)": KV compressed 4x
 *             by softmax-gated pooling with a learned positional bias; a
 *             lightning indexer (FP4, ReLU-scored multi-head dot products) picks
 *             the top-k compressed blocks per query; a sliding-window branch
 *             covers recent uncompressed tokens.
 *   [RN-HCA]  same page, section "重度壓縮注意力 (HCA)": 128x compression, dense
 *             attention over every compressed block, plus a sliding window.
 *   [RN-IMPL] same page, section "架構實現": most KV entries stored in FP8, the
 *             CSA indexer in FP4.
 *   [WIKI]    "DeepSeek V4: Towards Highly Efficient Million-Token Context
 *             Intelligence" (chenshi221.pages.dev wiki), section 关键技术方法 ›
 *             架构创新: m tokens become one entry, top-k + MQA, sliding window and
 *             attention sink; section 基础设施: MXFP4 on the indexer QK path, FP4
 *             to FP8 dequantisation is lossless.
 *   [OCP-FP8] OCP 8-bit Floating Point Specification (OFP8) v1.0, E4M3.
 *   [OCP-MX]  OCP Microscaling Formats (MX) v1.0: E2M1 elements, E8M0 scales,
 *             blocks of 32, shared exponent floor(log2 amax) - emax_elem.
 *
 * Where the pages leave a step open, the reading taken is stated next to the
 * function (gate = one scalar per token; K = V; sink = a per-head logit that adds
 * to the softmax denominator with a zero value vector and is not scaled; the
 * window is the last W raw tokens including the query's own; ties in top-k go to
 * the lower index).
 *
 * Parity status: every function below is pinned by CPU tests (closed forms,
 * library routines on special cases, brute force, exhaustive code tables); the
 * end-to-end pipeline has no printed value on the pages to pin against.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8E4M3 = 2, ORC_MXFP4 = 3 };

/* ------------------------------------------------------------------------- */
/* Codecs                                                                    */
/* ------------------------------------------------------------------------- */

/* [OCP-FP8] E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is
 * subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities; max 448. */
double orc_e4m3_value(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* [OCP-MX] E2M1 element values for codes 0..7 (sign in bit 3). */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int code) {
  double v = E2M1_MAG[code & 7];
  return (code & 8) ? -v : v;
}

/* Nearest of a sorted table of non-negative magnitudes (index = code), ties to
 * the even code, values beyond the last entry saturate to it.  Binary search for
 * the bracketing pair, then compare distances exactly in float64. */
static int nearest_even(const double* mag, int n, double a) {
  int lo = 0, hi = n - 1;
  if (a >= mag[n - 1]) return n - 1;
  while (hi - lo > 1) {          /* invariant: mag[lo] <= a < mag[hi] */
    int mid = (lo + hi) / 2;
    if (mag[mid] <= a) lo = mid; else hi = mid;
  }
  {
    double dl = a - mag[lo], dh = mag[hi] - a;
    if (dl < dh) return lo;
    if (dh < dl) return hi;
    return (lo % 2 == 0) ? lo : hi;
  }
}

static double E4M3_MAG[127];   /* codes 0x00..0x7E */
static int tables_ready = 0;
static void init_tables(void) {
  int c;
  if (tables_ready) return;
  for (c = 0; c < 127; ++c) E4M3_MAG[c] = orc_e4m3_value(c);
  tables_ready = 1;
}

/* RNE onto E4M3, saturating at +-448.  Input is a finite fp32 value. */
int orc_e4m3_encode(float y) {
  double a = fabs((double)y);
  int code;
  init_tables();
  code = nearest_even(E4M3_MAG, 127, a);
  if (signbit(y)) code |= 0x80;
  return code;
}

/* RNE onto E2M1, saturating at +-6; the sign bit follows the input's sign. */
int orc_e2m1_encode(double y) {
  double a = fabs(y);
  int code = nearest_even(E2M1_MAG, 8, a);
  if (signbit(y)) code |= 8;   /* the sign is kept, also for values that round to 0 */
  return code;
}

/* FP8 cache format (reading for "FP8 storage" [RN-IMPL]; the per-64 fp32 scale is
 * part of the task's configuration): per group of 64 fp32 values,
 *   amax = max|v|, s = fl32(amax / 448) (correctly rounded fp32 division),
 *   s = 1 when amax == 0, s = 2^-149 if the division underflows to zero,
 *   code = RNE_sat(fl32(v / s)), decoded value = e4m3(code) * s.            */
void orc_fp8_encode(const float* v, int64_t n, uint8_t* codes, float* scales) {
  int64_t g, i;
  for (g = 0; g < n / 64; ++g) {
    const float* x = v + g * 64;
    float amax = 0.0f, s;
    for (i = 0; i < 64; ++i) { float a = fabsf(x[i]); if (a > amax) amax = a; }
    if (amax == 0.0f) s = 1.0f;
    else {
      s = amax / 448.0f;
      if (s == 0.0f) s = ldexpf(1.0f, -149);
    }
    scales[g] = s;
    for (i = 0; i < 64; ++i) {
      float q = x[i] / s;
      codes[g * 64 + i] = (uint8_t)orc_e4m3_encode(q);
    }
  }
}

void orc_fp8_decode(const uint8_t* codes, const float* scales, int64_t n, double* out) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = orc_e4m3_value(codes[i]) * (double)scales[i / 64];
}

/* [OCP-MX] MXFP4: per block of 32 values, shared exponent
 *   X = floor(log2(amax)) - 2 (2 = exponent of the largest E2M1 value), clamped
 *   to the E8M0 range [-127, 127]; amax == 0 gives X = -127.  Elements are
 *   RNE_sat(v / 2^X) onto E2M1.  Codes are packed two per byte, element 2i in
 *   the low nibble.  The E8M0 byte is X + 127. */
void orc_mxfp4_encode(const float* v, int64_t n, uint8_t* codes, uint8_t* scales) {
  int64_t b, i;
  for (b = 0; b < n / 32; ++b) {
    const float* x = v + b * 32;
    double amax = 0.0;
    int X;
    for (i = 0; i < 32; ++i) { double a = fabs((double)x[i]); if (a > amax) amax = a; }
    if (amax == 0.0) X = -127;
    else {
      int E;
      frexp(amax, &E);          /* amax = f * 2^E, f in [0.5, 1) */
      X = (E - 1) - 2;
      if (X < -127) X = -127;
      if (X > 127) X = 127;
    }
    scales[b] = (uint8_t)(X + 127);
    for (i = 0; i < 32; i += 2) {
      int c0 = orc_e2m1_encode(ldexp((double)x[i], -X));
      int c1 = orc_e2m1_encode(ldexp((double)x[i + 1], -X));
      codes[b * 16 + i / 2] = (uint8_t)(c0 | (c1 << 4));
    }
  }
}

void orc_mxfp4_decode(const uint8_t* codes, const uint8_t* scales, int64_t n, double* out) {
  int64_t i;
  for (i = 0; i < n; ++i) {
    int byte = codes[i / 2];
    int c = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
    out[i] = ldexp(orc_e2m1_value(c), (int)scales[i / 32] - 127);
  }
}

/* bfloat16 storage: the top 16 bits of an fp32 value; encoding rounds an fp32
 * value to nearest-even on the dropped 16 bits (values here are finite). */
double orc_bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

uint16_t orc_bf16_encode(float f) {
  uint32_t u;
  double a, lo, hi;
  uint16_t t;
  memcpy(&u, &f, 4);
  t = (uint16_t)(u >> 16);                      /* truncation = one neighbour */
  lo = orc_bf16_value(t);
  a = (double)f;
  if (lo == a) return t;
  /* the other neighbour is one bf16 step further from zero */
  hi = orc_bf16_value((uint16_t)(t + 1));
  if (fabs(a - lo) < fabs(hi - a)) return t;
  if (fabs(hi - a) < fabs(a - lo)) return (uint16_t)(t + 1);
  return (t % 2 == 0) ? t : (uint16_t)(t + 1);
}

/* Decode n elements of any supported storage type to float64.
 * F32: float[n]; BF16: uint16[n]; FP8: uint8[n] + float scale per 64;
 * MXFP4: uint8[n/2] + uint8 E8M0 per 32. */
void orc_decode(const void* src, int dt, const void* scale, int64_t n, double* out) {
  int64_t i;
  switch (dt) {
    case ORC_F32: for (i = 0; i < n; ++i) out[i] = (double)((const float*)src)[i]; break;
    case ORC_BF16: for (i = 0; i < n; ++i) out[i] = orc_bf16_value(((const uint16_t*)src)[i]); break;
    case ORC_FP8E4M3: orc_fp8_decode((const uint8_t*)src, (const float*)scale, n, out); break;
    case ORC_MXFP4: orc_mxfp4_decode((const uint8_t*)src, (const uint8_t*)scale, n, out); break;
    default: for (i = 0; i < n; ++i) out[i] = NAN;
  }
}

/* Encode n fp32 values (n a multiple of 64) to a storage type. */
void orc_encode(const float* v, int64_t n, int dt, void* dst, void* scale) {
  int64_t i;
  switch (dt) {
    case ORC_F32: memcpy(dst, v, (size_t)n * 4); break;
    case ORC_BF16: for (i = 0; i < n; ++i) ((uint16_t*)dst)[i] = orc_bf16_encode(v[i]); break;
    case ORC_FP8E4M3: orc_fp8_encode(v, n, (uint8_t*)dst, (float*)scale); break;
    case ORC_MXFP4: orc_mxfp4_encode(v, n, (uint8_t*)dst, (uint8_t*)scale); break;
    default: break;
  }
}

/* ------------------------------------------------------------------------- */
/* O1: compression by softmax-gated pooling with a positional bias           */
/* [RN-CSA] (m = 4), [RN-HCA] (m = 128), [WIKI] (m tokens -> 1 entry).       */
/* Reading: one gate logit per raw token; non-overlapping blocks; an         */
/* incomplete tail block is not pooled.  For block j:                        */
/*   a_i = gate[jm+i] + bias[i];  w_i = exp(a_i - max a) / sum exp(a - max a) */
/*   c_j = sum_i w_i * x[jm+i]     (sums left to right over i)               */
/* ------------------------------------------------------------------------- */
void orc_pool(const double* x, const double* gate, const double* bias,
              int64_t nblk, int m, int D, double* out) {
  int64_t j;
  double* a = (double*)malloc(sizeof(double) * (size_t)m);
  double* e = (double*)malloc(sizeof(double) * (size_t)m);
  for (j = 0; j < nblk; ++j) {
    int i, d;
    double amax = -INFINITY, z = 0.0;
    for (i = 0; i < m; ++i) {
      a[i] = gate[j * m + i] + bias[i];
      if (a[i] > amax) amax = a[i];
    }
    for (i = 0; i < m; ++i) { e[i] = exp(a[i] - amax); z += e[i]; }
    for (d = 0; d < D; ++d) {
      double c = 0.0;
      for (i = 0; i < m; ++i) c += (e[i] / z) * x[(j * m + i) * D + d];
      out[j * D + d] = c;
    }
  }
  free(a);
  free(e);
}

/* ------------------------------------------------------------------------- */
/* O1 variants.  The pages name softmax-gated pooling with a learned          */
/* positional bias [RN-CSA] but give neither the gate's shape nor whether     */
/* blocks overlap; orc_pool takes one logit per token and disjoint blocks.    */
/* These are the two alternatives, alone or together:                         */
/*  - gate_pc = 1: one logit per token and channel, gate[t][d], with a bias   */
/*    per block position and channel, bias[u][d]; one softmax per channel;    */
/*  - overlap o (0 <= o <= m): block j pools the positions jm - o .. jm+m-1   */
/*    that exist (positions below 0 are left out of the softmax); the bias    */
/*    index of position t is u = t - (jm - o), so bias has m + o rows.        */
/* For block j and channel d, over the existing positions t_u:               */
/*   a_u = gate(t_u, d) + bias(u, d);  w_u = exp(a_u - max a) / sum exp(..)  */
/*   c_j[d] = sum_u w_u * x[t_u][d]     (sums in increasing u)               */
/* ------------------------------------------------------------------------- */
void orc_pool_variant(const double* x, const double* gate, int gate_pc, const double* bias,
                      int64_t nblk, int m, int o, int D, double* out) {
  int64_t j;
  double* a = (double*)malloc(sizeof(double) * (size_t)(m + o));
  for (j = 0; j < nblk; ++j) {
    const int64_t t0 = j * m - o;                       /* position of u = 0 */
    const int u0 = t0 < 0 ? (int)(-t0) : 0;             /* first existing u */
    int d, u;
    for (d = 0; d < D; ++d) {
      double amax = -INFINITY, z = 0.0, c = 0.0;
      for (u = u0; u < m + o; ++u) {
        const int64_t t = t0 + u;
        a[u] = (gate_pc ? gate[t * D + d] : gate[t]) + (gate_pc ? bias[(int64_t)u * D + d] : bias[u]);
        if (a[u] > amax) amax = a[u];
      }
      for (u = u0; u < m + o; ++u) z += exp(a[u] - amax);
      for (u = u0; u < m + o; ++u) c += (exp(a[u] - amax) / z) * x[(t0 + u) * D + d];
      out[j * D + d] = c;
    }
  }
  free(a);
}

/* ------------------------------------------------------------------------- */
/* O3: lightning-indexer score of entry j for one query [RN-CSA]             */
/*   r_h = max(0, sum_i q[h][i] * k[j][i])    (left to right over i)         */
/*   s_j = sum_h w[h] * r_h                   (left to right over h)         */
/* Products are formed then added (no fused multiply-add).                   */
/* ------------------------------------------------------------------------- */
double orc_index_score(const double* q, const double* w, const double* kj, int H, int d) {
  double s = 0.0;
  int h, i;
  for (h = 0; h < H; ++h) {
    double dot = 0.0, r, t;
    for (i = 0; i < d; ++i) { double p = q[h * d + i] * kj[i]; dot = dot + p; }
    r = dot > 0.0 ? dot : 0.0;
    t = w[h] * r;
    s = s + t;
  }
  return s;
}

/* ------------------------------------------------------------------------- */
/* O4: top-k.  Order entries by (score descending, index ascending), keep the */
/* first min(k, n_elig), emit them in ascending index order, pad with -1.    */
/* A library sort serves as the step.                                        */
/* ------------------------------------------------------------------------- */
typedef struct { double s; int64_t j; } scored_t;

static int cmp_rank(const void* pa, const void* pb) {
  const scored_t* a = (const scored_t*)pa;
  const scored_t* b = (const scored_t*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j < b->j) ? -1 : (a->j > b->j);
}

static int cmp_i32(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

void orc_select_topk(const double* s, int64_t n_elig, int k, int32_t* idx, double* sel_score) {
  int64_t j, nsel = n_elig < k ? n_elig : k;
  scored_t* v = (scored_t*)malloc(sizeof(scored_t) * (size_t)(n_elig > 0 ? n_elig : 1));
  for (j = 0; j < n_elig; ++j) { v[j].s = s[j]; v[j].j = j; }
  qsort(v, (size_t)n_elig, sizeof(scored_t), cmp_rank);
  for (j = 0; j < nsel; ++j) idx[j] = (int32_t)v[j].j;
  qsort(idx, (size_t)nsel, sizeof(int32_t), cmp_i32);
  for (j = nsel; j < k; ++j) idx[j] = -1;
  if (sel_score) {
    for (j = 0; j < k; ++j) sel_score[j] = idx[j] >= 0 ? s[idx[j]] : 0.0;
  }
  free(v);
}

/* Indexer + top-k over a batch of query rows.  Row r = b*Tq + t uses the key
 * cache of sequence b.  Keys are decoded one row at a time.
 *   qi   : decoded float64 [B*Tq][H][d]
 *   w    : float32 [B*Tq][H]
 *   keys : storage [B][N_cap][d] of type key_dt (+ scales)
 *   scores_out (optional): float64 [B*Tq][N_cap], eligible part filled        */
void orc_index_topk(const double* qi, const float* w, const void* keys, int key_dt,
                    const void* key_scale, const int32_t* n_elig, int B, int Tq, int H,
                    int d, int64_t N_cap, int k, int32_t* idx_out, double* sel_score,
                    double* scores_out) {
  int64_t r, R = (int64_t)B * Tq;
  /* rows one after another; the entries of a row are scored in parallel (each
   * score is its own left-to-right evaluation, so the split changes nothing) */
  for (r = 0; r < R; ++r) {
    int b = (int)(r / Tq);
    int64_t n = n_elig[r], j, h;
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double wd[64];
    for (h = 0; h < H; ++h) wd[h] = (double)w[r * H + h];
#pragma omp parallel
    {
      double* kj = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static)
      for (j = 0; j < n; ++j) {
        int64_t row = (int64_t)b * N_cap + j;
        if (key_dt == ORC_F32) orc_decode((const float*)keys + row * d, key_dt, NULL, d, kj);
        else if (key_dt == ORC_BF16) orc_decode((const uint16_t*)keys + row * d, key_dt, NULL, d, kj);
        else if (key_dt == ORC_FP8E4M3)
          orc_decode((const uint8_t*)keys + row * d, key_dt, (const float*)key_scale + row * (d / 64), d, kj);
        else
          orc_decode((const uint8_t*)keys + row * (d / 2), key_dt, (const uint8_t*)key_scale + row * (d / 32), d, kj);
        s[j] = orc_index_score(qi + r * H * d, wd, kj, H, d);
        if (scores_out) scores_out[r * N_cap + j] = s[j];
      }
      free(kj);
    }
    orc_select_topk(s, n, k, idx_out + r * k, sel_score ? sel_score + r * k : NULL);
    free(s);
  }
}

/* ------------------------------------------------------------------------- */
/* O5: attention of one query row over (selected entries U window U sink).    */
/* [WIKI] MQA over the selected entries, sliding window, attention sink;     */
/* [RN-CSA]/[RN-HCA] window of recent uncompressed tokens.                   */
/* Readings: one vector per entry/token serves as key and value; the sink is */
/* a per-head logit sigma_h, not multiplied by the softmax scale, whose value */
/* vector is zero.  For head h:                                              */
/*   l_j = tau * <q_h, c_j> (entries),  l_t = tau * <q_h, x_t> (window)       */
/*   M = max(sigma_h, all l);  Z = e^(sigma_h-M) + sum e^(l_j-M) + sum e^(l_t-M) */
/*   o_h = (sum e^(l_j-M) c_j + sum e^(l_t-M) x_t) / Z;  lse_h = M + log Z    */
/* Entries come first (in the order given), then window tokens, in every sum. */
/*   q   : [Hq][D]; ent: [n_ent][D] (already gathered); win: [n_win][D]      */
/* ------------------------------------------------------------------------- */
/* Separate values (a variant; the pages leave K vs V open and the reading   */
/* above takes K = V): the logits use ent / win as keys, the weighted sums    */
/* use ent_v / win_v (same shapes) as values.  NULL values: K = V.            */
void orc_attend_row_kv(const double* q, const double* ent, const double* ent_v, int64_t n_ent,
                       const double* win, const double* win_v, int64_t n_win, const float* sink,
                       double tau, int Hq, int D, double* o, double* lse);

void orc_attend_row(const double* q, const double* ent, int64_t n_ent, const double* win,
                    int64_t n_win, const float* sink, double tau, int Hq, int D,
                    double* o, double* lse) {
  orc_attend_row_kv(q, ent, NULL, n_ent, win, NULL, n_win, sink, tau, Hq, D, o, lse);
}

void orc_attend_row_kv(const double* q, const double* ent, const double* ent_v, int64_t n_ent,
                       const double* win, const double* win_v, int64_t n_win, const float* sink,
                       double tau, int Hq, int D, double* o, double* lse) {
  if (!ent_v) ent_v = ent;
  if (!win_v) win_v = win;
  int64_t n = n_ent + n_win;
  int h;
  /* heads are independent: they run in parallel, each with its own buffers */
#pragma omp parallel for schedule(static)
  for (h = 0; h < Hq; ++h) {
    double* l = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    const double* qh = q + (int64_t)h * D;
    double M = (double)sink[h], Z;
    int64_t t;
    int dd;
    for (t = 0; t < n; ++t) {
      const double* v = t < n_ent ? ent + t * D : win + (t - n_ent) * D;
      double dot = 0.0;
      for (dd = 0; dd < D; ++dd) { double pr = qh[dd] * v[dd]; dot = dot + pr; }
      l[t] = tau * dot;
      if (l[t] > M) M = l[t];
    }
    Z = exp((double)sink[h] - M);
    for (t = 0; t < n; ++t) { p[t] = exp(l[t] - M); Z = Z + p[t]; }
    for (dd = 0; dd < D; ++dd) {
      double acc = 0.0;
      for (t = 0; t < n; ++t) {
        const double* v = t < n_ent ? ent_v + t * D : win_v + (t - n_ent) * D;
        double pr = p[t] * v[dd];
        acc = acc + pr;
      }
      o[(int64_t)h * D + dd] = acc / Z;
    }
    if (lse) lse[h] = M + log(Z);
    free(l);
    free(p);
  }
}

/* Batched attention for the two attention calls.  Row r = b*Tq + t.
 *   q      : decoded float64 [B*Tq][Hq][D]
 *   kv     : storage [B][N_cap][D] of kv_dt (+ scales)
 *   sel    : int32 [B*Tq][k] (sparse: entries in the order given, -1 skipped),
 *            or NULL for dense: entries 0..n_elig[r]-1 (HCA)
 *   win    : storage [B][W_buf][D] of win_dt; row r uses tokens
 *            win_begin[r] .. win_begin[r]+win_len[r]-1 of sequence b
 *   o, lse : float64 [B*Tq][Hq][D], [B*Tq][Hq]                               */
static void orc_decode_row(const void* src, int dt, const float* scale, int64_t row, int D, double* dst) {
  if (dt == ORC_F32) orc_decode((const float*)src + row * D, dt, NULL, D, dst);
  else if (dt == ORC_BF16) orc_decode((const uint16_t*)src + row * D, dt, NULL, D, dst);
  else orc_decode((const uint8_t*)src + row * D, dt, scale + row * (D / 64), D, dst);
}

/* v / v_scale / win_v: separate values in the layouts of kv / kv_scale / win
 * (NULL: one vector per item is key and value). */
void orc_attend(const double* q, const void* kv, int kv_dt, const float* kv_scale,
                int64_t N_cap, const int32_t* sel, int k, const int32_t* n_elig,
                const void* win, int win_dt, int64_t W_buf, const int32_t* win_begin,
                const int32_t* win_len, const float* sink, double tau, int B, int Tq,
                int Hq, int D, double* o, double* lse, const void* v, const float* v_scale,
                const void* win_v) {
  int64_t r, R = (int64_t)B * Tq;
  /* rows one after another (the heads of a row run in parallel) */
  for (r = 0; r < R; ++r) {
    int b = (int)(r / Tq);
    int64_t ne = 0, nw = win_len[r], t;
    int64_t cap = sel ? k : n_elig[r];
    double* ent = (double*)malloc(sizeof(double) * (size_t)((cap > 0 ? cap : 1) * D));
    double* wv = (double*)malloc(sizeof(double) * (size_t)((nw > 0 ? nw : 1) * D));
    double* ent_v = v ? (double*)malloc(sizeof(double) * (size_t)((cap > 0 ? cap : 1) * D)) : NULL;
    double* wv_v = win_v ? (double*)malloc(sizeof(double) * (size_t)((nw > 0 ? nw : 1) * D)) : NULL;
    for (t = 0; t < cap; ++t) {
      int64_t j = sel ? sel[r * k + t] : t;
      int64_t row;
      if (j < 0) continue;
      row = (int64_t)b * N_cap + j;
      orc_decode_row(kv, kv_dt, kv_scale, row, D, ent + ne * D);
      if (v) orc_decode_row(v, kv_dt, v_scale, row, D, ent_v + ne * D);
      ne++;
    }
    for (t = 0; t < nw; ++t) {
      int64_t row = (int64_t)b * W_buf + win_begin[r] + t;
      orc_decode_row(win, win_dt, NULL, row, D, wv + t * D);
      if (win_v) orc_decode_row(win_v, win_dt, NULL, row, D, wv_v + t * D);
    }
    orc_attend_row_kv(q + r * Hq * D, ent, ent_v, ne, wv, wv_v, nw, sink, tau, Hq, D, o + r * Hq * D,
                      lse ? lse + r * Hq : NULL);
    free(ent);
    free(wv);
    free(ent_v);
    free(wv_v);
  }
}

/* Threads the parallel loops above use (a timing control: results do not
 * depend on it). */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
