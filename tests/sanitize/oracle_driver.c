/* oracle_driver.c -- runs every function of the CPU oracle on small inputs
 * (edge cases included) so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer checks the oracle's memory accesses and
 * arithmetic.  Test infrastructure: built and run by tests/test_sanitize.py.
 * Exit status 0 when every call returns and the few closed-form checks hold;
 * a sanitizer finding aborts the program. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

enum { F32 = 0, BF16 = 1, FP8 = 2, MXFP4 = 3 };

double orc_e4m3_value(int code);
double orc_e2m1_value(int code);
int orc_e4m3_encode(float y);
int orc_e2m1_encode(double y);
void orc_fp8_encode(const float* v, int64_t n, uint8_t* codes, float* scales);
void orc_fp8_decode(const uint8_t* codes, const float* scales, int64_t n, double* out);
void orc_mxfp4_encode(const float* v, int64_t n, uint8_t* codes, uint8_t* scales);
void orc_mxfp4_decode(const uint8_t* codes, const uint8_t* scales, int64_t n, double* out);
double orc_bf16_value(uint16_t h);
uint16_t orc_bf16_encode(float f);
void orc_decode(const void* src, int dt, const void* scale, int64_t n, double* out);
void orc_encode(const float* v, int64_t n, int dt, void* dst, void* scale);
void orc_pool(const double* x, const double* gate, const double* bias, int64_t nblk, int m, int D, double* out);
void orc_pool_variant(const double* x, const double* gate, int gate_pc, const double* bias, int64_t nblk, int m,
                      int o, int D, double* out);
double orc_index_score(const double* q, const double* w, const double* kj, int H, int d);
void orc_select_topk(const double* s, int64_t n_elig, int k, int32_t* idx, double* sel_score);
void orc_index_topk(const double* qi, const float* w, const void* keys, int key_dt, const void* key_scale,
                    const int32_t* n_elig, int B, int Tq, int H, int d, int64_t N_cap, int k, int32_t* idx_out,
                    double* sel_score, double* scores_out);
void orc_attend(const double* q, const void* kv, int kv_dt, const float* kv_scale, int64_t N_cap,
                const int32_t* sel, int k, const int32_t* n_elig, const void* win, int win_dt, int64_t W_buf,
                const int32_t* win_begin, const int32_t* win_len, const float* sink, double tau, int B, int Tq,
                int Hq, int D, double* o, double* lse, const void* v, const float* v_scale, const void* win_v);
void orc_set_threads(int n);

static uint64_t rng = 88172645463325252ull;
static double urand(void) {            /* xorshift64, uniform in [0, 1) */
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (double)(rng >> 11) * (1.0 / 9007199254740992.0);
}
static float nrand(void) { return (float)(sqrt(-2.0 * log(urand() + 1e-300)) * cos(6.283185307179586 * urand())); }

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void) {
  int i, j;
  orc_set_threads(2);
  /* codec tables and round trips */
  for (i = 0; i < 256; ++i) {
    const double v = orc_e4m3_value(i);
    if (!isnan(v)) CHECK(orc_e4m3_value(orc_e4m3_encode((float)v)) == v);
  }
  for (i = 0; i < 16; ++i) CHECK(orc_e2m1_value(orc_e2m1_encode(orc_e2m1_value(i))) == orc_e2m1_value(i));
  for (i = 0; i < 65536; i += 7) {
    const double v = orc_bf16_value((uint16_t)i);
    if (!isnan(v)) CHECK(orc_bf16_value(orc_bf16_encode((float)v)) == v);
  }
  {
    enum { N = 4 * 128 };
    float v[N];
    uint8_t c8[N], c4[N / 2], s4[N / 32];
    float s8[N / 64];
    double d[N];
    uint16_t b16[N];
    for (i = 0; i < N; ++i) v[i] = nrand() * (i < 128 ? 1e-30f : i < 256 ? 1e30f : 3.0f);
    v[300] = 0.0f; v[301] = -0.0f;
    for (i = 384; i < 448; ++i) v[i] = 0.0f;                 /* an all-zero group */
    v[448] = 1e-45f;                                        /* a subnormal amax */
    orc_fp8_encode(v, N, c8, s8); orc_fp8_decode(c8, s8, N, d);
    orc_mxfp4_encode(v, N, c4, s4); orc_mxfp4_decode(c4, s4, N, d);
    orc_encode(v, N, BF16, b16, NULL); orc_decode(b16, BF16, NULL, N, d);
    orc_encode(v, N, F32, d, NULL);
    orc_encode(v, N, FP8, c8, s8); orc_decode(c8, FP8, s8, N, d);
    orc_encode(v, N, MXFP4, c4, s4); orc_decode(c4, MXFP4, s4, N, d);
  }
  /* pooling: plain, per-channel gates, overlapping blocks (first block short) */
  {
    enum { T = 40, D = 8, M = 4, O = 2 };
    double x[T * D], g[T * D], bias[(M + O) * D], out[(T / M) * D];
    for (i = 0; i < T * D; ++i) { x[i] = nrand(); g[i] = nrand(); }
    for (i = 0; i < (M + O) * D; ++i) bias[i] = 0.1 * nrand();
    orc_pool(x, g, bias, T / M, M, D, out);
    orc_pool_variant(x, g, 0, bias, T / M, M, 0, D, out);
    orc_pool_variant(x, g, 1, bias, T / M, M, O, D, out);
    orc_pool_variant(x, g, 0, bias, T / M, M, O, D, out);
    orc_pool(x, g, bias, 1, 1, D, out);                     /* m = 1 */
  }
  /* indexer + top-k: ties, k >= n, n = 0, fp32 and MXFP4 keys */
  {
    enum { B = 2, Tq = 2, H = 4, d = 64, N = 300, K = 32 };
    double q[B * Tq * H * d];
    float w[B * Tq * H], keys[B * N * d];
    uint8_t kc[B * N * d / 2], ks[B * N * d / 32];
    int32_t n[B * Tq] = {N, 0, 17, N - 1}, idx[B * Tq * K];
    double sel[B * Tq * K], all[B * Tq * N], s[N];
    for (i = 0; i < B * Tq * H * d; ++i) q[i] = nrand();
    for (i = 0; i < B * Tq * H; ++i) w[i] = (float)urand();
    for (i = 0; i < B * N * d; ++i) keys[i] = nrand();
    memcpy(keys + 5 * d, keys + 9 * d, sizeof(float) * d);  /* equal keys: a tie */
    orc_index_topk(q, w, keys, F32, NULL, n, B, Tq, H, d, N, K, idx, sel, all);
    orc_mxfp4_encode(keys, B * N * d, kc, ks);
    orc_index_topk(q, w, kc, MXFP4, ks, n, B, Tq, H, d, N, K, idx, sel, NULL);
    for (j = 0; j < N; ++j) s[j] = (double)(j % 7);
    orc_select_topk(s, N, K, idx, sel);
    orc_select_topk(s, 10, K, idx, sel);                    /* k > n: -1 padding */
    CHECK(idx[10] == -1 && sel[10] == 0.0);
    orc_select_topk(s, 0, K, idx, NULL);
    CHECK(orc_index_score(q, w, q, 1, d) >= 0.0);
  }
  /* attention: sparse with padding, dense, empty and full windows, FP8 and
   * bf16 storage, separate values */
  {
    enum { B = 2, Tq = 2, Hq = 4, D = 128, N = 96, K = 16, W = 20 };
    double q[B * Tq * Hq * D], o[B * Tq * Hq * D], lse[B * Tq * Hq];
    float kvf[B * N * D], winf[B * W * D], sink[Hq], sc8[B * N * D / 64], vs8[B * N * D / 64];
    uint8_t kv8[B * N * D], v8[B * N * D];
    uint16_t win16[B * W * D], winv16[B * W * D];
    int32_t sel[B * Tq * K], n[B * Tq] = {N, 0, 50, 1}, wb[B * Tq] = {0, 5, 0, 19}, wl[B * Tq] = {W, 0, 15, 1};
    for (i = 0; i < B * Tq * Hq * D; ++i) q[i] = nrand();
    for (i = 0; i < B * N * D; ++i) kvf[i] = nrand();
    for (i = 0; i < B * W * D; ++i) winf[i] = nrand();
    for (i = 0; i < Hq; ++i) sink[i] = nrand();
    for (i = 0; i < B * Tq * K; ++i) sel[i] = (i % 5 == 0) ? -1 : (int32_t)(urand() * N);
    orc_fp8_encode(kvf, B * N * D, kv8, sc8);
    for (i = 0; i < B * N * D; ++i) kvf[i] = -kvf[i];
    orc_fp8_encode(kvf, B * N * D, v8, vs8);
    orc_encode(winf, B * W * D, BF16, win16, NULL);
    for (i = 0; i < B * W * D; ++i) winf[i] = 2.0f * winf[i];
    orc_encode(winf, B * W * D, BF16, winv16, NULL);
    orc_attend(q, kv8, FP8, sc8, N, sel, K, NULL, win16, BF16, W, wb, wl, sink, 0.088, B, Tq, Hq, D, o, lse,
               NULL, NULL, NULL);
    orc_attend(q, kv8, FP8, sc8, N, NULL, 0, n, win16, BF16, W, wb, wl, sink, 0.088, B, Tq, Hq, D, o, lse,
               NULL, NULL, NULL);
    orc_attend(q, kv8, FP8, sc8, N, sel, K, NULL, win16, BF16, W, wb, wl, sink, 0.088, B, Tq, Hq, D, o, NULL,
               v8, vs8, winv16);
    orc_attend(q, kvf, F32, NULL, N, NULL, 0, n, winf, F32, W, wb, wl, sink, 1.0, B, Tq, Hq, D, o, lse,
               NULL, NULL, NULL);
    /* row 1: no entry and an empty window -> sink only: o = 0, lse = sink */
    for (i = 0; i < Hq; ++i) CHECK(fabs(lse[1 * Hq + i] - (double)sink[i]) < 1e-12);
  }
  printf("oracle driver: ok\n");
  return 0;
}
