// index_common.h -- pieces shared by the decode and prefill indexer kernels:
// MXFP4 query/key operand loads, the exact MFMA scoring round, the float64
// head combine, and the block-wide exact radix selection with its streamed
// re-scoring source (the exact path every indexer row can fall back to).
#pragma once
#include "lca_device.h"

namespace lca {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int CAP = 128;           // candidate slots per chunk
constexpr int NDIRECT = 8192;      // rows with n_elig <= NDIRECT skip the chunk kernel
constexpr int SEL_THREADS = 1024;  // select kernel workgroup (16 wavefronts)
constexpr int SEL_WAVES = SEL_THREADS / WAVE;
constexpr int CMAX = 8192;         // candidates per row held in LDS by the select kernel
constexpr int LB = CMAX / SEL_THREADS;   // candidate loads per thread (one batch)
constexpr int MAXCH = 1024;        // chunks per row the candidate path handles
constexpr int KROW = 20;           // LDS floats per key in the transpose buffer (16 + pad)
constexpr int BITMAP_BITS = 1 << 18;


// Row r's eligible count, clamped where a kernel reads it to [0, N_cap], so
// that no value of the device-resident counts reads past the key cache.
__device__ __forceinline__ int idx_nelig(const IndexArgs& A, int64_t r) {
  return min(max(A.n_elig[r], 0), (int)A.N_cap);      // N_cap < 2^31
}

// ------------------------------------------------------------------------
// Query state of one wavefront (up to two query rows of one sequence).
// ------------------------------------------------------------------------
struct Rows {
  int b;            // sequence
  int r[2];         // query rows (r[1] < 0: absent)
  int n[2];         // n_elig per row (0 for absent rows)
};

struct MxQuery {
  int a[4];         // this lane's 16 bytes of the A operand
  int sa;           // this lane's E8M0 byte
  int dq, qmin, qmax;
};

// The query operand is loaded in two steps: mx_query_issue requests this
// lane's bytes (unconditionally, from row 0 where the lane has no query block,
// so the request count is fixed), mx_query_finish masks them and derives the
// exponent spread.
struct MxQueryRaw {
  int4 v;
  int sa;
  bool valid;
};
template <int HP>
__device__ __forceinline__ MxQueryRaw mx_query_issue(const IndexArgs& A, const Rows& rw) {
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, kb = lane >> 4;
  const int q = row / HP, h = row % HP;
  const int rq = q == 0 ? rw.r[0] : rw.r[1];     // (no dynamic indexing: keeps rw in registers)
  MxQueryRaw R;
  R.valid = (q < 2) && rq >= 0 && h < A.H && kb * 32 < A.d;
  const int64_t qrow = R.valid ? (int64_t)rq * A.H + h : 0;
  const int kbc = R.valid ? kb : 0;
  R.v = *(const int4*)((const uint8_t*)A.qi + qrow * (A.d / 2) + kbc * 16);
  R.sa = A.qi_scale[qrow * (A.d / 32) + kbc];
  return R;
}

__device__ __forceinline__ void mx_query_finish(const MxQueryRaw& R, MxQuery& Q) {
  const bool valid = R.valid;
  Q.a[0] = valid ? R.v.x : 0; Q.a[1] = valid ? R.v.y : 0; Q.a[2] = valid ? R.v.z : 0; Q.a[3] = valid ? R.v.w : 0;
  Q.sa = valid ? R.sa : 127;
  int smin = valid ? Q.sa : 1000, smax = valid ? Q.sa : -1000;
  // per (query, head): spread of the block exponents over the 4 lanes of a row
  int rmin = smin, rmax = smax;
  rmin = min(rmin, __shfl_xor(rmin, 16, WAVE)); rmax = max(rmax, __shfl_xor(rmax, 16, WAVE));
  rmin = min(rmin, __shfl_xor(rmin, 32, WAVE)); rmax = max(rmax, __shfl_xor(rmax, 32, WAVE));
  int dq = valid ? rmax - rmin : 0;
  int gmin = smin, gmax = smax;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    dq = max(dq, __shfl_xor(dq, o, WAVE));
    gmin = min(gmin, __shfl_xor(gmin, o, WAVE));
    gmax = max(gmax, __shfl_xor(gmax, o, WAVE));
  }
  Q.dq = dq; Q.qmin = gmin; Q.qmax = gmax;
}

template <int HP>
__device__ __forceinline__ void mx_load_query(const IndexArgs& A, const Rows& rw, MxQuery& Q) {
  mx_query_finish(mx_query_issue<HP>(A, rw), Q);
}

struct MxTiles {
  int4 code[4];
  int sc[4];
  uint32_t kscale;  // the scale bytes of key j0 + lane (for the exactness envelope)
};

// Head weights of a wavefront's NQ rows in registers, as float64, zero for
// heads >= H (wl: LDS weights [2][16], zero-filled beyond H).
template <int HP, int NQ>
struct MxW {
  double w[NQ][HP];
};
template <int HP, int NQ>
__device__ __forceinline__ void mx_load_weights(const float* wl, MxW<HP, NQ>& W) {
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int h = 0; h < HP; ++h) W.w[q][h] = (double)wl[q * 16 + h];
}

// The scale bytes of a key row as one word (d_I in {64, 128}: 2 or 4 bytes).
__device__ __forceinline__ uint32_t mx_scale_word(const uint8_t* ks, int d) {
  return d == 128 ? *(const uint32_t*)ks : (uint32_t)*(const uint16_t*)ks;
}

// A value that is uniform over the wavefront, moved to scalar registers.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Uniform addresses of a wavefront's key rows: row `base` of sequence b (b and
// base uniform over the wavefront) and the byte strides of the code and scale
// rows.  Rows up to 2^18 past `base` are addressed with 24-bit offset
// products.
struct MxRows {
  const uint8_t* code;
  const uint8_t* scale;
  int base;
  uint32_t cb, sb;
};
__device__ __forceinline__ MxRows mx_rows(const IndexArgs& A, int b, int base) {
  MxRows R;
  const int64_t row = (int64_t)b * A.N_cap + base;
  R.code = (const uint8_t*)A.ki + uniform_i64(row * (A.d / 2));
  R.scale = A.ki_scale + uniform_i64(row * (A.d / 32));
  R.base = base;
  R.cb = (uint32_t)A.d / 2;
  R.sb = (uint32_t)A.d / 32;
  return R;
}

// Load the B operands of 4 MFMA tiles = 64 keys [j0, j0+64), rows relative to
// R (R.base <= min(j0, jlim-1), j0 - R.base < 2^18).  The loads are
// unconditional (rows clamped into [0, jlim)) so that they all stay in flight;
// a lane past jlim scores a copy of the last row, which the caller's
// eligibility test discards.  K blocks past d_I load block 0 (the query
// operand is zero there, so they add nothing).
__device__ __forceinline__ void mx_load_round(const IndexArgs& A, const MxRows& R, int j0, int jlim, MxTiles& T) {
  const int lane = threadIdx.x & 63;
  const int kb = lane >> 4;
  const uint32_t kbc = kb * 32 < A.d ? kb : 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t jo = (uint32_t)(min(j0 + t * 16 + (lane & 15), jlim - 1) - R.base);
    const v4i v = __builtin_nontemporal_load((const v4i*)(R.code + (__umul24(jo, R.cb) + kbc * 16u)));
    T.code[t] = make_int4(v[0], v[1], v[2], v[3]);
    T.sc[t] = R.scale[__umul24(jo, R.sb) + kbc];
  }
  const uint32_t jo = (uint32_t)(min(j0 + lane, jlim - 1) - R.base);
  T.kscale = mx_scale_word(R.scale + __umul24(jo, R.sb), A.d);
}

// The same for a round anywhere in the sequence.
__device__ __forceinline__ void mx_load_round(const IndexArgs& A, int b, int j0, int jlim, MxTiles& T) {
  mx_load_round(A, mx_rows(A, b, min(j0, jlim - 1)), j0, jlim, T);
}

// Load the B operands of 4 MFMA tiles for an arbitrary list of entries: lane
// e < cnt names entry jmine; tile t covers the entries of lanes t*16..t*16+15.
// Loads stay unconditional (absent entries read row 0; the caller's
// eligibility test discards them).
__device__ __forceinline__ void mx_load_gather(const IndexArgs& A, int b, int jmine, int cnt, MxTiles& T) {
  const int lane = threadIdx.x & 63;
  const int kb = lane >> 4;
  const uint32_t kbc = kb * 32 < A.d ? kb : 0;
  const int64_t row0 = (int64_t)b * A.N_cap;
  const uint8_t* cbase = (const uint8_t*)A.ki + row0 * (A.d / 2);
  const uint8_t* sbase = A.ki_scale + row0 * (A.d / 32);
  const uint64_t cb = (uint32_t)A.d / 2, sb = (uint32_t)A.d / 32;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int src = t * 16 + (lane & 15);
    const int js = __shfl(jmine, src, WAVE);
    const uint64_t jo = (uint32_t)(src < cnt ? js : 0);
    const v4i v = *(const v4i*)(cbase + jo * cb + kbc * 16u);
    T.code[t] = make_int4(v[0], v[1], v[2], v[3]);
    T.sc[t] = sbase[jo * sb + kbc];
  }
  const uint64_t jo = (uint32_t)(lane < cnt ? jmine : 0);
  T.kscale = mx_scale_word(sbase + jo * sb, A.d);
}

__device__ __forceinline__ double mx_value(const uint8_t* codes, const uint8_t* scales, int i) {
  const uint32_t byte = codes[i >> 1];
  const uint32_t c = (i & 1) ? (byte >> 4) : (byte & 15u);
  return ldexp((double)e2m1_to_f32(c), (int)scales[i >> 5] - 127);
}

// Exact float64 dot product of query head (row qr, head h) and key row krow,
// left to right over the elements.
__device__ __forceinline__ double mx_dot_exact(const IndexArgs& A, int64_t qrow, const uint8_t* kc,
                                               const uint8_t* ks) {
  const uint8_t* qc = (const uint8_t*)A.qi + qrow * (A.d / 2);
  const uint8_t* qs = A.qi_scale + qrow * (A.d / 32);
  double dot = 0.0;
  for (int i = 0; i < A.d; ++i) dot = fma(mx_value(qc, qs, i), mx_value(kc, ks, i), dot);
  return dot;
}

__device__ __forceinline__ double mx_dot_exact(const IndexArgs& A, int64_t qrow, int64_t krow) {
  return mx_dot_exact(A, qrow, (const uint8_t*)A.ki + krow * (A.d / 2), A.ki_scale + krow * (A.d / 32));
}

// One step of the float64 head combine s = sum_h w_h * max(0, dot_h), taken in
// head order: multiply, then add (no contraction).
__device__ __forceinline__ double combine_step(double s, double dot, float w) {
#pragma clang fp contract(off)
  const double r = dot > 0.0 ? dot : 0.0;
  const double t = (double)w * r;
  return s + t;
}

// Score one round of 64 keys for the wave's NQ rows.  Lane L ends with the
// keys of entry j0+L (0 when not eligible).
// wbuf: this wave's LDS transpose buffer (64*KROW floats); wl: LDS weights
// [2][16].
__device__ __forceinline__ bool mx_exact(const MxQuery& Q, int kmin, int kmax) {
  return (Q.dq + kmax - kmin <= 9) && (Q.qmin + kmin >= 130) && (Q.qmax + kmax <= 368);
}

// Score one round of 64 keys for the wave's NQ rows.  Lane L ends with the
// key of entry j0+L (0 when not eligible).  The float64 head combine is taken
// in head order; each step is one fma, which equals multiply-then-add here
// because the product of two floats is exact in float64.  Heads >= H carry a
// zero weight and a zero dot and leave the sum unchanged (it is never -0).
// wbuf: this wave's LDS transpose buffer (64*KROW floats).
template <int HP, int NQ>
__device__ __forceinline__ void mx_score_round(const IndexArgs& A, const Rows& rw, const MxQuery& Q,
                                               const MxTiles& T, int j0, float* wbuf, const MxW<HP, NQ>& W,
                                               uint64_t* key, bool& inexact) {
  const int lane = threadIdx.x & 63;
  const v8i av = {Q.a[0], Q.a[1], Q.a[2], Q.a[3], 0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const v8i bv = {T.code[t].x, T.code[t].y, T.code[t].z, T.code[t].w, 0, 0, 0, 0};
    v4f c = {0.f, 0.f, 0.f, 0.f};
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, Q.sa, 0, T.sc[t]);
    float* dst = wbuf + (t * 16 + (lane & 15)) * KROW + 4 * (lane >> 4);
    *(float4*)dst = make_float4(c[0], c[1], c[2], c[3]);
  }
  // exponent envelope of this lane's key j0+lane from its own scale bytes
  uint32_t sw = T.kscale;
  if (A.d != 128) sw = (sw & 0xFFFFu) | ((sw & 0xFFu) * 0x01010000u);   // d_I = 64: repeat block 0
  int kmin = (int)(sw & 0xFFu), kmax = kmin;
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    const int v = (int)((sw >> (8 * i)) & 0xFFu);
    kmin = min(kmin, v);
    kmax = max(kmax, v);
  }
  const bool exact = mx_exact(Q, kmin, kmax);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int j = j0 + lane;
  const float4* mine = (const float4*)(wbuf + lane * KROW);
  float dv[NQ * HP];
#pragma unroll
  for (int i = 0; i < NQ * HP / 4; ++i) {
    const float4 v = mine[i];
    dv[4 * i] = v.x; dv[4 * i + 1] = v.y; dv[4 * i + 2] = v.z; dv[4 * i + 3] = v.w;
  }
  inexact = false;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    double sc = 0.0;
#pragma unroll
    for (int h = 0; h < HP; ++h) {
      const float r = __int_as_float(max(__float_as_int(dv[q * HP + h]), 0));   // ReLU (-0 -> +0)
      sc = fma(W.w[q][h], (double)r, sc);
    }
    const bool elig = rw.r[q] >= 0 && j < rw.n[q];
    key[q] = elig ? score_key(sc) : 0ull;
    inexact |= elig && !exact;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Exact float64 score of entry j for row q of the wave (keys outside the
// exact-MFMA envelope).
__device__ __forceinline__ uint64_t mx_score_exact(const IndexArgs& A, int qrow, int b, int j, const float* wlq) {
  double sc = 0.0;
  for (int h = 0; h < A.H; ++h)
    sc = combine_step(sc, mx_dot_exact(A, (int64_t)qrow * A.H + h, (int64_t)b * A.N_cap + j), wlq[h]);
  return score_key(sc);
}

// The same for a key row given by its codes and scale bytes.
__device__ __forceinline__ uint64_t mx_score_exact_row(const IndexArgs& A, int qrow, const uint8_t* kc,
                                                       const uint8_t* ks, const float* wlq) {
  double sc = 0.0;
  for (int h = 0; h < A.H; ++h) sc = combine_step(sc, mx_dot_exact(A, (int64_t)qrow * A.H + h, kc, ks), wlq[h]);
  return score_key(sc);
}

// F32 indexer: lane L scores entry j0+L for row 0 (F32 groups hold one row).
// qrow: the query row [H][d] (LDS or global; every lane reads the same
// addresses).
__device__ __forceinline__ void f32_score_round(const IndexArgs& A, const Rows& rw, int j0, const float* qrow,
                                                const float* wl, uint64_t& key0) {
  const int lane = threadIdx.x & 63;
  const int j = j0 + lane;
  key0 = 0;
  if (j >= rw.n[0]) return;
  const float* kr = (const float*)A.ki + ((int64_t)rw.b * A.N_cap + j) * A.d;
  double s = 0.0;
  for (int h = 0; h < A.H; ++h) {
    double dot = 0.0;
    for (int i = 0; i < A.d; ++i) dot = fma((double)qrow[h * A.d + i], (double)kr[i], dot);
    s = combine_step(s, dot, wl[h]);
  }
  key0 = score_key(s);
}

// The same evaluation with the lane's key row read 32 elements at a time by
// vector loads, all in flight (each head's dot product is still one float64
// chain over the elements in order): for callers that do not unroll it.
__device__ __forceinline__ void f32_score_round_vec(const IndexArgs& A, const Rows& rw, int j0, const float* qrow,
                                                    const float* wl, uint64_t& key0) {
  const int lane = threadIdx.x & 63;
  const int j = j0 + lane;
  const bool ok = j < rw.n[0];
  const float4* kr = (const float4*)((const float*)A.ki + ((int64_t)rw.b * A.N_cap + (ok ? j : 0)) * A.d);
  double s = 0.0;
  {
    // steps of (head, 32 elements of the row) in order; the next step's
    // elements load while these are multiplied
    const int nc = A.d / 32;
    const int nst = A.H * nc;
    float4 cur[8], nxt[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) cur[t] = kr[t];
    double dot = 0.0;
#pragma unroll 1
    for (int st = 0; st < nst; ++st) {
      const int h = st / nc, ci = st - h * nc;
      const bool more = st + 1 < nst;
      const int cn = ci + 1 == nc ? 0 : ci + 1;
      if (more) {
#pragma unroll
        for (int t = 0; t < 8; ++t) nxt[t] = kr[cn * 8 + t];
      }
      const float* q = qrow + h * A.d + ci * 32;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        dot = fma((double)q[4 * t], (double)cur[t].x, dot);
        dot = fma((double)q[4 * t + 1], (double)cur[t].y, dot);
        dot = fma((double)q[4 * t + 2], (double)cur[t].z, dot);
        dot = fma((double)q[4 * t + 3], (double)cur[t].w, dot);
      }
      if (ci + 1 == nc) {
        s = combine_step(s, dot, wl[h]);
        dot = 0.0;
      }
      if (more) {
#pragma unroll
        for (int t = 0; t < 8; ++t) cur[t] = nxt[t];
      }
    }
  }
  key0 = ok ? score_key(s) : 0ull;
}

// The same evaluation for the 64 entries j0 .. j0+63 of one wavefront with
// the key rows staged through a wavefront-private LDS tile, 16 elements of
// every row at a time: four lanes load a row's 64 contiguous bytes, so each
// load instruction reads 16 whole segments instead of 64 scattered ones (the
// per-lane row loads above are bound by the address unit when one workgroup
// scores a whole row).  The tile rows are padded to F32_TS floats, so the
// per-lane reads that follow hit 64 distinct banks.  Heads are taken four at
// a time (the rows are staged again for each group); each head keeps its own
// float64 chain over the elements in order, and the heads are combined in
// head order once their chains are complete: the same operations in the same
// order as f32_score_round.  Needs d % 16 == 0.
constexpr int F32_TS = 17;                 // tile row stride (floats)
constexpr int F32_TILE = 64 * F32_TS;      // tile floats per wavefront
__device__ __forceinline__ void f32_score_wave_lds(const IndexArgs& A, int b, int n, int j0, const float* qrow,
                                                   const float* wl, float* tile, uint64_t& key0) {
  const int lane = threadIdx.x & 63;
  const int d = A.d, H = A.H;
  const float* kb = (const float*)A.ki + (int64_t)b * A.N_cap * d;
  const int lr = lane >> 2, lf = lane & 3;   // load: row 16*t + lr, float4 lf of the 16 elements
  const int nc = d / 16;
  auto load = [&](int c, float4 (&v)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = min(j0 + 16 * t + lr, n - 1);       // rows past n: a valid row, never used
      v[t] = *(const float4*)(kb + (int64_t)row * d + c * 16 + lf * 4);
    }
  };
  double s = 0.0;
#pragma unroll 1
  for (int h0 = 0; h0 < H; h0 += 4) {
    double dot[4] = {0.0, 0.0, 0.0, 0.0};
    float4 cur[4], nxt[4];
    load(0, cur);
#pragma unroll 1
    for (int c = 0; c < nc; ++c) {
      if (c + 1 < nc) load(c + 1, nxt);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float* p = tile + (16 * t + lr) * F32_TS + 4 * lf;
        p[0] = cur[t].x; p[1] = cur[t].y; p[2] = cur[t].z; p[3] = cur[t].w;
      }
      // the LDS operations of one wavefront complete in issue order
      __builtin_amdgcn_wave_barrier();
      float kv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) kv[e] = tile[lane * F32_TS + e];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        if (h0 + hh < H) {
          const float* q = qrow + (h0 + hh) * d + c * 16;
#pragma unroll
          for (int e = 0; e < 16; ++e) dot[hh] = fma((double)q[e], (double)kv[e], dot[hh]);
        }
      }
      if (c + 1 < nc) {
#pragma unroll
        for (int t = 0; t < 4; ++t) cur[t] = nxt[t];
      }
    }
#pragma unroll
    for (int hh = 0; hh < 4; ++hh)
      if (h0 + hh < H) s = combine_step(s, dot[hh], wl[h0 + hh]);
  }
  key0 = j0 + lane < n ? score_key(s) : 0ull;
}

// ------------------------------------------------------------------------
// Wavefront bitonic sort of one u64 per lane, descending across lanes.
// ------------------------------------------------------------------------
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t o = shfl_xor_u64(v, j);
      const bool up = ((lane & k) == 0);         // this k-block sorts descending
      const bool lower = ((lane & j) == 0);
      // descending block: lower lane keeps the max
      const bool keep_max = (up == lower);
      v = keep_max ? (o > v ? o : v) : (o < v ? o : v);
    }
  }
  return v;
}

// ------------------------------------------------------------------------
// Chunk kernel.  A workgroup of 4 wavefronts owns one chunk of CH = 64*KPL
// consecutive entries for NQ query rows; each wavefront scores KPL/4 rounds
// of 64 entries (all its key tiles loaded up front), keeps its keys in
// registers, and contributes its 64 lane maxima (sorted) to the chunk
// threshold: the r-th largest of the chunk's 256 lane maxima, found by
// merging the four sorted lists with bitonic half-cleaners.
// ------------------------------------------------------------------------
constexpr int WBUF = 64 * KROW;           // floats per wave: dot-product transpose buffer

// Descending bitonic clean of a bitonic sequence held one value per lane.
__device__ __forceinline__ uint64_t wave_bitonic_clean_desc(uint64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) {
    const uint64_t o = shfl_xor_u64(v, j);
    const bool lower = (lane & j) == 0;
    v = lower ? (o > v ? o : v) : (o < v ? o : v);
  }
  return v;
}

// ------------------------------------------------------------------------
// Select kernel helpers (block of SEL_THREADS threads)
// ------------------------------------------------------------------------
struct SelShared {
  uint32_t hist[2048];
  uint32_t scan[SEL_WAVES];
  uint64_t red64[2][SEL_WAVES];
  int32_t off[MAXCH + 1];
  __align__(16) uint32_t bitmap[BITMAP_BITS / 32];   // (also fp32 rows' keys: 8-byte aligned)
  uint64_t rkey[64];           // items of the threshold bin, resolved exactly
  int32_t rj[64];
  uint32_t rank[64];
  uint32_t woff[SEL_WAVES];        // exclusive prefix of per-wavefront counts
  uint32_t wflag[SEL_WAVES];       // per-wavefront flags of the candidate exchange
  uint32_t ecnt[LB * SEL_WAVES];   // emission: items above the threshold per (pass, wavefront)
  uint32_t epre[LB * SEL_WAVES];   // and their exclusive prefix
  uint32_t ecnt2[LB * SEL_WAVES];  // tied items per (pass, wavefront)
  uint32_t epre2[LB * SEL_WAVES];
  int nres;
  int bcast[8];
  uint64_t bcast64[4];
};

// Block-wide max and min of one u64 per thread (min over values != ~0).
__device__ __forceinline__ void block_minmax_u64(uint64_t& mx, uint64_t& mn, SelShared& S) {
  mx = wave_max_u64_dpp(mx);
  mn = wave_min_u64_dpp(mn);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { S.red64[0][wave] = mx; S.red64[1][wave] = mn; }
  __syncthreads();
  mx = 0; mn = ~0ull;
#pragma unroll
  for (int i = 0; i < SEL_WAVES; ++i) {
    mx = S.red64[0][i] > mx ? S.red64[0][i] : mx;
    mn = S.red64[1][i] < mn ? S.red64[1][i] : mn;
  }
}

// Exclusive block scan of one int per thread; returns the exclusive prefix,
// total in *tot.
__device__ __forceinline__ int block_scan(int v, int* tot, SelShared& S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan_dpp(v);
  __syncthreads();
  if (lane == 63) S.scan[wave] = (uint32_t)incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < SEL_WAVES; ++i) {
    const int s = (int)S.scan[i];
    if (i < wave) before += s;
    all += s;
  }
  *tot = all;
  return before + incl - v;
}

// One radix digit step: among keys with (key & mask) == prefix, find the digit
// (nb bits at `shift`) holding the rem-th largest.  `src` is a functor
// for_each(fn(key, j)).  Returns via S.bcast: [0] digit, [1] count above,
// [2] count in digit.
template <class Src>
__device__ __forceinline__ void radix_digit(Src& src, uint64_t prefix, uint64_t mask, int shift, int nb, int rem, SelShared& S) {
  constexpr int BPT = 2048 / SEL_THREADS;       // bins per thread
  const int nbins = 1 << nb;
  for (int i = threadIdx.x; i < 2048; i += SEL_THREADS) S.hist[i] = 0;
  __syncthreads();
  src.for_each([&](uint64_t key, int j) {
    if (key != 0 && (key & mask) == prefix) atomicAdd(&S.hist[(key >> shift) & (uint64_t)(nbins - 1)], 1u);
  });
  __syncthreads();
  // thread t owns bins top-BPT*t .. top-BPT*t-BPT+1 (counted from the top bin)
  const int top = nbins - 1 - BPT * (int)threadIdx.x;
  int cnt[BPT], mine = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) { cnt[i] = (top - i >= 0) ? (int)S.hist[top - i] : 0; mine += cnt[i]; }
  int tot;
  int above = block_scan(mine, &tot, S);        // count in bins above this thread's bins
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    if (top - i >= 0 && above < rem && above + cnt[i] >= rem) {
      S.bcast[0] = top - i; S.bcast[1] = above; S.bcast[2] = cnt[i];
    }
    above += cnt[i];
  }
  __syncthreads();
}

// Smallest-j selection among ties (key == T): find the rem-th smallest j.
template <class Src>
__device__ int tie_select_j(Src& src, uint64_t T, int rem, SelShared& S) {
  constexpr int BPT = 2048 / SEL_THREADS;
  uint32_t prefix = 0, mask = 0;
  int shift = 31;
  while (shift > 0) {
    const int nb = shift >= 11 ? 11 : shift;
    shift -= nb;
    const uint32_t nbins = 1u << nb;
    for (int i = threadIdx.x; i < 2048; i += SEL_THREADS) S.hist[i] = 0;
    __syncthreads();
    src.for_each([&](uint64_t key, int j) {
      if (key == T && ((uint32_t)j & mask) == prefix) atomicAdd(&S.hist[((uint32_t)j >> shift) & (nbins - 1)], 1u);
    });
    __syncthreads();
    const int b0 = BPT * (int)threadIdx.x;
    int cnt[BPT], mine = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) { cnt[i] = (b0 + i < (int)nbins) ? (int)S.hist[b0 + i] : 0; mine += cnt[i]; }
    int tot;
    int below = block_scan(mine, &tot, S);
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (b0 + i < (int)nbins && below < rem && below + cnt[i] >= rem) { S.bcast[0] = b0 + i; S.bcast[1] = below; }
      below += cnt[i];
    }
    __syncthreads();
    const int dsel = S.bcast[0];
    rem -= S.bcast[1];
    prefix |= (uint32_t)dsel << shift;
    mask |= (nbins - 1) << shift;
    __syncthreads();
  }
  return (int)prefix;
}

// Threshold of a selection: items with key > T, or key == T and j <= Tj when
// low == 0; with low > 0, items with (key >> low) >= (T >> low).
struct Thr {
  uint64_t T;
  int low;
  int Tj;          // INT_MAX when all ties are taken
};

__device__ __forceinline__ bool selected(const Thr& th, uint64_t key, int j) {
  if (key == 0) return false;
  if (th.low > 0) return (key >> th.low) >= (th.T >> th.low);
  return key > th.T || (key == th.T && j <= th.Tj);
}

// Exact rank resolution inside one radix bin of at most 64 items: the items
// (key & mask) == prefix are gathered in LDS and the rem-th of them in the
// order (key desc, j asc) is found by counting, per item, the items before it.
template <class Src>
__device__ __forceinline__ void resolve_bin(Src& src, uint64_t prefix, uint64_t mask, int rem, SelShared& S) {
  if (threadIdx.x == 0) S.nres = 0;
  if (threadIdx.x < 64) S.rank[threadIdx.x] = 0;
  __syncthreads();
  src.for_each([&](uint64_t key, int j) {
    if (key != 0 && (key & mask) == prefix) {
      const int p = atomicAdd(&S.nres, 1);
      if (p < 64) { S.rkey[p] = key; S.rj[p] = j; }
    }
  });
  __syncthreads();
  const int n = min(S.nres, 64);
  {
    // thread (g, i): items before item i among items m = g*MPG .. g*MPG+MPG-1
    constexpr int MPG = 64 / SEL_WAVES;
    const int i = threadIdx.x & 63, g = threadIdx.x >> 6;
    if (i < n) {
      const uint64_t ki = S.rkey[i];
      const int ji = S.rj[i];
      int cnt = 0;
#pragma unroll
      for (int t = 0; t < MPG; ++t) {
        const int m = g * MPG + t;
        if (m < n) {
          const uint64_t km = S.rkey[m];
          cnt += (km > ki) || (km == ki && S.rj[m] < ji);
        }
      }
      if (cnt) atomicAdd(&S.rank[i], (uint32_t)cnt);
    }
  }
  __syncthreads();
  if (threadIdx.x < n && (int)S.rank[threadIdx.x] == rem - 1) {
    S.bcast64[0] = S.rkey[threadIdx.x];
    S.bcast[3] = S.rj[threadIdx.x];
  }
  __syncthreads();
}

// Exact selection threshold for the kk largest (by key desc, j asc) items.
template <class Src>
__device__ Thr find_threshold(Src& src, int kk, SelShared& S) {
  Thr th;
  uint64_t mx = 0, mn = ~0ull;
  src.for_each([&](uint64_t key, int j) {
    if (key != 0) { mx = key > mx ? key : mx; mn = key < mn ? key : mn; }
  });
  block_minmax_u64(mx, mn, S);
  th.Tj = 0x7FFFFFFF;
  if (mx == 0) { th.T = ~0ull; th.low = 0; return th; }   // nothing eligible
  if (mx == mn) {
    th.T = mx; th.low = 0;
  } else {
    const int hb = 63 - __clzll(mx ^ mn);
    int shift = hb + 1;
    uint64_t mask = (shift >= 64) ? 0 : ~((1ull << shift) - 1ull);
    uint64_t prefix = mx & mask;
    int rem = kk;
    bool early = false;
    while (shift > 0) {
      const int nb = shift >= 11 ? 11 : shift;
      shift -= nb;
      radix_digit(src, prefix, mask, shift, nb, rem, S);
      const int dsel = S.bcast[0], above = S.bcast[1], indig = S.bcast[2];
      __syncthreads();
      rem -= above;
      prefix |= (uint64_t)dsel << shift;
      mask |= (uint64_t)((1u << nb) - 1u) << shift;
      if (indig == rem) { early = shift > 0; break; }
      if (indig <= 64 && shift > 0) {
        // few items left in the bin: rank them exactly (ties by index)
        resolve_bin(src, prefix, mask, rem, S);
        th.T = S.bcast64[0];
        th.Tj = S.bcast[3];
        th.low = 0;
        __syncthreads();
        return th;
      }
    }
    th.T = prefix;
    th.low = early ? shift : 0;
    if (!early) {
      // count of items equal to T
      int cnt = 0;
      src.for_each([&](uint64_t key, int j) { cnt += (key == prefix); });
      int tot;
      block_scan(cnt, &tot, S);
      __syncthreads();
      if (tot > rem) th.Tj = tie_select_j(src, prefix, rem, S);
    }
  }
  return th;
}

// Write the selected indices in ascending order (LDS bitmap over segments of
// the index range), padded with -1, and optionally their scores.
template <class Src>
__device__ void emit_sorted(Src& src, const Thr& th, int n, int k, int32_t* out, double* sout, SelShared& S) {
  constexpr int WPT = BITMAP_BITS / 32 / SEL_THREADS;   // bitmap words per thread
  int written = 0;
  for (int seg0 = 0; seg0 < n; seg0 += BITMAP_BITS) {
    for (int i = threadIdx.x; i < BITMAP_BITS / 32; i += SEL_THREADS) S.bitmap[i] = 0;
    __syncthreads();
    src.for_each([&](uint64_t key, int j) {
      if (j >= seg0 && j < seg0 + BITMAP_BITS && selected(th, key, j))
        atomicOr(&S.bitmap[(j - seg0) >> 5], 1u << ((j - seg0) & 31));
    });
    __syncthreads();
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < WPT; ++w) cnt += __popc(S.bitmap[threadIdx.x * WPT + w]);
    int tot;
    int pos = written + block_scan(cnt, &tot, S);
    S.off[threadIdx.x] = pos;
#pragma unroll
    for (int w = 0; w < WPT; ++w) {
      uint32_t bits = S.bitmap[threadIdx.x * WPT + w];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        if (pos < k) out[pos] = seg0 + (threadIdx.x * WPT + w) * 32 + bit;
        ++pos;
      }
    }
    __syncthreads();
    if (sout) {
      src.for_each([&](uint64_t key, int j) {
        if (j >= seg0 && j < seg0 + BITMAP_BITS && selected(th, key, j)) {
          const int word = (j - seg0) >> 5, owner = word / WPT;
          int p = S.off[owner];
          for (int w = owner * WPT; w < word; ++w) p += __popc(S.bitmap[w]);
          p += __popc(S.bitmap[word] & ((1u << ((j - seg0) & 31)) - 1u));
          if (p < k) sout[p] = key_score(key);
        }
      });
      __syncthreads();
    }
    written += tot;
  }
  for (int i = written + threadIdx.x; i < k; i += SEL_THREADS) {
    out[i] = -1;
    if (sout) sout[i] = 0.0;
  }
}

// Candidates held in registers: item u of this thread is present when bit u
// of vm is set; slots u >= nu (uniform over the workgroup) are empty.
struct RegSrc {
  uint64_t (&key)[LB];
  int32_t (&j)[LB];
  uint32_t vm;
  int nu;
  template <class F> __device__ __forceinline__ void for_each(F&& f) {
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      if (u >= nu) break;
      if ((vm >> u) & 1u) f(key[u], j[u]);
    }
  }
};

// Source that re-scores every eligible entry of the row on each pass.
template <int DT, int HP>
struct StreamSrc {
  const IndexArgs* A;
  Rows rw;
  MxQuery Q;
  float* tbuf;     // per-wave buffers [SEL_WAVES][WBUF]
  const float* wl; // [32] weights (row 0)
  const float* ql; // F32 query in LDS
  template <class F> __device__ void for_each(F&& f) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = rw.n[0];
    MxW<HP, 1> W;
    if (DT == DT_MXFP4) mx_load_weights<HP, 1>(wl, W);
    for (int j0 = wave * 64; j0 < n; j0 += SEL_THREADS) {
      uint64_t k0;
      if (DT == DT_MXFP4) {
        MxTiles T;
        bool ix;
        mx_load_round(*A, rw.b, j0, n, T);
        mx_score_round<HP, 1>(*A, rw, Q, T, j0, tbuf + wave * WBUF, W, &k0, ix);
        if (ix) k0 = mx_score_exact(*A, rw.r[0], rw.b, j0 + lane, wl);
      } else {
        f32_score_round(*A, rw, j0, ql, wl, k0);
      }
      f(k0, j0 + lane);
    }
  }
};

__device__ __forceinline__ bool emit_regs(const uint64_t (&bk)[LB], const int32_t (&bj)[LB], uint32_t vm, int nu,
                                          const Thr& th, int ties, bool unsafe, int k, int32_t* out, double* sout,
                                          SelShared& S);

// Exact selection of one row from scratch (rows with few entries, and rows
// whose candidates failed the certification): an fp32 row of at most
// LB * SEL_THREADS entries is scored once into registers; otherwise every
// pass re-scores the row.
template <int DT, int HP>
__device__ __forceinline__ void select_streamed(const IndexArgs& A, int r, int n, int kk, int32_t* out, double* sout,
                                             SelShared& S, float* tbuf, const float* wl, const float* ql,
                                             bool all_selected) {
  StreamSrc<DT, HP> src;
  src.A = &A;
  src.rw.b = r / A.Tq;
  src.rw.r[0] = r; src.rw.r[1] = -1;
  src.rw.n[0] = n; src.rw.n[1] = 0;
  if (DT == DT_MXFP4) mx_load_query<HP>(A, src.rw, src.Q);
  src.tbuf = tbuf;
  src.wl = wl;
  src.ql = ql;
  if (all_selected) {
    // every eligible entry is selected: only the scores are needed
    for (int i = n + threadIdx.x; i < A.k; i += SEL_THREADS) sout[i] = 0.0;
    src.for_each([&](uint64_t key, int j) { if (j < n) sout[j] = key_score(key); });
    return;
  }
  if (DT == DT_F32 && n <= LB * SEL_THREADS) {
    // an fp32 row that fits the registers: every eligible entry scored once
    // (item u*SEL_THREADS + tid = entry j, in the order of the streamed
    // passes), then the radix select and the emission over the registers
    // (the MXFP4 scoring state does not leave room for the keys)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint64_t bk[LB];
    int32_t bj[LB];
    uint32_t vm = 0;
    // the keys go through LDS, so that the scoring loop is not unrolled:
    // rows of up to 4096 entries keep them in the (here unused) bitmap and
    // stage their key rows through per-wavefront tiles in the scoring
    // buffers' region; longer rows keep them in that region and load each
    // lane's row directly
    constexpr int KL_BITMAP = BITMAP_BITS / 64;         // keys the bitmap holds
    const bool tiles = n <= KL_BITMAP && A.d % 16 == 0;
    uint64_t* kl = tiles ? (uint64_t*)S.bitmap : (uint64_t*)tbuf;
#pragma unroll 1
    for (int u = 0; u < LB; ++u) {
      const int j0 = u * SEL_THREADS + wave * 64;
      if (j0 >= n) break;                 // uniform over the wavefront
      uint64_t k0;
      if (tiles) f32_score_wave_lds(A, src.rw.b, n, j0, ql, wl, tbuf + wave * F32_TILE, k0);
      else f32_score_round_vec(A, src.rw, j0, ql, wl, k0);
      kl[u * SEL_THREADS + threadIdx.x] = k0;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int j = u * SEL_THREADS + threadIdx.x;
      const bool ok = j < n;
      bk[u] = ok ? kl[j] : 0ull;          // key 0: no entry
      bj[u] = j;
      vm |= (uint32_t)ok << u;
    }
    const int nu = (n + SEL_THREADS - 1) / SEL_THREADS;
    if (threadIdx.x == 0) S.bcast[6] = 0;  // emit_regs' "unsafe" flag (find_threshold's barriers order this)
    RegSrc rs{bk, bj, vm, nu};
    const Thr th = find_threshold(rs, kk, S);
    emit_regs(bk, bj, vm, nu, th, -1, false, A.k, out, sout, S);
    return;
  }
  const Thr th = find_threshold(src, kk, S);
  emit_sorted(src, th, n, A.k, out, sout, S);
}

// Emission for candidates stored in ascending index order: a block scan over
// the selection flags of contiguous slices keeps that order, so no sorting is
// needed.  Items equal to the threshold key are taken in array (= index)
// order until `ties` of them are in.
// Emission, in ascending candidate order, of the register-held items that th
// selects, when no excluded entry is unsafe (block-wide OR of `unsafe`).  With
// ties >= 0 (a full key T with more ties than places) the items equal to T
// are taken in candidate order until `ties` of them are in.  Item i =
// u*SEL_THREADS + tid belongs to pass u; one exchange of per-(pass, wavefront)
// counts of items above the threshold and of tied items gives every item its
// output position.  Returns false (nothing written) when unsafe.
__device__ __forceinline__ bool emit_regs(const uint64_t (&bk)[LB], const int32_t (&bj)[LB], uint32_t vm, int nu,
                                          const Thr& th, int ties, bool unsafe, int k, int32_t* out, double* sout,
                                          SelShared& S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // per slot: taken (a) or a tie at a full key (e), without branches; the
  // wavefront's 2*LB counts go to lanes 0 .. 2*LB-1 and one LDS store
  uint32_t fa = 0, fe = 0;
  int cnts = 0;
  const bool tmode = ties >= 0;
  const uint64_t Thi = th.low > 0 ? th.T >> th.low : 0ull;
#pragma unroll
  for (int u = 0; u < LB; ++u) {
    if (u >= nu) break;                   // empty in every thread
    const uint64_t key = bk[u];
    const bool valid = (vm >> u) & 1u;
    const bool gt = key > th.T, eq = key == th.T;
    const bool sel = key != 0 && (th.low > 0 ? (key >> th.low) >= Thi : (gt || (eq && bj[u] <= th.Tj)));
    const bool a = valid && (tmode ? gt : sel);
    const bool e = valid && tmode && eq;
    fa |= (uint32_t)a << u;
    fe |= (uint32_t)e << u;
    const int ca = __popcll(__ballot(a)), ce = __popcll(__ballot(e));
    cnts = lane == u ? ca : (lane == LB + u ? ce : cnts);
  }
  if (lane < LB) S.ecnt[lane * SEL_WAVES + wave] = (uint32_t)cnts;
  else if (lane < 2 * LB) S.ecnt2[(lane - LB) * SEL_WAVES + wave] = (uint32_t)cnts;
  if (unsafe) S.bcast[6] = 1;
  __syncthreads();
  if (S.bcast[6]) return false;
  if (wave == 0) {
    // exclusive prefixes over (pass, wavefront), two entries per lane
    static_assert(LB * SEL_WAVES == 128, "two prefix entries per lane");
    const int a0 = (int)S.ecnt[2 * lane], a1 = (int)S.ecnt[2 * lane + 1];
    const int ia = wave_incl_scan_dpp(a0 + a1);
    S.epre[2 * lane] = (uint32_t)(ia - a0 - a1);
    S.epre[2 * lane + 1] = (uint32_t)(ia - a1);
    const int e0 = (int)S.ecnt2[2 * lane], e1 = (int)S.ecnt2[2 * lane + 1];
    const int ie = wave_incl_scan_dpp(e0 + e1);
    S.epre2[2 * lane] = (uint32_t)(ie - e0 - e1);
    S.epre2[2 * lane + 1] = (uint32_t)(ie - e1);
    if (lane == 63) { S.bcast[5] = ia; S.bcast[2] = ie; }
  }
  __syncthreads();
  const int tot = S.bcast[5] + (ties >= 0 ? min(S.bcast[2], ties) : 0);
#pragma unroll
  for (int u = 0; u < LB; ++u) {
    if (u >= nu) break;
    const bool a = (fa >> u) & 1u, e = (fe >> u) & 1u;
    const uint64_t ba = __ballot(a), be = __ballot(e);
    if (a || e) {
      const int pa = (int)S.epre[u * SEL_WAVES + wave] + lanes_below(ba);
      int pe = 0;
      if (ties >= 0) pe = (int)S.epre2[u * SEL_WAVES + wave] + lanes_below(be);
      const int pos = pa + (ties >= 0 ? min(pe, ties) : 0);
      if ((a || pe < ties) && pos < k) {
        out[pos] = bj[u];
        if (sout) sout[pos] = key_score(bk[u]);
      }
    }
  }
  for (int i = tot + threadIdx.x; i < k; i += SEL_THREADS) {
    out[i] = -1;
    if (sout) sout[i] = 0.0;
  }
  return true;
}

// The prefill path (index_prefill.hip): many query rows per sequence.
bool index_prefill_applies(const IndexArgs& a);
size_t index_prefill_ws_bytes(int B, int Tq, int64_t N_cap, int k);
hipError_t launch_index_prefill(const IndexArgs& a, hipStream_t s);

// Dynamic LDS of a workgroup running the block-wide selection.
static inline size_t select_smem(int dt, int H, int d) {
  (void)dt; (void)H; (void)d;
  size_t region = 12 * (size_t)CMAX;                                   // candidate keys + indices
  const size_t stream = sizeof(float) * SEL_WAVES * WBUF;              // scoring buffers (aliased)
  if (stream > region) region = stream;
  static_assert(sizeof(float) * SEL_WAVES * F32_TILE <= 12 * (size_t)CMAX, "fp32 key tiles fit below the weights");
  return sizeof(SelShared) + region + sizeof(float) * 32;
}

}  // namespace lca
