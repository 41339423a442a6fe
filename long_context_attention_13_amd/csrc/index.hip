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
#include "lca_device.h"

namespace lca {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int CAP = 128;           // candidate slots per chunk
constexpr int NDIRECT = 8192;      // rows with n_elig <= NDIRECT skip the chunk kernel
constexpr int SEL_THREADS = 1024;  // select kernel workgroup
constexpr int SEL_WAVES = SEL_THREADS / WAVE;
constexpr int RMAX = 16;           // candidate slots per select thread
constexpr int KROW = 20;           // LDS floats per key in the transpose buffer (16 + pad)
constexpr int BITMAP_BITS = 1 << 18;

struct IdxWs {
  int32_t* cnt;   // [R][NCH]
  uint64_t* mex;  // [R][NCH]
  uint64_t* ckey; // [R][NCH][CAP]
  int32_t* cidx;  // [R][NCH][CAP]
};

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static IdxWs carve(void* ws, int64_t R, int64_t NCH) {
  IdxWs w;
  char* p = (char*)ws;
  w.cnt = (int32_t*)p; p += align256(sizeof(int32_t) * R * NCH);
  w.mex = (uint64_t*)p; p += align256(sizeof(uint64_t) * R * NCH);
  w.ckey = (uint64_t*)p; p += align256(sizeof(uint64_t) * R * NCH * CAP);
  w.cidx = (int32_t*)p;
  return w;
}

static size_t carve_bytes(int64_t R, int64_t NCH) {
  return align256(sizeof(int32_t) * R * NCH) + align256(sizeof(uint64_t) * R * NCH) +
         align256(sizeof(uint64_t) * R * NCH * CAP) + align256(sizeof(int32_t) * R * NCH * CAP);
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

template <int HP>
__device__ __forceinline__ void mx_load_query(const IndexArgs& A, const Rows& rw, MxQuery& Q) {
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, kb = lane >> 4;
  const int q = row / HP, h = row % HP;
  const bool valid = (q < 2) && rw.r[q] >= 0 && h < A.H && kb * 32 < A.d;
  Q.a[0] = Q.a[1] = Q.a[2] = Q.a[3] = 0;
  Q.sa = 127;
  int smin = 1000, smax = -1000;
  if (valid) {
    const int64_t qrow = (int64_t)rw.r[q] * A.H + h;
    const int4 v = *(const int4*)((const uint8_t*)A.qi + qrow * (A.d / 2) + kb * 16);
    Q.a[0] = v.x; Q.a[1] = v.y; Q.a[2] = v.z; Q.a[3] = v.w;
    Q.sa = A.qi_scale[qrow * (A.d / 32) + kb];
    smin = smax = Q.sa;
  }
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

struct MxTiles {
  int4 code[4];
  int sc[4];
};

// Load the B operands of 4 MFMA tiles = 64 keys [j0, j0+64).
__device__ __forceinline__ void mx_load_round(const IndexArgs& A, int b, int j0, int jlim, MxTiles& T) {
  const int lane = threadIdx.x & 63;
  const int kb = lane >> 4;
  const bool kbok = kb * 32 < A.d;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = j0 + t * 16 + (lane & 15);
    T.code[t] = make_int4(0, 0, 0, 0);
    T.sc[t] = 127;
    if (j < jlim && kbok) {
      const int64_t row = (int64_t)b * A.N_cap + j;
      T.code[t] = *(const int4*)((const uint8_t*)A.ki + row * (A.d / 2) + kb * 16);
      T.sc[t] = A.ki_scale[row * (A.d / 32) + kb];
    }
  }
}

__device__ __forceinline__ double mx_value(const uint8_t* codes, const uint8_t* scales, int i) {
  const uint32_t byte = codes[i >> 1];
  const uint32_t c = (i & 1) ? (byte >> 4) : (byte & 15u);
  return ldexp((double)e2m1_to_f32(c), (int)scales[i >> 5] - 127);
}

// Exact float64 dot product of query head (row qr, head h) and key row krow,
// left to right over the elements.
__device__ double mx_dot_exact(const IndexArgs& A, int64_t qrow, int64_t krow) {
  const uint8_t* qc = (const uint8_t*)A.qi + qrow * (A.d / 2);
  const uint8_t* qs = A.qi_scale + qrow * (A.d / 32);
  const uint8_t* kc = (const uint8_t*)A.ki + krow * (A.d / 2);
  const uint8_t* ks = A.ki_scale + krow * (A.d / 32);
  double dot = 0.0;
  for (int i = 0; i < A.d; ++i) dot = fma(mx_value(qc, qs, i), mx_value(kc, ks, i), dot);
  return dot;
}

// One step of the float64 head combine s = sum_h w_h * max(0, dot_h), taken in
// head order: multiply, then add (no contraction).
__device__ __forceinline__ double combine_step(double s, double dot, float w) {
#pragma clang fp contract(off)
  const double r = dot > 0.0 ? dot : 0.0;
  const double t = (double)w * r;
  return s + t;
}

// Score one round of 64 keys for the wave's rows.  Lane L ends with the keys
// of entry j0+L for row 0 and row 1 (0 when not eligible).
// wbuf: this wave's LDS transpose buffer (64*KROW floats); wl: LDS weights
// [2][16] for the two rows.
template <int HP>
__device__ __forceinline__ void mx_score_round(const IndexArgs& A, const Rows& rw, const MxQuery& Q,
                                               const MxTiles& T, int j0, float* wbuf, const float* wl,
                                               uint64_t& key0, uint64_t& key1) {
  const int lane = threadIdx.x & 63;
  v8i av = {Q.a[0], Q.a[1], Q.a[2], Q.a[3], 0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v8i bv = {T.code[t].x, T.code[t].y, T.code[t].z, T.code[t].w, 0, 0, 0, 0};
    v4f c = {0.f, 0.f, 0.f, 0.f};
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, Q.sa, 0, T.sc[t]);
    float* dst = wbuf + (t * 16 + (lane & 15)) * KROW + 4 * (lane >> 4);
    *(float4*)dst = make_float4(c[0], c[1], c[2], c[3]);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int j = j0 + lane;
  const float* mine = wbuf + lane * KROW;
  key0 = key1 = 0;
  // exactness envelope of this key
  bool exact = true;
  if (j < max(rw.n[0], rw.n[1])) {
    const uint8_t* ks = A.ki_scale + ((int64_t)rw.b * A.N_cap + j) * (A.d / 32);
    int kmin = 1000, kmax = -1000;
    for (int i = 0; i < A.d / 32; ++i) { const int s = ks[i]; kmin = min(kmin, s); kmax = max(kmax, s); }
    exact = (Q.dq + kmax - kmin <= 9) && (Q.qmin + kmin >= 130) && (Q.qmax + kmax <= 368);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (rw.r[q] < 0 || j >= rw.n[q]) continue;
    double s = 0.0;
    if (exact) {
#pragma unroll
      for (int h = 0; h < HP; ++h)
        if (h < A.H) s = combine_step(s, (double)mine[q * HP + h], wl[q * 16 + h]);
    } else {
      for (int h = 0; h < A.H; ++h)
        s = combine_step(s, mx_dot_exact(A, (int64_t)rw.r[q] * A.H + h, (int64_t)rw.b * A.N_cap + j),
                         wl[q * 16 + h]);
    }
    const uint64_t kk = score_key(s);
    if (q == 0) key0 = kk; else key1 = kk;
  }
  __builtin_amdgcn_wave_barrier();
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
// Chunk kernel
// ------------------------------------------------------------------------
template <int DT, int KPL, int HP>
__global__ __launch_bounds__(256) void index_chunk_kernel(IndexArgs A, IdxWs W, int NCH, int groups_per_b,
                                                          int qpm) {
  constexpr int CH = 64 * KPL;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + wave;
  const int g = blockIdx.y;
  __shared__ float tbuf[4][64 * KROW];
  __shared__ float wl_s[4][32];

  Rows rw;
  rw.b = g / groups_per_b;
  const int t0 = (g % groups_per_b) * qpm;
  rw.r[0] = rw.b * A.Tq + t0;
  rw.r[1] = (qpm == 2 && t0 + 1 < A.Tq) ? rw.r[0] + 1 : -1;
  rw.n[0] = A.n_elig[rw.r[0]];
  rw.n[1] = rw.r[1] >= 0 ? A.n_elig[rw.r[1]] : 0;
  // rows with few entries are done by the select kernel alone
  if (rw.n[0] <= NDIRECT) rw.n[0] = 0;
  if (rw.n[1] <= NDIRECT) rw.n[1] = 0;
  const int jlim = max(rw.n[0], rw.n[1]);
  const int jbeg = c * CH;
  if (jbeg >= jlim || c >= NCH) return;

  float* wl = wl_s[wave];
  if (lane < 32) {
    const int q = lane >> 4, h = lane & 15;
    wl[lane] = (rw.r[q] >= 0 && h < A.H) ? A.w[(int64_t)rw.r[q] * A.H + h] : 0.f;
  }
  __builtin_amdgcn_wave_barrier();

  uint64_t k0[KPL], k1[KPL];
  if (DT == DT_MXFP4) {
    MxQuery Q;
    mx_load_query<HP>(A, rw, Q);
    MxTiles cur, nxt;
    mx_load_round(A, rw.b, jbeg, jlim, cur);
#pragma unroll
    for (int rr = 0; rr < KPL; ++rr) {
      if (rr + 1 < KPL) mx_load_round(A, rw.b, jbeg + (rr + 1) * 64, jlim, nxt);
      mx_score_round<HP>(A, rw, Q, cur, jbeg + rr * 64, tbuf[wave], wl, k0[rr], k1[rr]);
      if (rr + 1 < KPL) cur = nxt;
    }
  } else {
    const float* qrow = (const float*)A.qi + (int64_t)rw.r[0] * A.H * A.d;
#pragma unroll
    for (int rr = 0; rr < KPL; ++rr) {
      f32_score_round(A, rw, jbeg + rr * 64, qrow, wl, k0[rr]);
      k1[rr] = 0;
    }
  }

  // per row: threshold from the lane maxima, emit, record the best excluded key
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (rw.r[q] < 0 || rw.n[q] == 0 || jbeg >= rw.n[q]) continue;
    const uint64_t* kq = q == 0 ? k0 : k1;
    uint64_t lmax = 0;
#pragma unroll
    for (int rr = 0; rr < KPL; ++rr) lmax = kq[rr] > lmax ? kq[rr] : lmax;
    const uint64_t sorted = wave_sort_desc(lmax);
    const float lam = (float)A.k * (float)CH / (float)rw.n[q];
    int rsel = (int)ceilf(lam + 6.0f * sqrtf(lam) + 8.0f);
    rsel = rsel > 64 ? 64 : rsel;
    const uint32_t tlo = __shfl((uint32_t)sorted, rsel - 1, WAVE);
    const uint32_t thi = __shfl((uint32_t)(sorted >> 32), rsel - 1, WAVE);
    uint64_t thr = ((uint64_t)thi << 32) | tlo;
    if (thr == 0) thr = 1;     // key 0 marks "no entry"; never emit those
    int total = 0;
    uint64_t exmax = 0;
#pragma unroll
    for (int rr = 0; rr < KPL; ++rr) {
      const bool f = kq[rr] >= thr;
      total += __popcll(__ballot(f));
      if (!f && kq[rr] > exmax) exmax = kq[rr];
    }
    exmax = wave_max_u64(exmax);
    const int64_t slot = (int64_t)rw.r[q] * NCH + c;
    if (total > CAP) {
      if (lane == 0) { W.cnt[slot] = -1; W.mex[slot] = ~0ull; }
      continue;
    }
    int base = 0;
#pragma unroll
    for (int rr = 0; rr < KPL; ++rr) {
      const bool f = kq[rr] >= thr;
      const uint64_t bal = __ballot(f);
      if (f) {
        const int pos = base + lanes_below(bal);
        W.ckey[slot * CAP + pos] = kq[rr];
        W.cidx[slot * CAP + pos] = jbeg + rr * 64 + lane;
      }
      base += __popcll(bal);
    }
    if (lane == 0) { W.cnt[slot] = total; W.mex[slot] = exmax; }
  }
}

// ------------------------------------------------------------------------
// Select kernel helpers (block of SEL_THREADS threads)
// ------------------------------------------------------------------------
struct SelShared {
  uint32_t hist[2048];
  uint32_t scan[SEL_WAVES];
  uint64_t red64[SEL_WAVES];
  int32_t off[SEL_THREADS + 1];
  uint32_t bitmap[BITMAP_BITS / 32];
  int bcast[8];
  uint64_t bcast64[4];
};

__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, SelShared& S) {
  v = wave_max_u64(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) S.red64[wave] = v;
  __syncthreads();
  uint64_t m = 0;
  for (int i = 0; i < SEL_WAVES; ++i) m = S.red64[i] > m ? S.red64[i] : m;
  return m;
}

__device__ __forceinline__ uint64_t block_min_u64(uint64_t v, SelShared& S) {
  // min over valid keys; callers pass ~0 for invalid
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t t = shfl_xor_u64(v, o);
    v = t < v ? t : v;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) S.red64[wave] = v;
  __syncthreads();
  uint64_t m = ~0ull;
  for (int i = 0; i < SEL_WAVES; ++i) m = S.red64[i] < m ? S.red64[i] : m;
  return m;
}

// Exclusive block scan of one int per thread; returns the exclusive prefix,
// total in *tot.
__device__ __forceinline__ int block_scan(int v, int* tot, SelShared& S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, WAVE);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) S.scan[wave] = (uint32_t)incl;
  __syncthreads();
  int before = 0, all = 0;
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
__device__ void radix_digit(Src& src, uint64_t prefix, uint64_t mask, int shift, int nb, int rem, SelShared& S) {
  const int nbins = 1 << nb;
  for (int i = threadIdx.x; i < 2048; i += SEL_THREADS) S.hist[i] = 0;
  __syncthreads();
  src.for_each([&](uint64_t key, int j) {
    if (key != 0 && (key & mask) == prefix) atomicAdd(&S.hist[(key >> shift) & (uint64_t)(nbins - 1)], 1u);
  });
  __syncthreads();
  // suffix sums: thread t owns bins 2t, 2t+1 (counted from the top)
  const int t = threadIdx.x;
  const int bhi = nbins - 1 - 2 * t, blo = bhi - 1;
  const int c_hi = (bhi >= 0) ? (int)S.hist[bhi] : 0;
  const int c_lo = (blo >= 0) ? (int)S.hist[blo] : 0;
  int tot;
  const int above = block_scan(c_hi + c_lo, &tot, S);   // count in bins above bhi
  if (bhi >= 0 && above < rem && above + c_hi >= rem) {
    S.bcast[0] = bhi; S.bcast[1] = above; S.bcast[2] = c_hi;
  }
  if (blo >= 0 && above + c_hi < rem && above + c_hi + c_lo >= rem) {
    S.bcast[0] = blo; S.bcast[1] = above + c_hi; S.bcast[2] = c_lo;
  }
  __syncthreads();
}

// Smallest-j selection among ties (key == T): find the rem-th smallest j.
template <class Src>
__device__ int tie_select_j(Src& src, uint64_t T, int rem, SelShared& S) {
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
    const int t = threadIdx.x;
    const int b0 = 2 * t, b1 = b0 + 1;
    const int c0 = b0 < (int)nbins ? (int)S.hist[b0] : 0;
    const int c1 = b1 < (int)nbins ? (int)S.hist[b1] : 0;
    int tot;
    const int below = block_scan(c0 + c1, &tot, S);
    if (b0 < (int)nbins && below < rem && below + c0 >= rem) { S.bcast[0] = b0; S.bcast[1] = below; }
    if (b1 < (int)nbins && below + c0 < rem && below + c0 + c1 >= rem) { S.bcast[0] = b1; S.bcast[1] = below + c0; }
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

// Exact selection threshold for the kk largest (by key desc, j asc) items.
template <class Src>
__device__ Thr find_threshold(Src& src, int kk, SelShared& S) {
  Thr th;
  uint64_t mx = 0, mn = ~0ull;
  src.for_each([&](uint64_t key, int j) {
    if (key != 0) { mx = key > mx ? key : mx; mn = key < mn ? key : mn; }
  });
  mx = block_max_u64(mx, S);
  mn = block_min_u64(mn, S);
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

// Source over candidates held in registers.
struct RegSrc {
  uint64_t key[RMAX];
  int j[RMAX];
  template <class F> __device__ __forceinline__ void for_each(F&& f) {
#pragma unroll
    for (int s = 0; s < RMAX; ++s) f(key[s], j[s]);
  }
};

// Source that re-scores every eligible entry of the row on each pass.
template <int DT, int HP>
struct StreamSrc {
  const IndexArgs* A;
  Rows rw;
  MxQuery Q;
  float* tbuf;     // per-wave transpose buffers [SEL_WAVES][64*KROW]
  const float* wl; // [32] weights (row 0)
  const float* ql; // F32 query in LDS
  template <class F> __device__ void for_each(F&& f) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = rw.n[0];
    for (int j0 = wave * 64; j0 < n; j0 += SEL_THREADS) {
      uint64_t k0, k1;
      if (DT == DT_MXFP4) {
        MxTiles T;
        mx_load_round(*A, rw.b, j0, n, T);
        mx_score_round<HP>(*A, rw, Q, T, j0, tbuf + wave * 64 * KROW, wl, k0, k1);
      } else {
        f32_score_round(*A, rw, j0, ql, wl, k0);
      }
      f(k0, j0 + lane);
    }
  }
};

template <int DT, int HP>
__global__ __launch_bounds__(SEL_THREADS) void index_select_kernel(IndexArgs A, IdxWs W, int NCH, int CH) {
  extern __shared__ __align__(16) char smem[];
  SelShared& S = *(SelShared*)smem;
  float* tbuf = (float*)(smem + sizeof(SelShared));               // [SEL_WAVES][64*KROW]
  float* wl = tbuf + SEL_WAVES * 64 * KROW;                        // [32]
  float* ql = wl + 32;                                             // F32 query [H*d]

  const int r = blockIdx.x;
  const int n = A.n_elig[r];
  const int kk = n < A.k ? n : A.k;
  int32_t* out = A.idx_out + (int64_t)r * A.k;
  double* sout = A.score_out ? A.score_out + (int64_t)r * A.k : nullptr;

  if (threadIdx.x < 32) wl[threadIdx.x] = (threadIdx.x < (unsigned)A.H) ? A.w[(int64_t)r * A.H + threadIdx.x] : 0.f;
  if (DT == DT_F32)
    for (int i = threadIdx.x; i < A.H * A.d; i += SEL_THREADS) ql[i] = ((const float*)A.qi)[(int64_t)r * A.H * A.d + i];
  __syncthreads();

  bool done = false;
  if (n <= A.k) {
    // every eligible entry is selected; scores only if asked for
    for (int i = threadIdx.x; i < A.k; i += SEL_THREADS) out[i] = i < n ? i : -1;
    if (sout) {
      StreamSrc<DT, HP> src;
      src.A = &A;
      src.rw.b = r / A.Tq;
      src.rw.r[0] = r; src.rw.r[1] = -1;
      src.rw.n[0] = n; src.rw.n[1] = 0;
      if (DT == DT_MXFP4) mx_load_query<HP>(A, src.rw, src.Q);
      src.tbuf = tbuf; src.wl = wl; src.ql = ql;
      for (int i = n + threadIdx.x; i < A.k; i += SEL_THREADS) sout[i] = 0.0;
      src.for_each([&](uint64_t key, int j) { if (j < n) sout[j] = key_score(key); });
    }
    done = true;
  } else if (n > NDIRECT) {
    // ---------------- candidate path ----------------
    const int nch = (n + CH - 1) / CH;
    int bad = 0;
    // prefix offsets of the chunk counts
    int total = 0;
    for (int c0 = 0; c0 < nch; c0 += SEL_THREADS) {
      const int c = c0 + threadIdx.x;
      int v = 0;
      if (c < nch) {
        v = W.cnt[(int64_t)r * NCH + c];
        if (v < 0) { bad = 1; v = 0; }
      }
      int tot;
      const int ex = block_scan(v, &tot, S);
      if (nch <= SEL_THREADS) S.off[threadIdx.x] = ex;
      total += tot;
    }
    if (nch <= SEL_THREADS && threadIdx.x == 0) S.off[nch] = total;
    bad = __syncthreads_or(bad);
    if (!bad && nch <= SEL_THREADS && total <= RMAX * SEL_THREADS && total >= kk) {
      RegSrc src;
#pragma unroll
      for (int s = 0; s < RMAX; ++s) {
        const int i = s * SEL_THREADS + threadIdx.x;
        src.key[s] = 0;
        src.j[s] = 0x7FFFFFFF;
        if (i < total) {
          int lo = 0, hi = nch;      // find chunk c with off[c] <= i < off[c+1]
          while (hi - lo > 1) { const int mid = (lo + hi) >> 1; if (S.off[mid] <= i) lo = mid; else hi = mid; }
          const int64_t slot = (int64_t)r * NCH + lo;
          const int p = i - S.off[lo];
          src.key[s] = W.ckey[slot * CAP + p];
          src.j[s] = W.cidx[slot * CAP + p];
        }
      }
      const Thr th = find_threshold(src, kk, S);
      // certification: no excluded entry may reach the threshold
      int unsafe = 0;
      for (int c = threadIdx.x; c < nch; c += SEL_THREADS) {
        const uint64_t m = W.mex[(int64_t)r * NCH + c];
        if (m != 0) {
          if (th.low > 0) unsafe |= (m >> th.low) >= (th.T >> th.low);
          else unsafe |= m >= th.T;
        }
      }
      unsafe = __syncthreads_or(unsafe);
      if (!unsafe) {
        emit_sorted(src, th, n, A.k, out, sout, S);
        done = true;
      }
    }
  }
  if (!done) {
    // ---------------- exact streamed path ----------------
    StreamSrc<DT, HP> src;
    src.A = &A;
    src.rw.b = r / A.Tq;
    src.rw.r[0] = r; src.rw.r[1] = -1;
    src.rw.n[0] = n; src.rw.n[1] = 0;
    if (DT == DT_MXFP4) mx_load_query<HP>(A, src.rw, src.Q);
    src.tbuf = tbuf;
    src.wl = wl;
    src.ql = ql;
    const Thr th = find_threshold(src, kk, S);
    emit_sorted(src, th, n, A.k, out, sout, S);
  }
}

// ------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------
static int choose_kpl(const IndexArgs& a, int qpm) {
  const int64_t groups = (int64_t)a.B * ((a.Tq + qpm - 1) / qpm);
  const int64_t waves16 = groups * ((a.N_cap + 1023) / 1024);
  return waves16 >= 1024 ? 16 : 4;
}

static int qpm_of(int dt, int H) { return (dt == DT_MXFP4 && H <= 8) ? 2 : 1; }

size_t index_ws_bytes(int B, int Tq, int H, int d, int64_t N_cap, int k, int dt) {
  IndexArgs a{};
  a.B = B; a.Tq = Tq; a.H = H; a.d = d; a.N_cap = N_cap; a.k = k;
  const int kpl = choose_kpl(a, qpm_of(dt, H));
  const int64_t NCH = (N_cap + 64 * kpl - 1) / (64 * kpl);
  return carve_bytes((int64_t)B * Tq, NCH > 0 ? NCH : 1);
}

static size_t select_smem(int dt, int H, int d) {
  size_t s = sizeof(SelShared) + sizeof(float) * (SEL_WAVES * 64 * KROW + 32);
  if (dt == DT_F32) s += sizeof(float) * H * d;
  return s;
}

template <int DT, int KPL, int HP>
static hipError_t launch_t(const IndexArgs& a, hipStream_t s, int qpm) {
  const int CH = 64 * KPL;
  const int64_t NCH = (a.N_cap + CH - 1) / CH;
  IdxWs W = carve(a.ws, (int64_t)a.B * a.Tq, NCH > 0 ? NCH : 1);
  const int gpb = (a.Tq + qpm - 1) / qpm;
  if (a.N_cap > NDIRECT) {
    dim3 grid((unsigned)((NCH + 3) / 4), (unsigned)(a.B * gpb));
    hipLaunchKernelGGL((index_chunk_kernel<DT, KPL, HP>), grid, dim3(256), 0, s, a, W, (int)NCH, gpb, qpm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t smem = select_smem(DT, a.H, a.d);
  hipLaunchKernelGGL((index_select_kernel<DT, HP>), dim3((unsigned)(a.B * a.Tq)), dim3(SEL_THREADS), smem, s, a, W,
                     (int)NCH, CH);
  return hipGetLastError();
}

hipError_t launch_index(const IndexArgs& a, hipStream_t s) {
  if ((int64_t)a.B * a.Tq == 0) return hipSuccess;
  const int qpm = qpm_of(a.dt, a.H);
  const int kpl = choose_kpl(a, qpm);
  if (a.dt == DT_MXFP4) {
    if (a.H <= 8) return kpl == 16 ? launch_t<DT_MXFP4, 16, 8>(a, s, qpm) : launch_t<DT_MXFP4, 4, 8>(a, s, qpm);
    return kpl == 16 ? launch_t<DT_MXFP4, 16, 16>(a, s, qpm) : launch_t<DT_MXFP4, 4, 16>(a, s, qpm);
  }
  return kpl == 16 ? launch_t<DT_F32, 16, 16>(a, s, 1) : launch_t<DT_F32, 4, 16>(a, s, 1);
}

}  // namespace lca
