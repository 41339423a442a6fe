// index_prefill.hip -- lightning indexer and exact top-k for many query rows
// of one sequence (chunked prefill) on gfx950.
//
// [release notes (agentlenshq.com), 壓縮稀疏注意力 (CSA): FP4, ReLU-scored
//  multi-head dot products choose the top-k compressed blocks per query;
//  wiki (chenshi221), 基础设施: MXFP4 on the indexer QK path.]
//
// The result is the one the decode path gives (the top-k by (s desc, j asc)
// of the float64 score, bit for bit); the work is organised as a dense
// contraction so that it runs on the FP4 matrix cores:
//
//   sample  each row scores a strided sample of its eligible keys (one key in
//           sigma = k/16) and takes the 32nd largest sampled score, rounded
//           down, as its candidate threshold t: about 32*sigma entries of the
//           row reach it.  A workgroup samples 16 rows (the MFMA's columns), or
//           fewer when the rows' samples would not fit its LDS (16 rows up
//           to about 4200 samples a row, 8 up to 8400, ... 2 up to 33700).
//   score   a workgroup holds 64 query rows (16 per wavefront, the MFMA's
//           column operand, one operand per indexer head) and streams a range
//           of keys through LDS in stages of 512 (direct global->LDS loads,
//           double buffered).  Each 16-key tile is one scaled FP4 MFMA per
//           head; the fp32 head combine s32 = sum_h w_h * max(0, dot_h) runs
//           in the lane that holds the dots (4 keys of one row); keys with
//           s32 >= t go to a per-(row, key range, lane group) candidate list.
//   select  one wavefront per row: exact radix select of the k-th largest
//           s32 (T) over the row's candidates, then a certified band.  The
//           per-head dots are exact (the exactness envelope is checked for
//           every key against the workgroup's queries) and the combine adds
//           non-negative terms with fused multiply-adds, so
//           |s32 - s| <= eps * s with eps = (H + 1) * 2^-24.  Entries with
//           s32 above T(1+eps)/(1-eps) are in, entries below T(1-eps)/(1+eps)
//           are out, and the few in between are re-scored exactly (MFMA dots
//           + float64 combine) and ranked by (s desc, j asc).  The candidate
//           set is complete when T(1-eps) >= t(1+eps).
//   fallback rows failing any check (a candidate list overflowed, too few or
//           too many candidates, a wide band, a negative head weight, a key
//           outside the exactness envelope) are queued; the first PF_QFAST of
//           them are selected by the decode path's scan and select over
//           their key rows (a workgroup per chunk and queued row, then one per
//           row), any further ones by re-scoring every entry exactly in one
//           workgroup per row.
#include "index_common.h"
#include "index_select.h"

namespace lca {

constexpr int PF_QROWS = 64;          // query rows per score workgroup (16 per wavefront)
constexpr int PF_STAGE = 256;         // keys per LDS stage (3 workgroups per CU: the registers allow 3, the LDS 4)
constexpr int PF_CODE_B = PF_STAGE * 64;
constexpr int PF_STAGE_B = PF_CODE_B + PF_STAGE * 4;
constexpr int PF_NKC = 16;            // key ranges per row
constexpr int PF_LCAP = 96;           // candidates per (row, key range, lane group)
constexpr int PF_SROWS_LDS = 132 * 1024;     // LDS for the sampled scores of one sample workgroup
constexpr int PF_SPAD = 16;                  // padding of a row of samples (16-bit scores)
// sampled keys per row at most: a row of them, rounded up to 64 and padded,
// fits half of PF_SROWS_LDS (two rows a workgroup)
constexpr int PF_SMAX = (PF_SROWS_LDS / 2 / 2 - PF_SPAD) / 64 * 64;
constexpr int PF_RANK = 32;           // threshold = PF_RANK-th largest sampled score
constexpr int PF_QFAST = 16;          // queued rows the decode scan and select take
constexpr int PF_CAND = 3840;         // candidates per row the select pass holds
constexpr int PF_CPL = PF_CAND / 64;  // ... per lane
constexpr int PF_BAND = 64;           // band entries re-scored exactly
constexpr int PF_NMAX = 1 << 20;      // largest key cache the prefill path takes
constexpr int PF_FALLBACK_GRID = 128;
constexpr int PF_SWAVES = 8;         // wavefronts of the sample workgroup (16 rows)

struct PfWs {
  float* thr;       // [R] candidate threshold (fp32 score)
  int32_t* flags;   // [R] nonzero: the row is selected by the exact fallback
  int32_t* cnt;     // [R][PF_NKC][4] candidates per list (> PF_LCAP: overflow)
  uint64_t* cand;   // [R][PF_NKC][4][PF_LCAP] (fp32 score bits << 32) | j
  int32_t* queue;   // [1 + R] fallback queue: count, rows
  char* qws;        // [PF_QFAST] decode-scan workspaces of the queued rows (qslot bytes each)
};

static PfWs pf_carve(void* ws, int64_t R) {
  PfWs w;
  char* p = (char*)ws;
  w.thr = (float*)p; p += align256(sizeof(float) * R);
  w.flags = (int32_t*)p; p += align256(sizeof(int32_t) * R);
  w.cnt = (int32_t*)p; p += align256(sizeof(int32_t) * R * PF_NKC * 4);
  w.cand = (uint64_t*)p; p += align256(sizeof(uint64_t) * R * PF_NKC * 4 * PF_LCAP);
  w.queue = (int32_t*)p; p += align256(sizeof(int32_t) * (R + 1));
  w.qws = p;
  return w;
}

// The decode scan of PF_QFAST queued rows: its chunk size (chosen as for a
// call of PF_QFAST one-row sequences) and the workspace of one row.
struct PfQPlan {
  int kpl, NCH;
  size_t slot;
};
static PfQPlan pf_qplan(int64_t N_cap, int k) {
  IndexArgs v{};
  v.B = PF_QFAST; v.Tq = 1; v.N_cap = N_cap; v.k = k;
  PfQPlan q;
  q.kpl = choose_kpl(v, 1);
  const int64_t nch = (N_cap + 64 * q.kpl - 1) / (64 * q.kpl);
  q.NCH = (int)(nch > 0 ? nch : 1);
  q.slot = align256(carve_bytes(1, q.NCH));
  return q;
}

static size_t pf_bytes(int64_t R) {
  return align256(sizeof(float) * R) + align256(sizeof(int32_t) * R) + align256(sizeof(int32_t) * R * PF_NKC * 4) +
         align256(sizeof(uint64_t) * R * PF_NKC * 4 * PF_LCAP) + align256(sizeof(int32_t) * (R + 1));
}

// Sample stride: at least k/16 (so about 32*sigma <= 2k candidates per row
// at sigma = k/16) and enough to keep the sample within PF_SMAX keys.  The
// threshold misses a row's k-th largest score when 32 of its top-k entries
// fall in a sample that holds 16 of them on average, about once in 10^4
// rows; such a row is queued and selected by the decode scan.
static int pf_sigma(const IndexArgs& a) {
  int s = a.k / 16;
  const int64_t need = (a.N_cap + PF_SMAX - 1) / PF_SMAX;
  if (need > s) s = (int)need;
  return s < 1 ? 1 : s;
}

static int pf_key_range(const IndexArgs& a) {
  int64_t kc = (a.N_cap + PF_NKC - 1) / PF_NKC;
  kc = (kc + PF_STAGE - 1) / PF_STAGE * PF_STAGE;
  return (int)kc;
}

bool index_prefill_applies(const IndexArgs& a) {
  return a.dt == DT_MXFP4 && a.d == 128 && a.H >= 1 && a.H <= 16 && a.Tq >= PF_QROWS && a.k <= 1024 &&
         a.N_cap >= 64 && a.N_cap <= PF_NMAX && a.N_cap % 4 == 0;
}

size_t index_prefill_ws_bytes(int B, int Tq, int64_t N_cap, int k) {
  return pf_bytes((int64_t)B * Tq) + PF_QFAST * pf_qplan(N_cap, k).slot;
}

// ------------------------------------------------------------------------
// The lane's query operands: row c = lane & 15 of the wave's 16 rows,
// K-block g = lane >> 4, one 16-byte FP4 fragment and one E8M0 byte per head.
// ------------------------------------------------------------------------
template <int HP>
struct PfQuery {
  v8i bq[HP];
  int sb[HP];
  float wv[HP];
};

template <int HP>
__device__ __forceinline__ void pf_load_query(const IndexArgs& A, bool rv, int64_t r, PfQuery<HP>& P, bool& wneg) {
  const int g = (threadIdx.x & 63) >> 4;
  wneg = false;
#pragma unroll
  for (int h = 0; h < HP; ++h) {
    const bool ok = rv && h < A.H;
    const int64_t qrow = r * A.H + h;
    v4i v = {0, 0, 0, 0};
    if (ok) v = *(const v4i*)((const uint8_t*)A.qi + qrow * 64 + g * 16);
    P.bq[h] = (v8i){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
    P.sb[h] = ok ? (int)A.qi_scale[qrow * 4 + g] : 127;
    P.wv[h] = ok ? A.w[qrow] : 0.f;
    wneg |= P.wv[h] < 0.f;
  }
}

// s32 for the 4 keys of one MFMA tile held by this lane (rows 4g..4g+3 of the
// tile), one query row: fp32 fused multiply-adds in head order.
template <int HP>
__device__ __forceinline__ void pf_combine(const v4f (&acc)[HP], const PfQuery<HP>& P, float (&s)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = 0.f;
#pragma unroll
    for (int h = 0; h < HP; ++h) {
      // ReLU on the bit pattern: negative values (and -0) have negative int bits
      const float rl = __int_as_float(max(__float_as_int(acc[h][i]), 0));
      v = fmaf(P.wv[h], rl, v);
    }
    s[i] = v;
  }
}

// Digit of the rem-th largest value in a 256-bin LDS histogram (bins counted
// from the top), wave-wide.  Returns the digit; *above = count in higher bins.
__device__ __forceinline__ int pf_hist_digit(const uint32_t* hist, int rem, int* above_out) {
  const int lane = threadIdx.x & 63;
  const int top = 255 - 4 * lane;
  uint32_t c[4];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) { c[i] = hist[top - i]; mine += (int)c[i]; }
  const int incl = wave_incl_scan_dpp(mine);
  int above = incl - mine, d = -1, ab = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (d < 0 && above < rem && above + (int)c[i] >= rem) { d = top - i; ab = above; }
    above += (int)c[i];
  }
  const uint64_t m = __ballot(d >= 0);
  const int src = m ? __ffsll((unsigned long long)m) - 1 : 0;
  *above_out = __shfl(ab, src, WAVE);
  return __shfl(d, src, WAVE);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------------------
// Sample pass: 16 rows per workgroup; wave w scores sample tiles w, w+4, ...
// for all 16 rows, keeping the top 16 bits of each fp32 score (rounded down)
// in LDS; then each wave finds the thresholds of 4 rows.
// ------------------------------------------------------------------------
// Rows per sample workgroup: the most of 16, 8, 4, 2 whose samples (srow
// 16-bit scores a row) fit PF_SROWS_LDS.
static int pf_sample_rows(int srow) {
  int sr = 16;
  while (sr > 2 && (size_t)sr * srow * 2 > (size_t)PF_SROWS_LDS) sr >>= 1;
  return sr;
}

template <int HP>
__global__ __launch_bounds__(PF_SWAVES * 64) void pf_sample_kernel(IndexArgs A, PfWs W, int sigma, int srow, int sr) {
  extern __shared__ __align__(16) char smem[];
  uint16_t* sc = (uint16_t*)smem;                                  // [sr][srow]
  uint32_t* hist = (uint32_t*)(smem + (size_t)sr * srow * 2);      // [PF_SWAVES][256]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * sr;
  const int t = t0 + c;
  const bool rv = c < sr && t < A.Tq;            // columns sr .. 15 carry no query
  const int64_t r = (int64_t)b * A.Tq + (rv ? t : 0);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) W.queue[0] = 0;

  PfQuery<HP> P;
  bool wneg;
  pf_load_query<HP>(A, rv, r, P, wneg);
  const int nq = rv ? idx_nelig(A, r) : 0;
  int nmax = nq;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nmax = max(nmax, __shfl_xor(nmax, o, WAVE));
  const int S = nmax > 0 ? (nmax + sigma - 1) / sigma : 0;         // samples j = s * sigma < nmax
  const int ntile = (S + 15) / 16;
  // A operand of sample tile tt (16 sampled keys): lane = key c, K-block g
  auto ld = [&](int tt, v4i& av, int& ka) {
    const int sa = min(tt * 16 + c, S - 1);
    const int64_t krow = (int64_t)b * A.N_cap + (int64_t)sa * sigma;
    av = *(const v4i*)((const uint8_t*)A.ki + krow * 64 + g * 16);
    ka = A.ki_scale[krow * 4 + g];
  };
  v4i avc = {0, 0, 0, 0}, avn = {0, 0, 0, 0};
  int kac = 127, kan = 127;
  if (wave < ntile) ld(wave, avc, kac);
#pragma unroll 1
  for (int tt = wave; tt < ntile; tt += PF_SWAVES) {
    if (tt + PF_SWAVES < ntile) ld(tt + PF_SWAVES, avn, kan);
    const v8i a8 = {avc[0], avc[1], avc[2], avc[3], 0, 0, 0, 0};
    v4f acc[HP];
#pragma unroll
    for (int h = 0; h < HP; ++h) {
      const v4f z = {0.f, 0.f, 0.f, 0.f};
      acc[h] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, P.bq[h], z, 4, 4, 0, kac, 0, P.sb[h]);
    }
    float sv[4];
    pf_combine<HP>(acc, P, sv);
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int si = tt * 16 + 4 * g + i;
      const bool el = si < S && si * sigma < nq && !wneg;
      u[i] = el ? (__float_as_uint(sv[i]) >> 16) : 0u;
    }
    if (c < sr) *(uint2*)(sc + c * srow + tt * 16 + 4 * g) = make_uint2(u[0] | (u[1] << 16), u[2] | (u[3] << 16));
    avc = avn;
    kac = kan;
  }
  __syncthreads();

  uint32_t* hw = hist + wave * 256;
#pragma unroll 1
  for (int cq = wave; cq < sr; cq += PF_SWAVES) {
    const int tq = t0 + cq;
    if (tq >= A.Tq) break;
    const int64_t rq = (int64_t)b * A.Tq + tq;
    const int nqq = __shfl(nq, cq, WAVE);
    const bool neg = __shfl((int)wneg, cq, WAVE) != 0;
    const int Sq = min(S, (nqq + sigma - 1) / sigma);
    float thr = 0.f;
    if (Sq >= PF_RANK && !neg) {
      const uint16_t* v = sc + cq * srow;
      // exact radix select of the PF_RANK-th largest 16-bit score, digits of
      // at most 8 bits from the highest bit where the row's samples differ
      // (their common leading bits -- most of the exponent -- would put
      // nearly all of them in one bin and serialise the counting)
      // The smallest lane maximum vmn has at least 64 samples at or above it
      // when every lane holds one (and is 0 otherwise), so the PF_RANK-th
      // largest (PF_RANK <= 64) is >= vmn, and samples below vmn take no
      // part in the counting (they would pile into the lowest bins and
      // serialise the LDS atomics).
      static_assert(PF_RANK <= WAVE, "the smallest lane maximum bounds the rank");
      uint32_t vmx = 0;
      for (int i = lane; i < Sq; i += 64) vmx = max(vmx, (uint32_t)v[i]);
      uint32_t vmn = vmx;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        vmx = max(vmx, (uint32_t)__shfl_xor((int)vmx, o, WAVE));
        vmn = min(vmn, (uint32_t)__shfl_xor((int)vmn, o, WAVE));
      }
      int hi = vmx == vmn ? -1 : 31 - __clz(vmx ^ vmn);   // highest bit not yet resolved
      uint32_t prefix = hi < 0 ? vmx : vmx & ~((2u << hi) - 1u);
      int rem = PF_RANK;
#pragma unroll 1
      while (hi >= 0) {
        const int shift = hi >= 7 ? hi - 7 : 0;
        const uint32_t dmask = (2u << (hi - shift)) - 1u;     // this digit's bits
        const uint32_t pmask = ~((2u << hi) - 1u);            // the bits resolved above it
        for (int i = lane; i < 256; i += 64) hw[i] = 0;
        wave_lds_sync();
        for (int i = lane; i < Sq; i += 64) {
          const uint32_t x = v[i];
          if (x >= vmn && (x & pmask) == prefix) atomicAdd(&hw[(x >> shift) & dmask], 1u);
        }
        wave_lds_sync();
        int above;
        const int d = pf_hist_digit(hw, rem, &above);
        rem -= above;
        prefix |= (uint32_t)d << shift;
        wave_lds_sync();
        hi = shift - 1;
      }
      thr = __uint_as_float(prefix << 16);
    }
    if (lane == 0) {
      W.thr[rq] = neg ? __builtin_inff() : thr;
      W.flags[rq] = neg ? 1 : 0;
    }
  }
}

// ------------------------------------------------------------------------
// Score pass.
// ------------------------------------------------------------------------
template <int HP>
__global__ __launch_bounds__(256) void pf_score_kernel(IndexArgs A, PfWs W, int KC) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_red[4];
  __shared__ int s_q[3];                // query exponent summary: min, max, largest per-(row, head) spread
  __shared__ int s_bad;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int b = blockIdx.z, kc = blockIdx.y;
  const int t = blockIdx.x * PF_QROWS + wave * 16 + c;
  const bool rv = t < A.Tq;
  const int64_t r = (int64_t)b * A.Tq + (rv ? t : 0);
  const int nq = rv ? idx_nelig(A, r) : 0;
  const float thr = rv ? W.thr[r] : __builtin_inff();
  int nmax = nq;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nmax = max(nmax, __shfl_xor(nmax, o, WAVE));
  if (threadIdx.x == 0) { s_q[0] = 1 << 20; s_q[1] = -1; s_q[2] = 0; s_bad = 0; }
  if (lane == 0) s_red[wave] = nmax;
  __syncthreads();
  nmax = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
  const int j0 = kc * KC;
  const int j1 = min(j0 + KC, nmax);
  if (j0 >= j1) return;                 // uniform: no row of this workgroup reaches the range

  PfQuery<HP> P;
  bool wneg;
  pf_load_query<HP>(A, rv, r, P, wneg);
  {
    // exponent envelope of the workgroup's query operands
    int qmin = 1 << 20, qmax = -1, dq = 0;
#pragma unroll
    for (int h = 0; h < HP; ++h) {
      if (!(rv && h < A.H)) continue;
      int mn = P.sb[h], mx = P.sb[h];
      mn = min(mn, __shfl_xor(mn, 16, WAVE)); mx = max(mx, __shfl_xor(mx, 16, WAVE));
      mn = min(mn, __shfl_xor(mn, 32, WAVE)); mx = max(mx, __shfl_xor(mx, 32, WAVE));
      qmin = min(qmin, mn); qmax = max(qmax, mx); dq = max(dq, mx - mn);
    }
    atomicMin(&s_q[0], qmin);
    atomicMax(&s_q[1], qmax);
    atomicMax(&s_q[2], dq);
  }
  const int nlim = min(nq, j1);
  int nlim_min = rv ? nlim : 1 << 30;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nlim_min = min(nlim_min, __shfl_xor(nlim_min, o, WAVE));
  nlim_min = __builtin_amdgcn_readfirstlane(nlim_min);
  // candidate lists of the wave's 16 rows: uniform base + 32-bit lane offset
  const int64_t r0 = (int64_t)b * A.Tq + blockIdx.x * PF_QROWS + wave * 16;
  char* wlist = (char*)(W.cand + (r0 * PF_NKC + kc) * 4 * PF_LCAP);
  const uint32_t lane_off = (uint32_t)(((c * PF_NKC) * 4 + g) * PF_LCAP) * 8u;
  uint64_t* const lp = (uint64_t*)(wlist + lane_off);   // this lane's list
  uint32_t cnt = 0;

  const int nst = (j1 - j0 + PF_STAGE - 1) / PF_STAGE;
  const uint8_t* kbase = (const uint8_t*)A.ki + (int64_t)b * A.N_cap * 64;
  const uint8_t* sbase = A.ki_scale + (int64_t)b * A.N_cap * 4;
  // direct global -> LDS loads of one stage: codes in tile-major, block-major
  // order (chunk = (tile*4 + block)*16 + key), then the 4 scale bytes per key
  auto issue = [&](int st) {
    const int sj = j0 + st * PF_STAGE;
    char* base = smem + (st & 1) * PF_STAGE_B;
#pragma unroll
    for (int u = 0; u < PF_STAGE / 64; ++u) {
      const int ci = wave * PF_STAGE + u * 64 + lane;
      const int tile = ci >> 6, blk = (ci >> 4) & 3, kt = ci & 15;
      const int j = min(sj + tile * 16 + kt, (int)A.N_cap - 1);
      __builtin_amdgcn_global_load_lds((const void*)(kbase + (int64_t)j * 64 + blk * 16),
                                       (void*)(base + (wave * PF_STAGE + u * 64) * 16), 16, 0, 0);
    }
    if (wave * 64 + lane < PF_STAGE / 4) {      // 16 bytes = the scales of 4 keys a lane
      const int j = min(sj + 4 * (wave * 64 + lane), (int)A.N_cap - 4);
      __builtin_amdgcn_global_load_lds((const void*)(sbase + (int64_t)j * 4),
                                       (void*)(base + PF_CODE_B + wave * 64 * 16), 16, 0, 0);
    }
  };

  issue(0);
#pragma unroll 1
  for (int st = 0; st < nst; ++st) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (st + 1 < nst) issue(st + 1);
    const int sj = j0 + st * PF_STAGE;
    const char* base = smem + (st & 1) * PF_STAGE_B;
    const int nk = min(PF_STAGE, j1 - sj);
    {
      // exactness envelope of this stage's keys against the workgroup's queries
      const int qmin = s_q[0], qmax = s_q[1], dq = s_q[2];
      int bad = 0;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int key = u * 256 + threadIdx.x;
        if (key < nk) {
          const uint32_t w4 = *(const uint32_t*)(base + PF_CODE_B + key * 4);
          const int e0 = w4 & 255, e1 = (w4 >> 8) & 255, e2 = (w4 >> 16) & 255, e3 = w4 >> 24;
          const int kmin = min(min(e0, e1), min(e2, e3)), kmax = max(max(e0, e1), max(e2, e3));
          bad |= (dq + kmax - kmin > 9) || (qmin + kmin < 130) || (qmax + kmax > 368);
        }
      }
      if (bad) s_bad = 1;
    }
    const int ntl = (nk + 15) / 16;
    // A operand of tile tt from LDS: lane = key c of the tile, K-block g
    auto frag = [&](int tt, v8i& a8, int& ka) {
      const v4i av = *(const v4i*)(base + ((tt * 4 + g) * 16 + c) * 16);
      a8 = (v8i){av[0], av[1], av[2], av[3], 0, 0, 0, 0};
      ka = (int)(uint8_t)base[PF_CODE_B + (tt * 16 + c) * 4 + g];
    };
    auto mfma = [&](const v8i& a8, int ka, v4f (&acc)[HP]) {
#pragma unroll
      for (int h = 0; h < HP; ++h) {
        const v4f z = {0.f, 0.f, 0.f, 0.f};
        acc[h] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, P.bq[h], z, 4, 4, 0, ka, 0, P.sb[h]);
      }
    };
    auto epilogue = [&](const v4f (&acc)[HP], int tt) {
      float sc[4];
      pf_combine<HP>(acc, P, sc);
      const int jt = sj + tt * 16;
      const uint32_t jb = (uint32_t)(jt + 4 * g);    // this lane's first key of the tile
      // an overflowing list sends the row to the fallback: clamping the slot is enough
      auto put = [&](int i) {
        lp[min(cnt, (uint32_t)PF_LCAP - 1u)] = ((uint64_t)__float_as_uint(sc[i]) << 32) | (jb + (uint32_t)i);
        ++cnt;
      };
      if (jt + 16 <= nlim_min) {
        // (uniform) every key of the tile is eligible for every row: the
        // threshold alone decides
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (sc[i] >= thr) put(i);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (sc[i] >= thr && jt + 4 * g + i < nlim) put(i);
      }
    };
    // software pipeline: the next tile's fragment is read from LDS and its
    // MFMAs issued before this tile's combine and filter run on the vector ALU
    v8i fa, fb;
    int ka, kb2;
    v4f accA[HP], accB[HP];
    frag(0, fa, ka);
    if (ntl > 1) frag(1, fb, kb2);
    mfma(fa, ka, accA);
#pragma unroll 1
    for (int tt = 0; tt < ntl; tt += 2) {
      if (tt + 1 < ntl) mfma(fb, kb2, accB);
      if (tt + 2 < ntl) frag(tt + 2, fa, ka);
      __builtin_amdgcn_sched_barrier(0);
      epilogue(accA, tt);
      __builtin_amdgcn_sched_barrier(0);
      if (tt + 1 < ntl) {
        if (tt + 2 < ntl) mfma(fa, ka, accA);
        if (tt + 3 < ntl) frag(tt + 3, fb, kb2);
        __builtin_amdgcn_sched_barrier(0);
        epilogue(accB, tt + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __syncthreads();
  if (rv) {
    W.cnt[(r * PF_NKC + kc) * 4 + g] = (int)min(cnt, (uint32_t)PF_LCAP + 1u);
    if (s_bad && g == 0) atomicOr(&W.flags[r], 2);
  }
}

// ------------------------------------------------------------------------
// Select pass: one workgroup of PS_NW wavefronts per row.  The candidate
// lists are gathered into LDS, every thread holds PS_CPT of them in
// registers (item tid + PS_NT*m), and the phases -- radix select of the
// fp32 threshold, certification, band re-score, ascending emission through a
// bitmap over [0, n) -- are split over the workgroup; the band re-score (at
// most 64 entries) is wavefront 0's.  Every decision is the same in every
// wavefront (all read the same LDS), so the exits are uniform.
// ------------------------------------------------------------------------
constexpr int PS_NW = 4;
constexpr int PS_NT = PS_NW * 64;
constexpr int PS_CPT = PF_CAND / PS_NT;   // candidates per thread
static_assert(PS_CPT * PS_NT == PF_CAND, "candidates split evenly");

struct PfSelShared {
  uint32_t cs[PF_CAND];     // candidate scores (fp32 bits); then the MFMA transpose
                            // buffer, then the bitmap (the scores live in registers)
  int32_t cj[PF_CAND];      // candidate indices; later the output list
  uint32_t hist[256];
  float wl[32];
  int32_t bj[PF_BAND];
  uint32_t rmax[PS_NW], rmin[PS_NW];
  int nin, nband, wsum[PS_NW];
};
static_assert(sizeof(float) * WBUF <= sizeof(uint32_t) * PF_CAND, "transpose buffer fits the score array");
constexpr int PF_BM_BITS = PF_CAND * 32;   // entries one bitmap pass of the emission covers

template <int HP>
__global__ __launch_bounds__(PS_NT) void pf_select_kernel(IndexArgs A, PfWs W, int KC) {
  extern __shared__ __align__(16) char smem[];
  PfSelShared& L = *(PfSelShared*)smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t r = blockIdx.x;
  const int n = idx_nelig(A, r);
  const int kk = min(n, A.k);
  int32_t* out = A.idx_out + r * A.k;
  double* sout = A.score_out ? A.score_out + r * A.k : nullptr;
  auto enqueue = [&]() {
    if (tid == 0) {
      const int p = atomicAdd(&W.queue[0], 1);
      W.queue[1 + p] = (int)r;
    }
  };
  if (n <= A.k) {
    for (int i = tid; i < A.k; i += PS_NT) out[i] = i < n ? i : -1;
    if (sout) enqueue();                  // scores of every entry: the fallback computes them
    return;
  }
  if (W.flags[r] != 0) { enqueue(); return; }
  // list counts and offsets: the same in every wavefront
  const int nl = ((n + KC - 1) / KC) * 4;                 // lists (key range, lane group)
  const int cl = lane < nl ? W.cnt[r * PF_NKC * 4 + lane] : 0;
  if (__ballot(cl > PF_LCAP)) { enqueue(); return; }
  const int incl = wave_incl_scan_dpp(cl);
  const int total = __shfl(incl, 63, WAVE);
  if (total > PF_CAND || total < kk) { enqueue(); return; }
  const int loff = incl - cl;
  // gather the lists into LDS with direct global->LDS dword loads: the high
  // halves (scores) into cs, the low halves (indices) into cj, every list at
  // its flat offset; wavefront w takes lists w, w + PS_NW, ...
  const uint32_t* lw = (const uint32_t*)(W.cand + r * PF_NKC * 4 * PF_LCAP);
#pragma unroll 1
  for (int Lx = wave; Lx < nl; Lx += PS_NW) {
    const int cn = __builtin_amdgcn_readlane(cl, Lx);
    const int o = __builtin_amdgcn_readlane(loff, Lx);
    const uint32_t* src = lw + (int64_t)Lx * PF_LCAP * 2;
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      if (e2 * 64 >= cn) break;
      const int e = lane + 64 * e2;
      if (e < cn) {
        __builtin_amdgcn_global_load_lds((const void*)(src + 2 * e), (void*)(L.cj + o + 64 * e2), 4, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(src + 2 * e + 1), (void*)(L.cs + o + 64 * e2), 4, 0, 0);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t sv[PS_CPT];
#pragma unroll
  for (int m = 0; m < PS_CPT; ++m) {
    const int i = tid + PS_NT * m;
    sv[m] = i < total ? L.cs[i] : 0u;
  }
  // exact radix select (8-bit digits) of the kk-th largest s32, from the first
  // byte where the largest and smallest candidate differ
  uint32_t vmax = 0, vmin = ~0u;
#pragma unroll
  for (int m = 0; m < PS_CPT; ++m) {
    if (tid + PS_NT * m < total) { vmax = max(vmax, sv[m]); vmin = min(vmin, sv[m]); }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    vmax = max(vmax, (uint32_t)__shfl_xor((int)vmax, o, WAVE));
    vmin = min(vmin, (uint32_t)__shfl_xor((int)vmin, o, WAVE));
  }
  if (lane == 0) { L.rmax[wave] = vmax; L.rmin[wave] = vmin; }
  for (int i = tid; i < 256; i += PS_NT) L.hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < PS_NW; ++w) { vmax = max(vmax, L.rmax[w]); vmin = min(vmin, L.rmin[w]); }
  const int top = vmax == vmin ? 0 : (31 - __clz(vmax ^ vmin)) / 8 * 8;
  uint32_t mask = top == 24 ? 0u : ~((1u << (top + 8)) - 1u);
  uint32_t prefix = vmax & mask;
  int rem = kk;
#pragma unroll 1
  for (int shift = top; shift >= 0; shift -= 8) {
#pragma unroll
    for (int m = 0; m < PS_CPT; ++m) {
      const int i = tid + PS_NT * m;
      if (i < total && (sv[m] & mask) == prefix) atomicAdd(&L.hist[(sv[m] >> shift) & 255u], 1u);
    }
    __syncthreads();
    // every wavefront finds the same digit from the same histogram
    int above;
    const int d = pf_hist_digit(L.hist, rem, &above);
    rem -= above;
    prefix |= (uint32_t)d << shift;
    mask |= 255u << shift;
    __syncthreads();
    if (shift > 0)
      for (int i = tid; i < 256; i += PS_NT) L.hist[i] = 0;
    __syncthreads();
  }
  const double eps = (double)(A.H + 1) * 0x1p-24 * 1.001;
  const double Td = (double)__uint_as_float(prefix);
  const double t = (double)W.thr[r];
  if (!(Td * (1.0 - eps) >= t * (1.0 + eps))) { enqueue(); return; }
  const double hi = Td * (1.0 + eps) / (1.0 - eps);
  const double lo = Td * (1.0 - eps) / (1.0 + eps);
  // definitely-in count and the band (its order does not matter: the band
  // is ranked by (score, index) and emitted through the bitmap)
  if (tid == 0) { L.nin = 0; L.nband = 0; }
  __syncthreads();
  int nin = 0;
#pragma unroll
  for (int m = 0; m < PS_CPT; ++m) {
    const int i = tid + PS_NT * m;
    const double x = (double)__uint_as_float(sv[m]);
    const bool valid = i < total;
    nin += __popcll(__ballot(valid && x > hi));
    const bool inb = valid && x >= lo && x <= hi;
    const uint64_t bm = __ballot(inb);
    if (bm) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&L.nband, __popcll(bm));
      base = __shfl(base, 0, WAVE);
      if (inb) {
        const int p = base + lanes_below(bm);
        if (p < PF_BAND) L.bj[p] = L.cj[i];
      }
    }
  }
  if (lane == 0) atomicAdd(&L.nin, nin);
  if (lane < 32 && wave == 0) L.wl[lane] = lane < A.H ? A.w[r * A.H + lane] : 0.f;
  __syncthreads();
  const int nband = L.nband;
  nin = L.nin;
  const int need = kk - nin;
  if (nband > PF_BAND || need < 1 || need > nband) { enqueue(); return; }
  // exact scores of the band, wavefront 0 (MFMA dots are exact here: the
  // score pass checked the envelope; a key outside it would have flagged the row)
  Rows rw;
  rw.b = (int)(r / A.Tq);
  rw.r[0] = (int)r; rw.r[1] = -1;
  rw.n[0] = nband; rw.n[1] = 0;
  MxQuery Q;
  int jm = 0;
  bool bsel = false;
  if (wave == 0) {
    mx_load_query<HP>(A, rw, Q);
    jm = lane < nband ? L.bj[lane] : 0;
    uint64_t key;
    {
      MxTiles T;
      bool ix;
      MxW<HP, 1> Wt;
      mx_load_weights<HP, 1>(L.wl, Wt);
      mx_load_gather(A, rw.b, jm, nband, T);
      mx_score_round<HP, 1>(A, rw, Q, T, 0, (float*)L.cs, Wt, &key, ix);
      if (ix) key = mx_score_exact(A, (int)r, rw.b, jm, L.wl);
      if (lane >= nband) key = 0;
    }
    int rank = 0;
#pragma unroll 1
    for (int e = 0; e < nband; ++e) {
      const uint64_t ke = ((uint64_t)readlane_u32((uint32_t)(key >> 32), e) << 32) | readlane_u32((uint32_t)key, e);
      const int je = (int)readlane_u32((uint32_t)jm, e);
      rank += (ke > key) || (ke == key && je < jm);
    }
    bsel = lane < nband && rank < need;
  }
  // the candidates' indices in registers: the emission below writes the
  // output list over L.cj
  int32_t cjv[PS_CPT];
#pragma unroll
  for (int m = 0; m < PS_CPT; ++m) {
    const int i = tid + PS_NT * m;
    cjv[m] = (i < total && (double)__uint_as_float(sv[m]) > hi) ? L.cj[i] : -1;
  }
  __syncthreads();                        // the transpose buffer becomes the bitmap
  // ascending emission through a bitmap over [0, n), PF_BM_BITS entries at a
  // time (the bitmap lives in the score array)
  uint32_t* bitmap = L.cs;
  int32_t* outl = L.cj;
  int written = 0;
#pragma unroll 1
  for (int seg0 = 0; seg0 < n; seg0 += PF_BM_BITS) {
    const int nw = (min(n - seg0, PF_BM_BITS) + 31) >> 5;
    for (int i = tid; i < nw; i += PS_NT) bitmap[i] = 0;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < PS_CPT; ++m) {
      const int j = cjv[m] - seg0;
      if (cjv[m] >= 0 && j >= 0 && j < PF_BM_BITS) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
    }
    if (bsel && jm >= seg0 && jm - seg0 < PF_BM_BITS) atomicOr(&bitmap[(jm - seg0) >> 5], 1u << ((jm - seg0) & 31));
    __syncthreads();
    // thread t owns words [t*wpt, (t+1)*wpt); the workgroup scan of their
    // counts gives each its first output position
    const int wpt = (nw + PS_NT - 1) / PS_NT;
    const int w0 = tid * wpt, w1 = min(nw, w0 + wpt);
    int mine = 0;
    for (int w = w0; w < w1; ++w) mine += __popc(bitmap[w]);
    const int winc = wave_incl_scan_dpp(mine);
    if (lane == 63) L.wsum[wave] = winc;
    __syncthreads();
    int pos = written + winc - mine;
    int segtot = 0;
    for (int w = 0; w < PS_NW; ++w) {
      if (w < wave) pos += L.wsum[w];
      segtot += L.wsum[w];
    }
    for (int w = w0; w < w1; ++w) {
      uint32_t bits = bitmap[w];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        if (pos < A.k) {
          out[pos] = seg0 + w * 32 + bit;
          if (sout) outl[pos] = seg0 + w * 32 + bit;
        }
        ++pos;
      }
    }
    written += segtot;
    __syncthreads();                      // the bitmap and the sums are reused
  }
  if (sout) {
    // exact scores of every selected entry, 64 at a time, wavefront 0
    __syncthreads();
    if (wave == 0) {
#pragma unroll 1
      for (int i0 = 0; i0 < kk; i0 += 64) {
        const int cntr = min(64, kk - i0);
        const int je = lane < cntr ? outl[i0 + lane] : 0;
        rw.n[0] = cntr;
        MxTiles T;
        bool ix;
        uint64_t k2;
        MxW<HP, 1> Wt;
        mx_load_weights<HP, 1>(L.wl, Wt);
        mx_load_gather(A, rw.b, je, cntr, T);
        mx_score_round<HP, 1>(A, rw, Q, T, 0, (float*)L.cs, Wt, &k2, ix);
        if (ix) k2 = mx_score_exact(A, (int)r, rw.b, je, L.wl);
        if (lane < cntr) sout[i0 + lane] = key_score(k2);
      }
    }
  }
}

// ------------------------------------------------------------------------
// Fallback pass: rows queued by the select pass, selected exactly by
// re-scoring every entry (one 1024-thread workgroup per row).
// ------------------------------------------------------------------------
template <int HP>
__global__ __launch_bounds__(SEL_THREADS) void pf_fallback_kernel(IndexArgs A, PfWs W) {
  extern __shared__ __align__(16) char smem[];
  SelShared& S = *(SelShared*)smem;
  char* region = smem + sizeof(SelShared);
  float* tbuf = (float*)region;
  float* wl = (float*)(region + 12 * CMAX);
  const int qn = W.queue[0];
#pragma unroll 1
  for (int i = PF_QFAST + blockIdx.x; i < qn; i += gridDim.x) {
    const int r = W.queue[1 + i];
    __syncthreads();
    if (threadIdx.x < 32) wl[threadIdx.x] = (threadIdx.x < (unsigned)A.H) ? A.w[(int64_t)r * A.H + threadIdx.x] : 0.f;
    __syncthreads();
    const int n = idx_nelig(A, r);
    const int kk = n < A.k ? n : A.k;
    int32_t* out = A.idx_out + (int64_t)r * A.k;
    double* sout = A.score_out ? A.score_out + (int64_t)r * A.k : nullptr;
    select_streamed<DT_MXFP4, HP>(A, r, n, kk, out, sout, S, tbuf, wl, nullptr, n <= A.k);
  }
}

// The queued row r as a call of one sequence with one query row (the decode
// scan and select read the row through it).
__device__ __forceinline__ IndexArgs pf_row_view(const IndexArgs& A, int64_t r) {
  IndexArgs v = A;
  const int64_t b = r / A.Tq;
  v.B = 1;
  v.Tq = 1;
  v.qi = (const uint8_t*)A.qi + r * A.H * (A.d / 2);
  v.qi_scale = A.qi_scale + r * A.H * (A.d / 32);
  v.w = A.w + r * A.H;
  v.n_elig = A.n_elig + r;
  v.ki = (const uint8_t*)A.ki + b * A.N_cap * (A.d / 2);
  v.ki_scale = A.ki_scale + b * A.N_cap * (A.d / 32);
  v.idx_out = A.idx_out + r * A.k;
  v.score_out = A.score_out ? A.score_out + r * A.k : nullptr;
  return v;
}

// Chunk c of queued row g (g < PF_QFAST; slots past the queue exit at once).
template <int KPL, int HP>
__global__ __launch_bounds__(256) void pf_qscan_kernel(IndexArgs A, PfWs W, size_t slot, int NCH) {
  __shared__ ChunkShared<1> sm;
  const int g = blockIdx.y;
  if (g >= min(W.queue[0], PF_QFAST)) return;
  const IndexArgs v = pf_row_view(A, W.queue[1 + g]);
  index_chunk_body<DT_MXFP4, KPL, HP, 1>(v, carve(W.qws + g * slot, 1, NCH), NCH, 1, blockIdx.x, 0, sm);
}

// The selection of queued row g over its chunks' candidates.
template <int HP>
__global__ __launch_bounds__(SEL_THREADS) void pf_qselect_kernel(IndexArgs A, PfWs W, size_t slot, int NCH, int CH) {
  extern __shared__ __align__(16) char smem[];
  const int g = blockIdx.x;
  if (g >= min(W.queue[0], PF_QFAST)) return;
  const IndexArgs v = pf_row_view(A, W.queue[1 + g]);
  index_select_body<DT_MXFP4, HP>(v, carve(W.qws + g * slot, 1, NCH), NCH, CH, 0, smem);
}

// ------------------------------------------------------------------------
template <int HP>
static hipError_t launch_pf(const IndexArgs& a, hipStream_t s) {
  const int64_t R = (int64_t)a.B * a.Tq;
  PfWs W = pf_carve(a.ws, R);
  const int sigma = pf_sigma(a);
  const int smax = (int)((a.N_cap + sigma - 1) / sigma);
  // a row's samples, padded by 8 dwords: the 16 rows' stores of one tile then
  // spread evenly over the LDS banks
  const int srow = (smax + 63) / 64 * 64 + PF_SPAD;
  const int KC = pf_key_range(a);
  const int sr = pf_sample_rows(srow);
  const size_t smem0 = (size_t)sr * srow * 2 + PF_SWAVES * 256 * 4;
  hipLaunchKernelGGL((pf_sample_kernel<HP>), dim3((unsigned)((a.Tq + sr - 1) / sr), (unsigned)a.B),
                     dim3(PF_SWAVES * 64), smem0, s, a, W, sigma, srow, sr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((pf_score_kernel<HP>), dim3((unsigned)((a.Tq + PF_QROWS - 1) / PF_QROWS), PF_NKC, (unsigned)a.B),
                     dim3(256), (size_t)2 * PF_STAGE_B, s, a, W, KC);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((pf_select_kernel<HP>), dim3((unsigned)R), dim3(PS_NT), sizeof(PfSelShared), s, a, W, KC);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // the first PF_QFAST queued rows: decode scan (when the rows are long
  // enough to use it) and select
  const PfQPlan q = pf_qplan(a.N_cap, a.k);
  const int qn = (int)(R < PF_QFAST ? R : PF_QFAST);
  if (a.N_cap > NDIRECT) {
    const dim3 qg((unsigned)q.NCH, (unsigned)qn);
    switch (q.kpl) {
      case 32: hipLaunchKernelGGL((pf_qscan_kernel<32, HP>), qg, dim3(256), 0, s, a, W, q.slot, q.NCH); break;
      case 16: hipLaunchKernelGGL((pf_qscan_kernel<16, HP>), qg, dim3(256), 0, s, a, W, q.slot, q.NCH); break;
      default: hipLaunchKernelGGL((pf_qscan_kernel<4, HP>), qg, dim3(256), 0, s, a, W, q.slot, q.NCH); break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((pf_qselect_kernel<HP>), dim3((unsigned)qn), dim3(SEL_THREADS), select_smem(a.dt, a.H, a.d), s, a,
                     W, q.slot, q.NCH, 64 * q.kpl);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned fg = (unsigned)(R < PF_FALLBACK_GRID ? R : PF_FALLBACK_GRID);
  hipLaunchKernelGGL((pf_fallback_kernel<HP>), dim3(fg), dim3(SEL_THREADS), select_smem(a.dt, a.H, a.d), s, a, W);
  return hipGetLastError();
}

hipError_t launch_index_prefill(const IndexArgs& a, hipStream_t s) {
  return a.H <= 8 ? launch_pf<8>(a, s) : launch_pf<16>(a, s);
}

}  // namespace lca
