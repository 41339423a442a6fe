// index_chunk.h -- the decode scan of the lightning indexer (one workgroup per
// chunk of keys and query-row group) and its workspace layout, shared by the
// indexer kernels and the fused decode-step kernel.  The method and its
// sources are described in index.hip.
#pragma once
#include "index_common.h"

namespace lca {

struct IdxWs {
  int32_t* cnt;   // [R][NCH] candidates emitted by each chunk (-1: overflow)
  uint64_t* mex;  // [R][NCH] largest key a chunk did not emit (0: none)
  uint64_t* cmax; // [R][NCH] largest key of a chunk
  uint64_t* cthr; // [R][NCH] emission threshold of a chunk (every candidate >= it)
  uint64_t* ckey; // [R][NCH][CAP] candidates, ascending index within a chunk
  int32_t* cidx;  // [R][NCH][CAP]
};

__host__ __device__ inline IdxWs carve(void* ws, int64_t R, int64_t NCH) {
  IdxWs w;
  char* p = (char*)ws;
  w.cnt = (int32_t*)p; p += align256(sizeof(int32_t) * R * NCH);
  w.mex = (uint64_t*)p; p += align256(sizeof(uint64_t) * R * NCH);
  w.cmax = (uint64_t*)p; p += align256(sizeof(uint64_t) * R * NCH);
  w.cthr = (uint64_t*)p; p += align256(sizeof(uint64_t) * R * NCH);
  w.ckey = (uint64_t*)p; p += align256(sizeof(uint64_t) * R * NCH * CAP);
  w.cidx = (int32_t*)p;
  return w;
}

inline size_t carve_bytes(int64_t R, int64_t NCH) {
  return align256(sizeof(int32_t) * R * NCH) + 3 * align256(sizeof(uint64_t) * R * NCH) +
         align256(sizeof(uint64_t) * R * NCH * CAP) + align256(sizeof(int32_t) * R * NCH * CAP);
}

// A key row that the scan takes from elsewhere than the key cache (j < 0:
// none): the decode step computes the row its own compress job writes in the
// same launch, and hands the scan that copy (codes and scale bytes, any
// address space).
struct FreshKey {
  int j;
  const uint8_t* code;
  const uint8_t* sc;
};

// Replace, in a round of key tiles loaded for entries [j0, j0 + 64), the
// operands of entry F.j (the same per-lane layout as mx_load_round).
__device__ __forceinline__ void mx_patch_round(MxTiles& T, int j0, int jlim, const FreshKey& F, int d) {
  const int lane = threadIdx.x & 63;
  const int kb = lane >> 4;
  const uint32_t kbc = kb * 32 < d ? kb : 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (min(j0 + t * 16 + (lane & 15), jlim - 1) == F.j) {
      T.code[t] = *(const int4*)(F.code + kbc * 16);
      T.sc[t] = F.sc[kbc];
    }
  }
  if (min(j0 + lane, jlim - 1) == F.j) T.kscale = mx_scale_word(F.sc, d);
}

template <int NQ>
struct ChunkShared {
  __align__(16) float tbuf[4][WBUF];
  float wl[32];
  uint64_t lists[NQ][4][64];
  int wcnt[NQ][4];
  uint64_t wmex[NQ][4];
  uint64_t thr_s[NQ], top_s[NQ];
};

// Rounds of key tiles a wavefront keeps in flight (each round: 64 keys, 21
// registers per lane): the decode scan is bound by memory latency, so the
// deeper the ring the closer to the HBM rate.
constexpr int SCAN_DEPTH = 2;
constexpr int scan_depth(int KPL, int NQ) {
  const int d = NQ == 1 ? SCAN_DEPTH : 2;
  return d < KPL / 4 ? d : (KPL / 4 < 2 ? 2 : KPL / 4);
}

// Chunk c of query-row group g: one workgroup of 256 threads.
template <int DT, int KPL, int HP, int NQ>
__device__ __forceinline__ void index_chunk_body(const IndexArgs& A, const IdxWs& W, int NCH, int groups_per_b,
                                                 int c, int g, ChunkShared<NQ>& sm,
                                                 const FreshKey& F = FreshKey{-1, nullptr, nullptr}) {
  constexpr int CH = 64 * KPL;
  constexpr int RPW = KPL / 4;            // rounds per wavefront
  static_assert(KPL % 4 == 0, "four wavefronts share a chunk");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  auto& tbuf = sm.tbuf;
  float* wl = sm.wl;
  auto& lists = sm.lists;
  auto& wcnt = sm.wcnt;
  auto& wmex = sm.wmex;
  auto& thr_s = sm.thr_s;
  auto& top_s = sm.top_s;

  Rows rw;
  rw.b = g / groups_per_b;
  const int t0 = (g % groups_per_b) * NQ;
  rw.r[0] = rw.b * A.Tq + t0;
  rw.r[1] = (NQ == 2 && t0 + 1 < A.Tq) ? rw.r[0] + 1 : -1;
  // everything that does not depend on the row lengths is requested before
  // they arrive, in a fixed order: row lengths, head weights, the query
  // operand, then the first round of key tiles (rows up to N_cap exist, and
  // entries past a row's length are discarded by the eligibility test)
  rw.n[0] = idx_nelig(A, rw.r[0]);
  rw.n[1] = idx_nelig(A, rw.r[1] >= 0 ? rw.r[1] : rw.r[0]);
  const int wq = (threadIdx.x >> 4) & 1, wh = threadIdx.x & 15;
  const int rwq = wq == 0 ? rw.r[0] : rw.r[1];    // (no dynamic indexing: keeps rw in registers)
  const int wrow = (wq < NQ && rwq >= 0) ? rwq : rw.r[0];
  const float wv = A.w[(int64_t)wrow * A.H + (wh < A.H ? wh : 0)];
  MxQueryRaw QR{};
  if (DT == DT_MXFP4) QR = mx_query_issue<HP>(A, rw);
  const int jbeg = c * CH;                  // < N_cap: the grid covers N_cap
  const int jl = min((int)A.N_cap, jbeg + CH);
  const int jw = jbeg + wave * RPW * 64;    // this wavefront's first entry
  MxRows R{};
  // SD rounds of key tiles in flight per wavefront (a ring of stages; all
  // indices are compile-time constants once the round loop is unrolled)
  constexpr int SD = scan_depth(KPL, NQ);
  MxTiles st[SD];
  if (DT == DT_MXFP4) {
    R = mx_rows(A, rw.b, min(jw, jl - 1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i + 1 < SD; ++i) mx_load_round(A, R, min(jw + i * 64, jl), jl, st[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (rw.r[1] < 0) rw.n[1] = 0;
  // rows with few entries are done by the select kernel alone
  if (rw.n[0] <= NDIRECT) rw.n[0] = 0;
  if (rw.n[1] <= NDIRECT) rw.n[1] = 0;
  const int jlim = max(rw.n[0], rw.n[1]);
  if (jbeg >= jlim) return;                 // uniform over the workgroup

  if (threadIdx.x < 32) wl[threadIdx.x] = (wq < NQ && rwq >= 0 && wh < A.H) ? wv : 0.f;
  __syncthreads();

  uint64_t kq[NQ][RPW];
  if (DT == DT_MXFP4) {
    MxQuery Q;
    mx_query_finish(QR, Q);
    MxW<HP, NQ> Wt;
    mx_load_weights<HP, NQ>(wl, Wt);
    // the round SD-1 ahead loads while this one is scored
    uint32_t fix = 0;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      uint64_t kk[NQ];
      bool ix;
      if (rr + SD - 1 < RPW) mx_load_round(A, R, min(jw + (rr + SD - 1) * 64, jl), jl, st[(rr + SD - 1) % SD]);
      MxTiles& cur = st[rr % SD];
      if (F.j >= jw + rr * 64 && F.j < jw + rr * 64 + 64) mx_patch_round(cur, min(jw + rr * 64, jl), jl, F, A.d);
      mx_score_round<HP, NQ>(A, rw, Q, cur, jw + rr * 64, tbuf[wave], Wt, kk, ix);
#pragma unroll
      for (int q = 0; q < NQ; ++q) kq[q][rr] = kk[q];
      fix |= __ballot(ix) ? 1u << rr : 0u;
    }
    if (fix) {
      // rare: keys outside the exact-MFMA envelope, re-scored in float64
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        if (!((fix >> rr) & 1u)) continue;
        const int j = jw + rr * 64 + lane;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          if (kq[q][rr] == 0) continue;
          const bool fresh = j == F.j;
          const uint8_t* ks = fresh ? F.sc : A.ki_scale + ((int64_t)rw.b * A.N_cap + j) * (A.d / 32);
          int kmin = 1000, kmax = -1000;
          for (int i = 0; i < A.d / 32; ++i) { kmin = min(kmin, (int)ks[i]); kmax = max(kmax, (int)ks[i]); }
          if (!mx_exact(Q, kmin, kmax))
            kq[q][rr] = fresh ? mx_score_exact_row(A, rw.r[q], F.code, F.sc, wl + q * 16)
                              : mx_score_exact(A, rw.r[q], rw.b, j, wl + q * 16);
        }
      }
    }
  } else {
    const float* qrow = (const float*)A.qi + (int64_t)rw.r[0] * A.H * A.d;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) f32_score_round(A, rw, jw + rr * 64, qrow, wl, kq[0][rr]);
  }

  // chunk threshold per row from the 256 lane maxima
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    uint64_t lmax = 0;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) lmax = kq[q][rr] > lmax ? kq[q][rr] : lmax;
    lists[q][wave][lane] = wave_sort_desc(lmax);
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      uint64_t cur = lists[q][0][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const uint64_t o = lists[q][w][63 - lane];
        cur = wave_bitonic_clean_desc(cur > o ? cur : o);
      }
      const int n = rw.n[q];
      const float lam = n > 0 ? (float)A.k * (float)CH / (float)n : 0.f;
      int rsel = (int)ceilf(lam + 5.0f * sqrtf(lam) + 6.0f);
      rsel = rsel > 64 ? 64 : (rsel < 1 ? 1 : rsel);
      const uint64_t thr = ((uint64_t)readlane_u32((uint32_t)(cur >> 32), rsel - 1) << 32) |
                           readlane_u32((uint32_t)cur, rsel - 1);
      const uint64_t top = ((uint64_t)readlane_u32((uint32_t)(cur >> 32), 0) << 32) | readlane_u32((uint32_t)cur, 0);
      if (lane == 0) { thr_s[q] = thr == 0 ? 1 : thr; top_s[q] = top; }   // key 0 marks "no entry"
    }
  }
  __syncthreads();
  // counts and the best excluded key per wavefront
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const uint64_t thr = thr_s[q];
    int cnt = 0;
    uint64_t ex = 0;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const bool f = kq[q][rr] >= thr;
      cnt += __popcll(__ballot(f));
      if (!f && kq[q][rr] > ex) ex = kq[q][rr];
    }
    ex = wave_max_u64_dpp(ex);
    if (lane == 0) { wcnt[q][wave] = cnt; wmex[q][wave] = ex; }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (rw.r[q] < 0 || rw.n[q] == 0 || jbeg >= rw.n[q]) continue;
    const int64_t slot = (int64_t)rw.r[q] * NCH + c;
    const int total = wcnt[q][0] + wcnt[q][1] + wcnt[q][2] + wcnt[q][3];
    if (total > CAP) {
      if (threadIdx.x == 0) { W.cnt[slot] = -1; W.mex[slot] = ~0ull; }
      continue;
    }
    const uint64_t thr = thr_s[q];
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wcnt[q][w];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const bool f = kq[q][rr] >= thr;
      const uint64_t bal = __ballot(f);
      if (f) {
        const int pos = base + lanes_below(bal);
        W.ckey[slot * CAP + pos] = kq[q][rr];
        W.cidx[slot * CAP + pos] = jw + rr * 64 + lane;
      }
      base += __popcll(bal);
    }
    if (threadIdx.x == 0) {
      uint64_t m = wmex[q][0];
      for (int w = 1; w < 4; ++w) m = wmex[q][w] > m ? wmex[q][w] : m;
      W.cnt[slot] = total;
      W.mex[slot] = m;
      W.cmax[slot] = top_s[q];
      W.cthr[slot] = thr;
    }
  }
}

// Rows per wavefront: two query rows share the MFMA A operand when the heads
// fit in 8 rows and there is more than one query per sequence.
inline int nq_of(int dt, int H, int Tq) { return (dt == DT_MXFP4 && H <= 8 && Tq > 1) ? 2 : 1; }

inline int choose_kpl(const IndexArgs& a, int nq) {
  // the largest chunk (fewer candidates for the select kernel) that still
  // gives at least 2048 wavefronts and keeps the expected top-k count of a
  // full-length chunk (lambda) low enough for the per-chunk rank to stay <= 64
  const int64_t groups = (int64_t)a.B * ((a.Tq + nq - 1) / nq);
  for (int kpl : {32, 16}) {
    const int64_t ch = 64 * kpl;
    const double lam = (double)a.k * (double)ch / (double)(a.N_cap > 0 ? a.N_cap : 1);
    if (groups * ((a.N_cap + ch - 1) / ch) * 4 >= 2048 && lam <= 24.0) return kpl;
  }
  return 4;
}

// The decode scan of one indexer call: chunk size, rows per wavefront and the
// carved workspace.
struct ScanPlan {
  int kpl, nq, CH, NCH, gpb;
  IdxWs W;
};
inline ScanPlan index_scan_plan(const IndexArgs& a) {
  ScanPlan p;
  p.nq = nq_of(a.dt, a.H, a.Tq);
  p.kpl = choose_kpl(a, p.nq);
  p.CH = 64 * p.kpl;
  const int64_t nch = (a.N_cap + p.CH - 1) / p.CH;
  p.NCH = (int)(nch > 0 ? nch : 1);
  p.gpb = (a.Tq + p.nq - 1) / p.nq;
  p.W = carve(a.ws, (int64_t)a.B * a.Tq, p.NCH);
  return p;
}

bool index_scan_fusable(const IndexArgs& a);
hipError_t launch_index_select(const IndexArgs& a, const ScanPlan& p, hipStream_t s);
// The same, with the merge of mb's split jobs in the same launch (mb's merge
// plan filled: S, items, ml, po, mblk0).
hipError_t launch_index_select_merge(const IndexArgs& a, const ScanPlan& p, const AttendBatch& mb, hipStream_t s);

}  // namespace lca
