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
#include "attend_mfma.h"
#include "index_chunk.h"

namespace lca {

template <int DT, int KPL, int HP, int NQ>
__global__ __launch_bounds__(256) void index_chunk_kernel(IndexArgs A, IdxWs W, int NCH, int groups_per_b) {
  __shared__ ChunkShared<NQ> sm;
  index_chunk_body<DT, KPL, HP, NQ>(A, W, NCH, groups_per_b, blockIdx.x, blockIdx.y, sm);
}

// The selection of query row r (one workgroup of SEL_THREADS threads).
template <int DT, int HP>
__device__ __forceinline__ void index_select_body(const IndexArgs& A, const IdxWs& W, int NCH, int CH, int r,
                                                  char* smem) {
  SelShared& S = *(SelShared*)smem;
  // the candidate arrays (candidate path) and the scoring buffers (streamed
  // path) share one region
  char* region = smem + sizeof(SelShared);
  uint64_t* ckey_l = (uint64_t*)region;                            // [CMAX]
  int32_t* cidx_l = (int32_t*)(region + sizeof(uint64_t) * CMAX);  // [CMAX]
  float* tbuf = (float*)region;                                    // [SEL_WAVES][WBUF]
  float* wl = (float*)(region + 12 * CMAX);                        // [32]
  const float* ql = (const float*)A.qi + (int64_t)r * A.H * A.d;   // F32 query row (global)

  // the row length and head weights first (waits for them then do not wait
  // for the larger requests behind), then the per-chunk summaries
  const int n = A.n_elig[r];
  const float wv = (threadIdx.x < (unsigned)A.H) ? A.w[(int64_t)r * A.H + threadIdx.x] : 0.f;
  constexpr int CPTH = MAXCH / SEL_THREADS;          // chunks per thread
  int cv[CPTH];
  uint64_t mv[CPTH], xv[CPTH], tv[CPTH];
  const bool cand_ok = NCH <= MAXCH;
  const int64_t rc0 = (int64_t)r * NCH;                 // this row's first chunk slot
#pragma unroll
  for (int i = 0; i < CPTH; ++i) {
    const int c = i * SEL_THREADS + threadIdx.x;
    const int cc = (cand_ok && c < NCH) ? c : 0;
    cv[i] = W.cnt[rc0 + cc];
    mv[i] = W.mex[rc0 + cc];
    xv[i] = W.cmax[rc0 + cc];
    tv[i] = W.cthr[rc0 + cc];
  }
  // and, speculatively, the first SPEC slots of every chunk (SPEC: a power of
  // two with NCH * SPEC <= CMAX, at least 8), copied by DMA straight into the
  // candidate arrays at position c * SPEC + slot; chunks with more candidates
  // are gathered again once the counts are known
  int spec_sh = 3;
  while (spec_sh < 7 && (NCH << (spec_sh + 1)) <= CMAX) ++spec_sh;
  const int spec = 1 << spec_sh;
  {
    // a fixed number of copies per wavefront (all CMAX slots; slots past
    // NCH*SPEC repeat the last real one and are never read), so that waits
    // on the earlier requests stay exact
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nst = cand_ok ? NCH << spec_sh : 4;          // staged slots
    const uint64_t* krow = W.ckey + (cand_ok ? rc0 * CAP : 0);
    const int32_t* jrow = W.cidx + (cand_ok ? rc0 * CAP : 0);
    // keys: 128 per instruction (2 per lane); indices: 256 (4 per lane)
#pragma unroll
    for (int t = 0; t < CMAX / 128 / SEL_WAVES; ++t) {
      const int q = wave + t * SEL_WAVES;
      const int i = min(q * 128 + 2 * lane, nst - 2);
      const uint32_t a = (uint32_t)(i >> spec_sh) * CAP + (i & (spec - 1));
      __builtin_amdgcn_global_load_lds((const void*)(krow + a), (void*)(ckey_l + q * 128), 16, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < CMAX / 256 / SEL_WAVES; ++t) {
      const int q = wave + t * SEL_WAVES;
      const int i = min(q * 256 + 4 * lane, nst - 4);
      const uint32_t a = (uint32_t)(i >> spec_sh) * CAP + (i & (spec - 1));
      __builtin_amdgcn_global_load_lds((const void*)(jrow + a), (void*)(cidx_l + q * 256), 16, 0, 0);
    }
  }
  for (int i = threadIdx.x; i < 2048; i += SEL_THREADS) S.hist[i] = 0;
  if (threadIdx.x == 0) { S.bcast[6] = 0; S.bcast[7] = 0; }
  const int kk = n < A.k ? n : A.k;
  int32_t* out = A.idx_out + (int64_t)r * A.k;
  double* sout = A.score_out ? A.score_out + (int64_t)r * A.k : nullptr;

  const int nch = (n + CH - 1) / CH;
  const bool cand_path = n > A.k && n > NDIRECT && nch <= MAXCH && cand_ok;
  if (!cand_path) {
    // the slot copies must land before the region is reused; the weights
    // are only needed by the re-scoring paths
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x < 32) wl[threadIdx.x] = wv;
    __syncthreads();
  }
  if (n <= A.k) {
    // every eligible entry is selected
    for (int i = threadIdx.x; i < A.k; i += SEL_THREADS) out[i] = i < n ? i : -1;
    if (sout) select_streamed<DT, HP>(A, r, n, kk, out, sout, S, tbuf, wl, ql, true);
    return;
  }
  bool done = false;
  if (cand_path) {
    // ---------------- candidate path ----------------
    // chunk offsets, the key range [gmin, gmax] of all candidates and the
    // flags (a chunk over its slots: bit 0; a chunk over the speculative
    // slots: bit 1), in one exchange of per-wavefront partials
    static_assert(CPTH == 1, "one chunk per thread");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c0 = threadIdx.x;
    int v = c0 < nch ? cv[0] : 0;
    const bool bad_c = v < 0;
    if (bad_c) v = 0;
    const uint64_t bal_bad = __ballot(bad_c), bal_over = __ballot(v > spec);
    const int incl = wave_incl_scan_dpp(v);
    const uint64_t wmx = wave_max_u64_dpp(v > 0 ? xv[0] : 0ull);
    const uint64_t wmn = wave_min_u64_dpp(v > 0 ? tv[0] : ~0ull);
    if (lane == 63) S.scan[wave] = (uint32_t)incl;
    if (lane == 0) {
      S.red64[0][wave] = wmx;
      S.red64[1][wave] = wmn;
      if (bal_bad | bal_over) atomicOr(&S.bcast[7], (bal_bad ? 1 : 0) | (bal_over ? 2 : 0));
    }
    __syncthreads();
    if (wave == 0) {
      // one wavefront combines the per-wavefront partials
      const int t = lane < SEL_WAVES ? (int)S.scan[lane] : 0;
      const int ti = wave_incl_scan_dpp(t);
      const uint64_t gx = wave_max_u64_dpp(lane < SEL_WAVES ? S.red64[0][lane] : 0ull);
      const uint64_t gn = wave_min_u64_dpp(lane < SEL_WAVES ? S.red64[1][lane] : ~0ull);
      if (lane < SEL_WAVES) S.woff[lane] = ti - t;
      if (lane == SEL_WAVES - 1) { S.bcast[4] = ti; S.bcast64[1] = gx; S.bcast64[2] = gn; }
    }
    __syncthreads();
    const int total = S.bcast[4];
    const uint64_t gmax = S.bcast64[1], gmin = S.bcast64[2];
    const int flags = S.bcast[7];
    if (c0 < nch) S.off[c0] = (int)S.woff[wave] + incl - v;
    if (c0 == 0) S.off[nch] = total;
    __builtin_amdgcn_s_waitcnt(0);            // this wavefront's slot copies have landed
    __syncthreads();
    if (!(flags & 1) && total <= CMAX && total >= kk && gmax >= gmin) {
      // Every thread holds up to LB candidates in registers: item i =
      // u*SEL_THREADS + tid in candidate order (ascending entry index).
      uint64_t bk[LB];
      int32_t bj[LB];
      uint32_t vm = 0;
      if (!(flags & 2)) {
        // staged layout (slot c*SPEC + e of chunk c): valid when e < count
#pragma unroll
        for (int u = 0; u < LB; ++u) {
          const int i = u * SEL_THREADS + threadIdx.x;
          const int c = i >> spec_sh, e = i & (spec - 1);
          const int cc = c < nch ? c : 0;
          const bool ok = c < nch && e < S.off[cc + 1] - S.off[cc];
          bk[u] = ckey_l[i];
          bj[u] = cidx_l[i];
          vm |= (uint32_t)ok << u;
        }
      } else {
        // some chunk has more than SPEC candidates: gather all of them in
        // dense order; a chunk map (candidate slot -> chunk, written one
        // chunk per wavefront into the bitmap area) gives each its address
        uint16_t* cmap = (uint16_t*)S.bitmap;
#pragma unroll 1
        for (int c = wave; c < nch; c += SEL_WAVES) {
          const int o = S.off[c], cnt = S.off[c + 1] - o;
          for (int e = lane; e < cnt; e += 64) cmap[o + e] = (uint16_t)c;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < LB; ++u) {
          const int i = u * SEL_THREADS + threadIdx.x;
          const int c = i < total ? cmap[i] : 0;
          const int64_t a = (rc0 + c) * CAP + (i < total ? i - S.off[c] : 0);
          bk[u] = W.ckey[a];
          bj[u] = W.cidx[a];
          vm |= (uint32_t)(i < total) << u;
        }
      }
      RegSrc src{bk, bj, vm};
      // first radix digit: the 11 bits below the common prefix of the range
      const int hb = gmax == gmin ? -1 : 63 - __clzll(gmax ^ gmin);
      int shift = hb + 1 > 11 ? hb + 1 - 11 : 0;
      const int nb = hb + 1 - shift;
      uint64_t mask = (hb + 1 >= 64) ? 0 : ~((1ull << (hb + 1)) - 1ull);
      uint64_t prefix = gmax & mask;
      if (nb > 0) src.for_each([&](uint64_t kv, int) { atomicAdd(&S.hist[(kv >> shift) & ((1ull << nb) - 1ull)], 1u); });
      __syncthreads();
      Thr th;
      th.Tj = 0x7FFFFFFF;
      int rem = kk, ties = 0;
      bool have = false, tie_break = false;
      if (nb == 0) {
        // every candidate has the same key
        th.T = gmax; th.low = 0; ties = rem; have = true; tie_break = total > rem;
      } else {
        // digit holding the rem-th largest, found by one wavefront: lane l
        // holds the 32 bins nbins-1-32l .. nbins-32-32l (counted from the top)
        if (wave == 0) {
          const int nbins = 1 << nb;
          const int hi = nbins - 1 - 32 * lane;
          uint32_t hb32[32];
          if (hi >= 31) {
            const uint4* hp = (const uint4*)&S.hist[hi - 31];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const uint4 h = hp[q];
              hb32[4 * q] = h.x; hb32[4 * q + 1] = h.y; hb32[4 * q + 2] = h.z; hb32[4 * q + 3] = h.w;
            }
          } else {
#pragma unroll
            for (int q = 0; q < 32; ++q) hb32[q] = (hi - 31 + q >= 0) ? S.hist[hi - 31 + q] : 0u;
          }
          int cnt32 = 0;
#pragma unroll
          for (int q = 0; q < 32; ++q) cnt32 += (int)hb32[q];
          const int inc = wave_incl_scan_dpp(cnt32);
          if (inc - cnt32 < rem && inc >= rem) {
            int above = inc - cnt32;
            bool found = false;
#pragma unroll
            for (int q = 31; q >= 0; --q) {
              const int cb = (int)hb32[q];
              if (!found && above + cb >= rem) {
                S.bcast[0] = hi - 31 + q; S.bcast[1] = above; S.bcast[2] = cb;
                found = true;
              }
              above += cb;
            }
          }
        }
        __syncthreads();
        int dsel = S.bcast[0], indig = S.bcast[2];
        rem -= S.bcast[1];
        prefix |= (uint64_t)dsel << shift;
        mask |= (uint64_t)((1u << nb) - 1u) << shift;
        // narrow down until the threshold is exact
        while (!have) {
          if (indig == rem) {                     // the whole bin is in
            th.T = prefix; th.low = shift; ties = rem; have = true;
          } else if (shift == 0) {                // a full key with more ties than needed
            th.T = prefix; th.low = 0; ties = rem; have = true; tie_break = true;
          } else if (indig <= 64) {               // few items: rank them exactly
            resolve_bin(src, prefix, mask, rem, S);
            // exact: the rem-th item of the bin is (T, Tj); ties up to Tj are in
            th.T = S.bcast64[0]; th.low = 0; th.Tj = S.bcast[3];
            have = true;
          } else {
            const int nb2 = shift >= 11 ? 11 : shift;
            shift -= nb2;
            radix_digit(src, prefix, mask, shift, nb2, rem, S);
            dsel = S.bcast[0]; indig = S.bcast[2];
            const int above2 = S.bcast[1];
            rem -= above2;
            prefix |= (uint64_t)dsel << shift;
            mask |= (uint64_t)((1u << nb2) - 1u) << shift;
          }
        }
      }
      // certification: no excluded entry may reach the threshold
      bool unsafe = false;
      if (c0 < nch && mv[0] != 0) {
        if (th.low > 0) unsafe = (mv[0] >> th.low) >= (th.T >> th.low);
        else unsafe = mv[0] >= th.T;
      }
      done = emit_regs(bk, bj, vm, th, tie_break ? ties : -1, unsafe, A.k, out, sout, S);
    }
  }
  if (!done) {
    __syncthreads();
    if (threadIdx.x < 32) wl[threadIdx.x] = wv;
    __syncthreads();
    select_streamed<DT, HP>(A, r, n, kk, out, sout, S, tbuf, wl, ql, false);
  }
}

template <int DT, int HP>
__global__ __launch_bounds__(SEL_THREADS) void index_select_kernel(IndexArgs A, IdxWs W, int NCH, int CH) {
  extern __shared__ __align__(16) char smem[];
  index_select_body<DT, HP>(A, W, NCH, CH, blockIdx.x, smem);
}

// The selection of the decode step with the merge of the dense attention
// jobs' split partials in the same launch (they are complete once the scan
// launch is, and the selection occupies one workgroup per row): blocks
// [0, B*Tq) select a row each; each later block merges SEL_THREADS / 128
// (row, head) units, 128 threads per unit.
template <int DT, int HP>
__global__ __launch_bounds__(SEL_THREADS) void index_select_merge_kernel(IndexArgs A, IdxWs W, int NCH, int CH,
                                                                         AttendBatch mb) {
  extern __shared__ __align__(16) char smem[];
  const int nsel = A.B * A.Tq;
  if ((int)blockIdx.x < nsel) {
    index_select_body<DT, HP>(A, W, NCH, CH, blockIdx.x, smem);
    return;
  }
  constexpr int UPB = SEL_THREADS / 128;
  const int units = mb.mblk0[mb.njobs];
  const int g = threadIdx.x >> 7;
  int u = ((int)blockIdx.x - nsel) * UPB + g;
  const bool real = u < units;
  if (!real) u = units - 1;               // takes part in the barriers only
  int j = 0;
  while (j + 1 < mb.njobs && u >= mb.mblk0[j + 1]) ++j;
  MgShared& sm = ((MgShared*)smem)[g];
  attend_merge_body<16, 16>(mb.job[j], mb.S[j], mb.items[j], mb.ml[j], mb.po[j], u - mb.mblk0[j], sm, real);
}

// ------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------
size_t index_ws_bytes(int B, int Tq, int H, int d, int64_t N_cap, int k, int dt) {
  IndexArgs a{};
  a.B = B; a.Tq = Tq; a.H = H; a.d = d; a.N_cap = N_cap; a.k = k; a.dt = dt;
  if (index_prefill_applies(a)) return index_prefill_ws_bytes(B, Tq);
  const int kpl = choose_kpl(a, nq_of(dt, H, Tq));
  const int64_t NCH = (N_cap + 64 * kpl - 1) / (64 * kpl);
  return carve_bytes((int64_t)B * Tq, NCH > 0 ? NCH : 1);
}

template <int DT, int KPL, int HP, int NQ>
static hipError_t launch_t(const IndexArgs& a, hipStream_t s) {
  const int CH = 64 * KPL;
  const int64_t NCH = (a.N_cap + CH - 1) / CH;
  IdxWs W = carve(a.ws, (int64_t)a.B * a.Tq, NCH > 0 ? NCH : 1);
  const int gpb = (a.Tq + NQ - 1) / NQ;
  if (a.N_cap > NDIRECT) {
    dim3 grid((unsigned)NCH, (unsigned)(a.B * gpb));
    hipLaunchKernelGGL((index_chunk_kernel<DT, KPL, HP, NQ>), grid, dim3(256), 0, s, a, W, (int)NCH, gpb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t smem = select_smem(DT, a.H, a.d);
  hipLaunchKernelGGL((index_select_kernel<DT, HP>), dim3((unsigned)(a.B * a.Tq)), dim3(SEL_THREADS), smem, s, a, W,
                     (int)NCH, CH);
  return hipGetLastError();
}

template <int DT, int HP, int NQ>
static hipError_t launch_k(const IndexArgs& a, hipStream_t s) {
  switch (choose_kpl(a, NQ)) {
    case 32: return launch_t<DT, 32, HP, NQ>(a, s);
    case 16: return launch_t<DT, 16, HP, NQ>(a, s);
    default: return launch_t<DT, 4, HP, NQ>(a, s);
  }
}

// The decode chunk path of an MXFP4 indexer with at most 8 heads, whose scan
// a fused launch can run (the select then runs on its own).
bool index_scan_fusable(const IndexArgs& a) {
  return (int64_t)a.B * a.Tq > 0 && !index_prefill_applies(a) && a.dt == DT_MXFP4 && a.H <= 8 && a.N_cap > NDIRECT;
}

hipError_t launch_index_select_merge(const IndexArgs& a, const ScanPlan& p, const AttendBatch& mb, hipStream_t s) {
  constexpr int UPB = SEL_THREADS / 128;
  static_assert(UPB * sizeof(MgShared) <= sizeof(SelShared) + 12 * (size_t)CMAX, "merge units fit the LDS");
  const int units = mb.mblk0[mb.njobs];
  const size_t smem = select_smem(DT_MXFP4, a.H, a.d);
  const unsigned nb = (unsigned)(a.B * a.Tq + (units + UPB - 1) / UPB);
  hipLaunchKernelGGL((index_select_merge_kernel<DT_MXFP4, 8>), dim3(nb), dim3(SEL_THREADS), smem, s, a, p.W, p.NCH,
                     p.CH, mb);
  return hipGetLastError();
}

hipError_t launch_index_select(const IndexArgs& a, const ScanPlan& p, hipStream_t s) {
  const size_t smem = select_smem(DT_MXFP4, a.H, a.d);
  hipLaunchKernelGGL((index_select_kernel<DT_MXFP4, 8>), dim3((unsigned)(a.B * a.Tq)), dim3(SEL_THREADS), smem, s, a,
                     p.W, p.NCH, p.CH);
  return hipGetLastError();
}

hipError_t launch_index(const IndexArgs& a, hipStream_t s) {
  if ((int64_t)a.B * a.Tq == 0) return hipSuccess;
  if (index_prefill_applies(a)) return launch_index_prefill(a, s);
  const int nq = nq_of(a.dt, a.H, a.Tq);
  if (a.dt == DT_MXFP4) {
    if (a.H <= 8) return nq == 2 ? launch_k<DT_MXFP4, 8, 2>(a, s) : launch_k<DT_MXFP4, 8, 1>(a, s);
    return launch_k<DT_MXFP4, 16, 1>(a, s);
  }
  return launch_k<DT_F32, 16, 1>(a, s);
}

}  // namespace lca
