// index_select.h -- the exact top-k selection of one query row of the decode
// indexer (one workgroup of SEL_THREADS threads) over the candidates of the
// chunk scan, with the certification and the streamed fallback; shared by the
// decode select kernels (index.hip) and the prefill path's queued rows
// (index_prefill.hip).  The method and its sources are described in
// index.hip.
#pragma once
#include "index_chunk.h"

namespace lca {

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
  const int n = idx_nelig(A, r);
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
  if (threadIdx.x == 0) S.bcast[6] = 0;
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
    // slots: bit 1), in one exchange of per-wavefront partials (the flags
    // as well: a word cleared by one thread could otherwise be set by another
    // wavefront before the clear)
    static_assert(CPTH == 1, "one chunk per thread");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c0 = threadIdx.x;
    int v = c0 < nch ? cv[0] : 0;
    const bool bad_c = v < 0;
    if (bad_c) v = 0;
    const int wfl = (__ballot(bad_c) ? 1 : 0) | (__ballot(v > spec) ? 2 : 0);
    const int incl = wave_incl_scan_dpp(v);
    const uint64_t wmx = wave_max_u64_dpp(v > 0 ? xv[0] : 0ull);
    const uint64_t wmn = wave_min_u64_dpp(v > 0 ? tv[0] : ~0ull);
    if (lane == 63) S.scan[wave] = (uint32_t)incl;
    if (lane == 0) {
      S.red64[0][wave] = wmx;
      S.red64[1][wave] = wmn;
      S.wflag[wave] = (uint32_t)wfl;
    }
    __syncthreads();
    if (wave == 0) {
      // one wavefront combines the per-wavefront partials
      const int t = lane < SEL_WAVES ? (int)S.scan[lane] : 0;
      const int ti = wave_incl_scan_dpp(t);
      const uint64_t gx = wave_max_u64_dpp(lane < SEL_WAVES ? S.red64[0][lane] : 0ull);
      const uint64_t gn = wave_min_u64_dpp(lane < SEL_WAVES ? S.red64[1][lane] : ~0ull);
      const uint32_t f = lane < SEL_WAVES ? S.wflag[lane] : 0u;
      const int fl = (__ballot(f & 1u) ? 1 : 0) | (__ballot(f & 2u) ? 2 : 0);
      if (lane < SEL_WAVES) S.woff[lane] = ti - t;
      if (lane == SEL_WAVES - 1) { S.bcast[4] = ti; S.bcast[7] = fl; S.bcast64[1] = gx; S.bcast64[2] = gn; }
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
      // u*SEL_THREADS + tid of the candidates in dense order (ascending entry
      // index), present when i < total; the slots u >= nu are empty in every
      // thread and are skipped by all the passes below.
      const int nu = __builtin_amdgcn_readfirstlane((total + SEL_THREADS - 1) / SEL_THREADS);
      uint64_t bk[LB];
      int32_t bj[LB];
      uint32_t vm = 0;
      if (!(flags & 2)) {
        // staged layout (slot c*SPEC + e of chunk c, valid when e < count):
        // compacted in place to the dense order (all slots read, then the
        // valid ones written at off[c] + e)
        int dpos[LB];
#pragma unroll
        for (int u = 0; u < LB; ++u) {
          const int i = u * SEL_THREADS + threadIdx.x;
          const int c = i >> spec_sh, e = i & (spec - 1);
          const int cc = c < nch ? c : 0;
          const bool ok = c < nch && e < S.off[cc + 1] - S.off[cc];
          bk[u] = ckey_l[i];
          bj[u] = cidx_l[i];
          dpos[u] = ok ? S.off[cc] + e : -1;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < LB; ++u)
          if (dpos[u] >= 0) { ckey_l[dpos[u]] = bk[u]; cidx_l[dpos[u]] = bj[u]; }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < LB; ++u) {
          const int i = u * SEL_THREADS + threadIdx.x;
          if (u < nu) { bk[u] = ckey_l[i]; bj[u] = cidx_l[i]; }
          vm |= (uint32_t)(i < total) << u;
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
      RegSrc src{bk, bj, vm, nu};
      // first radix digit: the (at most) 9 bits below the common prefix of
      // the range
      const int hb = gmax == gmin ? -1 : 63 - __clzll(gmax ^ gmin);
      int shift = hb + 1 > 9 ? hb + 1 - 9 : 0;
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
        // holds the 8 bins nbins-1-8l .. nbins-8-8l (counted from the top)
        if (wave == 0) {
          constexpr int BPL = 8;
          const int nbins = 1 << nb;
          const int hi = nbins - 1 - BPL * lane;
          uint32_t hb8[BPL];
          if (hi >= BPL - 1) {
            const uint4* hp = (const uint4*)&S.hist[hi - (BPL - 1)];
#pragma unroll
            for (int q = 0; q < BPL / 4; ++q) {
              const uint4 h = hp[q];
              hb8[4 * q] = h.x; hb8[4 * q + 1] = h.y; hb8[4 * q + 2] = h.z; hb8[4 * q + 3] = h.w;
            }
          } else {
#pragma unroll
            for (int q = 0; q < BPL; ++q) hb8[q] = (hi - (BPL - 1) + q >= 0) ? S.hist[hi - (BPL - 1) + q] : 0u;
          }
          int cnt8 = 0;
#pragma unroll
          for (int q = 0; q < BPL; ++q) cnt8 += (int)hb8[q];
          const int inc = wave_incl_scan_dpp(cnt8);
          if (inc - cnt8 < rem && inc >= rem) {
            int above = inc - cnt8;
            bool found = false;
#pragma unroll
            for (int q = BPL - 1; q >= 0; --q) {
              const int cb = (int)hb8[q];
              if (!found && above + cb >= rem) {
                S.bcast[0] = hi - (BPL - 1) + q; S.bcast[1] = above; S.bcast[2] = cb;
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
      done = emit_regs(bk, bj, vm, nu, th, tie_break ? ties : -1, unsafe, A.k, out, sout, S);
    }
  }
  if (!done) {
    __syncthreads();
    if (threadIdx.x < 32) wl[threadIdx.x] = wv;
    __syncthreads();
    select_streamed<DT, HP>(A, r, n, kk, out, sout, S, tbuf, wl, ql, false);
  }
}

}  // namespace lca
