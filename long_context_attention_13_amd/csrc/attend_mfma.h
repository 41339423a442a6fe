// attend_mfma.h -- the bf16-MFMA attention workgroup body (one query-row group
// and one split of its list) and the split merge, shared by the attention
// kernels and the fused decode-step kernel.  The method and its sources are
// described in attend.hip.
#pragma once
#include "lca_device.h"

namespace lca {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Split plan.  One split per row for a call shaped for prefill (at least
// ATT_PREFILL_TQ query rows per sequence; its dense rows are then grouped to
// share staged tiles) and for lists of at most two tiles; otherwise a row's
// list (entries, then window tokens; its length is bounded by the capacity
// n_kv_max + W_buf) is cut into splits of a fixed size: one 64-item tile up
// to 2048 items, two tiles beyond (decode lists are latency-bound, so short
// splits spread them over many compute units), larger only when needed to
// keep a row within the merge's 1024 splits.  The plan depends on the call's
// list capacity and query rows per sequence only -- never on the number of
// sequences, nor on the data -- so a sequence gives the same bits in any
// batch (splits past a row's actual list return at once and are not merged).
struct Plan { int S; int items; };

constexpr int ATT_PREFILL_TQ = 64;
constexpr int ATT_MAX_SPLITS = 1024;

inline Plan att_plan(int64_t Tq, int64_t n_kv_max, int64_t W_buf) {
  const int64_t L = n_kv_max + W_buf;
  if (Tq >= ATT_PREFILL_TQ || L <= 128) return Plan{1, (int)(L < 1 ? 1 : L)};
  int64_t items = L <= 2048 ? 64 : 128;
  if ((L + items - 1) / items > ATT_MAX_SPLITS) items = (L + 64 * ATT_MAX_SPLITS - 1) / (64 * ATT_MAX_SPLITS) * 64;
  return Plan{(int)((L + items - 1) / items), (int)items};
}

// Device-resident sizes are clamped where a kernel reads them, so that no
// value sends a read outside the buffers the call describes: a row's
// eligible count to [0, N_cap], its window slice to rows of [0, W_buf) (the
// begin to a row that exists, as the loads of a tile read the slice's first
// row even when it is empty).
// (N_cap and W_buf are below 2^31.)
__device__ __forceinline__ int att_nelig(const AttendArgs& A, int r) {
  return min(max(A.n_elig[r], 0), (int)A.N_cap);
}
// (begin, length) of row r's window slice
__device__ __forceinline__ int2 att_window(const AttendArgs& A, int r) {
  const int W = (int)A.W_buf;
  const int wb = min(max(A.win_begin[r], 0), max(W - 1, 0));
  const int wl = min(max(A.win_len[r], 0), W - wb);
  return make_int2(wb, wl);
}

__device__ __forceinline__ void store_out(const AttendArgs& A, int64_t i, float v) {
  if (A.out_dt == DT_F32) ((float*)A.out)[i] = v;
  else ((uint16_t*)A.out)[i] = f32_to_bf16(v);
}

// Rows that share staged tiles: dense lists with many query rows per
// sequence and no split (the prefill case); at most 512 threads a group.
template <int HQ>
constexpr int att_qb() { return HQ * 4 * 4 <= 512 ? 4 : 512 / (HQ * 4); }

// ------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int MT_TE = 64;                 // items per tile
constexpr int MT_KROW = 136;              // bf16 per K row in LDS (128 + pad)
constexpr int MT_VROW = 72;               // bf16 per V^T row in LDS (64 + pad)

// Rows of one tile fetched into registers.  A task is a pair of adjacent
// items and one 16-dim chunk (32 pairs x 8 chunks = 256 tasks per tile);
// each thread owns CPT tasks.  Entry and window loads are both issued
// unconditionally (from clamped, valid addresses) and the right one is picked
// when the tile is written to LDS, so every load of a tile is in flight at
// once.
constexpr int MT_TASKS = MT_TE / 2 * 8;

template <int KVDT, int CPT, bool SV = false>
struct MtRegs {
  int4 ent[CPT][2][KVDT == DT_FP8 ? 1 : 2];
  int4 win[CPT][2][2];
  float2 sc[CPT][2];
  int kind[CPT][2];       // 0 entry, 1 window token, -1 nothing
  // separate values (SV): the value rows of the same items
  int4 vent[SV ? CPT : 1][2][KVDT == DT_FP8 ? 1 : 2];
  int4 vwin[SV ? CPT : 1][2][2];
  float2 vsc[SV ? CPT : 1][2];
};

// An entry row that the attention takes from elsewhere than the entry cache
// (j < 0: none): the decode step computes the row its own compress job writes
// in the same launch.  code: the row in kv_dt's layout; sc: its two FP8 scales.
struct FreshEnt {
  int j;
  const uint8_t* code;
  const float* sc;
};

// SV: the value rows come from A.v / A.v_scale / A.win_v (the layouts of
// A.kv / A.kv_scale / A.win).
template <int KVDT, int NT, int CPT, bool SV = false>
__device__ __forceinline__ void mt_fetch(const AttendArgs& A, int b, int64_t wbase, int nkv, int e_lo, const int* idxl,
                                         int t0, int p1, MtRegs<KVDT, CPT, SV>& R,
                                         const FreshEnt& fe = FreshEnt{-1, nullptr, nullptr}) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int task = c * NT + tid;
    const int pr = task & 31, ch = (task >> 5) & 7;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = 2 * pr + u;
      const int p = t0 + e;
      int kind = -1;
      int64_t j = 0;
      if (p < p1 && task < MT_TASKS) {
        if (p < nkv) {
          j = A.sparse ? (int64_t)idxl[p - e_lo] : (int64_t)p;
          kind = (j >= 0 && j < A.N_cap) ? 0 : -1;
        } else {
          kind = 1;
        }
      }
      R.kind[c][u] = kind;
      // which sources the tile touches is uniform over the workgroup, so
      // these branches do not split the loads
      if (t0 < nkv) {
        const int64_t erow = (int64_t)b * A.N_cap + (kind == 0 ? j : 0);
        if (KVDT == DT_FP8) {
          R.ent[c][u][0] = *(const int4*)((const uint8_t*)A.kv + erow * 128 + ch * 16);
          R.sc[c][u] = *(const float2*)(A.kv_scale + erow * 2);
          if (SV) {
            R.vent[c][u][0] = *(const int4*)((const uint8_t*)A.v + erow * 128 + ch * 16);
            R.vsc[c][u] = *(const float2*)(A.v_scale + erow * 2);
          }
        } else {
          R.ent[c][u][0] = *(const int4*)((const uint16_t*)A.kv + erow * 128 + ch * 16);
          R.ent[c][u][1] = *(const int4*)((const uint16_t*)A.kv + erow * 128 + ch * 16 + 8);
          if (SV) {
            R.vent[c][u][0] = *(const int4*)((const uint16_t*)A.v + erow * 128 + ch * 16);
            R.vent[c][u][1] = *(const int4*)((const uint16_t*)A.v + erow * 128 + ch * 16 + 8);
          }
        }
        if (!SV && kind == 0 && j == fe.j) {
          if (KVDT == DT_FP8) {
            R.ent[c][u][0] = *(const int4*)(fe.code + ch * 16);
            R.sc[c][u] = *(const float2*)fe.sc;
          } else {
            R.ent[c][u][0] = *(const int4*)((const uint16_t*)fe.code + ch * 16);
            R.ent[c][u][1] = *(const int4*)((const uint16_t*)fe.code + ch * 16 + 8);
          }
        }
      }
      if (t0 + MT_TE > nkv && A.W_buf > 0) {
        const int64_t wrow = wbase + (kind == 1 ? p - nkv : 0);
        R.win[c][u][0] = *(const int4*)((const uint16_t*)A.win + wrow * 128 + ch * 16);
        R.win[c][u][1] = *(const int4*)((const uint16_t*)A.win + wrow * 128 + ch * 16 + 8);
        if (SV) {
          R.vwin[c][u][0] = *(const int4*)((const uint16_t*)A.win_v + wrow * 128 + ch * 16);
          R.vwin[c][u][1] = *(const int4*)((const uint16_t*)A.win_v + wrow * 128 + ch * 16 + 8);
        }
      }
    }
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2_from_fp8x2(uint32_t two_codes) {
  const float2 f = fp8x2_to_f32(two_codes);
  return __builtin_amdgcn_perm(__float_as_uint(f.y), __float_as_uint(f.x), 0x07060302u);
}

// Staged layouts: K row-major (item x 128 dims, padded rows); V^T dim-major
// with the items of a row in the order the P operand takes them (item
// 32k + 16h + 4g + i at column 32k + 8g + 4h + i, so each lane's 8 items of
// one dim are contiguous).  The permutation keeps item pairs (2m, 2m+1)
// adjacent, so one 32-bit store writes both items of a pair for one dim.
// The bf16 pieces of one staged row: FP8 codes converted exactly (the
// scales are applied to the products), bf16 rows as they are.
template <int KVDT>
__device__ __forceinline__ void mt_row_pieces(const int4 (&ent)[KVDT == DT_FP8 ? 1 : 2], int4& v0, int4& v1) {
  if (KVDT == DT_FP8) {
    const int4 q = ent[0];
    v0.x = (int)pack_bf16x2_from_fp8x2((uint32_t)q.x & 0xFFFFu);
    v0.y = (int)pack_bf16x2_from_fp8x2((uint32_t)q.x >> 16);
    v0.z = (int)pack_bf16x2_from_fp8x2((uint32_t)q.y & 0xFFFFu);
    v0.w = (int)pack_bf16x2_from_fp8x2((uint32_t)q.y >> 16);
    v1.x = (int)pack_bf16x2_from_fp8x2((uint32_t)q.z & 0xFFFFu);
    v1.y = (int)pack_bf16x2_from_fp8x2((uint32_t)q.z >> 16);
    v1.z = (int)pack_bf16x2_from_fp8x2((uint32_t)q.w & 0xFFFFu);
    v1.w = (int)pack_bf16x2_from_fp8x2((uint32_t)q.w >> 16);
  } else {
    v0 = ent[0];
    v1 = ent[KVDT == DT_FP8 ? 0 : 1];
  }
}

// SV: the value rows go to V^T and their scales to vsclo / vschi; otherwise
// the key rows serve as values too (vsclo / vschi unused).
template <int KVDT, int NT, int CPT, bool SV = false>
__device__ __forceinline__ void mt_store(const MtRegs<KVDT, CPT, SV>& R, __bf16* Kl, __bf16* Vt, float* sclo, float* schi,
                                         int* okl, float* vsclo = nullptr, float* vschi = nullptr) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int task = c * NT + tid;
    if (task >= MT_TASKS) break;
    const int pr = task & 31, ch = task >> 5;
    int4 v[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = 2 * pr + u;
      const int kind = R.kind[c][u];
      int4 v0 = make_int4(0, 0, 0, 0), v1 = make_int4(0, 0, 0, 0);
      int4 w0 = v0, w1 = v0;              // the value row (SV)
      float slo = 1.f, shi = 1.f, vlo = 1.f, vhi = 1.f;
      if (kind == 0) {
        mt_row_pieces<KVDT>(R.ent[c][u], v0, v1);
        if (KVDT == DT_FP8) { slo = R.sc[c][u].x; shi = R.sc[c][u].y; }
        if (SV) {
          mt_row_pieces<KVDT>(R.vent[c][u], w0, w1);
          if (KVDT == DT_FP8) { vlo = R.vsc[c][u].x; vhi = R.vsc[c][u].y; }
        }
      } else if (kind == 1) {
        v0 = R.win[c][u][0];
        v1 = R.win[c][u][1];
        if (SV) { w0 = R.vwin[c][u][0]; w1 = R.vwin[c][u][1]; }
      }
      *(int4*)&Kl[e * MT_KROW + ch * 16] = v0;
      *(int4*)&Kl[e * MT_KROW + ch * 16 + 8] = v1;
      v[u][0] = SV ? w0 : v0;
      v[u][1] = SV ? w1 : v1;
      if (ch == 0) {
        sclo[e] = slo; schi[e] = shi; okl[e] = kind >= 0;
        if (SV) { vsclo[e] = vlo; vschi[e] = vhi; }
      }
    }
    const int e0 = 2 * pr;
    const int ep = (e0 & ~31) | ((e0 & 12) << 1) | ((e0 & 16) >> 2) | (e0 & 3);   // even column of the pair
    uint32_t* vt = (uint32_t*)Vt + ep / 2;
    const uint32_t* a = (const uint32_t*)&v[0][0];     // item 2pr: dims ch*16 .. +15 as 8 dwords
    const uint32_t* bb = (const uint32_t*)&v[1][0];    // item 2pr+1
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      // dwords a[q] = (dim 2q+1 | dim 2q) of item e0, bb[q] the same of item e0+1
      vt[(ch * 16 + 2 * q) * (MT_VROW / 2)] = __builtin_amdgcn_perm(bb[q], a[q], 0x05040100u);
      vt[(ch * 16 + 2 * q + 1) * (MT_VROW / 2)] = __builtin_amdgcn_perm(bb[q], a[q], 0x07060302u);
    }
  }
}

template <int QB>
struct MtShared {
  __align__(16) __bf16 Kl[MT_TE * MT_KROW];
  __align__(16) __bf16 Vt[128 * MT_VROW];
  __align__(16) float sclo[MT_TE];
  __align__(16) float schi[MT_TE];
  __align__(16) int okl[MT_TE];
  int idxl[QB == 1 ? 2048 : 1];
};

// The same with the value scales of a separate-values call.
template <int QB>
struct MtSharedSV {
  MtShared<QB> m;
  __align__(16) float vsclo[MT_TE];
  __align__(16) float vschi[MT_TE];
};

// Split `split` of query-row group `grp` of one attention call.
// SV: separate values (A.v, A.v_scale, A.win_v); vsclo / vschi: LDS for the
// value scales of a tile (MtSharedSV).
template <int KVDT, int HQ, int QB, bool SV = false>
__device__ __forceinline__ void attend_mfma_body(const AttendArgs& A, int S, int split_items, float* part_ml,
                                                 float* part_o, int split, int grp, MtShared<QB>& sm,
                                                 const FreshEnt& fe = FreshEnt{-1, nullptr, nullptr},
                                                 float* vsclo = nullptr, float* vschi = nullptr) {
  // QB query rows of one sequence share each staged tile (dense lists only):
  // the workgroup's list is entries 0 .. max n_elig - 1 followed by the union
  // of the rows' window slices, and every row masks what is not its own.
  constexpr int NT = HQ * 4 * QB;                  // threads (HQ/16 waves per row)
  constexpr int CPT = (MT_TASKS + NT - 1) / NT;    // staging tasks per thread and tile
  const int ngrp = (A.Tq + QB - 1) / QB;
  const int b = grp / ngrp;
  const int t0r = (grp % ngrp) * QB;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, col = lane & 15;
  const int qrow = wave / (HQ / 16);                // this wave's row within the group
  const bool rvalid = t0r + qrow < A.Tq;
  const int r = b * A.Tq + (rvalid ? t0r + qrow : t0r);
  const int nkv_r = A.sparse ? A.k : att_nelig(A, r);
  const int2 ws_r = att_window(A, r);
  const int wb_r = ws_r.x, wl_r = ws_r.y;
  int nkv = nkv_r, wlo = wb_r, whi = wb_r + wl_r;
  if (QB > 1) {
    // the same for every wave of the group (uniform loop bounds)
    nkv = 0; wlo = 0x7FFFFFFF; whi = 0;
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      if (t0r + q >= A.Tq) break;
      const int rq = b * A.Tq + t0r + q;
      nkv = max(nkv, att_nelig(A, rq));
      const int2 wq = att_window(A, rq);
      wlo = min(wlo, wq.x);
      whi = max(whi, wq.x + wq.y);
    }
    if (whi < wlo) whi = wlo;
  }
  __bf16* Kl = sm.Kl;
  __bf16* Vt = sm.Vt;
  float* sclo = sm.sclo;
  float* schi = sm.schi;
  int* okl = sm.okl;
  int* idxl = sm.idxl;

  // the selected indices of this split's entry range, staged once; their
  // bound does not depend on the window, so they are requested together with
  // the row's window bounds
  const int p0 = split * split_items;
  const int e_lo = p0;
  if (QB == 1 && A.sparse) {
    const int e_end = min(p0 + split_items, A.k);
    for (int i = tid; i < e_end - e_lo; i += NT) idxl[i] = A.idx[(int64_t)r * A.k + e_lo + i];
  }

  const int L = nkv + (whi - wlo);
  const int64_t wbase = (int64_t)b * A.W_buf + wlo;
  const int p1 = S == 1 ? L : min(L, p0 + split_items);
  if (S > 1 && p0 >= L) return;             // an empty split: the merge does not read it

  // Q^T operand: this lane's head = (wave % (HQ/16))*16 + col, dims 32*ks + 8*g .. +7
  const int head = (wave % (HQ / 16)) * 16 + col;
  bf16x8 qv[4];
  {
    const uint16_t* qp = (const uint16_t*)A.q + ((int64_t)r * HQ + head) * 128;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int4 v = *(const int4*)(qp + 32 * ks + 8 * g);
      qv[ks] = *(const bf16x8*)&v;
    }
  }
  const float scale2 = A.scale * LOG2E;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  MtRegs<KVDT, CPT, SV> R;
  if (p0 < p1) mt_fetch<KVDT, NT, CPT, SV>(A, b, wbase, nkv, e_lo, idxl, p0, p1, R, fe);
  for (int t0 = p0; t0 < p1; t0 += MT_TE) {
    __syncthreads();
    mt_store<KVDT, NT, CPT, SV>(R, Kl, Vt, sclo, schi, okl, vsclo, vschi);
    __syncthreads();
    if (t0 + MT_TE < p1) mt_fetch<KVDT, NT, CPT, SV>(A, b, wbase, nkv, e_lo, idxl, t0 + MT_TE, p1, R, fe);

    // ---- S^T = K Q^T for 4 subtiles of 16 items: per K-step the four
    // subtiles' fragments are read together and feed four independent
    // accumulators (FP8: dims 0-63 and 64-127 carry separate scales, so two
    // sets of sums)
    f32x4 clo[4], chi[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) { clo[st] = f32x4{0.f, 0.f, 0.f, 0.f}; chi[st] = clo[st]; }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 kf[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) kf[st] = *(const bf16x8*)&Kl[(st * 16 + col) * MT_KROW + 8 * g + 32 * ks];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (KVDT != DT_FP8 || ks < 2) clo[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[st], qv[ks], clo[st], 0, 0, 0);
        else chi[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[st], qv[ks], chi[st], 0, 0, 0);
      }
    }
    float sv[4][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      // per-item data of this lane's 4 items (4 consecutive items)
      const float4 slo4 = *(const float4*)&sclo[st * 16 + 4 * g];
      const float4 shi4 = *(const float4*)&schi[st * 16 + 4 * g];
      const int4 ok4 = *(const int4*)&okl[st * 16 + 4 * g];
      const float sl[4] = {slo4.x, slo4.y, slo4.z, slo4.w}, sh[4] = {shi4.x, shi4.y, shi4.z, shi4.w};
      const int okv[4] = {ok4.x, ok4.y, ok4.z, ok4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = st * 16 + 4 * g + i;
        const float sdot = KVDT == DT_FP8 ? clo[st][i] * sl[i] + chi[st][i] * sh[i] : clo[st][i];
        bool ok = okv[i] != 0;
        if (QB > 1) {
          // the item must belong to this wave's row
          const int p = t0 + e;
          const int wpos = wlo + (p - nkv);
          ok = ok && rvalid && (p < nkv ? p < nkv_r : (wpos >= wb_r && wpos < wb_r + wl_r));
        }
        sv[st][i] = ok ? sdot * scale2 : -INFINITY;
      }
    }
    // ---- online softmax for head `head`
    float tmax = -INFINITY;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sv[st][i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // base-2 exponentials (the logits carry the factor log2 e); a running
    // max of -inf (nothing attended yet) is replaced by 0 so that masked
    // items give exp2(-inf) = 0 without a test per item
    const float m_new = fmaxf(m_run, tmax);
    const float mb = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - mb);
    m_run = m_new;
    float lsum = 0.f;
    float pv[4][4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pe = exp2f(sv[st][i] - mb);
        pv[st][i] = pe;
        lsum += pe;
      }
    l_run = l_run * alpha + lsum;
    // rescale only when some lane's running max moved (usually only the
    // first tiles)
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= alpha;
    }

    // ---- O^T += V^T P^T, two K-steps of 32 items
#pragma unroll
    for (int kap = 0; kap < 2; ++kap) {
      bf16x8 plo, phi;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int st = 2 * kap + (jj >> 2), i = jj & 3;
        const int e = st * 16 + 4 * g + i;
        if (KVDT == DT_FP8) {
          plo[jj] = (__bf16)(pv[st][i] * (SV ? vsclo : sclo)[e]);   // the V scale folds into P
          phi[jj] = (__bf16)(pv[st][i] * (SV ? vschi : schi)[e]);
        } else {
          plo[jj] = (__bf16)pv[st][i];
          phi[jj] = plo[jj];
        }
      }
      bf16x8 vf[8];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) vf[mt] = *(const bf16x8*)&Vt[(mt * 16 + col) * MT_VROW + 32 * kap + 8 * g];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[mt], mt < 4 ? plo : phi, acc[mt], 0, 0, 0);
    }
  }

  // ---- finish: the per-head sum over the 4 lanes that share the head
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!rvalid) return;
  if (S == 1) {
    const float sk = A.sink[head] * LOG2E;
    const float M = fmaxf(m_run, sk);
    const float em = (m_run == -INFINITY) ? 0.f : exp2f(m_run - M);
    const float Z = exp2f(sk - M) + l_run * em;
    const float f = em / Z;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_out(A, ((int64_t)r * HQ + head) * 128 + mt * 16 + 4 * g + i, acc[mt][i] * f);
    if (A.lse && g == 0) A.lse[(int64_t)r * HQ + head] = (M + log2f(Z)) * LN2;
  } else {
    // partial outputs in bf16 (half the bytes written here and read by the
    // merge; the rounding is far inside the bf16 / FP8 tolerance), a (row,
    // head)'s splits side by side ([row][head][split][dim]: the merge reads
    // them as one contiguous run); maxima and sums in fp32, [row][split][head]
    const int64_t base = ((int64_t)r * S + split) * HQ + head;
    const int64_t obase = ((int64_t)r * HQ + head) * S + split;
    uint16_t* pob = (uint16_t*)part_o;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      *(uint2*)&pob[obase * 128 + mt * 16 + 4 * g] =
          make_uint2((uint32_t)f32_to_bf16(acc[mt][0]) | ((uint32_t)f32_to_bf16(acc[mt][1]) << 16),
                     (uint32_t)f32_to_bf16(acc[mt][2]) | ((uint32_t)f32_to_bf16(acc[mt][3]) << 16));
    if (g == 0) { part_ml[base * 2] = m_run; part_ml[base * 2 + 1] = l_run; }
  }
}

// ------------------------------------------------------------------------
// merge: combine the split partials of one row in split order with the sink
// ------------------------------------------------------------------------
struct MgShared {
  float wsp[1024];
  float red[2][2];
};

// one workgroup per (row, head) = blk; thread d owns output dim d.  Only the
// splits that hold items of the row's list (length L = list + window) are
// read: a later split is empty and contributes nothing.  Every load (the split
// maxima and sums, and the first MG_PRE splits' outputs) is issued before any
// of them is used.
// `store` false: the unit only takes part in the workgroup's barriers (a
// workgroup that merges several units, one per 128 threads, with fewer units
// left than groups).
// MG_PRE partial outputs are loaded up front, the rest MG_STEP at a time
// (fewer registers where the merge shares a kernel with other work).
// Even splits are summed into o0 and odd ones into o1, each in increasing
// order, whatever MG_PRE and MG_STEP are (both even), so every variant of the
// body gives the same bits.
// BF: the partial outputs are bf16 in [row][head][split][dim] order (the
// matrix-core kernels); thread d then loads the dword holding dims d & ~1 and
// d | 1 (the two lanes of a pair read the same dword) and takes its half.
// Otherwise fp32 in [row][split][head][dim] order (the fp32 kernel).
template <bool BF, int MG_PRE = 64, int MG_STEP = 32>
__device__ __forceinline__ void attend_merge_body(const AttendArgs& A, int S_all, int split_items,
                                                  const float* part_ml, const float* part_o, int blk, MgShared& sm,
                                                  bool store = true) {
  static_assert(MG_PRE % 2 == 0 && MG_STEP % 2 == 0, "even prefetch and step");
  const int r = blk / A.Hq, h = blk % A.Hq;
  const int d = threadIdx.x & 127;
  // the row's list length is requested with the partials, which are read for
  // every planned split (all inside the workspace) and masked once it arrives
  const int L = (A.sparse ? A.k : att_nelig(A, r)) + att_window(A, r).y;
  float* wsp = sm.wsp;
  auto& red = sm.red;
  const float sk = A.sink[h] * LOG2E;                       // partial maxima are base-2 logits
  const int64_t base0 = (int64_t)r * S_all * A.Hq + h;      // partial (r, s, h) = base0 + s*Hq
  const int64_t ost = (int64_t)A.Hq * A.D;
  const float* po = part_o + base0 * A.D + d;
  const uint32_t* pw =
      (const uint32_t*)((const uint16_t*)part_o + ((int64_t)r * A.Hq + h) * S_all * A.D) + (d >> 1);
  const int hs = (d & 1) ? 0 : 16;          // the shift that puts this dim's bf16 in the high half
  // partial s as loaded (its word; fp32 bits or the bf16 pair), and as a value
  // (taken only where it is summed, so that every load is issued first)
  auto raw = [&](int s) -> uint32_t { return BF ? pw[s * (A.D >> 1)] : __float_as_uint(po[s * ost]); };
  auto val = [&](uint32_t w) -> float { return BF ? __uint_as_float((w << hs) & 0xFFFF0000u) : __uint_as_float(w); };
  uint32_t ov[MG_PRE];
#pragma unroll
  for (int i = 0; i < MG_PRE; ++i) ov[i] = i < S_all ? raw(i) : 0u;
  float mv[8], lv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int s = d + 128 * i;
    mv[i] = s < S_all ? part_ml[(base0 + (int64_t)s * A.Hq) * 2] : -INFINITY;
    lv[i] = s < S_all ? part_ml[(base0 + (int64_t)s * A.Hq) * 2 + 1] : 0.f;
  }
  const int S = min(S_all, (L + split_items - 1) / split_items);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (d + 128 * i >= S) { mv[i] = -INFINITY; lv[i] = 0.f; }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) mx = fmaxf(mx, mv[i]);
  mx = wave_max(mx);
  if ((d & 63) == 0) red[0][d >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(sk, fmaxf(red[0][0], red[0][1]));
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int s = d + 128 * i;
    if (s < S) {
      const float e = (mv[i] == -INFINITY) ? 0.f : exp2f(mv[i] - M);
      wsp[s] = e;
      z += lv[i] * e;
    }
  }
  z = wave_sum(z);
  if ((d & 63) == 0) red[1][d >> 6] = z;
  __syncthreads();
  const float Z = exp2f(sk - M) + red[1][0] + red[1][1];
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int i = 0; i < MG_PRE; i += 2) {
    if (i < S) o0 = fmaf(val(ov[i]), wsp[i], o0);
    if (i + 1 < S) o1 = fmaf(val(ov[i + 1]), wsp[i + 1], o1);
  }
  for (int s0 = MG_PRE; s0 < S; s0 += MG_STEP) {
    uint32_t ot[MG_STEP];
#pragma unroll
    for (int i = 0; i < MG_STEP; ++i) ot[i] = s0 + i < S ? raw(s0 + i) : 0u;
#pragma unroll
    for (int i = 0; i < MG_STEP; i += 2) {
      if (s0 + i < S) o0 = fmaf(val(ot[i]), wsp[s0 + i], o0);
      if (s0 + i + 1 < S) o1 = fmaf(val(ot[i + 1]), wsp[s0 + i + 1], o1);
    }
  }
  const float o = o0 + o1;
  if (!store) return;
  store_out(A, ((int64_t)r * A.Hq + h) * A.D + d, o / Z);
  if (A.lse && d == 0) A.lse[(int64_t)r * A.Hq + h] = (M + log2f(Z)) * LN2;
}

// The dense attention of many query rows of one sequence with 64 heads and
// bf16 entries, a wavefront per row (attend_dense.hip): used for the grouped
// (single-split) dense layout when it applies.
bool attend_dense_wide_applies(const AttendArgs& a);
hipError_t launch_attend_dense_wide(const AttendArgs& a, hipStream_t s);
// The same for the sparse lists of many query rows (one list per row).
bool attend_sparse_wide_applies(const AttendArgs& a);
hipError_t launch_attend_sparse_wide(const AttendArgs& a, hipStream_t s);

}  // namespace lca
