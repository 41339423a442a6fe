// attend_dense.hip -- the dense attention of many consecutive query rows of
// one sequence (HCA over a prefill chunk): 64 query heads, bf16 entries and
// window.
//
// [release notes (agentlenshq.com), 重度壓縮注意力 (HCA): the 128x compressed
//  sequence is short enough to attend densely; every query row of a chunk
//  attends over (nearly) the same entries.  wiki (chenshi221.pages.dev),
//  关键技术方法 › 架构创新: one KV head shared by all query heads, plus the
//  sliding window and the sink.]
//
// A workgroup of 8 wavefronts takes 4 consecutive query rows; wavefront w is
// row w / 2 with heads 32*(w % 2) .. +31.  The group's list (entries
// 0 .. max n_elig - 1, then the union of the rows' windows) is staged in LDS
// in tiles of 64 items (two tile buffers, one barrier per tile) by all 512
// threads, and each wavefront computes with 32x32x16 bf16 MFMA:
//   S^T (64 items x 32 heads) = K (items x dims) Q^T, 2 x 8 products;
//   O^T (128 dims x 32 heads) += V^T (dims x items) P^T, 4 x 4 products.
// The result layout of the first product puts, in lane l, items
// 32*ib + 8*q + 4*(l/32) + i of head l % 32; the staged V^T columns hold the
// items of each 16-item step with bits 2 and 3 of the offset swapped, so the
// probabilities of step s are result registers 8*(s%2) .. +7 of block s/2 as
// they stand.  Online softmax in base 2 per head, the running max kept in
// scaled units; the sink enters at the end.
#include "attend_mfma.h"

namespace lca {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int DW_ROWS = 4;                   // query rows per workgroup
constexpr int DW_NT = DW_ROWS * 128;         // threads: (row, half of the heads) per wavefront
constexpr int DW_KROW = 136;                 // bf16 per staged K row (128 + pad)
constexpr int DW_VROW = 72;                  // bf16 per staged V^T row (64 + pad)

struct DwShared {
  struct Tile {
    __align__(16) __bf16 Kl[MT_TE * DW_KROW];
    __align__(16) __bf16 Vt[128 * DW_VROW];
    __align__(16) int okl[MT_TE];
  } t[2];
};

// column of item e of a tile in the staged V^T rows: bits 2 and 3 swapped
__device__ __forceinline__ int dw_col(int e) { return (e & ~15) | (e & 3) | ((e & 4) << 1) | ((e & 8) >> 1); }

// Staging of a tile by NT threads: task (pr, cq) = items 2*pr, 2*pr + 1 of
// the tile, dims 8*cq .. +7 (32 x 16 tasks); thread t takes pr = t % 32 and
// cq = t / 32 + (NT / 32) * c.  An item is an entry (kind 0), a window token
// (1) or nothing (-1); each load reads a valid row.  A tile whose items are
// all entries (`full`, the same for every thread: most tiles of a long list)
// takes a path without the per-item source selects and masks.
template <int NT>
struct DwRegs {
  int4 v[512 / NT][2];
  int kind[2];
  bool full;
};

template <int NT>
__device__ __forceinline__ void dw_fetch(const AttendArgs& A, int b, int64_t wbase, int nkv, int t0, int L,
                                         DwRegs<NT>& R) {
  const int t = threadIdx.x, pr = t & 31, cq0 = t >> 5;
  R.full = t0 + MT_TE <= nkv && t0 + MT_TE <= A.N_cap;      // (then also <= L)
  if (R.full) {
    const uint16_t* row = (const uint16_t*)A.kv + ((int64_t)b * A.N_cap + t0 + 2 * pr) * 128;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int c = 0; c < 512 / NT; ++c) R.v[c][u] = *(const int4*)(row + u * 128 + (cq0 + (NT / 32) * c) * 8);
      R.kind[u] = 0;
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p = t0 + 2 * pr + u;
    const int kind = p < L ? (p < nkv ? (p < A.N_cap ? 0 : -1) : 1) : -1;
    const uint16_t* row = kind == 1 ? (const uint16_t*)A.win + (wbase + (p - nkv)) * 128
                                    : (const uint16_t*)A.kv + ((int64_t)b * A.N_cap + (kind == 0 ? p : 0)) * 128;
#pragma unroll
    for (int c = 0; c < 512 / NT; ++c) R.v[c][u] = *(const int4*)(row + (cq0 + (NT / 32) * c) * 8);
    R.kind[u] = kind;
  }
}

template <int NT, bool FULL>
__device__ __forceinline__ void dw_store_t(const DwRegs<NT>& R, DwShared::Tile& T) {
  const int t = threadIdx.x, pr = t & 31, cq0 = t >> 5;
  uint32_t* vt = (uint32_t*)T.Vt + dw_col(2 * pr) / 2;
#pragma unroll
  for (int c = 0; c < 512 / NT; ++c) {
    const int cq = cq0 + (NT / 32) * c;
    int4 v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      v[u] = FULL || R.kind[u] >= 0 ? R.v[c][u] : make_int4(0, 0, 0, 0);
      *(int4*)&T.Kl[(2 * pr + u) * DW_KROW + cq * 8] = v[u];
    }
    // V^T: dword (row d, column pair) = dim d of items 2pr (low half) and 2pr + 1
    const uint32_t* a = (const uint32_t*)&v[0];
    const uint32_t* e = (const uint32_t*)&v[1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      vt[(cq * 8 + 2 * q) * (DW_VROW / 2)] = __builtin_amdgcn_perm(e[q], a[q], 0x05040100u);
      vt[(cq * 8 + 2 * q + 1) * (DW_VROW / 2)] = __builtin_amdgcn_perm(e[q], a[q], 0x07060302u);
    }
  }
  if (cq0 == 0) {
    T.okl[2 * pr] = FULL || R.kind[0] >= 0;
    T.okl[2 * pr + 1] = FULL || R.kind[1] >= 0;
  }
}

template <int NT>
__device__ __forceinline__ void dw_store(const DwRegs<NT>& R, DwShared::Tile& T) {
  if (R.full) dw_store_t<NT, true>(R, T);          // uniform
  else dw_store_t<NT, false>(R, T);
}

__device__ __forceinline__ void dw_store4(const AttendArgs& A, int64_t i, f32x16 acc, int j0, float f) {
  if (A.out_dt == DT_F32) {
    *(float4*)((float*)A.out + i) = make_float4(acc[j0] * f, acc[j0 + 1] * f, acc[j0 + 2] * f, acc[j0 + 3] * f);
  } else {
    const uint32_t lo = f32_to_bf16(acc[j0] * f) | ((uint32_t)f32_to_bf16(acc[j0 + 1] * f) << 16);
    const uint32_t hi = f32_to_bf16(acc[j0 + 2] * f) | ((uint32_t)f32_to_bf16(acc[j0 + 3] * f) << 16);
    *(uint2*)((uint16_t*)A.out + i) = make_uint2(lo, hi);
  }
}

// ---- the per-tile work of a wavefront (lane l: head half*32 + l % 32)

// S^T = K Q^T for the staged tile: items 32*ib .. +31 in s[ib]
__device__ __forceinline__ void dw_qk(const DwShared::Tile& T, const bf16x8 (&qv)[8], f32x16 (&s)[2]) {
  const int lane = threadIdx.x & 63, h = lane >> 5, n = lane & 31;
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int j = 0; j < 16; ++j) s[ib][j] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const bf16x8 kf = *(const bf16x8*)&T.Kl[(32 * ib + n) * DW_KROW + 16 * ks + 8 * h];
      s[ib] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qv[ks], s[ib], 0, 0, 0);
    }
}

// online softmax of the tile's logits (masked items -inf) for the lane's
// head (lanes n and n + 32 share it), then O^T += V^T P^T in steps of 16
// items.  exp2 is the hardware instruction: a weight below 2^-126 of the
// running reference contributes nothing.
__device__ __forceinline__ void dw_softmax_pv(const DwShared::Tile& T, f32x16 (&s)[2], float scale2, float& m_run,
                                              float& l_run, f32x16 (&acc)[4]) {
  const int lane = threadIdx.x & 63, h = lane >> 5, n = lane & 31;
  float tmax = -INFINITY;
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, s[ib][j]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
  // the reference max moves only when the tile's max exceeds it by more than
  // 8 (base 2): the weights then stay below 2^8 (exact range in bf16 and
  // fp32), and the accumulator is rescaled on few tiles
  const float m_new = (tmax * scale2 > m_run + 8.f) ? tmax * scale2 : m_run;
  const float mb = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m_run - mb);
  m_run = m_new;
  float lsum = 0.f;
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float pe = __builtin_amdgcn_exp2f(fmaf(s[ib][j], scale2, -mb));
      s[ib][j] = pe;
      lsum += pe;
    }
  l_run = l_run * alpha + lsum;
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) acc[m4] *= alpha;
  }
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    bf16x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = (__bf16)s[st >> 1][8 * (st & 1) + e];
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
      const bf16x8 vf = *(const bf16x8*)&T.Vt[(32 * m4 + n) * DW_VROW + 16 * st + 8 * h];
      acc[m4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[m4], 0, 0, 0);
    }
  }
}

// the sum over the two lanes of the head, the sink, the stores of row r
__device__ __forceinline__ void dw_finish(const AttendArgs& A, int r, int head, bool store, float m_run, float l_run,
                                          const f32x16 (&acc)[4]) {
  const int h = (threadIdx.x & 63) >> 5;
  l_run += __shfl_xor(l_run, 32, 64);
  if (!store) return;
  const float sk = A.sink[head] * LOG2E;
  const float M = fmaxf(m_run, sk);
  const float em = (m_run == -INFINITY) ? 0.f : exp2f(m_run - M);
  const float Z = exp2f(sk - M) + l_run * em;
  const float f = em / Z;
  const int64_t o0 = ((int64_t)r * 64 + head) * 128;
  // register 4*q + i of acc[m4] is dim 32*m4 + 8*q + 4*h + i
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4)
#pragma unroll
    for (int q = 0; q < 4; ++q) dw_store4(A, o0 + 32 * m4 + 8 * q + 4 * h, acc[m4], 4 * q, f);
  if (A.lse && h == 0) A.lse[(int64_t)r * 64 + head] = (M + log2f(Z)) * LN2;
}

__global__ __launch_bounds__(DW_NT, 512 / DW_NT) void attend_dense_wide_kernel(AttendArgs A) {
  __shared__ DwShared sm;
  const int ngrp = (A.Tq + DW_ROWS - 1) / DW_ROWS;
  const int b = blockIdx.x / ngrp;
  const int t0r = (blockIdx.x % ngrp) * DW_ROWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, n = lane & 31;
  const int qrow = wave >> 1, head = (wave & 1) * 32 + n;
  const bool rvalid = t0r + qrow < A.Tq;
  const int r = b * A.Tq + (rvalid ? t0r + qrow : t0r);
  const int nkv_r = att_nelig(A, r);
  const int2 ws_r = att_window(A, r);
  const int wb_r = ws_r.x, wl_r = ws_r.y;
  // the group's list bounds, the same for every wavefront
  int nkv = 0, wlo = 0x7FFFFFFF, whi = 0;
#pragma unroll
  for (int q = 0; q < DW_ROWS; ++q) {
    if (t0r + q >= A.Tq) break;
    const int rq = b * A.Tq + t0r + q;
    nkv = max(nkv, att_nelig(A, rq));
    const int2 wq = att_window(A, rq);
    wlo = min(wlo, wq.x);
    whi = max(whi, wq.x + wq.y);
  }
  if (whi < wlo) whi = wlo;
  const int L = nkv + (whi - wlo);
  const int64_t wbase = (int64_t)b * A.W_buf + wlo;

  // Q^T operand of step ks: head `head`, dims 16*ks + 8*h .. +7
  bf16x8 qv[8];
  {
    const uint16_t* qp = (const uint16_t*)A.q + ((int64_t)r * 64 + head) * 128 + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int4 v = *(const int4*)(qp + 16 * ks);
      qv[ks] = *(const bf16x8*)&v;
    }
  }
  const float scale2 = A.scale * LOG2E;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[m4][j] = 0.f;

  // tile 0 is staged before the loop; in the loop, after the barrier (every
  // wavefront is done with the tile before the current one, and tile t0 is
  // written), tile t0 + 64 goes to the other buffer, tile t0 + 128 is
  // requested, and tile t0 is computed
  DwRegs<DW_NT> R;
  if (L > 0) {
    dw_fetch(A, b, wbase, nkv, 0, L, R);
    dw_store(R, sm.t[0]);
    if (MT_TE < L) dw_fetch(A, b, wbase, nkv, MT_TE, L, R);
  }
  for (int t0 = 0, cur = 0; t0 < L; t0 += MT_TE, cur ^= 1) {
    __syncthreads();
    if (t0 + MT_TE < L) {
      dw_store(R, sm.t[cur ^ 1]);
      if (t0 + 2 * MT_TE < L) dw_fetch(A, b, wbase, nkv, t0 + 2 * MT_TE, L, R);
    }
    const DwShared::Tile& T = sm.t[cur];

    f32x16 s[2];
    dw_qk(T, qv, s);

    // ---- this lane's 32 items: 32*ib + 8*q + 4*h + i in register 4*q + i
    // of s[ib].  A tile inside the row's entries (and the cache) needs no
    // masks; otherwise an item counts if it was staged and belongs to the row
    if (!(t0 + MT_TE <= nkv_r && t0 + MT_TE <= A.N_cap)) {
      uint32_t okm = 0;
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int4 ok4 = *(const int4*)&T.okl[32 * ib + 8 * q + 4 * h];
          const int okv[4] = {ok4.x, ok4.y, ok4.z, ok4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int p = t0 + 32 * ib + 8 * q + 4 * h + i;
            const int wpos = wlo + (p - nkv);
            const bool o = okv[i] != 0 && rvalid && (p < nkv ? p < nkv_r : (wpos >= wb_r && wpos < wb_r + wl_r));
            okm |= (uint32_t)o << (16 * ib + 4 * q + i);
          }
        }
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[ib][j] = (okm >> (16 * ib + j)) & 1u ? s[ib][j] : -INFINITY;
    }

    dw_softmax_pv(T, s, scale2, m_run, l_run, acc);
  }

  dw_finish(A, r, head, rvalid, m_run, l_run, acc);
}

// ------------------------------------------------------------------------
// Sparse (CSA) rows of a prefill chunk: every row has its own list (its k
// selected entries, then its window), so a workgroup is one row: 2
// wavefronts of 32 heads, and its 128 threads stage each tile (4 tasks a
// thread: item pair t % 32, dims 8*(t/32 + 4c) .. +7).  The selected indices
// of a tile are requested one tile ahead of its entry rows.
// [release notes (agentlenshq.com), 壓縮稀疏注意力 (CSA): MQA over the
//  top-k entries chosen per query plus the sliding window and the sink.]
constexpr int DS_NT = 128;

struct DsRegs {
  int4 v[4][2];
  int kind[2];
};

__device__ __forceinline__ void ds_idx(const int32_t* idr, int k, int t0, int (&j)[2]) {
  const int pr = threadIdx.x & 31;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p = t0 + 2 * pr + u;
    j[u] = p < k ? idr[p] : -1;
  }
}

__device__ __forceinline__ void ds_fetch(const AttendArgs& A, int b, int64_t wbase, int t0, int L, const int (&j)[2],
                                         DsRegs& R) {
  const int t = threadIdx.x, pr = t & 31, cq0 = t >> 5;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p = t0 + 2 * pr + u;
    const int kind = p < A.k ? ((j[u] >= 0 && j[u] < A.N_cap) ? 0 : -1) : (p < L ? 1 : -1);
    const uint16_t* row = kind == 1 ? (const uint16_t*)A.win + (wbase + (p - A.k)) * 128
                                    : (const uint16_t*)A.kv + ((int64_t)b * A.N_cap + (kind == 0 ? j[u] : 0)) * 128;
#pragma unroll
    for (int c = 0; c < 4; ++c) R.v[c][u] = *(const int4*)(row + (cq0 + 4 * c) * 8);
    R.kind[u] = kind;
  }
}

__device__ __forceinline__ void ds_store(const DsRegs& R, DwShared::Tile& T) {
  const int t = threadIdx.x, pr = t & 31, cq0 = t >> 5;
  uint32_t* vt = (uint32_t*)T.Vt + dw_col(2 * pr) / 2;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int cq = cq0 + 4 * c;
    int4 v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      v[u] = R.kind[u] >= 0 ? R.v[c][u] : make_int4(0, 0, 0, 0);
      *(int4*)&T.Kl[(2 * pr + u) * DW_KROW + cq * 8] = v[u];
    }
    const uint32_t* a = (const uint32_t*)&v[0];
    const uint32_t* e = (const uint32_t*)&v[1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      vt[(cq * 8 + 2 * q) * (DW_VROW / 2)] = __builtin_amdgcn_perm(e[q], a[q], 0x05040100u);
      vt[(cq * 8 + 2 * q + 1) * (DW_VROW / 2)] = __builtin_amdgcn_perm(e[q], a[q], 0x07060302u);
    }
  }
  if (cq0 == 0) {
    T.okl[2 * pr] = R.kind[0] >= 0;
    T.okl[2 * pr + 1] = R.kind[1] >= 0;
  }
}

__global__ __launch_bounds__(DS_NT) __attribute__((amdgpu_waves_per_eu(2))) void attend_sparse_wide_kernel(AttendArgs A) {
  __shared__ DwShared::Tile T;
  const int r = blockIdx.x;                    // query row b * Tq + t
  const int b = r / A.Tq;
  const int lane = threadIdx.x & 63, h = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int head = wave * 32 + n;
  const int2 ws_r = att_window(A, r);
  const int wb_r = ws_r.x, wl_r = ws_r.y;
  const int L = A.k + wl_r;
  const int64_t wbase = (int64_t)b * A.W_buf + wb_r;
  const int32_t* idr = A.idx + (int64_t)r * A.k;

  bf16x8 qv[8];
  {
    const uint16_t* qp = (const uint16_t*)A.q + ((int64_t)r * 64 + head) * 128 + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int4 v = *(const int4*)(qp + 16 * ks);
      qv[ks] = *(const bf16x8*)&v;
    }
  }
  const float scale2 = A.scale * LOG2E;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[m4][j] = 0.f;

  // tile t0's rows are in flight while tile t0 - 64 is computed; the indices
  // of tile t0 + 64 are requested with them
  DsRegs R;
  int jn[2];
  if (L > 0) {
    ds_idx(idr, A.k, 0, jn);
    ds_fetch(A, b, wbase, 0, L, jn, R);
    ds_idx(idr, A.k, MT_TE, jn);
  }
  for (int t0 = 0; t0 < L; t0 += MT_TE) {
    if (t0 > 0) __syncthreads();               // every wavefront is done with the previous tile
    ds_store(R, T);
    __syncthreads();
    if (t0 + MT_TE < L) {
      ds_fetch(A, b, wbase, t0 + MT_TE, L, jn, R);
      ds_idx(idr, A.k, t0 + 2 * MT_TE, jn);
    }
    f32x16 s[2];
    dw_qk(T, qv, s);
    // items that are not entries of the cache or window tokens (a -1 index,
    // past the list) are masked
    uint32_t okm = 0;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int4 ok4 = *(const int4*)&T.okl[32 * ib + 8 * q + 4 * h];
        okm |= ((uint32_t)(ok4.x != 0) | ((uint32_t)(ok4.y != 0) << 1) | ((uint32_t)(ok4.z != 0) << 2) |
                ((uint32_t)(ok4.w != 0) << 3)) << (16 * ib + 4 * q);
      }
    if (__ballot(okm != 0xFFFFFFFFu)) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[ib][j] = (okm >> (16 * ib + j)) & 1u ? s[ib][j] : -INFINITY;
    }
    dw_softmax_pv(T, s, scale2, m_run, l_run, acc);
  }
  dw_finish(A, r, head, true, m_run, l_run, acc);
}

bool attend_sparse_wide_applies(const AttendArgs& a) {
  return a.sparse && a.Hq == 64 && a.D == 128 && a.q_dt == DT_BF16 && a.win_dt == DT_BF16 && a.kv_dt == DT_BF16 &&
         a.scale > 0.f;
}

hipError_t launch_attend_sparse_wide(const AttendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attend_sparse_wide_kernel, dim3((unsigned)(a.B * a.Tq)), dim3(DS_NT), 0, s, a);
  return hipGetLastError();
}

// bf16 entries and window (the staging copies rows as they are), 64 heads of
// 128 dims, and a positive scale (the running max is taken before scaling).
bool attend_dense_wide_applies(const AttendArgs& a) {
  return !a.sparse && a.Hq == 64 && a.D == 128 && a.Tq >= DW_ROWS && a.q_dt == DT_BF16 && a.win_dt == DT_BF16 &&
         a.kv_dt == DT_BF16 && a.scale > 0.f;
}

hipError_t launch_attend_dense_wide(const AttendArgs& a, hipStream_t s) {
  const unsigned nblk = (unsigned)(a.B * ((a.Tq + DW_ROWS - 1) / DW_ROWS));
  hipLaunchKernelGGL(attend_dense_wide_kernel, dim3(nblk), dim3(DW_NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace lca
