// append_body.h -- the token append of one sequence of one raw-token stream,
// shared by the append kernel and the fused append + compress kernel.  The
// method, its source and the ring layout are described in append.hip.
#pragma once
#include "lca_device.h"

namespace lca {

// All threads of the workgroup take part (strided copy); the new length and
// the derived step arguments are written by thread 0 after a barrier, so
// every thread has read the old length first.  The caller puts a barrier
// after this before reading what it wrote.
__device__ __forceinline__ void append_token(const AppendArgs& a, int b) {
  const int64_t pos = a.len[b];          // the new token's position
  const int64_t r0 = pos % a.R;
  const int64_t row0 = (int64_t)b * 2 * a.R + r0, row1 = row0 + a.R;
  const int esz = a.x_dt == DT_F32 ? 4 : 2;
  const char* src = (const char*)a.x_new + (int64_t)b * a.D * esz;
  char* ring = (char*)a.ring;
  for (int i = threadIdx.x; i < a.D * esz / 4; i += blockDim.x) {
    const uint32_t v = ((const uint32_t*)src)[i];
    ((uint32_t*)(ring + row0 * a.D * esz))[i] = v;
    ((uint32_t*)(ring + row1 * a.D * esz))[i] = v;
  }
  if (a.g_new && a.gate_pc) {            // one gate logit per channel
    for (int i = threadIdx.x; i < a.D; i += blockDim.x) {
      const float g = a.g_new[(int64_t)b * a.D + i];
      a.gring[row0 * a.D + i] = g;
      a.gring[row1 * a.D + i] = g;
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  if (a.g_new && !a.gate_pc) {
    const float g = a.g_new[b];
    a.gring[row0] = g;
    a.gring[row1] = g;
  }
  const int64_t L = pos + 1;
  a.len[b] = L;
  if (a.m > 0) {
    if (a.nblk) a.nblk[b] = (L % a.m == 0) ? 1 : 0;
    // first ring row of the block's span (its m tokens and the overlap
    // tokens before them; for the first block those rows are not read)
    if (a.x_tok0) a.x_tok0[b] = (int32_t)(L >= a.m ? ((L - a.m - a.overlap) % a.R + a.R) % a.R : 0);
    if (a.dst_row0) a.dst_row0[b] = L / a.m - 1 >= 0 ? L / a.m - 1 : 0;
    if (a.n_elig) a.n_elig[b] = (int32_t)(L / a.m);
  }
  if (a.win_begin) {
    const int64_t wl = L < a.W ? L : a.W;
    a.win_begin[b] = (int32_t)((L - wl) % a.R);
    a.win_len[b] = (int32_t)wl;
  }
}

}  // namespace lca
