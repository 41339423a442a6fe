// append.hip -- the token append of a decode loop: one new raw token per
// sequence and stream goes into a doubled ring, and the step's arguments
// for the compress jobs, the indexer and the attention are derived on the
// device (so that a captured step graph can be replayed step after step).
//
// [release notes (agentlenshq.com), 壓縮稀疏注意力 (CSA): the most recent
//  tokens stay uncompressed in a sliding window, and every complete block of
//  m tokens becomes one compressed entry (m = 4 for CSA, 128 for HCA).]
//
// Ring layout: token t of a sequence is stored at rows t % R and t % R + R
// of its [2R][D] ring (and of its [2R] gate ring), so that every run of at
// most R consecutive tokens -- a block being compressed, the window -- is
// one contiguous row range.
#include "lca_device.h"

namespace lca {

__global__ __launch_bounds__(128) void decode_append_kernel(AppendBatch bt) {
  const AppendArgs& a = bt.job[blockIdx.y];
  const int b = blockIdx.x;
  if (b >= a.B) return;
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
  __syncthreads();                        // every thread has read len[b]
  if (threadIdx.x != 0) return;
  if (a.g_new) {
    const float g = a.g_new[b];
    a.gring[row0] = g;
    a.gring[row1] = g;
  }
  const int64_t L = pos + 1;
  a.len[b] = L;
  if (a.m > 0) {
    if (a.nblk) a.nblk[b] = (L % a.m == 0) ? 1 : 0;
    if (a.x_tok0) a.x_tok0[b] = (int32_t)(L >= a.m ? (L - a.m) % a.R : 0);
    if (a.dst_row0) a.dst_row0[b] = L / a.m - 1 >= 0 ? L / a.m - 1 : 0;
    if (a.n_elig) a.n_elig[b] = (int32_t)(L / a.m);
  }
  if (a.win_begin) {
    const int64_t wl = L < a.W ? L : a.W;
    a.win_begin[b] = (int32_t)((L - wl) % a.R);
    a.win_len[b] = (int32_t)wl;
  }
}

hipError_t launch_decode_append(const AppendBatch& bt, hipStream_t s) {
  int gx = 0;
  for (int j = 0; j < bt.njobs; ++j) gx = bt.job[j].B > gx ? bt.job[j].B : gx;
  if (bt.njobs == 0 || gx == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_append_kernel, dim3((unsigned)gx, (unsigned)bt.njobs), dim3(128), 0, s, bt);
  return hipGetLastError();
}

}  // namespace lca
