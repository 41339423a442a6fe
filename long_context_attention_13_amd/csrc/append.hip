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
#include "append_body.h"

namespace lca {

__global__ __launch_bounds__(128) void decode_append_kernel(AppendBatch bt) {
  const AppendArgs& a = bt.job[blockIdx.y];
  if ((int)blockIdx.x < a.B) append_token(a, blockIdx.x);
}

hipError_t launch_decode_append(const AppendBatch& bt, hipStream_t s) {
  int gx = 0;
  for (int j = 0; j < bt.njobs; ++j) gx = bt.job[j].B > gx ? bt.job[j].B : gx;
  if (bt.njobs == 0 || gx == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_append_kernel, dim3((unsigned)gx, (unsigned)bt.njobs), dim3(128), 0, s, bt);
  return hipGetLastError();
}

}  // namespace lca
