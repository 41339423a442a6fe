// compress.hip -- softmax-gated pooling with positional bias, fused with the
// cache encoders (FP8 E4M3 + per-64 fp32 scale, MXFP4, bf16, fp32).
//
// [release notes (agentlenshq.com), 壓縮稀疏注意力 (CSA): KV compressed 4x along
//  the sequence by softmax-gated pooling with a learned positional bias;
//  重度壓縮注意力 (HCA): the same at 128x; 架構實現: most KV entries in FP8, the
//  indexer in FP4.]
//
// One workgroup pools one block of m raw tokens: the m gate weights are
// formed once in LDS, token rows are read in 16-byte pieces by token groups
// of threads and accumulated in fp32, the group partials are summed in LDS,
// and the encoder
// runs on the pooled row while it is still in registers: a wavefront is
// exactly one 64-channel FP8 scale group, a half wavefront one 32-channel MX
// block.  The kernel is HBM-bound (every raw token read once).
#include "append_body.h"
#include "compress_body.h"

namespace lca {

template <int XDT, int ODT, int D>
__global__ __launch_bounds__(PE_THREADS) void pool_encode_kernel(CompressArgs a) {
  __shared__ PeShared S;
  pool_encode_block<XDT, ODT, D>(a, blockIdx.y, blockIdx.x, S);
}

// Several compress calls in one launch: blockIdx.z is the job; every job has
// the input type XDT and width D, the output type is taken per job.
template <int XDT, int D>
__global__ __launch_bounds__(PE_THREADS) void pool_encode_batch_kernel(CompressBatch bt) {
  __shared__ PeShared S;
  const CompressArgs& a = bt.job[blockIdx.z];
  if ((int)blockIdx.y >= a.B || (int)blockIdx.x >= a.nblk_max) return;
  switch (a.dst_dt) {
    case DT_F32: pool_encode_block<XDT, DT_F32, D>(a, blockIdx.y, blockIdx.x, S); break;
    case DT_BF16: pool_encode_block<XDT, DT_BF16, D>(a, blockIdx.y, blockIdx.x, S); break;
    case DT_FP8: pool_encode_block<XDT, DT_FP8, D>(a, blockIdx.y, blockIdx.x, S); break;
    default: pool_encode_block<XDT, DT_MXFP4, D>(a, blockIdx.y, blockIdx.x, S); break;
  }
}

// The compress launch of a decode-loop step: blockIdx.z < njobs is compress
// job z, whose block 0 of sequence b first appends sequence b's new token to
// the job's ring (append job mp.of[z]) and then compresses with the block
// arguments it has just derived; z >= njobs is an append job that no compress
// job reads.  The append's barrier and the one below order its global writes
// before the workgroup reads them.
template <int XDT, int D>
__global__ __launch_bounds__(PE_THREADS) void append_compress_kernel(AppendBatch ab, AppendMap mp,
                                                                     CompressBatch bt) {
  __shared__ PeShared S;
  const int z = blockIdx.z, b = blockIdx.y, i = blockIdx.x;
  if (z >= bt.njobs) {
    const AppendArgs& a = ab.job[mp.extra[z - bt.njobs]];
    if (i == 0 && b < a.B) append_token(a, b);
    return;
  }
  const CompressArgs& a = bt.job[z];
  if (b >= a.B || i >= a.nblk_max) return;
  if (mp.of[z] >= 0) {
    append_token(ab.job[mp.of[z]], b);
    __syncthreads();
  }
  switch (a.dst_dt) {
    case DT_F32: pool_encode_block<XDT, DT_F32, D>(a, b, i, S); break;
    case DT_BF16: pool_encode_block<XDT, DT_BF16, D>(a, b, i, S); break;
    case DT_FP8: pool_encode_block<XDT, DT_FP8, D>(a, b, i, S); break;
    default: pool_encode_block<XDT, DT_MXFP4, D>(a, b, i, S); break;
  }
}

template <int XDT, int ODT>
static hipError_t launch_d(const CompressArgs& a, hipStream_t s) {
  dim3 grid(a.nblk_max, a.B);
  if (a.D == 64) hipLaunchKernelGGL((pool_encode_kernel<XDT, ODT, 64>), grid, dim3(PE_THREADS), 0, s, a);
  else hipLaunchKernelGGL((pool_encode_kernel<XDT, ODT, 128>), grid, dim3(PE_THREADS), 0, s, a);
  return hipGetLastError();
}

template <int XDT>
static hipError_t launch_o(const CompressArgs& a, hipStream_t s) {
  switch (a.dst_dt) {
    case DT_F32: return launch_d<XDT, DT_F32>(a, s);
    case DT_BF16: return launch_d<XDT, DT_BF16>(a, s);
    case DT_FP8: return launch_d<XDT, DT_FP8>(a, s);
    default: return launch_d<XDT, DT_MXFP4>(a, s);
  }
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (a.nblk_max == 0 || a.B == 0) return hipSuccess;
  return a.x_dt == DT_F32 ? launch_o<DT_F32>(a, s) : launch_o<DT_BF16>(a, s);
}

hipError_t launch_compress_batch(const CompressBatch& bt, hipStream_t s) {
  int gx = 0, gy = 0;
  for (int j = 0; j < bt.njobs; ++j) {
    gx = bt.job[j].nblk_max > gx ? bt.job[j].nblk_max : gx;
    gy = bt.job[j].B > gy ? bt.job[j].B : gy;
  }
  if (bt.njobs == 0 || gx == 0 || gy == 0) return hipSuccess;
  const dim3 grid(gx, gy, bt.njobs);
  const bool f32 = bt.job[0].x_dt == DT_F32, d64 = bt.job[0].D == 64;
  if (f32 && d64) hipLaunchKernelGGL((pool_encode_batch_kernel<DT_F32, 64>), grid, dim3(PE_THREADS), 0, s, bt);
  else if (f32) hipLaunchKernelGGL((pool_encode_batch_kernel<DT_F32, 128>), grid, dim3(PE_THREADS), 0, s, bt);
  else if (d64) hipLaunchKernelGGL((pool_encode_batch_kernel<DT_BF16, 64>), grid, dim3(PE_THREADS), 0, s, bt);
  else hipLaunchKernelGGL((pool_encode_batch_kernel<DT_BF16, 128>), grid, dim3(PE_THREADS), 0, s, bt);
  return hipGetLastError();
}

hipError_t launch_append_compress(const AppendBatch& ab, const AppendMap& mp, const CompressBatch& bt,
                                  hipStream_t s) {
  int gx = 1, gy = 0;
  for (int j = 0; j < bt.njobs; ++j) {
    gx = bt.job[j].nblk_max > gx ? bt.job[j].nblk_max : gx;
    gy = bt.job[j].B > gy ? bt.job[j].B : gy;
  }
  for (int e = 0; e < mp.nextra; ++e) gy = ab.job[mp.extra[e]].B > gy ? ab.job[mp.extra[e]].B : gy;
  const int gz = bt.njobs + mp.nextra;
  if (gz == 0 || gy == 0) return hipSuccess;
  const dim3 grid(gx, gy, gz);
  const bool f32 = bt.njobs > 0 && bt.job[0].x_dt == DT_F32, d64 = bt.njobs > 0 && bt.job[0].D == 64;
  if (f32 && d64) hipLaunchKernelGGL((append_compress_kernel<DT_F32, 64>), grid, dim3(PE_THREADS), 0, s, ab, mp, bt);
  else if (f32) hipLaunchKernelGGL((append_compress_kernel<DT_F32, 128>), grid, dim3(PE_THREADS), 0, s, ab, mp, bt);
  else if (d64) hipLaunchKernelGGL((append_compress_kernel<DT_BF16, 64>), grid, dim3(PE_THREADS), 0, s, ab, mp, bt);
  else hipLaunchKernelGGL((append_compress_kernel<DT_BF16, 128>), grid, dim3(PE_THREADS), 0, s, ab, mp, bt);
  return hipGetLastError();
}

}  // namespace lca
