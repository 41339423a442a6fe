// lca_internal.h -- declarations shared by the C-ABI layer (abi.cpp) and the
// kernel translation units.  Not part of the public interface.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lca {

enum Dt : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_MXFP4 = 3 };

struct CompressArgs {
  const void* x; int x_dt; int64_t x_rows;
  const float* gate; const float* bias; int m;
  const int32_t* x_tok0; const int32_t* nblk; const int64_t* dst_row0;
  int B; int nblk_max; int D;
  void* dst; int dst_dt; void* dst_scale; int64_t dst_rows;
  float* pooled;
  int gate_pc;                        // 1: gate [B][x_rows][D], bias [m + overlap][D]
  int overlap;                        // block i pools m + overlap tokens from x_tok0 + i*m
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);

constexpr int MAX_COMPRESS_JOBS = 8;
struct CompressBatch {                // jobs share x_dt and D
  CompressArgs job[MAX_COMPRESS_JOBS];
  int njobs;
};
hipError_t launch_compress_batch(const CompressBatch& bt, hipStream_t s);

struct IndexArgs {
  const void* qi; int dt; const uint8_t* qi_scale;
  const float* w;
  const void* ki; const uint8_t* ki_scale;
  const int32_t* n_elig;
  int B, Tq, H, d; int64_t N_cap; int k;
  int32_t* idx_out; double* score_out;
  void* ws; size_t ws_bytes;
};
size_t index_ws_bytes(int B, int Tq, int H, int d, int64_t N_cap, int k, int dt);
hipError_t launch_index(const IndexArgs& a, hipStream_t s);

struct AttendArgs {
  const void* q; int q_dt;
  const void* kv; int kv_dt; const float* kv_scale; int64_t N_cap;
  int sparse;                         // 1: CSA list idx[r][0..k), 0: HCA entries 0..n_elig[r)
  const int32_t* idx; int k;
  const int32_t* n_elig;
  const void* win; int win_dt; int64_t W_buf;
  const int32_t* win_begin; const int32_t* win_len;
  const float* sink; float scale;
  int B, Tq, Hq, D;
  void* out; int out_dt; float* lse;
  void* ws; size_t ws_bytes;
  // separate values (NULL: one vector per item is key and value): layouts of
  // kv / kv_scale / win; not batched (single calls only)
  const void* v; const float* v_scale; const void* win_v;
};
size_t attend_ws_bytes(int B, int Tq, int Hq, int D, int64_t n_kv_max, int64_t W_buf);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);

constexpr int MAX_ATTEND_JOBS = 4;
struct AttendBatch {                  // jobs share kv_dt and Hq; plans filled by the launcher
  AttendArgs job[MAX_ATTEND_JOBS];
  int S[MAX_ATTEND_JOBS], items[MAX_ATTEND_JOBS];
  float* ml[MAX_ATTEND_JOBS];
  float* po[MAX_ATTEND_JOBS];
  int blk0[MAX_ATTEND_JOBS + 1], mblk0[MAX_ATTEND_JOBS + 1];
  int njobs;
};
bool attend_batchable(const AttendArgs& a);
hipError_t launch_attend_batch(const AttendBatch& bt, hipStream_t s);
// the stages of launch_attend_batch: plans (splits, partial buffers, block
// offsets), the attention launch over bt's blocks, the merge launch
void attend_batch_plan(AttendBatch& bt);
hipError_t launch_attend_batch_mfma(const AttendBatch& bt, hipStream_t s);
hipError_t launch_attend_batch_merge(const AttendBatch& bt, hipStream_t s);

// Token append of a decode loop (one new token per sequence and stream into
// a doubled ring of R rows, and the step's derived arguments).
struct AppendArgs {
  const void* x_new; int x_dt; const float* g_new;
  void* ring; float* gring; int64_t R;
  int64_t* len; int m; int W;
  int32_t* x_tok0; int32_t* nblk; int64_t* dst_row0; int32_t* n_elig;
  int32_t* win_begin; int32_t* win_len;
  int B, D;
  int overlap;                        // the stream's compress jobs pool m + overlap tokens
  int gate_pc;                        // 1: g_new [B][D], gring [B][2R][D]
};
constexpr int MAX_APPEND_JOBS = 8;
struct AppendBatch {
  AppendArgs job[MAX_APPEND_JOBS];
  int njobs;
};
hipError_t launch_decode_append(const AppendBatch& bt, hipStream_t s);

// The appends of a decode-loop step run in the compress launch: compress job
// j appends for append job of[j] (-1: none) before it compresses (the job
// reads that stream's ring and takes its block arguments from the append);
// the append jobs extra[0 .. nextra) that no compress job reads get blocks of
// their own in the same launch.
struct AppendMap {
  int of[MAX_COMPRESS_JOBS];
  int extra[MAX_APPEND_JOBS];
  int nextra;
};
hipError_t launch_append_compress(const AppendBatch& ab, const AppendMap& mp, const CompressBatch& cb,
                                  hipStream_t s);

// Scratch memory of the allocation-free decode step: a file-scope device
// array of NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.
// noalloc_scratch returns the current device's copy (its address is resolved
// once per device).
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

// Events recorded on the launch stream around the launches of a decode step
// (measurement): ev[0] before the first launch, ev[i] after launch i, whose
// kernel names[i - 1] names.  At most cap - 1 launches are logged.
struct LaunchLog {
  hipEvent_t* ev;
  int cap;
  int n;
  const char** names;
};
hipError_t log_start(LaunchLog* lg, hipStream_t s);
hipError_t log_launch(LaunchLog* lg, hipStream_t s, const char* name);

// One decode step: the compress jobs, the indexer call, the attention jobs, in
// that order and with the results of the three calls; the dense attention jobs
// may run beside the indexer's scan.
// With `app` (and its map) the appends run first, in the compress launch.
// With `lg`, events are recorded around the launches.
hipError_t launch_decode_step(const AppendBatch* app, const AppendMap* mp, const CompressBatch& cb,
                              const IndexArgs& ia, const AttendBatch& ab, hipStream_t s, LaunchLog* lg = nullptr);

}  // namespace lca
