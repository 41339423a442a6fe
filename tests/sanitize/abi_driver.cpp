// abi_driver.cpp -- drives every entry point of include/lca.h through valid
// calls (which reach the host stand-ins of abi_stubs.cpp instead of a GPU)
// and invalid ones (which must fail validation with the documented status),
// so that a build of csrc/abi.cpp with AddressSanitizer and
// UndefinedBehaviorSanitizer checks the C-ABI layer's own host code: argument
// validation, job marshalling, workspace checks and error reporting.  Device
// pointers are fake aligned addresses that the layer never dereferences.
// Test infrastructure: built and run by tests/test_sanitize.py.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/lca.h"

extern "C" int lca_stub_launches(void);

static int g_fail = 0;
#define EXPECT(call, want)                                                                       \
  do {                                                                                           \
    const int got_ = (int)(call);                                                               \
    if (got_ != (want)) {                                                                        \
      fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, got_, (want), \
              lca_last_error());                                                                 \
      g_fail = 1;                                                                                \
    }                                                                                            \
  } while (0)

// a fake device address; distinct offsets are 256 MiB apart, so no two
// buffers of the calls below overlap
static char* F(uintptr_t off = 0) { return (char*)(uintptr_t)(0x100000 + off * ((uintptr_t)1 << 28)); }

static lca_compress_job cjob(lca_dtype dst_dt, void* dst, void* sc, int64_t rows, int m = 4) {
  lca_compress_job j;
  memset(&j, 0, sizeof(j));
  j.x = F(1); j.x_dt = LCA_BF16; j.x_rows = 4096; j.gate = (const float*)F(2); j.pos_bias = (const float*)F(3);
  j.m = m; j.x_tok0 = (const int32_t*)F(4); j.nblk = (const int32_t*)F(5); j.dst_row0 = (const int64_t*)F(6);
  j.B = 4; j.nblk_max = 1; j.D = 128; j.dst = dst; j.dst_dt = dst_dt; j.dst_scale = sc; j.dst_rows = rows;
  return j;
}

static lca_attend_job ajob(int sparse, void* out, void* ws) {
  lca_attend_job a;
  memset(&a, 0, sizeof(a));
  a.sparse = sparse; a.q = F(20); a.q_dt = LCA_BF16; a.kv = F(21); a.kv_dt = LCA_FP8E4M3;
  a.kv_scale = (const float*)F(22); a.N_cap = sparse ? 262144 : 8192;
  a.idx = sparse ? (const int32_t*)F(23) : nullptr; a.k = sparse ? 1024 : 0;
  a.n_elig = (const int32_t*)F(24); a.win = F(25); a.win_dt = LCA_BF16; a.W_buf = 256;
  a.win_begin = (const int32_t*)F(26); a.win_len = (const int32_t*)F(27); a.sink = (const float*)F(28);
  a.scale = 0.088f; a.B = 4; a.Tq = 1; a.Hq = 64; a.D = 128; a.out = out; a.out_dt = LCA_BF16;
  a.ws = ws; a.ws_bytes = (size_t)1 << 30;
  return a;
}

static lca_index_job ijob() {
  lca_index_job i;
  memset(&i, 0, sizeof(i));
  i.qi = F(40); i.qi_dt = LCA_MXFP4; i.qi_scale = (const uint8_t*)F(41); i.w = (const float*)F(42);
  i.ki = F(43); i.ki_dt = LCA_MXFP4; i.ki_scale = (const uint8_t*)F(44); i.n_elig = (const int32_t*)F(45);
  i.B = 4; i.Tq = 1; i.H_I = 8; i.d_I = 128; i.N_cap = 262144; i.k = 1024; i.idx_out = (int32_t*)F(23);
  i.ws = F(47); i.ws_bytes = (size_t)1 << 30;
  return i;
}

int main() {
  EXPECT(lca_abi_version(), 3);
  // compress: valid, then invalid
  EXPECT(lca_csa_compress(F(1), LCA_F32, 64, (float*)F(2), (float*)F(3), 4, (int32_t*)F(4), (int32_t*)F(5),
                          (int64_t*)F(6), 2, 16, 128, F(7), LCA_FP8E4M3, F(8), 16, nullptr, nullptr), 0);
  EXPECT(lca_hca_compress(F(1), LCA_BF16, 4096, (float*)F(2), (float*)F(3), 128, (int32_t*)F(4), (int32_t*)F(5),
                          (int64_t*)F(6), 2, 32, 128, F(7), LCA_MXFP4, F(8), 32, (float*)F(9), nullptr), 0);
  EXPECT(lca_csa_compress(nullptr, LCA_F32, 64, (float*)F(2), (float*)F(3), 4, (int32_t*)F(4), (int32_t*)F(5),
                          (int64_t*)F(6), 2, 16, 128, F(7), LCA_F32, nullptr, 16, nullptr, nullptr), 1);
  EXPECT(lca_csa_compress(F(1), LCA_F32, 64, (float*)F(2), (float*)F(3), 65, (int32_t*)F(4), (int32_t*)F(5),
                          (int64_t*)F(6), 2, 1, 128, F(7), LCA_F32, nullptr, 16, nullptr, nullptr), 2);
  if (strlen(lca_last_error()) == 0) { fprintf(stderr, "no error message\n"); g_fail = 1; }
  // compress batch with the variants
  {
    lca_compress_job j[3] = {cjob(LCA_FP8E4M3, F(60), F(61), 262144), cjob(LCA_MXFP4, F(62), F(63), 262144),
                             cjob(LCA_FP8E4M3, F(64), F(65), 8192, 128)};
    j[1].gate_pc = 1; j[1].overlap = 4;
    EXPECT(lca_compress_batch(j, 3, nullptr), 0);
    EXPECT(lca_compress_batch(j, 0, nullptr), 1);
    EXPECT(lca_compress_batch(j, 9, nullptr), 1);
    j[2].D = 64;
    EXPECT(lca_compress_batch(j, 3, nullptr), 2);
  }
  // indexer
  EXPECT(lca_lightning_index_topk(F(40), LCA_MXFP4, (uint8_t*)F(41), (float*)F(42), F(43), LCA_MXFP4,
                                  (uint8_t*)F(44), (int32_t*)F(45), 4, 1, 8, 128, 262144, 1024, (int32_t*)F(46),
                                  (double*)F(49), F(47), (size_t)1 << 30, nullptr), 0);
  EXPECT(lca_lightning_index_topk(F(40), LCA_F32, nullptr, (float*)F(42), F(43), LCA_F32, nullptr,
                                  (int32_t*)F(45), 1, 1, 4, 64, 1024, 64, (int32_t*)F(46), nullptr, F(47),
                                  (size_t)1 << 30, nullptr), 0);
  EXPECT(lca_lightning_index_topk(F(40), LCA_F32, nullptr, (float*)F(42), F(43), LCA_F32, nullptr,
                                  (int32_t*)F(45), 1, 1, 17, 64, 1024, 64, (int32_t*)F(46), nullptr, F(47),
                                  (size_t)1 << 30, nullptr), 2);
  EXPECT(lca_lightning_index_topk(F(40), LCA_MXFP4, (uint8_t*)F(41), (float*)F(42), F(43), LCA_MXFP4,
                                  (uint8_t*)F(44), (int32_t*)F(45), 4, 1, 8, 128, 262144, 1024, (int32_t*)F(46),
                                  nullptr, F(47), 16, nullptr), 4);
  if (lca_index_topk_ws(4, 1, 8, 128, 262144, 1024) == 0) { fprintf(stderr, "zero workspace\n"); g_fail = 1; }
  // attention single calls
  EXPECT(lca_sparse_mqa_attend(F(20), LCA_BF16, F(21), LCA_FP8E4M3, (float*)F(22), 262144, (int32_t*)F(23), 1024,
                               F(25), LCA_BF16, 256, (int32_t*)F(26), (int32_t*)F(27), (float*)F(28), 0.088f, 4, 1,
                               64, 128, F(29), LCA_BF16, (float*)F(30), F(31), (size_t)1 << 30, nullptr), 0);
  EXPECT(lca_hca_attend(F(20), LCA_F32, F(21), LCA_F32, nullptr, 8192, (int32_t*)F(24), F(25), LCA_F32, 256,
                        (int32_t*)F(26), (int32_t*)F(27), (float*)F(28), 0.088f, 2, 3, 16, 128, F(29), LCA_F32,
                        nullptr, F(31), (size_t)1 << 30, nullptr), 0);
  EXPECT(lca_attend_separate_v(1, F(20), LCA_BF16, F(21), F(32), LCA_FP8E4M3, (float*)F(22), (float*)F(33),
                               262144, (int32_t*)F(23), 1024, nullptr, F(25), F(34), LCA_BF16, 256,
                               (int32_t*)F(26), (int32_t*)F(27), (float*)F(28), 0.088f, 4, 1, 64, 128, F(29),
                               LCA_BF16, nullptr, F(31), (size_t)1 << 30, nullptr), 0);
  EXPECT(lca_window_attend(F(20), LCA_BF16, F(25), LCA_BF16, 256, (int32_t*)F(26), (int32_t*)F(27), (float*)F(28),
                           0.088f, 4, 1, 64, 128, F(29), LCA_BF16, nullptr, F(31), (size_t)1 << 30, nullptr), 0);
  EXPECT(lca_sparse_mqa_attend(F(20), LCA_BF16, F(21), LCA_FP8E4M3, (float*)F(22), 262144, (int32_t*)F(23), 1024,
                               F(25), LCA_BF16, 256, (int32_t*)F(26), (int32_t*)F(27), (float*)F(28), 0.088f, 4, 1,
                               64, 64, F(29), LCA_BF16, (float*)F(30), F(31), (size_t)1 << 30, nullptr), 2);
  if (lca_attend_ws(4, 1, 64, 128, 1024, 128) == 0) { fprintf(stderr, "zero attention workspace\n"); g_fail = 1; }
  // attention batch
  {
    lca_attend_job a[2] = {ajob(1, F(70), F(71)), ajob(0, F(72), F(73))};
    EXPECT(lca_attend_batch(a, 2, nullptr), 0);
    EXPECT(lca_attend_batch(a, 5, nullptr), 1);
    a[1].Hq = 32;
    EXPECT(lca_attend_batch(a, 2, nullptr), 2);
  }
  // the decode step, its event and allocation-free forms, the append and the loop step
  {
    lca_compress_job c[3] = {cjob(LCA_FP8E4M3, F(21), F(22), 262144), cjob(LCA_MXFP4, F(43), F(44), 262144),
                             cjob(LCA_FP8E4M3, F(80), F(81), 8192, 128)};
    lca_index_job ix = ijob();
    lca_attend_job a[2] = {ajob(1, F(70), F(71)), ajob(0, F(72), F(73))};
    a[1].kv = F(80); a[1].kv_scale = (const float*)F(81);
    EXPECT(lca_decode_step(c, 3, &ix, a, 2, nullptr), 0);
    EXPECT(lca_decode_step(c, 3, nullptr, a + 1, 1, nullptr), 0);
    EXPECT(lca_decode_step_noalloc(c, 3, &ix, a, 2, nullptr), 0);
    void* ev[LCA_MAX_STEP_LAUNCHES + 1];
    for (int i = 0; i <= LCA_MAX_STEP_LAUNCHES; ++i) ev[i] = F(90 + i);
    const char* names[LCA_MAX_STEP_LAUNCHES];
    int32_t nl = -1;
    EXPECT(lca_decode_step_events(c, 3, &ix, a, 2, ev, LCA_MAX_STEP_LAUNCHES + 1, names, &nl, nullptr), 0);
    EXPECT(lca_decode_step_events(c, 3, &ix, a, 2, ev, 2, names, &nl, nullptr), 1);
    a[1].out = F(23);                                  // a dense job writing the indexer's output
    EXPECT(lca_decode_step(c, 3, &ix, a, 2, nullptr), 1);
    lca_append_job ap;
    memset(&ap, 0, sizeof(ap));
    ap.x_new = F(100); ap.x_dt = LCA_BF16; ap.g_new = (const float*)F(101); ap.ring = F(102);
    ap.gring = (float*)F(103); ap.R = 256; ap.len = (int64_t*)F(104); ap.m = 4; ap.W = 128;
    ap.x_tok0 = (int32_t*)F(105); ap.nblk = (int32_t*)F(106); ap.dst_row0 = (int64_t*)F(107);
    ap.n_elig = (int32_t*)F(108); ap.win_begin = (int32_t*)F(109); ap.win_len = (int32_t*)F(110);
    ap.B = 4; ap.D = 128;
    EXPECT(lca_decode_append(&ap, 1, nullptr), 0);
    ap.D = 96;
    EXPECT(lca_decode_append(&ap, 1, nullptr), 2);
  }
  if (lca_stub_launches() < 10) { fprintf(stderr, "only %d launches reached\n", lca_stub_launches()); g_fail = 1; }
  if (!g_fail) printf("abi driver: ok (%d launches)\n", lca_stub_launches());
  return g_fail;
}
