// abi_stubs.cpp -- host-only stand-ins for the kernel launchers and the
// device-side helpers that the C-ABI layer (csrc/abi.cpp) calls, so that the
// layer can be built with AddressSanitizer and UndefinedBehaviorSanitizer and
// exercised on a machine without a GPU.  Each launcher counts its call and
// returns success; the workspace sizes follow a simple fixed rule.  Test
// infrastructure: built and run by tests/test_sanitize.py.
#include "../../long_context_attention_13_amd/csrc/lca_internal.h"

namespace lca {

int g_launches = 0;
static char g_scratch[256];

hipError_t launch_compress(const CompressArgs& a, hipStream_t) { g_launches += a.B > 0; return hipSuccess; }
hipError_t launch_compress_batch(const CompressBatch& bt, hipStream_t) { g_launches += bt.njobs > 0; return hipSuccess; }
size_t index_ws_bytes(int B, int Tq, int H, int d, int64_t N_cap, int k, int dt) {
  (void)H; (void)d; (void)k; (void)dt;
  return 256 + (size_t)B * Tq * (size_t)(N_cap / 64 + 1) * 64;
}
hipError_t launch_index(const IndexArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
size_t attend_ws_bytes(int B, int Tq, int Hq, int D, int64_t n_kv_max, int64_t W_buf) {
  const int64_t L = n_kv_max + W_buf;
  return L <= 128 || Tq >= 64 ? 0 : (size_t)B * Tq * Hq * (D + 2) * 4 * (size_t)((L + 63) / 64);
}
hipError_t launch_attend(const AttendArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
bool attend_batchable(const AttendArgs& a) {
  return a.q_dt == DT_BF16 && a.win_dt == DT_BF16 && (a.kv_dt == DT_BF16 || a.kv_dt == DT_FP8) && !a.v &&
         a.Tq < 64;
}
hipError_t launch_attend_batch(const AttendBatch&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode_append(const AppendBatch&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t noalloc_scratch(void** ptr) { *ptr = g_scratch; return hipSuccess; }
hipError_t launch_decode_step(const AppendBatch*, const AppendMap*, const CompressBatch&, const IndexArgs&,
                              const AttendBatch&, hipStream_t, LaunchLog* lg) {
  ++g_launches;
  if (lg) lg->n = 0;
  return hipSuccess;
}

}  // namespace lca

extern "C" int lca_stub_launches(void) { return lca::g_launches; }
