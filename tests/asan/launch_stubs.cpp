// Host-only stand-ins for the kernel launchers and the one HIP runtime call
// of the C-ABI front end, for an AddressSanitizer / UBSan build of api.cpp
// without device code. The host ABI tests only make calls that validation
// rejects, so any launch reaching these stubs is a failure: they abort.
#include <stdio.h>
#include <stdlib.h>

#include "qblk_internal.h"

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

namespace {
[[noreturn]] void launched(const char* what) {
  fprintf(stderr, "launch reached in a host-only test build: %s\n", what);
  abort();
}
}  // namespace

namespace qblk {
hipError_t launch_quantize_act(const float*, int64_t, int64_t, int64_t, void*, hipStream_t) {
  launched("quantize_act");
}
hipError_t launch_pack_weights(int, const float*, int64_t, int64_t, int64_t, void*, int64_t, hipStream_t) {
  launched("pack_weights");
}
hipError_t launch_kv_scores(int, const void*, int64_t, int64_t, int64_t, int64_t, const void*, int64_t, float*,
                            int64_t, hipStream_t) {
  launched("kv_scores");
}
hipError_t launch_gemv(int, const void*, int64_t, int64_t, const void*, int64_t, float*, int64_t, hipStream_t) {
  launched("gemv");
}
hipError_t launch_gemv_f32(int, const void*, int64_t, int64_t, const float*, int64_t, int64_t, float*, int64_t,
                           const GemvWork&, int64_t, hipStream_t) {
  launched("gemv_f32");
}
hipError_t gemv_scratch_work(hipStream_t, GemvWork*) { launched("gemv_scratch_work"); }
hipError_t launch_gemv_multi(int, const GemvDesc*, int, int64_t, hipStream_t) { launched("gemv_multi"); }
hipError_t launch_gemv_float(int, const void*, int64_t, int64_t, const float*, int64_t, int64_t, float*, int64_t,
                             hipStream_t) {
  launched("gemv_float");
}
hipError_t launch_gemm(int, const void*, int64_t, int64_t, const void*, int64_t, float*, int64_t, hipStream_t) {
  launched("gemm");
}
hipError_t launch_gemm_small(int, const void*, int64_t, int64_t, const void*, int64_t, float*, int64_t,
                             hipStream_t) {
  launched("gemm_small");
}
hipError_t launch_block_sums(int, const void*, int64_t, int64_t, const void*, int64_t, int32_t*, hipStream_t) {
  launched("block_sums");
}
}  // namespace qblk
