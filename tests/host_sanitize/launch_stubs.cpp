// Stand-ins for the kernel launch functions and the device-array entry point,
// for a host-only build of kk_host.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer.  The host ABI tests never reach a launch; each
// stand-in aborts with a message so that one which does fails loudly.
#include <cstdio>
#include <cstdlib>

#include "kk.h"
#include "kk_internal.h"

namespace {
[[noreturn]] void reached(const char* what) {
  std::fprintf(stderr, "host-only build: %s reached (no kernels in this build)\n", what);
  std::abort();
}
}  // namespace

namespace kk {
hipError_t launch_write(const WriteArgs&, hipStream_t) { reached("launch_write"); }
hipError_t launch_gqa_write(const GqaWriteArgs&, hipStream_t) { reached("launch_gqa_write"); }
hipError_t launch_append(const AppendArgs&, hipStream_t) { reached("launch_append"); }
hipError_t launch_epilogue_gemm(const EpiArgs&, hipStream_t) { reached("launch_epilogue_gemm"); }
hipError_t launch_epilogue_gemm_wide(const EpiArgs&, hipStream_t) { reached("launch_epilogue_gemm_wide"); }
hipError_t launch_decode(const DecodeArgs&, const DecodeLaunch&, hipStream_t) { reached("launch_decode"); }
hipError_t launch_store(uint32_t*, const uint32_t*, int64_t, hipStream_t) { reached("launch_store"); }
}  // namespace kk

extern "C" kk_status kk_decode_attn_noalloc(const kk_model_cfg*, const kk_cache*, int32_t, int32_t, const int32_t*,
                                            int32_t, const void*, const void*, kk_dtype, float*, int32_t,
                                            hipStream_t) {
  reached("kk_decode_attn_noalloc");
}
