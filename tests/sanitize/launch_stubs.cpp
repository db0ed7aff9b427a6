// Host-only stand-ins for the kernel launchers of the C ABI layer, for the
// sanitizer build of its argument validation (no GPU, no device code): each
// records that it was reached and returns the status the driver asks for.
#include "launch.hpp"

extern "C" int g_stub_calls;
extern "C" int g_stub_status;
extern "C" void* g_stub_ws;  // the workspace the last prefill launcher was given
int g_stub_calls = 0;
int g_stub_status = 0;
void* g_stub_ws = nullptr;
extern "C" void* const g_stub_scratch;
void* const g_stub_scratch = (void*)(uintptr_t(5) << 40);

namespace qgemv {

static hipError_t reached() {
  ++g_stub_calls;
  return (hipError_t)g_stub_status;
}

hipError_t launch_q4k_gemv(const void*, const void*, const OutF32&, int64_t, int64_t, hipStream_t) { return reached(); }
hipError_t launch_q4k_gemv(const void*, const void*, const OutEx&, int64_t, int64_t, hipStream_t) { return reached(); }
hipError_t launch_nvfp4_gemv(const void*, const void*, const OutF32&, int64_t, int64_t, hipStream_t) { return reached(); }
hipError_t launch_nvfp4_gemv(const void*, const void*, const OutEx&, int64_t, int64_t, hipStream_t) { return reached(); }
hipError_t launch_tq1_gemv(const void*, const void*, const OutF32&, int64_t, int64_t, hipStream_t) { return reached(); }
hipError_t launch_tq1_gemv(const void*, const void*, const OutEx&, int64_t, int64_t, hipStream_t) { return reached(); }
hipError_t launch_dense_gemv(bool, const void*, const void*, const OutF32&, int64_t, int64_t, hipStream_t) {
  return reached();
}
hipError_t launch_dense_gemv(bool, const void*, const void*, const OutEx&, int64_t, int64_t, hipStream_t) {
  return reached();
}
hipError_t launch_q4k_get_rows(const void*, int64_t, int64_t, const int32_t*, int64_t, void*, int, hipStream_t) {
  return reached();
}
hipError_t launch_nvfp4_get_rows(const void*, int64_t, int64_t, const int32_t*, int64_t, void*, int, hipStream_t) {
  return reached();
}
hipError_t launch_tq1_get_rows(const void*, int64_t, int64_t, const int32_t*, int64_t, void*, int, hipStream_t) {
  return reached();
}
hipError_t launch_q4k_prefill(const void*, const void*, float*, int64_t, int64_t, int64_t, void* ws, hipStream_t) {
  g_stub_ws = ws;
  return reached();
}
hipError_t launch_nvfp4_prefill(const void*, const void*, float*, int64_t, int64_t, int64_t, void* ws, hipStream_t) {
  g_stub_ws = ws;
  return reached();
}
hipError_t launch_tq1_prefill(const void*, const void*, float*, int64_t, int64_t, int64_t, void* ws, hipStream_t) {
  g_stub_ws = ws;
  return reached();
}
hipError_t launch_read_ceiling(const void*, int64_t, float*, hipStream_t) { return reached(); }
int64_t read_sink_len(int64_t bytes) { return (bytes + 32767) / 32768; }
// stands in for the library's device array: a fixed fake address
hipError_t scratch_address(hipStream_t, void** ptr) {
  *ptr = g_stub_scratch;
  return hipSuccess;
}

}  // namespace qgemv
