// Host-side launchers of the gfx950 kernels.  Arguments are validated by the
// C-ABI layer before these are called; each enqueues on `s` and returns the
// HIP status of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qgemv {

hipError_t launch_q4k_gemv(const void* w, const void* x, float* y, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_nvfp4_gemv(const void* w, const void* x, float* y, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_tq1_gemv(const void* w, const void* x, float* y, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_q4k_dequant(const void* w, float* out, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_nvfp4_dequant(const void* w, float* out, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_tq1_dequant(const void* w, float* out, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_read_ceiling(const void* buf, int64_t bytes, float* sink, hipStream_t s);
int64_t read_sink_len(int64_t bytes);

}  // namespace qgemv
