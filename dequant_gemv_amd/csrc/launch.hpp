// Host-side launchers of the gfx950 kernels.  Arguments are validated by the
// C-ABI layer before these are called; each enqueues on `s` and returns the
// HIP status of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "epilogue.hpp"

namespace qgemv {

hipError_t launch_q4k_gemv(const void* w, const void* x, const OutF32& y, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_q4k_gemv(const void* w, const void* x, const OutEx& y, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_nvfp4_gemv(const void* w, const void* x, const OutF32& y, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_nvfp4_gemv(const void* w, const void* x, const OutEx& y, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_tq1_gemv(const void* w, const void* x, const OutF32& y, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_tq1_gemv(const void* w, const void* x, const OutEx& y, int64_t n, int64_t k, hipStream_t s);
// Largest K of the dense GEMV: the workgroup's activation copy (2K bytes,
// rounded up to 1 KiB) must fit in LDS.
constexpr int64_t kDenseMaxK = 65536;

hipError_t launch_dense_gemv(bool bf16, const void* w, const void* x, const OutF32& y, int64_t n, int64_t k,
                             hipStream_t s);
hipError_t launch_dense_gemv(bool bf16, const void* w, const void* x, const OutEx& y, int64_t n, int64_t k,
                             hipStream_t s);
// Rows rows[0..nrows) (rows == NULL: rows 0..nrows-1) of the weights as
// element type `dtype` (kF32 / kF16 / kBF16) into out[nrows][k].
hipError_t launch_q4k_get_rows(const void* w, int64_t n, int64_t k, const int32_t* rows, int64_t nrows, void* out,
                               int dtype, hipStream_t s);
hipError_t launch_nvfp4_get_rows(const void* w, int64_t n, int64_t k, const int32_t* rows, int64_t nrows,
                                 void* out, int dtype, hipStream_t s);
hipError_t launch_tq1_get_rows(const void* w, int64_t n, int64_t k, const int32_t* rows, int64_t nrows, void* out,
                               int dtype, hipStream_t s);
// Prefill: y[t][r] (fp32, [T][n]) = x[t] . dequant(W)[r] for T activation rows.
constexpr int64_t kPrefillMaxK = int64_t(1) << 20;
// Prefill; ws: NULL (K splits add into y with atomics) or a workspace of at
// least prefill_workspace_bytes(t, n, k) bytes (prefill_plan.hpp), whose
// contents need no initialisation (every byte read is written first).
hipError_t launch_q4k_prefill(const void* w, const void* x, float* y, int64_t t, int64_t n, int64_t k, void* ws,
                              hipStream_t s);
hipError_t launch_nvfp4_prefill(const void* w, const void* x, float* y, int64_t t, int64_t n, int64_t k, void* ws,
                                hipStream_t s);
hipError_t launch_tq1_prefill(const void* w, const void* x, float* y, int64_t t, int64_t n, int64_t k, void* ws,
                              hipStream_t s);
// The library's own prefill workspace: kScratchBytes of device memory per
// device, reserved until the process ends.  *ptr = its address on the device
// that runs stream s (looked up once per device, then cached).
constexpr int64_t kScratchBytes = int64_t(32) << 20;
hipError_t scratch_address(hipStream_t s, void** ptr);
hipError_t launch_read_ceiling(const void* buf, int64_t bytes, float* sink, hipStream_t s);
int64_t read_sink_len(int64_t bytes);

}  // namespace qgemv
