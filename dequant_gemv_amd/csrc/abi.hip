// C ABI of libqgemv: argument validation in plain host code, then one launch on
// the caller's stream.  See include/qgemv.h for the contract of each call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "prefill_plan.hpp"
#include "qgemv.h"

#ifndef QGEMV_BUILD_ID
#define QGEMV_BUILD_ID "unknown"
#endif

namespace {

thread_local int g_last_hip_error = 0;

// Largest K any entry point accepts: keeps every per-wave byte offset of the
// kernels' 32-bit buffer descriptors below 2^31.
constexpr int64_t kMaxK = int64_t(1) << 24;
constexpr int64_t kMaxM = (int64_t(1) << 31) - 1;

enum Fmt { kQ4k, kNvfp4, kTq1, kDenseF16, kDenseBF16 };

bool dense(Fmt f) { return f == kDenseF16 || f == kDenseBF16; }

int64_t k_multiple(Fmt f) {
  switch (f) {
    case kNvfp4: return 32;
    case kDenseF16:
    case kDenseBF16: return 8;
    default: return 256;
  }
}

int64_t k_max(Fmt f) { return dense(f) ? qgemv::kDenseMaxK : kMaxK; }

int64_t weight_bytes(Fmt f, int64_t m, int64_t k) {
  switch (f) {
    case kQ4k: return m * (k / 256) * 144;
    case kTq1: return m * (k / 256) * 54;
    case kNvfp4: return m * (k / 2) + m * (k / 16);
    default: return 2 * m * k;
  }
}

bool valid_dtype(int32_t t) { return t == QGEMV_F32 || t == QGEMV_F16 || t == QGEMV_BF16; }

int64_t dtype_size(int32_t t) { return t == QGEMV_F32 ? 4 : 2; }

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

int check_shape(Fmt f, int64_t m, int64_t k) {
  if (m < 0 || m > kMaxM || k <= 0 || k > k_max(f) || k % k_multiple(f) != 0) return QGEMV_E_SHAPE;
  return QGEMV_OK;
}

int finish(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return QGEMV_E_HIP;
  }
  return QGEMV_OK;
}

template <typename Out>
hipError_t launch_gemv(Fmt f, const void* w, const void* x, const Out& y, int64_t m, int64_t k, hipStream_t s) {
  switch (f) {
    case kQ4k: return qgemv::launch_q4k_gemv(w, x, y, m, k, s);
    case kNvfp4: return qgemv::launch_nvfp4_gemv(w, x, y, m, k, s);
    case kTq1: return qgemv::launch_tq1_gemv(w, x, y, m, k, s);
    default: return qgemv::launch_dense_gemv(f == kDenseBF16, w, x, y, m, k, s);
  }
}

int gemv(Fmt f, const void* w, const void* x, float* y, int64_t m, int64_t k, hipStream_t s) {
  int rc = check_shape(f, m, k);
  if (rc != QGEMV_OK) return rc;
  if (m == 0) return QGEMV_OK;
  if (!w || !x || !y) return QGEMV_E_NULL;
  if (misaligned(w, 16) || misaligned(x, 16) || misaligned(y, 4)) return QGEMV_E_ALIGN;
  if (overlap(y, m * 4, w, weight_bytes(f, m, k)) || overlap(y, m * 4, x, k * 2)) return QGEMV_E_ALIAS;
  return finish(launch_gemv(f, w, x, qgemv::OutF32{y}, m, k, s));
}

int gemv_ex(Fmt f, const void* w, const void* x, void* y, int64_t m, int64_t k, const qgemv_epilogue* ep,
            hipStream_t s) {
  const qgemv_epilogue plain = {1.f, 0.f, nullptr, QGEMV_F32, QGEMV_F32};
  const qgemv_epilogue e = ep ? *ep : plain;
  int rc = check_shape(f, m, k);
  if (rc != QGEMV_OK) return rc;
  if (!valid_dtype(e.y_dtype) || (e.beta != 0.f && !valid_dtype(e.c_dtype))) return QGEMV_E_DTYPE;
  if (m == 0) return QGEMV_OK;
  const bool use_c = e.beta != 0.f;
  if (!w || !x || !y || (use_c && !e.c)) return QGEMV_E_NULL;
  const int64_t ysz = dtype_size(e.y_dtype);
  if (misaligned(w, 16) || misaligned(x, 16) || misaligned(y, (uintptr_t)ysz)) return QGEMV_E_ALIGN;
  if (use_c && misaligned(e.c, (uintptr_t)dtype_size(e.c_dtype))) return QGEMV_E_ALIGN;
  if (overlap(y, m * ysz, w, weight_bytes(f, m, k)) || overlap(y, m * ysz, x, k * 2)) return QGEMV_E_ALIAS;
  if (use_c && overlap(y, m * ysz, e.c, m * dtype_size(e.c_dtype)) && !(e.c == y && e.c_dtype == e.y_dtype))
    return QGEMV_E_ALIAS;
  const qgemv::OutEx out{y, use_c ? e.c : nullptr, e.alpha, e.beta, use_c ? (int)e.c_dtype : (int)QGEMV_F32,
                         (int)e.y_dtype};
  return finish(launch_gemv(f, w, x, out, m, k, s));
}

int get_rows(Fmt f, const void* w, int64_t m, int64_t k, const int32_t* rows, int64_t nrows, void* out,
             int32_t dtype, hipStream_t s) {
  int rc = check_shape(f, m, k);
  if (rc != QGEMV_OK) return rc;
  if (nrows < 0 || nrows > kMaxM || (!rows && nrows > m)) return QGEMV_E_SHAPE;
  if (!valid_dtype(dtype)) return QGEMV_E_DTYPE;
  if (nrows == 0) return QGEMV_OK;
  // tasks of 16 output bytes each, in workgroups of up to 256
  const int64_t tasks = k * dtype_size(dtype) / 16;
  const int64_t per_wg = tasks < 256 ? tasks : 256;
  if (nrows * ((tasks + per_wg - 1) / per_wg) > kMaxM) return QGEMV_E_SHAPE;
  if ((m > 0 && !w) || !out) return QGEMV_E_NULL;
  if (misaligned(w, 16) || misaligned(out, 16) || misaligned(rows, 4)) return QGEMV_E_ALIGN;
  const int64_t out_bytes = nrows * k * dtype_size(dtype);
  if (overlap(out, out_bytes, w, weight_bytes(f, m, k)) || (rows && overlap(out, out_bytes, rows, nrows * 4)))
    return QGEMV_E_ALIAS;
  switch (f) {
    case kQ4k: return finish(qgemv::launch_q4k_get_rows(w, m, k, rows, nrows, out, dtype, s));
    case kNvfp4: return finish(qgemv::launch_nvfp4_get_rows(w, m, k, rows, nrows, out, dtype, s));
    default: return finish(qgemv::launch_tq1_get_rows(w, m, k, rows, nrows, out, dtype, s));
  }
}

// Where the partial sums of tiles split over K go: added into y with atomics
// (qgemm_*), a caller's workspace (qgemm_*_ws) or the library's own array
// (qgemm_q4k_noalloc).
enum Split { kAtomics, kCallerWs, kScratchWs };

int gemm(Fmt f, const void* w, const void* x, float* y, int64_t t, int64_t m, int64_t k, Split mode, void* ws,
         int64_t ws_bytes, hipStream_t s) {
  int rc = check_shape(f, m, k);
  if (rc != QGEMV_OK) return rc;
  // the grid's y dimension counts tiles of 256 or 512 activation rows (at
  // most 65535); an activation tile spans at most 512 * 2K <= 2^30 bytes
  if (t < 0 || t > 65535 * int64_t(128) || k > qgemv::kPrefillMaxK) return QGEMV_E_SHAPE;
  if (f == kNvfp4 && k % 64 != 0) return QGEMV_E_SHAPE;  // whole 64-weight steps
  if (t == 0 || m == 0) return QGEMV_OK;
  if (!w || !x || !y) return QGEMV_E_NULL;
  if (misaligned(w, 16) || misaligned(x, 16) || misaligned(y, 4)) return QGEMV_E_ALIGN;
  const int64_t yb = t * m * 4, wb = weight_bytes(f, m, k), xb = t * k * 2;
  if (overlap(y, yb, w, wb) || overlap(y, yb, x, xb)) return QGEMV_E_ALIAS;
  void* wsp = nullptr;
  const int64_t need = mode == kAtomics ? 0 : qgemv::prefill_workspace_bytes(t, m, k);
  if (need > 0 && mode == kCallerWs) {
    if (!ws) return QGEMV_E_NULL;
    if (misaligned(ws, 256)) return QGEMV_E_ALIGN;
    if (ws_bytes < need) return QGEMV_E_WORKSPACE;
    if (overlap(ws, need, y, yb) || overlap(ws, need, w, wb) || overlap(ws, need, x, xb)) return QGEMV_E_ALIAS;
    wsp = ws;
  } else if (need > 0) {
    if (need > qgemv::kScratchBytes) return QGEMV_E_WORKSPACE;
    const hipError_t e = qgemv::scratch_address(s, &wsp);
    if (e != hipSuccess) return finish(e);
  }
  switch (f) {
    case kQ4k: return finish(qgemv::launch_q4k_prefill(w, x, y, t, m, k, wsp, s));
    case kNvfp4: return finish(qgemv::launch_nvfp4_prefill(w, x, y, t, m, k, wsp, s));
    case kTq1: return finish(qgemv::launch_tq1_prefill(w, x, y, t, m, k, wsp, s));
    default: return QGEMV_E_SHAPE;
  }
}

int dequant(Fmt f, const void* w, float* out, int64_t m, int64_t k, hipStream_t s) {
  int rc = check_shape(f, m, k);
  if (rc != QGEMV_OK) return rc;
  if (m == 0) return QGEMV_OK;
  if (!w || !out) return QGEMV_E_NULL;
  return get_rows(f, w, m, k, nullptr, m, out, QGEMV_F32, s);
}

}  // namespace

extern "C" {

int qgemv_q4k(const void* w, const void* x, float* y, int64_t M, int64_t K, struct ihipStream_t* s) {
  return gemv(kQ4k, w, x, y, M, K, s);
}
int qgemv_nvfp4(const void* w, const void* x, float* y, int64_t M, int64_t K, struct ihipStream_t* s) {
  return gemv(kNvfp4, w, x, y, M, K, s);
}
int qgemv_tq1(const void* w, const void* x, float* y, int64_t M, int64_t K, struct ihipStream_t* s) {
  return gemv(kTq1, w, x, y, M, K, s);
}
int qdequant_q4k(const void* w, float* out, int64_t M, int64_t K, struct ihipStream_t* s) {
  return dequant(kQ4k, w, out, M, K, s);
}
int qdequant_nvfp4(const void* w, float* out, int64_t M, int64_t K, struct ihipStream_t* s) {
  return dequant(kNvfp4, w, out, M, K, s);
}
int qdequant_tq1(const void* w, float* out, int64_t M, int64_t K, struct ihipStream_t* s) {
  return dequant(kTq1, w, out, M, K, s);
}

int qgemv_q4k_ex(const void* w, const void* x, void* y, int64_t M, int64_t K, const qgemv_epilogue* ep,
                 struct ihipStream_t* s) {
  return gemv_ex(kQ4k, w, x, y, M, K, ep, s);
}
int qgemv_nvfp4_ex(const void* w, const void* x, void* y, int64_t M, int64_t K, const qgemv_epilogue* ep,
                   struct ihipStream_t* s) {
  return gemv_ex(kNvfp4, w, x, y, M, K, ep, s);
}
int qgemv_tq1_ex(const void* w, const void* x, void* y, int64_t M, int64_t K, const qgemv_epilogue* ep,
                 struct ihipStream_t* s) {
  return gemv_ex(kTq1, w, x, y, M, K, ep, s);
}
int qgemv_f16(const void* w, const void* x, float* y, int64_t M, int64_t K, struct ihipStream_t* s) {
  return gemv(kDenseF16, w, x, y, M, K, s);
}
int qgemv_bf16(const void* w, const void* x, float* y, int64_t M, int64_t K, struct ihipStream_t* s) {
  return gemv(kDenseBF16, w, x, y, M, K, s);
}
int qgemv_f16_ex(const void* w, const void* x, void* y, int64_t M, int64_t K, const qgemv_epilogue* ep,
                 struct ihipStream_t* s) {
  return gemv_ex(kDenseF16, w, x, y, M, K, ep, s);
}
int qgemv_bf16_ex(const void* w, const void* x, void* y, int64_t M, int64_t K, const qgemv_epilogue* ep,
                  struct ihipStream_t* s) {
  return gemv_ex(kDenseBF16, w, x, y, M, K, ep, s);
}
int qget_rows_q4k(const void* w, int64_t M, int64_t K, const int32_t* rows, int64_t nrows, void* out,
                  int32_t out_dtype, struct ihipStream_t* s) {
  return get_rows(kQ4k, w, M, K, rows, nrows, out, out_dtype, s);
}
int qget_rows_nvfp4(const void* w, int64_t M, int64_t K, const int32_t* rows, int64_t nrows, void* out,
                    int32_t out_dtype, struct ihipStream_t* s) {
  return get_rows(kNvfp4, w, M, K, rows, nrows, out, out_dtype, s);
}
int qget_rows_tq1(const void* w, int64_t M, int64_t K, const int32_t* rows, int64_t nrows, void* out,
                  int32_t out_dtype, struct ihipStream_t* s) {
  return get_rows(kTq1, w, M, K, rows, nrows, out, out_dtype, s);
}

int qgemm_q4k(const void* w, const void* x, float* y, int64_t T, int64_t M, int64_t K, struct ihipStream_t* s) {
  return gemm(kQ4k, w, x, y, T, M, K, kAtomics, nullptr, 0, s);
}
int qgemm_nvfp4(const void* w, const void* x, float* y, int64_t T, int64_t M, int64_t K, struct ihipStream_t* s) {
  return gemm(kNvfp4, w, x, y, T, M, K, kAtomics, nullptr, 0, s);
}
int qgemm_tq1(const void* w, const void* x, float* y, int64_t T, int64_t M, int64_t K, struct ihipStream_t* s) {
  return gemm(kTq1, w, x, y, T, M, K, kAtomics, nullptr, 0, s);
}

int64_t qgemm_workspace_bytes(int64_t T, int64_t M, int64_t K) {
  if (T < 0 || M < 0 || K <= 0 || T > 65535 * int64_t(128) || M > (int64_t(1) << 31) || K > qgemv::kPrefillMaxK)
    return QGEMV_E_SHAPE;
  return qgemv::prefill_workspace_bytes(T, M, K);
}
int qgemm_q4k_ws(const void* w, const void* x, float* y, int64_t T, int64_t M, int64_t K, void* ws, int64_t ws_bytes,
                 struct ihipStream_t* s) {
  return gemm(kQ4k, w, x, y, T, M, K, kCallerWs, ws, ws_bytes, s);
}
int qgemm_nvfp4_ws(const void* w, const void* x, float* y, int64_t T, int64_t M, int64_t K, void* ws,
                   int64_t ws_bytes, struct ihipStream_t* s) {
  return gemm(kNvfp4, w, x, y, T, M, K, kCallerWs, ws, ws_bytes, s);
}
int qgemm_tq1_ws(const void* w, const void* x, float* y, int64_t T, int64_t M, int64_t K, void* ws, int64_t ws_bytes,
                 struct ihipStream_t* s) {
  return gemm(kTq1, w, x, y, T, M, K, kCallerWs, ws, ws_bytes, s);
}

int qgemm_q4k_noalloc(const void* w, const void* x, float* y, int64_t T, int64_t M, int64_t K,
                      struct ihipStream_t* s) {
  return gemm(kQ4k, w, x, y, T, M, K, kScratchWs, nullptr, 0, s);
}

int64_t qgemv_read_sink_len(int64_t bytes) { return bytes > 0 ? qgemv::read_sink_len(bytes) : 0; }

int qgemv_read_ceiling(const void* buf, int64_t bytes, float* sink, struct ihipStream_t* s) {
  if (bytes < 0 || bytes % 16 != 0) return QGEMV_E_SHAPE;
  if (bytes == 0) return QGEMV_OK;
  if (!buf || !sink) return QGEMV_E_NULL;
  if (misaligned(buf, 16) || misaligned(sink, 4)) return QGEMV_E_ALIGN;
  if (qgemv::read_sink_len(bytes) > kMaxM) return QGEMV_E_SHAPE;
  if (overlap(sink, qgemv::read_sink_len(bytes) * 4, buf, bytes)) return QGEMV_E_ALIAS;
  return finish(qgemv::launch_read_ceiling(buf, bytes, sink, s));
}

const char* qgemv_strerror(int code) {
  switch (code) {
    case QGEMV_OK: return "ok";
    case QGEMV_E_NULL: return "a required pointer is NULL";
    case QGEMV_E_SHAPE: return "invalid shape (M < 0, K <= 0, K not a multiple of the block, or too large)";
    case QGEMV_E_ALIGN: return "misaligned pointer (weights, x and rows out need 16 bytes, y and c their element size)";
    case QGEMV_E_HIP: return "the HIP runtime rejected the launch (see qgemv_last_hip_error)";
    case QGEMV_E_ALIAS: return "the output overlaps an input";
    case QGEMV_E_DTYPE: return "unknown element type (QGEMV_F32, QGEMV_F16 or QGEMV_BF16)";
    case QGEMV_E_WORKSPACE: return "the workspace is smaller than qgemm_workspace_bytes asks for";
    default: return "unknown qgemv error code";
  }
}

int qgemv_last_hip_error(void) { return g_last_hip_error; }

const char* qgemv_build_id(void) { return QGEMV_BUILD_ID; }

}  // extern "C"
