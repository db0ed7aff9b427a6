// C ABI of libqgemv: argument validation in plain host code, then one launch on
// the caller's stream.  See include/qgemv.h for the contract of each call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
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

enum Fmt { kQ4k, kNvfp4, kTq1 };

int64_t k_multiple(Fmt f) { return f == kNvfp4 ? 32 : 256; }

int64_t weight_bytes(Fmt f, int64_t m, int64_t k) {
  switch (f) {
    case kQ4k: return m * (k / 256) * 144;
    case kTq1: return m * (k / 256) * 54;
    default: return m * (k / 2) + m * (k / 16);
  }
}

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

int check_shape(Fmt f, int64_t m, int64_t k) {
  if (m < 0 || m > kMaxM || k <= 0 || k > kMaxK || k % k_multiple(f) != 0) return QGEMV_E_SHAPE;
  // grid of the dequant kernels: at most m*k/16 threads in blocks of 256
  if (m > 0 && (m * (k / 16) + 255) / 256 > kMaxM) return QGEMV_E_SHAPE;
  return QGEMV_OK;
}

int finish(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return QGEMV_E_HIP;
  }
  return QGEMV_OK;
}

int gemv(Fmt f, const void* w, const void* x, float* y, int64_t m, int64_t k, hipStream_t s) {
  int rc = check_shape(f, m, k);
  if (rc != QGEMV_OK) return rc;
  if (m == 0) return QGEMV_OK;
  if (!w || !x || !y) return QGEMV_E_NULL;
  if (misaligned(w, 16) || misaligned(x, 16) || misaligned(y, 4)) return QGEMV_E_ALIGN;
  if (overlap(y, m * 4, w, weight_bytes(f, m, k)) || overlap(y, m * 4, x, k * 2)) return QGEMV_E_ALIAS;
  switch (f) {
    case kQ4k: return finish(qgemv::launch_q4k_gemv(w, x, y, m, k, s));
    case kNvfp4: return finish(qgemv::launch_nvfp4_gemv(w, x, y, m, k, s));
    default: return finish(qgemv::launch_tq1_gemv(w, x, y, m, k, s));
  }
}

int dequant(Fmt f, const void* w, float* out, int64_t m, int64_t k, hipStream_t s) {
  int rc = check_shape(f, m, k);
  if (rc != QGEMV_OK) return rc;
  if (m == 0) return QGEMV_OK;
  if (!w || !out) return QGEMV_E_NULL;
  if (misaligned(w, 16) || misaligned(out, 16)) return QGEMV_E_ALIGN;
  if (overlap(out, m * k * 4, w, weight_bytes(f, m, k))) return QGEMV_E_ALIAS;
  switch (f) {
    case kQ4k: return finish(qgemv::launch_q4k_dequant(w, out, m, k, s));
    case kNvfp4: return finish(qgemv::launch_nvfp4_dequant(w, out, m, k, s));
    default: return finish(qgemv::launch_tq1_dequant(w, out, m, k, s));
  }
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
    case QGEMV_E_ALIGN: return "misaligned pointer (weights and x need 16 bytes, y 4 bytes)";
    case QGEMV_E_HIP: return "the HIP runtime rejected the launch (see qgemv_last_hip_error)";
    case QGEMV_E_ALIAS: return "the output overlaps an input";
    default: return "unknown qgemv error code";
  }
}

int qgemv_last_hip_error(void) { return g_last_hip_error; }

const char* qgemv_build_id(void) { return QGEMV_BUILD_ID; }

}  // extern "C"
