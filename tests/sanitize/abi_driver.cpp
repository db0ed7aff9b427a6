// Drives the argument validation of every C ABI entry point (include/qgemv.h)
// under host AddressSanitizer / UndefinedBehaviorSanitizer, with the kernel
// launchers replaced by stubs (launch_stubs.cpp): valid calls must reach the
// launcher exactly once and return its status; invalid ones must return the
// documented error before it.  Host buffers stand in for device memory (the
// validation only looks at pointer values).  Exits non-zero on the first
// mismatch.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qgemv.h"

extern "C" int g_stub_calls;
extern "C" int g_stub_status;
extern "C" void* g_stub_ws;
extern "C" void* const g_stub_scratch;

static int g_fail = 0;

#define EXPECT(call, want_rc, want_calls)                                                          \
  do {                                                                                             \
    g_stub_calls = 0;                                                                              \
    const int rc_ = (call);                                                                        \
    if (rc_ != (want_rc) || g_stub_calls != (want_calls)) {                                        \
      fprintf(stderr, "line %d: %s -> %d (%d launches), want %d (%d)\n", __LINE__, #call, rc_,     \
              g_stub_calls, (int)(want_rc), (int)(want_calls));                                     \
      g_fail = 1;                                                                                  \
    }                                                                                              \
  } while (0)

typedef int (*gemv_fn)(const void*, const void*, float*, int64_t, int64_t, struct ihipStream_t*);
typedef int (*gemv_ex_fn)(const void*, const void*, void*, int64_t, int64_t, const qgemv_epilogue*,
                          struct ihipStream_t*);

struct Fmt {
  const char* name;
  gemv_fn gemv;
  gemv_ex_fn gemv_ex;
  int64_t kmul;  // K granularity
  int64_t kmax;
};

static unsigned char* buf(size_t n) {
  void* p = aligned_alloc(256, (n + 255) / 256 * 256);
  memset(p, 0, (n + 255) / 256 * 256);
  return (unsigned char*)p;
}

int main() {
  const Fmt fmts[] = {
      {"q4k", qgemv_q4k, qgemv_q4k_ex, 256, int64_t(1) << 24},
      {"nvfp4", qgemv_nvfp4, qgemv_nvfp4_ex, 32, int64_t(1) << 24},
      {"tq1", qgemv_tq1, qgemv_tq1_ex, 256, int64_t(1) << 24},
      {"f16", qgemv_f16, qgemv_f16_ex, 8, 65536},
      {"bf16", qgemv_bf16, qgemv_bf16_ex, 8, 65536},
  };
  unsigned char* w = buf(1 << 20);
  unsigned char* x = buf(1 << 16);
  unsigned char* y = buf(1 << 16);
  unsigned char* c = buf(1 << 16);
  const int64_t M = 37;
  for (const Fmt& f : fmts) {
    const int64_t K = 4 * f.kmul;
    // plain call
    EXPECT(f.gemv(w, x, (float*)y, M, K, nullptr), QGEMV_OK, 1);
    EXPECT(f.gemv(w, x, (float*)y, 0, K, nullptr), QGEMV_OK, 0);
    EXPECT(f.gemv(w, x, (float*)y, -1, K, nullptr), QGEMV_E_SHAPE, 0);
    EXPECT(f.gemv(w, x, (float*)y, (int64_t(1) << 31), K, nullptr), QGEMV_E_SHAPE, 0);
    EXPECT(f.gemv(w, x, (float*)y, M, 0, nullptr), QGEMV_E_SHAPE, 0);
    EXPECT(f.gemv(w, x, (float*)y, M, K + f.kmul / 2, nullptr), QGEMV_E_SHAPE, 0);
    EXPECT(f.gemv(w, x, (float*)y, M, f.kmax + f.kmul, nullptr), QGEMV_E_SHAPE, 0);
    EXPECT(f.gemv(w, x, (float*)y, INT64_MAX, INT64_MAX, nullptr), QGEMV_E_SHAPE, 0);
    EXPECT(f.gemv(nullptr, x, (float*)y, M, K, nullptr), QGEMV_E_NULL, 0);
    EXPECT(f.gemv(w, nullptr, (float*)y, M, K, nullptr), QGEMV_E_NULL, 0);
    EXPECT(f.gemv(w, x, nullptr, M, K, nullptr), QGEMV_E_NULL, 0);
    EXPECT(f.gemv(w + 8, x, (float*)y, M, K, nullptr), QGEMV_E_ALIGN, 0);
    EXPECT(f.gemv(w, x + 2, (float*)y, M, K, nullptr), QGEMV_E_ALIGN, 0);
    EXPECT(f.gemv(w, x, (float*)(y + 2), M, K, nullptr), QGEMV_E_ALIGN, 0);
    EXPECT(f.gemv(w, x, (float*)(w + 64), M, K, nullptr), QGEMV_E_ALIAS, 0);
    EXPECT(f.gemv(w, x, (float*)(x + 16), M, K, nullptr), QGEMV_E_ALIAS, 0);
    // the largest shape the calls accept (pointer values far apart, never
    // dereferenced): the size arithmetic must not overflow
    EXPECT(f.gemv((const void*)uintptr_t(0x1000), (const void*)(uintptr_t(1) << 61), (float*)(uintptr_t(1) << 62),
                  (int64_t(1) << 31) - 1, f.kmax, nullptr),
           QGEMV_OK, 1);
    // a launch the runtime rejects
    g_stub_status = 98;  // hipErrorInvalidDeviceFunction
    EXPECT(f.gemv(w, x, (float*)y, M, K, nullptr), QGEMV_E_HIP, 1);
    if (qgemv_last_hip_error() != 98) {
      fprintf(stderr, "%s: last hip error %d\n", f.name, qgemv_last_hip_error());
      g_fail = 1;
    }
    g_stub_status = 0;

    // output stage
    qgemv_epilogue e = {2.f, 0.5f, c, QGEMV_F32, QGEMV_F16};
    EXPECT(f.gemv_ex(w, x, y, M, K, &e, nullptr), QGEMV_OK, 1);
    EXPECT(f.gemv_ex(w, x, y, M, K, nullptr, nullptr), QGEMV_OK, 1);
    EXPECT(f.gemv_ex(w, x, y, 0, K, &e, nullptr), QGEMV_OK, 0);
    e.y_dtype = 3;
    EXPECT(f.gemv_ex(w, x, y, M, K, &e, nullptr), QGEMV_E_DTYPE, 0);
    e.y_dtype = QGEMV_BF16;
    e.c_dtype = -1;
    EXPECT(f.gemv_ex(w, x, y, M, K, &e, nullptr), QGEMV_E_DTYPE, 0);
    e.beta = 0.f;  // c is not read: its type and pointer do not matter
    e.c = nullptr;
    EXPECT(f.gemv_ex(w, x, y, M, K, &e, nullptr), QGEMV_OK, 1);
    e.beta = 1.f;
    e.c_dtype = QGEMV_F16;
    EXPECT(f.gemv_ex(w, x, y, M, K, &e, nullptr), QGEMV_E_NULL, 0);
    e.c = c + 1;
    EXPECT(f.gemv_ex(w, x, y, M, K, &e, nullptr), QGEMV_E_ALIGN, 0);
    e.c = y;  // in place: c is y itself, same type
    e.y_dtype = QGEMV_F16;
    EXPECT(f.gemv_ex(w, x, y, M, K, &e, nullptr), QGEMV_OK, 1);
    e.c_dtype = QGEMV_F32;  // c is y but of another type
    EXPECT(f.gemv_ex(w, x, y, M, K, &e, nullptr), QGEMV_E_ALIAS, 0);
    e.c = y + 8;  // partial overlap
    e.c_dtype = QGEMV_BF16;
    EXPECT(f.gemv_ex(w, x, y, M, K, &e, nullptr), QGEMV_E_ALIAS, 0);
    e.c = c;
    EXPECT(f.gemv_ex(w, x, y + 1, M, K, &e, nullptr), QGEMV_E_ALIGN, 0);
    EXPECT(f.gemv_ex(w, x, w, M, K, &e, nullptr), QGEMV_E_ALIAS, 0);
  }

  // dequantisation and row gathers
  typedef int (*deq_fn)(const void*, float*, int64_t, int64_t, struct ihipStream_t*);
  typedef int (*rows_fn)(const void*, int64_t, int64_t, const int32_t*, int64_t, void*, int32_t,
                         struct ihipStream_t*);
  const deq_fn deqs[] = {qdequant_q4k, qdequant_nvfp4, qdequant_tq1};
  const rows_fn rowfs[] = {qget_rows_q4k, qget_rows_nvfp4, qget_rows_tq1};
  unsigned char* out = buf(1 << 20);
  int32_t* idx = (int32_t*)buf(4096);
  for (int i = 0; i < 3; ++i) {
    EXPECT(deqs[i](w, (float*)out, 5, 512, nullptr), QGEMV_OK, 1);
    EXPECT(deqs[i](w, (float*)out, 0, 512, nullptr), QGEMV_OK, 0);
    EXPECT(deqs[i](w, nullptr, 5, 512, nullptr), QGEMV_E_NULL, 0);
    EXPECT(deqs[i](w, (float*)out, 5, 100, nullptr), QGEMV_E_SHAPE, 0);
    EXPECT(rowfs[i](w, 5, 512, idx, 9, out, QGEMV_F16, nullptr), QGEMV_OK, 1);
    EXPECT(rowfs[i](w, 5, 512, nullptr, 5, out, QGEMV_BF16, nullptr), QGEMV_OK, 1);
    EXPECT(rowfs[i](w, 5, 512, nullptr, 6, out, QGEMV_F32, nullptr), QGEMV_E_SHAPE, 0);
    EXPECT(rowfs[i](w, 5, 512, idx, -1, out, QGEMV_F32, nullptr), QGEMV_E_SHAPE, 0);
    EXPECT(rowfs[i](w, 5, 512, idx, 0, out, QGEMV_F32, nullptr), QGEMV_OK, 0);
    EXPECT(rowfs[i](w, 5, 512, idx, 9, out, 7, nullptr), QGEMV_E_DTYPE, 0);
    EXPECT(rowfs[i](w, 5, 512, idx + 1, 9, out, QGEMV_F32, nullptr), QGEMV_OK, 1);
    EXPECT(rowfs[i](w, 5, 512, (const int32_t*)((unsigned char*)idx + 2), 9, out, QGEMV_F32, nullptr),
           QGEMV_E_ALIGN, 0);
    EXPECT(rowfs[i](w, 5, 512, idx, 9, out + 8, QGEMV_F32, nullptr), QGEMV_E_ALIGN, 0);
    EXPECT(rowfs[i](w, 5, 512, idx, 9, nullptr, QGEMV_F32, nullptr), QGEMV_E_NULL, 0);
    EXPECT(rowfs[i](nullptr, 5, 512, idx, 9, out, QGEMV_F32, nullptr), QGEMV_E_NULL, 0);
    EXPECT(rowfs[i](nullptr, 0, 512, idx, 9, out, QGEMV_F32, nullptr), QGEMV_OK, 1);  // every index out of range
    EXPECT(rowfs[i](w, 5, 512, idx, 9, w, QGEMV_F32, nullptr), QGEMV_E_ALIAS, 0);
    EXPECT(rowfs[i](w, 5, 512, idx, 9, (unsigned char*)idx, QGEMV_F32, nullptr), QGEMV_E_ALIAS, 0);
    // more workgroups than a grid holds: 2^14 per row of 2^24 fp32 outputs
    EXPECT(rowfs[i](w, 5, int64_t(1) << 24, idx, (int64_t(1) << 17) + 1, out, QGEMV_F32, nullptr), QGEMV_E_SHAPE, 0);
  }

  // prefill
  typedef int (*gemm_fn)(const void*, const void*, float*, int64_t, int64_t, int64_t, struct ihipStream_t*);
  const gemm_fn gemms[] = {qgemm_q4k, qgemm_nvfp4, qgemm_tq1};
  for (int i = 0; i < 3; ++i) {
    EXPECT(gemms[i](w, x, (float*)out, 7, 5, 512, nullptr), QGEMV_OK, 1);
    EXPECT(gemms[i](w, x, (float*)out, 0, 5, 512, nullptr), QGEMV_OK, 0);
    EXPECT(gemms[i](w, x, (float*)out, 7, 0, 512, nullptr), QGEMV_OK, 0);
    EXPECT(gemms[i](w, x, (float*)out, -1, 5, 512, nullptr), QGEMV_E_SHAPE, 0);
    EXPECT(gemms[i](w, x, (float*)out, 65535 * int64_t(128) + 1, 5, 512, nullptr), QGEMV_E_SHAPE, 0);
    EXPECT(gemms[i](w, x, (float*)out, 7, 5, (int64_t(1) << 20) + 256, nullptr), QGEMV_E_SHAPE, 0);
    EXPECT(gemms[i](w, nullptr, (float*)out, 7, 5, 512, nullptr), QGEMV_E_NULL, 0);
    EXPECT(gemms[i](w, x + 8, (float*)out, 7, 5, 512, nullptr), QGEMV_E_ALIGN, 0);
    EXPECT(gemms[i](w, x, (float*)x, 7, 5, 512, nullptr), QGEMV_E_ALIAS, 0);
  }
  EXPECT(qgemm_nvfp4(w, x, (float*)out, 7, 5, 96, nullptr), QGEMV_E_SHAPE, 0);  // K % 64

  // prefill with a workspace: no K split at 7 x 5 x 512 (no workspace needed),
  // 130 tokens x 4096 rows x K 4096 splits each of its 32 tiles 6 ways (8
  // asked for, 64 steps rounded to whole 6-step iterations: 12 steps per
  // split; 6 x 32 partial tiles of 256 x 128 fp32); pointer values far apart
  // stand in for device memory
  if (qgemm_workspace_bytes(7, 5, 512) != 0 || qgemm_workspace_bytes(0, 5, 512) != 0 ||
      qgemm_workspace_bytes(130, 4096, 4096) != int64_t(32) * 6 * 256 * 128 * 4 ||
      qgemm_workspace_bytes(-1, 5, 512) != QGEMV_E_SHAPE || qgemm_workspace_bytes(7, 5, 0) != QGEMV_E_SHAPE)
    g_fail = 1;
  typedef int (*gemm_ws_fn)(const void*, const void*, float*, int64_t, int64_t, int64_t, void*, int64_t,
                            struct ihipStream_t*);
  const gemm_ws_fn gemm_wss[] = {qgemm_q4k_ws, qgemm_nvfp4_ws, qgemm_tq1_ws};
  const int64_t need = qgemm_workspace_bytes(130, 4096, 4096);
  const void* bw = (const void*)(uintptr_t(1) << 40);
  const void* bx = (const void*)(uintptr_t(2) << 40);
  float* by = (float*)(uintptr_t(3) << 40);
  void* bws = (void*)(uintptr_t(4) << 40);
  for (int i = 0; i < 3; ++i) {
    g_stub_ws = bws;
    EXPECT(gemm_wss[i](w, x, (float*)out, 7, 5, 512, nullptr, 0, nullptr), QGEMV_OK, 1);
    if (g_stub_ws != nullptr) g_fail = 1;  // nothing split: no workspace handed on
    EXPECT(gemm_wss[i](bw, bx, by, 130, 4096, 4096, bws, need, nullptr), QGEMV_OK, 1);
    if (g_stub_ws != bws) g_fail = 1;
    EXPECT(gemm_wss[i](bw, bx, by, 130, 4096, 4096, nullptr, need, nullptr), QGEMV_E_NULL, 0);
    EXPECT(gemm_wss[i](bw, bx, by, 130, 4096, 4096, (char*)bws + 16, need, nullptr), QGEMV_E_ALIGN, 0);
    EXPECT(gemm_wss[i](bw, bx, by, 130, 4096, 4096, bws, need - 1, nullptr), QGEMV_E_WORKSPACE, 0);
    EXPECT(gemm_wss[i](bw, bx, by, 130, 4096, 4096, (void*)((char*)by + 256), need, nullptr), QGEMV_E_ALIAS, 0);
    EXPECT(gemm_wss[i](bw, bx, by, 130, 4096, 4096, (void*)((char*)bw - 256), need, nullptr), QGEMV_E_ALIAS, 0);
    EXPECT(gemm_wss[i](bw, bx, by, 0, 4096, 4096, nullptr, 0, nullptr), QGEMV_OK, 0);
  }
  g_stub_ws = bws;
  EXPECT(qgemm_q4k(bw, bx, by, 130, 4096, 4096, nullptr), QGEMV_OK, 1);
  if (g_stub_ws != nullptr) g_fail = 1;  // the plain call splits with atomics

  // prefill through the library's own 32 MiB array: the argument checks come
  // first; a split needing more than the array is refused before any HIP call
  // (4608 x 8192 x 4096 asks for 64 MiB); an unsplit call needs no array
  EXPECT(qgemm_q4k_noalloc(bw, bx, by, 4608, 8192, 4096, nullptr), QGEMV_E_WORKSPACE, 0);
  EXPECT(qgemm_q4k_noalloc(bw, bx, by, 130, 4096, 4000, nullptr), QGEMV_E_SHAPE, 0);
  EXPECT(qgemm_q4k_noalloc(bw, bx, by, -1, 4096, 4096, nullptr), QGEMV_E_SHAPE, 0);
  EXPECT(qgemm_q4k_noalloc(nullptr, bx, by, 130, 4096, 4096, nullptr), QGEMV_E_NULL, 0);
  EXPECT(qgemm_q4k_noalloc(bw, bx, (float*)((char*)by + 2), 130, 4096, 4096, nullptr), QGEMV_E_ALIGN, 0);
  EXPECT(qgemm_q4k_noalloc(bw, bx, (float*)bx, 130, 4096, 4096, nullptr), QGEMV_E_ALIAS, 0);
  EXPECT(qgemm_q4k_noalloc(bw, bx, by, 0, 4096, 4096, nullptr), QGEMV_OK, 0);
  g_stub_ws = bws;
  EXPECT(qgemm_q4k_noalloc(w, x, (float*)out, 7, 5, 512, nullptr), QGEMV_OK, 1);
  if (g_stub_ws != nullptr) g_fail = 1;
  EXPECT(qgemm_q4k_noalloc(bw, bx, by, 130, 4096, 4096, nullptr), QGEMV_OK, 1);
  if (g_stub_ws != g_stub_scratch) g_fail = 1;  // the split goes through the array

  // read probe, strings
  EXPECT(qgemv_read_ceiling(w, 65536, (float*)out, nullptr), QGEMV_OK, 1);
  EXPECT(qgemv_read_ceiling(w, 0, (float*)out, nullptr), QGEMV_OK, 0);
  EXPECT(qgemv_read_ceiling(w, 100, (float*)out, nullptr), QGEMV_E_SHAPE, 0);
  EXPECT(qgemv_read_ceiling(w, -16, (float*)out, nullptr), QGEMV_E_SHAPE, 0);
  EXPECT(qgemv_read_ceiling(nullptr, 65536, (float*)out, nullptr), QGEMV_E_NULL, 0);
  EXPECT(qgemv_read_ceiling(w + 4, 65536, (float*)out, nullptr), QGEMV_E_ALIGN, 0);
  EXPECT(qgemv_read_ceiling(w, 65536, (float*)(w + 16), nullptr), QGEMV_E_ALIAS, 0);
  if (qgemv_read_sink_len(0) != 0 || qgemv_read_sink_len(-5) != 0 || qgemv_read_sink_len(65536) < 1) g_fail = 1;
  for (int code = -10; code <= 2; ++code)
    if (!qgemv_strerror(code) || !*qgemv_strerror(code)) g_fail = 1;
  if (!qgemv_build_id() || !*qgemv_build_id()) g_fail = 1;

  free(w);
  free(x);
  free(y);
  free(c);
  free(out);
  free(idx);
  if (g_fail) return 1;
  printf("abi validation: ok\n");
  return 0;
}
