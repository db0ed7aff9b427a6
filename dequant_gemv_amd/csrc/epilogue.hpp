// Output stages of the GEMV kernels: what happens to the finished dot product
// v_r = x . w_r of row r.  OutF32 stores it as fp32 (alpha = 1, beta = 0);
// OutEx evaluates the general form alpha * v_r + beta * c_r of "Writing a high
// performant GEMV + dequant for Metal" (section "What is a GEMV") and stores
// it as fp32, fp16 or bf16 (round to nearest even), the fp16 / bf16 outputs of
// that page's kernel and of the Mojo fp4_gemv page's final cast.
//
// Both are passed to the kernels by value; put() runs once per row on the one
// lane that stores it.  prefetch(row) lets a kernel fetch what put() will read
// for the row (c_r) early, so that the load's latency does not land on the
// end of every wave.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace qgemv {

// Element types of vectors and materialised rows (the QGEMV_F32 / QGEMV_F16 /
// QGEMV_BF16 values of the C interface).
enum Dtype : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

__host__ __device__ constexpr int dtype_bytes(int t) { return t == kF32 ? 4 : 2; }

struct OutF32 {
  float* y;
  struct Pre {};
  __device__ __forceinline__ Pre prefetch(int, int, bool) const { return {}; }
  __device__ __forceinline__ void put(int row, float v, Pre = {}) const { y[row] = v; }
};

struct OutEx {
  void* y;
  const void* c;  // read only when beta != 0
  float alpha;
  float beta;
  int c_dtype;
  int y_dtype;

  struct Pre {
    unsigned bits;  // c_r as stored (fp32 bits, or a 16-bit code)
  };
  // c of row row0 + j (row0 wave-uniform, 0 <= j < 64; only lanes with
  // `want` load); nothing is read when beta == 0
  __device__ __forceinline__ Pre prefetch(int row0, int j, bool want) const {
    Pre p{0u};
    if (beta != 0.f && want) {
      const int64_t sz = c_dtype == kF32 ? 4 : 2;
      const auto r = make_rsrc(static_cast<const unsigned char*>(c) + row0 * sz, (uint32_t)(64 * sz));
      p.bits = sz == 4 ? ld32(r, (uint32_t)j * 4u) : (unsigned)ld16(r, (uint32_t)j * 2u);
    }
    return p;
  }
  __device__ __forceinline__ float c_value(Pre p) const {
    if (c_dtype == kF32) return __builtin_bit_cast(float, p.bits);
    if (c_dtype == kF16) return (float)__builtin_bit_cast(_Float16, (unsigned short)p.bits);
    return (float)__builtin_bit_cast(__bf16, (unsigned short)p.bits);
  }
  __device__ __forceinline__ float load_c(int row) const {
    if (c_dtype == kF32) return static_cast<const float*>(c)[row];
    if (c_dtype == kF16) return (float)static_cast<const _Float16*>(c)[row];
    return (float)static_cast<const __bf16*>(c)[row];
  }
  __device__ __forceinline__ void put(int row, float v, Pre p) const {
    float r = alpha * v;
    if (beta != 0.f) r = __builtin_fmaf(beta, c_value(p), r);
    store(row, r);
  }
  __device__ __forceinline__ void put(int row, float v) const {
    float r = alpha * v;
    if (beta != 0.f) r = __builtin_fmaf(beta, load_c(row), r);
    store(row, r);
  }
  __device__ __forceinline__ void store(int row, float r) const {
    if (y_dtype == kF32)
      static_cast<float*>(y)[row] = r;
    else if (y_dtype == kF16)
      static_cast<_Float16*>(y)[row] = (_Float16)pin_f32(r);
    else
      static_cast<__bf16*>(y)[row] = (__bf16)pin_f32(r);
  }
};

}  // namespace qgemv
