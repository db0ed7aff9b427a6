// Shared pieces of the row-materialisation (GET_ROWS) kernels: output element
// conversion, 16-element vector stores and the launch geometry.
//
// Every format's kernel splits an output row into tasks of 16 or 32 weights
// that read one small contiguous piece of the packed row (a 16-byte nibble
// slice, a 16-element run of a ternary block) and write their outputs with
// 16-byte stores.  Workgroup b covers tasks [(b % bpr) * B, ...) of output
// row b / bpr, so no thread ever divides by a runtime value.
#pragma once
#include "device.hpp"
#include "epilogue.hpp"

namespace qgemv {

template <typename T>
__device__ __forceinline__ unsigned pack2(float a, float b) {
  if constexpr (sizeof(T) == 2) {
    const T lo = (T)pin_f32(a), hi = (T)pin_f32(b);  // fp32 value, then round to nearest even
    return (unsigned)__builtin_bit_cast(unsigned short, lo) | ((unsigned)__builtin_bit_cast(unsigned short, hi) << 16);
  } else {
    return 0u;  // unused
  }
}

// out[0..16) = v converted to T, with 16-byte stores (dst 16-byte aligned for
// fp32, 32-byte for 16-bit types: both hold for every task of these kernels).
template <typename T>
__device__ __forceinline__ void store16(T* dst, const float (&v)[16]) {
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < 16; i += 8)
      *reinterpret_cast<u32x4*>(dst + i) = u32x4{pack2<T>(v[i], v[i + 1]), pack2<T>(v[i + 2], v[i + 3]),
                                                 pack2<T>(v[i + 4], v[i + 5]), pack2<T>(v[i + 6], v[i + 7])};
  }
}

// 16 quiet NaNs (clear sign bit) of the output type: the row of an index
// outside [0, n).
template <typename T>
__device__ __forceinline__ void store16_nan(T* dst) {
  const unsigned q = sizeof(T) == 4 ? 0x7FC00000u : (__is_same(T, _Float16) ? 0x7E007E00u : 0x7FC07FC0u);
  const u32x4 v = {q, q, q, q};
#pragma unroll
  for (int i = 0; i < 16; i += 16 / (int)sizeof(T)) *reinterpret_cast<u32x4*>(dst + i) = v;
}

// Source row of output row j, or -1 when the index is outside [0, n).
__device__ __forceinline__ int source_row(const int32_t* rows, int j, int n) {
  const int r = rows ? rows[j] : j;
  return (unsigned)r < (unsigned)n ? r : -1;
}

struct RowsGeom {
  int block;  // threads per workgroup
  int bpr;    // workgroups per output row
  int64_t grid;
};

// Tasks per row -> workgroup size (a multiple of 64, at most 256) and count.
inline RowsGeom rows_geom(int64_t tasks, int64_t nrows_out) {
  RowsGeom g;
  const int64_t b = tasks < 256 ? (tasks + 63) / 64 * 64 : 256;
  g.block = (int)b;
  g.bpr = (int)((tasks + b - 1) / b);
  g.grid = nrows_out * g.bpr;
  return g;
}

}  // namespace qgemv
