// Shared pieces of the row-materialisation (GET_ROWS) kernels: output element
// conversion, vector stores and the launch geometry.
//
// Every format's kernel gives each thread 16 bytes of output: E = 8 weights
// for fp16 / bf16, 4 for fp32, consecutive in the row.  Consecutive threads
// own consecutive 16-byte pieces, so each wave-wide store writes one
// contiguous KiB; the packed bytes a thread needs are a few bytes of one
// block (plus its header), read with small loads that neighbouring lanes
// share.  A thread owns U such tasks, B apart (B = threads per workgroup), and
// issues the loads of all U before converting and storing any, so a wave keeps
// U times more bytes in flight than one task would (a single load-convert-store
// per thread leaves the kernel bound by load latency).  Workgroup b covers
// tasks [(b % bpr) * B * U, ...) of output row b / bpr, so no thread divides
// by a runtime value.
#pragma once
#include "device.hpp"
#include "epilogue.hpp"

namespace qgemv {

template <typename T>
__device__ __forceinline__ unsigned pack2(float a, float b) {
  if constexpr (sizeof(T) == 2) {
    // fp32 values, then both rounded to nearest even by one packed conversion
    // (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32); pinned, so that no multiply or
    // fma before them is fused into a single-rounding mixed-precision op
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef T t2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {pin_f32(a), pin_f32(b)};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, t2_t));
  } else {
    return 0u;  // unused
  }
}

// Outputs per thread (16 bytes of T).
template <typename T>
constexpr int kRowsE = 16 / (int)sizeof(T);

// dst[0..E) = v converted to T, one 16-byte store (dst 16-byte aligned).
template <typename T>
__device__ __forceinline__ void store_e(T* dst, const float (&v)[kRowsE<T>]) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    *reinterpret_cast<u32x4*>(dst) = u32x4{pack2<T>(v[0], v[1]), pack2<T>(v[2], v[3]), pack2<T>(v[4], v[5]),
                                           pack2<T>(v[6], v[7])};
  }
}

// E quiet NaNs (clear sign bit) of the output type: the piece of a row whose
// index is outside [0, n).
template <typename T>
__device__ __forceinline__ void store_e_nan(T* dst) {
  const unsigned q = sizeof(T) == 4 ? 0x7FC00000u : (__is_same(T, _Float16) ? 0x7E007E00u : 0x7FC07FC0u);
  *reinterpret_cast<u32x4*>(dst) = u32x4{q, q, q, q};
}

// Little-endian value of BYTES (2, 4 or 8) bytes at an even byte offset of a
// buffer, read as separate 16-bit buffer loads.  The ternary blocks are 54
// bytes, so their fields are only 2-byte aligned; plain 16-bit pointer loads
// would be merged by the compiler into dword / dwordx2 loads at addresses
// that are not 4-byte aligned, and those do not reliably return the bytes
// asked for.  Buffer-load intrinsics are never merged.
template <int BYTES>
__device__ __forceinline__ uint64_t load_le_a2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  uint64_t v = 0;
#pragma unroll
  for (int i = 0; i < BYTES / 2; ++i) v |= (uint64_t)ld16(r, off + 2u * (uint32_t)i) << (16 * i);
  return v;
}

// The same bytes from the BYTES / 4 + 1 dwords around them, read with ONE
// dword-aligned multi-dword load and realigned with alignbyte (off is 2-byte
// aligned).  The range check is per dword: a dword wholly or partly past the
// range reads as zero, so the bytes past the end of the range must not be
// needed.
template <int BYTES>
__device__ __forceinline__ uint64_t load_le_a2_dw(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  static_assert(BYTES == 4 || BYTES == 8, "4 or 8 bytes");
  const uint32_t al = off & ~3u, sh = off & 3u;
  if constexpr (BYTES == 4) {
    const auto d = __builtin_amdgcn_raw_buffer_load_b64(r, (int)al, 0, 0);
    return __builtin_amdgcn_alignbyte(d[1], d[0], sh);
  } else {
    const auto d = __builtin_amdgcn_raw_buffer_load_b96(r, (int)al, 0, 0);
    const unsigned lo = __builtin_amdgcn_alignbyte(d[1], d[0], sh);
    return (uint64_t)lo | ((uint64_t)__builtin_amdgcn_alignbyte(d[2], d[1], sh) << 32);
  }
}

// Source row of output row j, or -1 when the index is outside [0, n).
__device__ __forceinline__ int source_row(const int32_t* rows, int j, int n) {
  const int r = rows ? rows[j] : j;
  return (unsigned)r < (unsigned)n ? r : -1;
}

// Below this many tasks in a launch the kernels run one task per thread.
constexpr int64_t kRowsSmallTasks = int64_t(1) << 21;

struct RowsGeom {
  int block;  // threads per workgroup
  int bpr;    // workgroups per output row
  int64_t grid;
};

// Tasks per row and per thread (U) -> workgroup size (a multiple of 64, at
// most 256) and count.
inline RowsGeom rows_geom(int64_t tasks, int64_t nrows_out, int u) {
  RowsGeom g;
  const int64_t per_thread = (tasks + u - 1) / u;
  const int64_t b = per_thread < 256 ? (per_thread + 63) / 64 * 64 : 256;
  g.block = (int)b;
  g.bpr = (int)((tasks + b * u - 1) / (b * u));
  g.grid = nrows_out * g.bpr;
  return g;
}

// Runs a row-materialisation thread owning U tasks: load(t) fetches what task
// t needs, emit(t, in) converts and stores it, fill(t) stores task t's quiet
// NaNs.
template <int U, typename In, typename Load, typename Emit, typename Fill>
__device__ __forceinline__ void rows_thread(int bpr, int tasks, bool valid, Load&& load, Emit&& emit, Fill&& fill) {
  const int j = blockIdx.x / bpr;
  const int t0 = (blockIdx.x - j * bpr) * blockDim.x * U + threadIdx.x;
  In in[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = t0 + u * (int)blockDim.x;
    if (valid && t < tasks) in[u] = load(t);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = t0 + u * (int)blockDim.x;
    if (t < tasks) {
      if (valid)
        emit(t, in[u]);
      else
        fill(t);
    }
  }
}

}  // namespace qgemv
