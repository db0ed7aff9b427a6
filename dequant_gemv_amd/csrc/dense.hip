// Dense fp16 / bf16 GEMV for gfx950: y = x . W^T with W [N][K] row-major in
// the activations' type.  This is the uncompressed comparison point of the
// Mojo fp4_gemv page (its NVFP4 GEMV against a bf16 GEMV of the same shape):
// the same read-once weight stream, 2 bytes per weight instead of 0.5625.
//
// Work split.  A wave owns `rpw` consecutive rows, i.e. one contiguous run of
// rpw * 2K bytes, and walks it in 1 KiB units (lane i takes bytes 16i..16i+15
// of a unit, 8 weights): unit c of a row pairs with activation bytes
// [1024c, 1024c + 1024), which the workgroup keeps in LDS (copied once,
// zero-filled past K).  Weight loads go straight to VGPRs through a ring of
// DEPTH register quads: the load for unit u + DEPTH is issued as soon as
// unit u's registers are free, so DEPTH KiB per wave are always in flight and
// the compiler's own vmcnt waits (loads return in order) gate each unit.
// Each lane accumulates with v_dot2_f32_f16 / v_dot2_f32_bf16; at the end of
// a row the lane partials are summed across the wave with DPP and one lane
// hands the row to the output stage.  When 2K is not a multiple of 1 KiB the
// last unit of a row runs into the next row's bytes: those lanes' weights are
// replaced by zero.
#include "device.hpp"
#include "epilogue.hpp"
#include "launch.hpp"
#include "stream.hpp"

namespace qgemv {

#ifndef QGEMV_DENSE_DEPTH
#define QGEMV_DENSE_DEPTH 8  // 1 KiB weight loads in flight per wave
#endif
#ifndef QGEMV_DENSE_WAVES
#define QGEMV_DENSE_WAVES 8  // waves per workgroup (two per SIMD)
#endif
#ifndef QGEMV_DENSE_TARGET_WAVES
#define QGEMV_DENSE_TARGET_WAVES 2048  // about eight waves per CU, all resident at once
#endif

// (The bf16 pair is built from a by-value word: __builtin_bit_cast applied to a
// vector-element lvalue such as w.y reads element 0 with this compiler.)
__device__ __forceinline__ bf16x2 as_bf2(unsigned v) { return __builtin_bit_cast(bf16x2, v); }

template <bool BF>
__device__ __forceinline__ float dot8(const u32x4& w, const u32x4& x, float acc) {
  if constexpr (BF) {
    acc = dot2bf(as_bf2(w.x), x.x, acc);
    acc = dot2bf(as_bf2(w.y), x.y, acc);
    acc = dot2bf(as_bf2(w.z), x.z, acc);
    return dot2bf(as_bf2(w.w), x.w, acc);
  } else {
    acc = dot2h(w.x, x.x, acc);
    acc = dot2h(w.y, x.y, acc);
    acc = dot2h(w.z, x.z, acc);
    return dot2h(w.w, x.w, acc);
  }
}

template <int W, int D, bool BF, typename Out>
__global__ __launch_bounds__(64 * W) void dense_gemv_kernel(const uint8_t* __restrict__ w,
                                                            const uint8_t* __restrict__ x, Out out, int n,
                                                            int k, int rpw) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char xs[];
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_bytes = 2 * k;
  const int kc = (row_bytes + 1023) >> 10;  // units per row
  const int64_t row0_64 = ((int64_t)blockIdx.x * W + wave) * rpw;
  const int nrows = (int)max((int64_t)0, min((int64_t)rpw, (int64_t)n - row0_64));
  const int row0 = (int)min(row0_64, (int64_t)n);
  const int total = nrows * kc;
  // bytes of the last unit of a row that belong to the row
  const int tail = row_bytes - ((kc - 1) << 10);
  const bool tail_lane = 16 * lane < tail;

  // the output stage's input for the first row (a row's is fetched when the
  // previous row ends, a whole row of loads ahead of its use)
  auto pre = out.prefetch(row0, 0, nrows > 0);

  // Activation copy straight into LDS: piece P (1 KiB) by wave P % W; bytes
  // past 2K read as zero.
  const auto xr = make_rsrc(x, (uint32_t)row_bytes);
  for (int piece = wave; piece < kc; piece += W)
    ld128_lds(xr, xs + piece * 1024, (uint32_t)(piece * 1024 + 16 * lane));
  compiler_fence();

  // First DEPTH weight loads of the wave's run.  Loads are never skipped:
  // past the end of the run their offsets fall outside the descriptor and
  // read zero without touching memory, so the loop below has no data-dependent
  // branch around a load and every wait the compiler places is exact.
  const auto wr = make_rsrc(w + (int64_t)row0 * row_bytes, (uint32_t)(nrows * row_bytes));
  u32x4 buf[D];
  int lj = 0, lc = 0;  // row and unit of the next load
  auto next_off = [&]() {
    const uint32_t off = (uint32_t)(lj * row_bytes + (lc << 10) + 16 * lane);
    if (++lc == kc) {
      lc = 0;
      ++lj;
    }
    return off;
  };
#pragma unroll
  for (int i = 0; i < D; ++i) buf[i] = ld128w(wr, next_off());

  wait_vm<0>();  // the activation pieces (and the first weight units) are in
  __syncthreads();

  float acc = 0.f;
  int j = 0, c = 0;  // row and unit being consumed
  for (int base = 0; base < total; base += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + (c << 10) + 16 * lane);
      const bool keep = c != kc - 1 || tail_lane;
      acc = dot8<BF>(keep ? buf[i] : u32x4{0u, 0u, 0u, 0u}, xv, acc);
      // refill after the use, into the same registers (a refill issued before
      // the use would need fresh registers and a copy, i.e. a full wait, at
      // the loop's back edge)
      buf[i] = ld128w(wr, next_off());
      if (++c == kc) {  // row j done (units past the run belong to rows >= nrows)
        float a[1] = {acc};
        store_rows<1>(a, out, pre, row0 + j, j < nrows ? 1 : 0, 1.f, lane);
        acc = 0.f;
        c = 0;
        ++j;
        pre = out.prefetch(row0, j, j < nrows);
      }
    }
  }
}

template <bool BF, typename Out>
static hipError_t launch_dense(const void* w, const void* x, const Out& y, int64_t n, int64_t k, hipStream_t s) {
  constexpr int W = QGEMV_DENSE_WAVES;
  const int64_t waves = n < QGEMV_DENSE_TARGET_WAVES ? n : QGEMV_DENSE_TARGET_WAVES;
  int64_t rpw = (n + waves - 1) / waves;
  const int64_t rpw_max = ((int64_t(1) << 31) - 1) / (2 * k);  // a wave's run stays below 2 GiB
  if (rpw > rpw_max) rpw = rpw_max;
  const int64_t wgs = (n + rpw * W - 1) / (rpw * W);
  const size_t lds = (size_t)((2 * k + 1023) / 1024) * 1024;
  auto kernel = dense_gemv_kernel<W, QGEMV_DENSE_DEPTH, BF, Out>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(64 * W), lds, s, (const uint8_t*)w, (const uint8_t*)x, y, (int)n, (int)k, (int)rpw);
  return hipGetLastError();
}

hipError_t launch_dense_gemv(bool bf16, const void* w, const void* x, const OutF32& y, int64_t n, int64_t k,
                             hipStream_t s) {
  return bf16 ? launch_dense<true>(w, x, y, n, k, s) : launch_dense<false>(w, x, y, n, k, s);
}
hipError_t launch_dense_gemv(bool bf16, const void* w, const void* x, const OutEx& y, int64_t n, int64_t k,
                             hipStream_t s) {
  return bf16 ? launch_dense<true>(w, x, y, n, k, s) : launch_dense<false>(w, x, y, n, k, s);
}

}  // namespace qgemv
