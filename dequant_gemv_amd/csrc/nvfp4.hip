// NVFP4 W4A16 fused dequantise + GEMV and row materialisation for gfx950.
//
// Format (Mojo module "fp4_gemv"): E2M1 nibbles with one FP8 E4M3 scale per 16
// consecutive weights; weight = e2m1 * |scale|; bf16 activations, fp32
// accumulation.  Buffer: [M][K/2] nibble bytes (even element in the low
// nibble), then [M][K/16] scale bytes.
//
// GEMV work split.  As on that page each lane owns whole 16-weight scale
// blocks, but on a wave64 the lanes take contiguous 16-byte slices: a wave
// owns one K-chunk of 2048 weights (1 KiB of nibbles, fully coalesced) for R
// rows, lane l the 32 weights 32l..32l+31 of the chunk (two scale blocks).
// gfx950 converts two E2M1 codes to a bf16 pair in one instruction
// (v_cvt_scalef32_pk_bf16_fp4, scale 1.0: exact) and v_dot2_f32_bf16 multiplies
// them with the matching bf16 activation pair into an fp32 accumulator, so a
// weight costs one VALU slot.  |scale| is applied once per 16-weight block
// (algebraically equal to scaling each weight; only the rounding order moves).
#include "device.hpp"
#include "launch.hpp"
#include "rows.hpp"
#include "stream.hpp"

namespace qgemv {

// Rows per wave and waves per workgroup (tuning).
#ifndef QGEMV_NVFP4_R
#define QGEMV_NVFP4_R 8
#endif
#ifndef QGEMV_WG_WAVES
#define QGEMV_WG_WAVES 8
#endif

template <int R, typename Out>
__global__ __launch_bounds__(64 * QGEMV_WG_WAVES) void nvfp4_gemv_kernel(const uint8_t* __restrict__ w,
                                                         const uint16_t* __restrict__ x,
                                                         Out out, int n, int k,
                                                         int kc, int kw, int rg) {
  __shared__ float red[16 * 16];
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: keeps the buffer descriptors in SGPRs
  const int kwi = wave % kw;
  const int rgi = wave / kw;
  const int64_t nib_row = k / 2, sc_row = k / 16;
  const int row0 = blockIdx.x * rg * R + rgi * R;
  const int nrows = max(0, min(R, n - row0));
  const auto nr = make_rsrc(w + (int64_t)row0 * nib_row, (uint32_t)(nrows * nib_row));
  const auto sr = make_rsrc(w + (int64_t)n * nib_row + (int64_t)row0 * sc_row, (uint32_t)(nrows * sc_row));
  const auto xr = make_rsrc(x, (uint32_t)k * 2u);

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;

  for (int ch = kwi; ch < kc; ch += kw) {
    const int e0 = ch * 2048 + 32 * lane;
    // Lanes past K in a ragged chunk point at the end of the ranges: nibbles,
    // scales and activations all read as zero and add exactly 0.
    const bool valid = e0 < k;
    const uint32_t nib_off = valid ? (uint32_t)(ch * 1024 + 16 * lane) : (uint32_t)(nrows * nib_row);
    const uint32_t sc_off = valid ? (uint32_t)(ch * 128 + 2 * lane) : (uint32_t)(nrows * sc_row);
    // Activations first (loads complete in issue order), then all R rows.
    unsigned X[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = ld128(xr, (uint32_t)e0 * 2u + 16u * i);
      X[4 * i] = v.x; X[4 * i + 1] = v.y; X[4 * i + 2] = v.z; X[4 * i + 3] = v.w;
    }
    u32x4 nib[R];
    unsigned sc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      nib[r] = ld128w(nr, nib_off + (uint32_t)(r * nib_row));
      sc[r] = ld16(sr, sc_off + (uint32_t)(r * sc_row));
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const unsigned q[4] = {nib[r].x, nib[r].y, nib[r].z, nib[r].w};
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x2 p0 = fp4x2_bf16(q[j >> 2], j);
        a0 = dot2bf(p0, X[j], a0);
        const bf16x2 p1 = fp4x2_bf16(q[2 + (j >> 2)], j);
        a1 = dot2bf(p1, X[8 + j], a1);
      }
      const float s0 = __builtin_fabsf(__builtin_amdgcn_cvt_f32_fp8((int)sc[r], 0));
      const float s1 = __builtin_fabsf(__builtin_amdgcn_cvt_f32_fp8((int)sc[r], 1));
      acc[r] = __builtin_fmaf(s1, a1, __builtin_fmaf(s0, a0, acc[r]));
    }
  }

  wave_reduce_rows<R>(acc);
  constexpr int L = log2i<R>();
  constexpr int kLanesPerRow = 64 >> L;
  if ((lane & (kLanesPerRow - 1)) == 0)
    red[(rgi * kw + kwi) * R + (lane >> (6 - L))] = acc[0];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < rg * R) {
    const int g = t / R, r = t % R;
    float s = 0.f;
    for (int kk = 0; kk < kw; ++kk) s += red[(g * kw + kk) * R + r];
    const int row = blockIdx.x * rg * R + g * R + r;
    if (row < n) out.put(row, s);
  }
}


// Row-streaming variant (K <= 16384): a wave owns R whole rows.  Its nibbles
// are one contiguous run of R*K/2 bytes in which unit u = r*KC + ch (row r,
// K-chunk ch of up to 2048 weights) starts at r*K/2 + 1024 ch; its scales are
// a second run of R*K/16 bytes, loaded up front.  Both land in the wave's LDS
// stage.  The activations are copied once per workgroup into LDS with each
// 64-byte lane slice spread as four 16-byte granules 1 KiB apart (so each of
// a lane's four reads is one contiguous 1 KiB across the wave) and held in
// registers for every chunk.  Lane l takes weights 32l..32l+31 of each chunk
// as in the K-split kernel; row totals are summed with DPP.
#ifndef QGEMV_NVFP4_AHEAD
#define QGEMV_NVFP4_AHEAD 4
#endif
#ifndef QGEMV_NVFP4_AHEAD0
#define QGEMV_NVFP4_AHEAD0 QGEMV_NVFP4_AHEAD
#endif
#ifndef QGEMV_NVFP4_FIRST
#define QGEMV_NVFP4_FIRST 8  // loads issued right after the activation barrier (measured best of 4-12)
#endif

template <int KC, int R, int W>
struct Nvfp4Rows {
  using S = StreamSchedule<1024, R * KC, QGEMV_NVFP4_AHEAD0, QGEMV_NVFP4_AHEAD, QGEMV_NVFP4_FIRST>;
  static constexpr int kScLoads = (R * KC * 128 + 1023) / 1024;
  static constexpr int kStage = kScLoads * 1024 + S::kStage;
  static constexpr int kLds = W * kStage + KC * 4096;
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};

template <int KC, int R, int W, typename Out>
__global__ __launch_bounds__(64 * W) void nvfp4_gemv_rows_kernel(const uint8_t* __restrict__ w,
                                                                const uint16_t* __restrict__ x,
                                                                Out out, int n, int k) {
  using C = Nvfp4Rows<KC, R, W>;
  using S = typename C::S;  // assumes the longest rows (K = 2048 KC); shorter rows only end earlier
  const int kNibRow = k / 2, kScRow = k / 16;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::kLds];
  unsigned char* const xs = lds + W * C::kStage;
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned char* const sc_stage = lds + wave * C::kStage;
  unsigned char* const nib_stage = sc_stage + C::kScLoads * 1024;
  const int row0 = (blockIdx.x * W + wave) * R;
  const int nrows = max(0, min(R, n - row0));

  // activations: granule t of lane slot i of chunk c lands at c*4096 + t*1024 + 16 i
  load_shared_pieces<4 * KC, W>(make_rsrc(x, (uint32_t)k * 2u), xs, wave, lane, [](int piece, int i) {
    return (uint32_t)(((piece >> 2) * 256 + i * 4 + (piece & 3)) * 16);
  });
  // The scale run, then the first nibble loads.  The run is nrows*K/16
  // bytes, not always a multiple of 16.  Buffer loads check the range dword
  // by dword: dwords past the end, and a dword the end cuts through, read as
  // zero.  So the bytes of the run's last partial 16-byte piece (2..14 of
  // them) are fetched again with exact 2-byte loads and written over what the
  // 16-byte load left there once the piece is in.
  const uint32_t sc_len = (uint32_t)(nrows * kScRow);
  const uint32_t sc_full = sc_len & ~15u;
  const bool tail_lane = 2u * (uint32_t)lane < sc_len - sc_full;
  const auto sr = make_rsrc(w + (int64_t)n * kNibRow + (int64_t)row0 * kScRow, sc_len);
  stream_loads<0, C::kScLoads, QGEMV_WLOAD_AUX>(sr, sc_stage, lane);
  const unsigned short sc_tail = ld16(sr, tail_lane ? sc_full + 2u * lane : sc_len);
  compiler_fence();  // counted by the wait below: stays between the scale and nibble loads
  const auto nr = make_rsrc(w + (int64_t)row0 * kNibRow, (uint32_t)(nrows * kNibRow));
  stream_loads<0, S::kUpFront, QGEMV_WLOAD_AUX>(nr, nib_stage, lane);

  wait_vm<S::kUpFront>();  // activations, scales and the scale tail (issued first) are in
  if (tail_lane) *reinterpret_cast<unsigned short*>(sc_stage + sc_full + 2 * lane) = sc_tail;
  __builtin_amdgcn_s_barrier();  // ... every wave's activation pieces too
  // the output stage's input for the wave's rows, after the barrier's wait
  // (the stream's later waits only get stricter by this one load)
  const auto pre = prefetch_rows(out, row0, nrows, lane);
  stream_loads<S::kUpFront, S::issued_before(0), QGEMV_WLOAD_AUX>(nr, nib_stage, lane);

  unsigned X[KC][16];
#pragma unroll
  for (int ch = 0; ch < KC; ++ch)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xs + ch * 4096 + t * 1024 + 16 * lane);
      X[ch][4 * t] = v.x; X[ch][4 * t + 1] = v.y; X[ch][4 * t + 2] = v.z; X[ch][4 * t + 3] = v.w;
    }

  // lanes past K in a ragged last chunk: the next row's bytes meet zero
  // activations, and their scales are dropped (a NaN scale must not leak)
  const bool tail_ok = (KC - 1) * 2048 + 32 * lane < k;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  static_for<0, R * KC>([&](auto uc) {
    constexpr int U = decltype(uc)::value, r = U / KC, ch = U % KC;
    wait_vm<S::wait_count(U)>();
    // refill first: the stage holds the whole run (no unread byte is
    // overwritten) and the arithmetic stays off the load path
    stream_loads<S::issued_before(U), S::issued_before(U + 1), QGEMV_WLOAD_AUX>(nr, nib_stage, lane);
    const u32x4 nv = *reinterpret_cast<const u32x4*>(nib_stage + r * kNibRow + ch * 1024 + 16 * lane);
    const unsigned sc = *reinterpret_cast<const uint16_t*>(sc_stage + r * kScRow + ch * 128 + 2 * lane);
    const unsigned q[4] = {nv.x, nv.y, nv.z, nv.w};
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a0 = dot2bf(fp4x2_bf16(q[j >> 2], j), X[ch][j], a0);
      a1 = dot2bf(fp4x2_bf16(q[2 + (j >> 2)], j), X[ch][8 + j], a1);
    }
    float s0 = __builtin_fabsf(__builtin_amdgcn_cvt_f32_fp8((int)sc, 0));
    float s1 = __builtin_fabsf(__builtin_amdgcn_cvt_f32_fp8((int)sc, 1));
    if constexpr (ch == KC - 1) {
      s0 = tail_ok ? s0 : 0.f;
      s1 = tail_ok ? s1 : 0.f;
    }
    acc[r] = __builtin_fmaf(s1, a1, __builtin_fmaf(s0, a0, acc[r]));
  });
  store_rows<R>(acc, out, pre, row0, nrows, 1.f, lane);
}

// Row materialisation.  Task t of an output row makes weights
// [E t, E t + E) (E = 8 or 4): E/2 nibble bytes and the one scale byte of
// their 16-weight block; every weight e2m1 * |scale| is exact in fp32 (and in
// fp16 / bf16).
#ifndef QGEMV_NVFP4_ROWS_U
#define QGEMV_NVFP4_ROWS_U 2  // row-materialisation tasks per thread
#endif

struct Nvfp4RowIn {
  unsigned q;
  unsigned sc;
};

template <typename T, int U>
__global__ __launch_bounds__(256) void nvfp4_rows_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                         const int32_t* __restrict__ rows, T* __restrict__ out,
                                                         int bpr) {
  constexpr int E = kRowsE<T>;
  const int j = blockIdx.x / bpr;
  const int r = source_row(rows, j, n);
  const int64_t rr = r < 0 ? 0 : r;
  const uint8_t* const nib = w + rr * (k / 2);
  const uint8_t* const scl = w + (int64_t)n * (k / 2) + rr * (k / 16);
  T* const orow = out + (int64_t)j * k;
  rows_thread<U, Nvfp4RowIn>(
      bpr, k / E, r >= 0,
      [&](int t) {
        const int e0 = t * E;
        Nvfp4RowIn in;
        in.q = E == 8 ? *reinterpret_cast<const uint32_t*>(nib + e0 / 2)
                      : *reinterpret_cast<const uint16_t*>(nib + e0 / 2);
        in.sc = scl[e0 / 16];
        return in;
      },
      [&](int t, const Nvfp4RowIn& in) {
        const float s = __builtin_fabsf(__builtin_amdgcn_cvt_f32_fp8((int)in.sc, 0));
        float v[E];
#pragma unroll
        for (int i = 0; i < E / 2; ++i) {
          const f32x2 p = fp4x2_f32(in.q, i);
          v[2 * i] = p.x * s;
          v[2 * i + 1] = p.y * s;
        }
        store_e(orow + t * E, v);
      },
      [&](int t) { store_e_nan(orow + t * E); });
}

template <int R, typename Out>
static hipError_t launch_nvfp4_r(const void* w, const void* x, const Out& y, int64_t n, int64_t k,
                                 hipStream_t s) {
  const int kc = (int)((k + 2047) / 2048);
  const int kw = kc < QGEMV_WG_WAVES ? kc : QGEMV_WG_WAVES;
  const int rg = kw >= QGEMV_WG_WAVES ? 1 : QGEMV_WG_WAVES / kw;
  const int rows_per_wg = rg * R;
  const int64_t grid = (n + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((nvfp4_gemv_kernel<R, Out>), dim3((unsigned)grid), dim3(64 * kw * rg), 0, s,
                     (const uint8_t*)w, (const uint16_t*)x, y, (int)n, (int)k, kc, kw, rg);
  return hipGetLastError();
}

template <int KC, int R, int W, typename Out>
static hipError_t launch_nvfp4_rows_r(const void* w, const void* x, const Out& y, int64_t n, int64_t k, hipStream_t s) {
  const int64_t rows_per_wg = (int64_t)W * R;
  const int64_t grid = (n + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((nvfp4_gemv_rows_kernel<KC, R, W, Out>), dim3((unsigned)grid), dim3(64 * W), 0, s,
                     (const uint8_t*)w, (const uint16_t*)x, y, (int)n, (int)k);
  return hipGetLastError();
}

template <int KC, typename Out>
static hipError_t launch_nvfp4_rows(const void* w, const void* x, const Out& y, int64_t n, int64_t k, hipStream_t s) {
  constexpr int kRmax = largest_fitting_r([](int r) {
    return 8 * (((r * KC * 128 + 1023) / 1024) + r * KC) * 1024 + KC * 4096 <= 160 * 1024;
  });
  return dispatch_rows<kRmax>(n, [&](auto rc, auto wc) {
    return launch_nvfp4_rows_r<KC, decltype(rc)::value, decltype(wc)::value, Out>(w, x, y, n, k, s);
  });
}

#ifndef QGEMV_NVFP4_IMPL
#define QGEMV_NVFP4_IMPL 2  // 1: K-split kernel only, 2: row-streaming for K <= 16384
#endif

template <typename Out>
static hipError_t launch_nvfp4_gemv_out(const void* w, const void* x, const Out& y, int64_t n, int64_t k,
                                      hipStream_t s) {
  if (QGEMV_NVFP4_IMPL == 2) {
    switch ((k + 2047) / 2048) {
      case 1: return launch_nvfp4_rows<1, Out>(w, x, y, n, k, s);
      case 2: return launch_nvfp4_rows<2, Out>(w, x, y, n, k, s);
      case 3: return launch_nvfp4_rows<3, Out>(w, x, y, n, k, s);
      case 4: return launch_nvfp4_rows<4, Out>(w, x, y, n, k, s);
      case 5: return launch_nvfp4_rows<5, Out>(w, x, y, n, k, s);
      case 6: return launch_nvfp4_rows<6, Out>(w, x, y, n, k, s);
      case 7: return launch_nvfp4_rows<7, Out>(w, x, y, n, k, s);
      case 8: return launch_nvfp4_rows<8, Out>(w, x, y, n, k, s);
      default: break;
    }
  }
  return launch_nvfp4_r<QGEMV_NVFP4_R, Out>(w, x, y, n, k, s);
}

hipError_t launch_nvfp4_gemv(const void* w, const void* x, const OutF32& y, int64_t n, int64_t k, hipStream_t s) {
  return launch_nvfp4_gemv_out(w, x, y, n, k, s);
}
hipError_t launch_nvfp4_gemv(const void* w, const void* x, const OutEx& y, int64_t n, int64_t k, hipStream_t s) {
  return launch_nvfp4_gemv_out(w, x, y, n, k, s);
}

template <typename T, int U>
static hipError_t launch_nvfp4_rows_u(const void* w, int64_t n, int64_t k, const int32_t* rows, int64_t nrows,
                                    void* out, hipStream_t s) {
  const RowsGeom g = rows_geom(k / kRowsE<T>, nrows, U);
  hipLaunchKernelGGL((nvfp4_rows_kernel<T, U>), dim3((unsigned)g.grid), dim3(g.block), 0, s, (const uint8_t*)w,
                     (int)n, (int)k, rows, (T*)out, g.bpr);
  return hipGetLastError();
}

// Small launches (a few hundred gathered rows) take one task per thread so
// that they still spread over the whole chip.
template <typename T>
static hipError_t launch_nvfp4_rows_t(const void* w, int64_t n, int64_t k, const int32_t* rows, int64_t nrows,
                                    void* out, hipStream_t s) {
  if (nrows * (k / kRowsE<T>) < kRowsSmallTasks) return launch_nvfp4_rows_u<T, 1>(w, n, k, rows, nrows, out, s);
  return launch_nvfp4_rows_u<T, QGEMV_NVFP4_ROWS_U>(w, n, k, rows, nrows, out, s);
}

hipError_t launch_nvfp4_get_rows(const void* w, int64_t n, int64_t k, const int32_t* rows, int64_t nrows,
                                 void* out, int dtype, hipStream_t s) {
  if (dtype == kF16) return launch_nvfp4_rows_t<_Float16>(w, n, k, rows, nrows, out, s);
  if (dtype == kBF16) return launch_nvfp4_rows_t<__bf16>(w, n, k, rows, nrows, out, s);
  return launch_nvfp4_rows_t<float>(w, n, k, rows, nrows, out, s);
}

}  // namespace qgemv
