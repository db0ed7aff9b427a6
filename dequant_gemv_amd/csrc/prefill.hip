// Prefill (many activation rows at once) for gfx950: Y[t][r] = sum_k X[t][k] *
// dequant(W)[r][k], the M > 1 path of the Mojo fp4_gemv page (its cooperative
// shared-memory matmul) and the TQ1_0 page's prefill, where the weights are
// dequantised a block at a time into a tile that a matrix unit consumes.
//
// Unlike the batch-1 GEMV this is a dense contraction (2 T flops per weight
// byte pair), so it runs on MFMA: v_mfma_f32_16x16x32_{f16,bf16}, whose lane
// layout (checked on the part) is A[m][k] at lane m%16 + 16 (k/8) element k%8,
// B[k][n] at lane n%16 + 16 (k/8) element k%8, D[m][n] at lane n + 16 (m/4)
// register m%4 (m, n < 16, k < 32).  Tokens are the MFMA's M, weight rows its
// N, so a B fragment is 8 consecutive weights of one weight row.
//
// Work split.  A workgroup (4 waves) owns a tile of BT = 128 tokens x BN = 128
// weight rows and walks K in steps of 64 weights; each wave accumulates a
// 64 x 64 sub-tile (4 x 4 MFMA tiles) in registers.  Per step:
//  - the activations of the tile (128 x 64 values) go to LDS; row t's
//    16-byte granule g sits at position g ^ (t & 7) of its 128-byte LDS row,
//    so that the 16 lanes of a fragment read hit different banks;
//  - each thread dequantises 32 weights of one weight row of the step (the
//    format's functor: packed bytes straight from global memory into
//    registers, fp32 arithmetic, one rounding to the MFMA input type) and
//    writes them to LDS with the same swizzle;
//  - the waves read A and B fragments with ds_read_b128 and issue 32 MFMAs.
// Loads run several steps ahead (see prefill_kernel); one barrier per step.
#include "device.hpp"
#include "launch.hpp"

namespace qgemv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPfBT = 128;   // tokens per workgroup tile
constexpr int kPfBN = 128;   // weight rows per workgroup tile
constexpr int kPfKS = 64;    // weights per K step
constexpr int kPfRowB = 128; // LDS bytes per tile row per step (64 16-bit values)
constexpr int kPfTile = kPfBT * kPfRowB;  // 16 KiB

// LDS byte offset of 16-byte granule g (0..7) of tile row t.
__device__ __forceinline__ int pf_off(int t, int g) { return t * kPfRowB + 16 * (g ^ (t & 7)); }

// Two fp32 values -> two 16-bit codes of T (round to nearest even), packed.
template <typename T>
__device__ __forceinline__ unsigned pf_pack2(float a, float b) {
  const T lo = (T)pin_f32(a), hi = (T)pin_f32(b);
  return (unsigned)__builtin_bit_cast(unsigned short, lo) | ((unsigned)__builtin_bit_cast(unsigned short, hi) << 16);
}

// ---- per-format weight steps ------------------------------------------------
// A functor gives, for thread (row r of the tile, half h) and step s, the 32
// weights [64 s + 32 h, 64 s + 32 h + 32) of the row as 16 packed 16-bit
// codes.  load() only issues loads (raw packed bytes); make() does the
// arithmetic once they are in.

// Q4_K ("Writing a high performant GEMV + dequant for Metal", sections "What
// is a weight block?" and "Kernel code"): step s is chunk c = s % 4 of block
// b = s / 4; half h = the low (h = 0) or high nibbles of its 32 qs bytes,
// i.e. group 2c + h.
struct Q4kPrefill {
  using T = _Float16;
  static constexpr bool kBf16 = false;
  static constexpr int kKMultiple = 256;
  static constexpr bool kWaveHalf = false;  // neighbouring lanes: the two halves of one row
  struct Desc {
    __amdgpu_buffer_rsrc_t r;  // the tile's rows
    uint32_t row_bytes;
  };
  struct Raw {
    u32x4 hdr, q0, q1;
  };
  static __device__ __forceinline__ Desc desc(const uint8_t* w, int, int k, int n0, int nv) {
    const uint32_t rb = (uint32_t)(k / 256 * 144);
    return Desc{make_rsrc(w + (int64_t)n0 * rb, (uint32_t)nv * rb), rb};
  }
  static __device__ __forceinline__ Raw load(const Desc& d, int r, int s, int) {
    const uint32_t blk = (uint32_t)r * d.row_bytes + (uint32_t)(s >> 2) * 144u;
    const uint32_t qo = blk + 16u + 32u * (uint32_t)(s & 3);
    Raw raw;
    raw.hdr = ld128(d.r, blk);
    raw.q0 = ld128(d.r, qo);
    raw.q1 = ld128(d.r, qo + 16u);
    return raw;
  }
  static __device__ __forceinline__ void make(const Raw& raw, int s, int h, unsigned (&out)[16]) {
    const int c = s & 3;
    // 6-bit scale and min of group 2c + h (same packing as the GEMV kernels)
    const bool hi = c >= 2;
    const unsigned sh = 16u * (unsigned)(c & 1) + 8u * (unsigned)h;
    const unsigned ma = hi ? 0x0Fu : 0x3Fu;
    const unsigned sa = hi ? raw.hdr.w : raw.hdr.y, mb = hi ? raw.hdr.w : raw.hdr.z;
    const unsigned sg = ((sa >> sh) & ma) | (hi ? (((raw.hdr.y >> (sh + 6)) & 3u) << 4) : 0u);
    const unsigned mg = ((mb >> (sh + (hi ? 4u : 0u))) & ma) | (hi ? (((raw.hdr.z >> (sh + 6)) & 3u) << 4) : 0u);
    const float ds = f16lo(raw.hdr.x) * (float)sg, dm = f16hi(raw.hdr.x) * (float)mg;
    const unsigned q[8] = {raw.q0.x, raw.q0.y, raw.q0.z, raw.q0.w, raw.q1.x, raw.q1.y, raw.q1.z, raw.q1.w};
    const unsigned nsh = 4u * (unsigned)h;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned v = (q[i] >> nsh) & 0x0F0F0F0Fu;  // four nibbles, one per byte
      const float w0 = __builtin_fmaf(ds, (float)(v & 0xFFu), -dm);
      const float w1 = __builtin_fmaf(ds, (float)((v >> 8) & 0xFFu), -dm);
      const float w2 = __builtin_fmaf(ds, (float)((v >> 16) & 0xFFu), -dm);
      const float w3 = __builtin_fmaf(ds, (float)(v >> 24), -dm);
      out[2 * i] = pf_pack2<T>(w0, w1);
      out[2 * i + 1] = pf_pack2<T>(w2, w3);
    }
  }
};

// NVFP4 (Mojo module "fp4_gemv"): step s, half h = weights [64 s + 32 h, +32)
// of a row: 16 nibble bytes and the 2 scale bytes of their two 16-weight
// blocks.  Every e2m1 * |scale| is exact in fp32 and in bf16, so the bf16
// weights are exact and the MFMA runs on bf16 (the activations' type).
struct Nvfp4Prefill {
  using T = __bf16;
  static constexpr bool kBf16 = true;
  static constexpr int kKMultiple = 64;
  static constexpr bool kWaveHalf = false;
  struct Desc {
    __amdgpu_buffer_rsrc_t nib, sc;  // the tile's nibble rows, its scale rows
    uint32_t nib_row, sc_row;
  };
  struct Raw {
    u32x4 q;
    unsigned short sc;
  };
  static __device__ __forceinline__ Desc desc(const uint8_t* w, int n, int k, int n0, int nv) {
    const uint32_t nr = (uint32_t)(k / 2), sr = (uint32_t)(k / 16);
    return Desc{make_rsrc(w + (int64_t)n0 * nr, (uint32_t)nv * nr),
                make_rsrc(w + (int64_t)n * nr + (int64_t)n0 * sr, (uint32_t)nv * sr), nr, sr};
  }
  static __device__ __forceinline__ Raw load(const Desc& d, int r, int s, int h) {
    Raw raw;
    raw.q = ld128(d.nib, (uint32_t)r * d.nib_row + 32u * (uint32_t)s + 16u * (uint32_t)h);
    raw.sc = ld16(d.sc, (uint32_t)r * d.sc_row + 4u * (uint32_t)s + 2u * (uint32_t)h);
    return raw;
  }
  static __device__ __forceinline__ void make(const Raw& raw, int, int, unsigned (&out)[16]) {
    const float s0 = __builtin_fabsf(__builtin_amdgcn_cvt_f32_fp8((int)raw.sc, 0));
    const float s1 = __builtin_fabsf(__builtin_amdgcn_cvt_f32_fp8((int)raw.sc, 1));
    const unsigned q[4] = {raw.q.x, raw.q.y, raw.q.z, raw.q.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // byte i: weights 2i, 2i + 1 (block i / 8)
      const f32x2 e = fp4x2_f32(q[i >> 2], i);
      const float sc = i < 8 ? s0 : s1;
      out[i] = pf_pack2<T>(e.x * sc, e.y * sc);
    }
  }
};


// TQ1_0 ("metal: TQ1_0 kernel performance", sections 1, 2 and "Not
// applicable"): step s covers elements [64 c, 64 c + 64) of block b = s / 4
// (c = s % 4); half h the 32 starting at e0 = 64 c + 32 h, which are one
// digit of qs[0..31] (e0 < 160), two digits of qs[32..47] (e0 = 160, 192),
// or digit 4 of qs[32..47] followed by the four digits of qh[0..3] (e0 =
// 224).  The block is only 2-byte aligned, so the bytes from qs[0] (or
// qs[32]) on are read as nine aligned dwords (single-dword loads: one past
// the range reads zero and is never needed) and realigned with alignbyte; d
// is a 16-bit load.  Each weight is one of d * -1, d * 0, d * 1, exact in
// fp16: two weights' digits come from one packed 16-bit multiply and one
// byte permute picks their fp16 codes (as in the row materialisation).
struct Tq1Prefill {
  using T = _Float16;
  static constexpr bool kBf16 = false;
  static constexpr int kKMultiple = 256;
  static constexpr bool kWaveHalf = true;  // make() branches on the half: one half per wave
  struct Desc {
    __amdgpu_buffer_rsrc_t r;  // the tile's rows
    uint32_t row_bytes;
  };
  struct Raw {
    unsigned wd[9];
    unsigned short d;
    unsigned char sh;  // bytes to drop at the front of the window
  };
  static __device__ __forceinline__ Desc desc(const uint8_t* w, int, int k, int n0, int nv) {
    const uint32_t rb = (uint32_t)(k / 256 * 54);
    return Desc{make_rsrc(w + (int64_t)n0 * rb, (uint32_t)nv * rb), rb};
  }
  static __device__ __forceinline__ Raw load(const Desc& d, int r, int s, int h) {
    const uint32_t blk = (uint32_t)r * d.row_bytes + (uint32_t)(s >> 2) * 54u;
    const int e0 = 64 * (s & 3) + 32 * h;
    const uint32_t a = blk + (e0 < 160 ? 0u : 32u);
    const uint32_t al = a & ~3u;
    Raw raw;
#pragma unroll
    for (int i = 0; i < 9; ++i) raw.wd[i] = ld32(d.r, al + 4u * (uint32_t)i);
    raw.d = ld16(d.r, blk + 52u);
    raw.sh = (unsigned char)(a & 3u);
    return raw;
  }
  // weights (2 pr, 2 pr + 1) from bytes bi, bi + 1 of the stream, digit k
  static __device__ __forceinline__ unsigned pair(const unsigned (&q)[8], int bi, int k, unsigned vm, unsigned vp) {
    const unsigned word = q[bi >> 2];
    const unsigned b = (unsigned)(bi & 3);
    const unsigned pr = __builtin_amdgcn_perm(0u, word, 0x0C000C00u | b | ((b + 1u) << 16));
    const u16x2 dg = tq1_digits2(__builtin_bit_cast(u16x2, pr), pow3_u16(k));
    const u16x2 sel = dg * u16x2{0x0202, 0x0202} + u16x2{0x0100, 0x0100};
    return __builtin_amdgcn_perm(vp, vm, __builtin_bit_cast(unsigned, sel));
  }
  static __device__ __forceinline__ void make(const Raw& raw, int s, int h, unsigned (&out)[16]) {
    unsigned q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = __builtin_amdgcn_alignbyte(raw.wd[j + 1], raw.wd[j], raw.sh);
    const float d = (float)__builtin_bit_cast(_Float16, raw.d);
    const unsigned vm = pf_pack2<T>(d * -1.f, d * 0.f);  // codes of d*(t-1), t = 0, 1
    const unsigned vp = pf_pack2<T>(d * 1.f, 0.f);        // and t = 2
    const int e0 = 64 * (s & 3) + 32 * h;  // the same for the whole wave
    if (e0 < 160) {
      const int k = e0 >> 5;
#pragma unroll
      for (int p = 0; p < 16; ++p) out[p] = pair(q, 2 * p, k, vm, vp);
    } else if (e0 < 224) {
      const int k0 = (e0 - 160) >> 4;
#pragma unroll
      for (int p = 0; p < 16; ++p) out[p] = pair(q, (2 * p) & 15, k0 + (p >> 3), vm, vp);
    } else {
#pragma unroll
      for (int p = 0; p < 8; ++p) out[p] = pair(q, 2 * p, 4, vm, vp);
#pragma unroll
      for (int p = 8; p < 16; ++p) out[p] = pair(q, 16 + ((2 * p - 16) & 3), (2 * p - 16) >> 2, vm, vp);
    }
  }
};

// ---- the kernel ---------------------------------------------------------------

#ifndef QGEMV_PREFILL_INTERLEAVE
#define QGEMV_PREFILL_INTERLEAVE 4  // ALU instructions placed after each MFMA (0: no placement)
#endif
#ifndef QGEMV_PREFILL_DEPTH
#define QGEMV_PREFILL_DEPTH 2  // K steps of loads in flight
#endif

// P = steps of loads in flight: step s + P is issued while step s is
// multiplied.  Loads go to registers only (a P-deep rotation of activation
// and packed-weight registers); both tiles are written to LDS with ds_write
// one step before they are used, into double-buffered stages.  (Loading the
// activations with LDS-DMA instead makes the compiler wait for every DMA in
// flight before any LDS access it cannot prove disjoint, which drains the
// pipeline every step.)
template <typename F, int P>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const uint8_t* __restrict__ w,
                                                        const uint16_t* __restrict__ x, float* __restrict__ y,
                                                        int t_count, int n, int k, int split_steps) {
  __shared__ __attribute__((aligned(1024))) unsigned char xs0[2 * kPfTile];
  __shared__ __attribute__((aligned(1024))) unsigned char ws0[2 * kPfTile];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.y * kPfBT, n0 = blockIdx.x * kPfBN;
  // K split z of gridDim.z: steps [z * split_steps, ...) of the K / 64 steps
  const int s_begin = blockIdx.z * split_steps;
  const int steps = min(split_steps, k / kPfKS - s_begin);
  const uint32_t xrow = (uint32_t)k * 2u;  // bytes per activation row

  // activations of the tile: rows t0.. (zero past T); weights: rows n0.. (zero past n)
  const int tv = min(kPfBT, t_count - t0), nv = min(kPfBN, n - n0);
  const auto xr = make_rsrc(x + (int64_t)t0 * k, (uint32_t)tv * xrow);
  const typename F::Desc wd = F::desc(w, n, k, n0, nv);

  // this thread's slots: activation granules 4 xh .. 4 xh + 3 of tile row
  // xr_ = tid / 2 (64 contiguous bytes), and weights [32 dh, 32 dh + 32) of
  // weight row dr: the two halves of a row on neighbouring lanes (their
  // packed bytes are next to each other), or, for a format whose
  // dequantisation branches on the half, one half per wave
  const int xr_ = tid >> 1, xh = tid & 1;
  const int dr = F::kWaveHalf ? (tid & 127) : (tid >> 1), dh = F::kWaveHalf ? (tid >> 7) : (tid & 1);
  const uint32_t xoff = (uint32_t)xr_ * xrow + 64u * (uint32_t)xh;

  struct XRaw {
    u32x4 g[4];
  };
  auto load_x = [&](int s) {
    XRaw v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v.g[i] = ld128(xr, xoff + (uint32_t)(s_begin + s) * 128u + 16u * (uint32_t)i);
    return v;
  };
  auto store_x = [&](const XRaw& v, int b) {
    unsigned char* const base = xs0 + b * kPfTile;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(base + pf_off(xr_, 4 * xh + i)) = v.g[i];
  };
  auto store_w = [&](const unsigned (&v)[16], int b) {
    unsigned char* const base = ws0 + b * kPfTile;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<u32x4*>(base + pf_off(dr, 4 * dh + g)) = u32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // wave sub-tile: tokens 64 (wave & 1) .., rows 64 (wave >> 1) ..
  const int wt = 64 * (wave & 1), wn = 64 * (wave >> 1);
  const int fl = lane & 15, fq = lane >> 4;  // fragment row / column and k-granule

  // prologue: steps 0 .. P-1 in flight, step 0 into stage 0
  XRaw xq[P];
  typename F::Raw wq[P];
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < steps) {
      xq[p] = load_x(p);
      wq[p] = F::load(wd, dr, s_begin + p, dh);
    }
  {
    store_x(xq[0], 0);
    unsigned v[16];
    F::make(wq[0], s_begin, dh, v);
    store_w(v, 0);
  }
  lds_barrier();

  for (int s0 = 0; s0 < steps; s0 += P) {
    static_for<0, P>([&](auto ic) {
      constexpr int I = decltype(ic)::value;
      const int s = s0 + I;
      if (s < steps) {
        // Straight-line step (one scheduling region): step s + P into the
        // registers step s used (stored at the end of step s - 1); past the
        // end these are harmless range-checked reads and the last step's
        // stores go to a stage nobody reads.
        xq[I] = load_x(s + P);
        wq[I] = F::load(wd, dr, s_begin + s + P, dh);
        const unsigned char* const xb = xs0 + (s & 1) * kPfTile;
        const unsigned char* const wb = ws0 + (s & 1) * kPfTile;
        // step s + 1's dequantisation, interleaved below with this step's MFMAs
        constexpr int J = (I + 1) % P;
        unsigned v[16];
        F::make(wq[J], s_begin + s + 1, dh, v);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int g = 4 * kh + fq;
          u32x4 af[4], bf[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const u32x4*>(xb + pf_off(wt + 16 * i + fl, g));
#pragma unroll
          for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const u32x4*>(wb + pf_off(wn + 16 * j + fl, g));
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if constexpr (F::kBf16)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                                     __builtin_bit_cast(bf16x8, bf[j]), acc[i][j],
                                                                     0, 0, 0);
              else
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, af[i]),
                                                                    __builtin_bit_cast(half8, bf[j]), acc[i][j], 0,
                                                                    0, 0);
            }
        }
        store_x(xq[J], (s + 1) & 1);
        store_w(v, (s + 1) & 1);
        // issue order: fragment reads, then each MFMA followed by a few of the
        // dequantisation's ALU instructions (in-order issue would otherwise
        // run them all after the last MFMA)
#if QGEMV_PREFILL_INTERLEAVE
        static_for<0, 2>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x0100, 8, 0);  // 8 DS reads
          static_for<0, 16>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x0002, QGEMV_PREFILL_INTERLEAVE, 0);  // VALU
          });
        });
#endif
        lds_barrier();  // this step's LDS reads and the next step's stores are done
      }
    });
  }

  // D[m][n] of tile (i, j) sits at lane n + 16 (m / 4), register m % 4
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int t = t0 + wt + 16 * i + 4 * fq + a;
      if (t < t_count) {
        float* const yr = y + (int64_t)t * n;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + wn + 16 * j + fl;
          if (col < n) {
            if (gridDim.z == 1)
              yr[col] = acc[i][j][a];
            else
              atomicAdd(yr + col, acc[i][j][a]);  // partial sum of one K split (y zeroed first)
          }
        }
      }
    }
}

__global__ __launch_bounds__(256) void prefill_zero_kernel(float* __restrict__ y, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) y[i] = 0.f;
}

// Tiles of 128 x 128.  When there are fewer tiles than CUs, K is split as
// well (about two workgroups per CU, at least 8 steps per split) and the
// splits add their partial sums into y with fp32 atomics, y being cleared by
// a fill kernel first (a kernel, so that the sequence can be captured in a
// graph); the order of those few additions varies from run to run.
template <typename F>
static hipError_t launch_prefill(const void* w, const void* x, float* y, int64_t t, int64_t n, int64_t k,
                                 hipStream_t s) {
  const int64_t tiles = ((n + kPfBN - 1) / kPfBN) * ((t + kPfBT - 1) / kPfBT);
  const int64_t steps = k / kPfKS;
  int64_t split = 1;
  if (tiles < 256) split = (512 + tiles - 1) / tiles;  // fewer tiles than CUs
  split = min(split, max(int64_t(1), steps / 8));
  split = min(split, int64_t(16));
  const int64_t split_steps = (steps + split - 1) / split;
  split = (steps + split_steps - 1) / split_steps;
  if (split > 1) {
    const int64_t count = t * n;
    hipLaunchKernelGGL(prefill_zero_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, y, count);
  }
  const dim3 grid((unsigned)((n + kPfBN - 1) / kPfBN), (unsigned)((t + kPfBT - 1) / kPfBT), (unsigned)split);
  hipLaunchKernelGGL((prefill_kernel<F, QGEMV_PREFILL_DEPTH>), grid, dim3(256), 0, s, (const uint8_t*)w,
                     (const uint16_t*)x, y, (int)t, (int)n, (int)k, (int)split_steps);
  return hipGetLastError();
}

hipError_t launch_q4k_prefill(const void* w, const void* x, float* y, int64_t t, int64_t n, int64_t k, hipStream_t s) {
  return launch_prefill<Q4kPrefill>(w, x, y, t, n, k, s);
}
hipError_t launch_nvfp4_prefill(const void* w, const void* x, float* y, int64_t t, int64_t n, int64_t k,
                                hipStream_t s) {
  return launch_prefill<Nvfp4Prefill>(w, x, y, t, n, k, s);
}
hipError_t launch_tq1_prefill(const void* w, const void* x, float* y, int64_t t, int64_t n, int64_t k, hipStream_t s) {
  return launch_prefill<Tq1Prefill>(w, x, y, t, n, k, s);
}

}  // namespace qgemv
