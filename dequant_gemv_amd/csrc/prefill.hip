// Prefill (many activation rows at once) for gfx950: Y[t][r] = sum_k X[t][k] *
// dequant(W)[r][k], the M > 1 path of the Mojo fp4_gemv page (its cooperative
// shared-memory matmul) and the TQ1_0 page's prefill, where the weights are
// dequantised a block at a time into a tile that a matrix unit consumes.
//
// Unlike the batch-1 GEMV this is a dense contraction (2 T flops per weight),
// so it runs on MFMA: v_mfma_f32_32x32x16_{f16,bf16}, whose lane layout
// (checked on the part) is A[m][k] at lane m + 32 (k/8) element k%8, B[k][n]
// at lane n + 32 (k/8) element k%8, D[m][n] at lane n + 32 ((m/4) % 2)
// register 4 (m/8) + m%4 (m, n < 32, k < 16).  Tokens are the MFMA's M,
// weight rows its N, so a B fragment is 8 consecutive weights of one weight
// row.  (This shape sustains about 78% of the unit's peak from one wave per
// SIMD on the part, 16x16x32 about half.)
//
// Work split.  A workgroup of 8 waves (two per SIMD, so that one wave's
// loads, decode and barrier waits overlap the other's MFMAs) owns a tile of
// BT = 256 or 512 tokens x 128 weight rows and walks K in steps of 64
// weights; each wave accumulates a BT/4 x 64 sub-tile (BT/128 x 2 MFMA tiles
// of 32 x 32).  Per step:
//  - the activations of the tile (BT x 64 values, 32 or 64 KiB) go straight from
//    global memory into LDS (buffer loads with the LDS bit, no registers);
//    row t's 16-byte granule g sits at position g ^ ((t / 2) % 8) of its
//    128-byte LDS row, so that the lanes of a fragment read hit different
//    banks;
//  - each thread dequantises 16 weights of one weight row of the step (the
//    format's functor: packed bytes straight from global memory into
//    registers, one rounding to the MFMA input type) and writes them to LDS
//    with the same swizzle;
//  - each wave reads 16 A and B fragments (ds_read_b128) and issues 16 MFMAs.
// Each packed weight is decoded once per BT tokens.

#include "device.hpp"
#include "launch.hpp"
#include "prefill_plan.hpp"

namespace qgemv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfRowB = 128;  // LDS bytes per tile row per step (64 16-bit values)
constexpr int kPfWTile = kPfBN * kPfRowB;  // 16 KiB of weights per stage
constexpr int kPfWaves = 8;

// A load whose step lies past the end of the K range starts at this offset,
// which is beyond every descriptor's range (each covers < 2^31 bytes): it
// reads zero without touching memory.
constexpr uint32_t kPfDead = 0x80000000u;

// LDS byte offset of 16-byte granule g (0..7) of tile row t.  Rows are 128
// bytes, so the 256-byte bank space of the LDS holds two: the granules of a
// row pair are permuted by (t / 2) % 8, and any 16 consecutive rows put a
// given granule in 16 different 16-byte bank groups (a fragment read of 16
// rows, or the 16 lanes of a store, is conflict-free).
__device__ __forceinline__ int pf_off(int t, int g) { return t * kPfRowB + 16 * (g ^ ((t >> 1) & 7)); }

// fp16 pair (fma(a_H, s, m), fma(b_H, s, m)), each rounded once from the
// exact value, where a_H, b_H are the fp16 values in half H of a and b:
// v_fma_mix reads an fp16 operand from either half of a register and writes
// either half of the result (the compiler forms the low write but packs the
// high one with a shift and an or).
template <int H>
__device__ __forceinline__ unsigned mix_pair(unsigned a, unsigned b, float s, float m, Int<H>) {
  unsigned d;
  if constexpr (H == 0) {
    __asm__("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(a), "v"(s), "v"(m));
    __asm__("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "+v"(d) : "v"(b), "v"(s), "v"(m));
  } else {
    __asm__("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(a), "v"(s), "v"(m));
    __asm__("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(d) : "v"(b), "v"(s), "v"(m));
  }
  return d;
}

// Two fp32 values -> two 16-bit codes of T (round to nearest even), packed.
template <typename T>
__device__ __forceinline__ unsigned pf_pack2(float a, float b) {
  const T lo = (T)pin_f32(a), hi = (T)pin_f32(b);
  return (unsigned)__builtin_bit_cast(unsigned short, lo) | ((unsigned)__builtin_bit_cast(unsigned short, hi) << 16);
}

// ---- per-format weight steps ------------------------------------------------
// A functor gives, for thread (row r of the tile, quarter q) and step s, the
// 16 weights [64 s + 16 q, 64 s + 16 q + 16) of the row as 8 packed 16-bit
// codes.  load() only issues loads (raw packed bytes, kLoads of them; all
// zero when `live` is false); make() does the arithmetic once they are in,
// and turns zero bytes into zero weights.  Offsets split into a per-thread
// part (voff) and a wave-uniform part (soff, an SGPR).  The four quarters of
// a row sit on neighbouring lanes, so their packed bytes are next to each
// other in a load.

// Q4_K ("Writing a high performant GEMV + dequant for Metal", sections "What
// is a weight block?" and "Kernel code"): step s is chunk c = s % 4 of block
// b = s / 4, i.e. the 32 qs bytes whose low nibbles are group 2c and whose
// high nibbles are group 2c + 1; quarter q = nibbles h = q / 2 of qs bytes
// 32 c + 16 (q % 2) .. + 16.
struct Q4kPrefill {
  using T = _Float16;
  static constexpr bool kBf16 = false;
  static constexpr int kKMultiple = 256;
  static constexpr int kLoads = 2;
  struct Desc {
    __amdgpu_buffer_rsrc_t r;  // the tile's rows
    uint32_t row_bytes;
  };
  struct Raw {
    u32x4 hdr, qs;
  };
  static __device__ __forceinline__ Desc desc(const uint8_t* w, int, int k, int n0, int nv) {
    const uint32_t rb = (uint32_t)(k / 256 * 144);
    return Desc{make_rsrc(w + (int64_t)n0 * rb, (uint32_t)nv * rb), rb};
  }
  static __device__ __forceinline__ Raw load(const Desc& d, int r, int s, int q, bool live) {
    const uint32_t ro = (uint32_t)r * d.row_bytes;
    const uint32_t so = live ? (uint32_t)(s >> 2) * 144u : kPfDead;
    Raw raw;
    raw.hdr = ld128s(d.r, ro, so);
    raw.qs = ld128s(d.r, ro + 16u * (uint32_t)(q & 1), so + 16u + 32u * (uint32_t)(s & 3));
    return raw;
  }
  // weight = d * scale * q - dmin * min, rounded once from the exact value to
  // fp16: a nibble masked in place is the fp16 subnormal q * 2^-24 (low
  // nibble) or q * 2^-20 (high nibble), exact, and one mixed-precision fma
  // (v_fma_mix) multiplies it by the fp32 d * scale * 2^24 (or 2^20), adds
  // -dmin * min and rounds once to fp16.
  static __device__ __forceinline__ void make(const Raw& raw, int s, int q, unsigned (&out)[8]) {
    const int c = s & 3;
    const unsigned h = (unsigned)q >> 1;
    // 6-bit scale and min of group 2c + h (same packing as the GEMV kernels)
    const bool hi = c >= 2;
    const unsigned sh = 16u * (unsigned)(c & 1) + 8u * h;
    const unsigned ma = hi ? 0x0Fu : 0x3Fu;
    const unsigned sa = hi ? raw.hdr.w : raw.hdr.y, mb = hi ? raw.hdr.w : raw.hdr.z;
    const unsigned sg = ((sa >> sh) & ma) | (hi ? (((raw.hdr.y >> (sh + 6)) & 3u) << 4) : 0u);
    const unsigned mg = ((mb >> (sh + (hi ? 4u : 0u))) & ma) | (hi ? (((raw.hdr.z >> (sh + 6)) & 3u) << 4) : 0u);
    // d * scale (exact in fp32: 11 x 6 significant bits) times 2^24 / 2^20
    const float ds = f16lo(raw.hdr.x) * (float)sg * (h ? 1048576.f : 16777216.f);
    const float ndm = -(f16hi(raw.hdr.x) * (float)mg);
    const unsigned mask = h ? 0x00F000F0u : 0x000F000Fu;
    const unsigned qw[4] = {raw.qs.x, raw.qs.y, raw.qs.z, raw.qs.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned a = qw[i] & mask;         // elements 4i, 4i + 2 of the 16
      const unsigned b = (qw[i] >> 8) & mask;  // elements 4i + 1, 4i + 3
      out[2 * i] = mix_pair(a, b, ds, ndm, Int<0>{});
      out[2 * i + 1] = mix_pair(a, b, ds, ndm, Int<1>{});
    }
  }
};

// NVFP4 (Mojo module "fp4_gemv"): step s, quarter q = weights [64 s + 16 q,
// +16) of a row, one 16-weight block: 8 nibble bytes and its scale byte.
// Every e2m1 * |scale| is exact in fp32 and in bf16, so the bf16 weights are
// exact and the MFMA runs on bf16 (the activations' type).
struct Nvfp4Prefill {
  using T = __bf16;
  static constexpr bool kBf16 = true;
  static constexpr int kKMultiple = 64;
  static constexpr int kLoads = 2;
  struct Desc {
    __amdgpu_buffer_rsrc_t nib, sc;  // the tile's nibble rows, its scale rows
    uint32_t nib_row, sc_row;
  };
  struct Raw {
    u32x2 q;
    unsigned char sc;
  };
  static __device__ __forceinline__ Desc desc(const uint8_t* w, int n, int k, int n0, int nv) {
    const uint32_t nr = (uint32_t)(k / 2), sr = (uint32_t)(k / 16);
    return Desc{make_rsrc(w + (int64_t)n0 * nr, (uint32_t)nv * nr),
                make_rsrc(w + (int64_t)n * nr + (int64_t)n0 * sr, (uint32_t)nv * sr), nr, sr};
  }
  static __device__ __forceinline__ Raw load(const Desc& d, int r, int s, int q, bool live) {
    Raw raw;
    raw.q = ld64s(d.nib, (uint32_t)r * d.nib_row + 8u * (uint32_t)q, live ? 32u * (uint32_t)s : kPfDead);
    raw.sc = ld8s(d.sc, (uint32_t)r * d.sc_row + (uint32_t)q, live ? 4u * (uint32_t)s : kPfDead);
    return raw;
  }
  static __device__ __forceinline__ void make(const Raw& raw, int, int, unsigned (&out)[8]) {
    const float sc = __builtin_fabsf(__builtin_amdgcn_cvt_f32_fp8((int)raw.sc, 0));
    const unsigned q[2] = {raw.q.x, raw.q.y};
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // byte i: weights 2i, 2i + 1
      const f32x2 e = fp4x2_f32(q[i >> 2], i);
      out[i] = pf_pack2<T>(e.x * sc, e.y * sc);
    }
  }
};

// TQ1_0 ("metal: TQ1_0 kernel performance", sections 1, 2 and "Not
// applicable"): step s covers elements [64 c, 64 c + 64) of block b = s / 4
// (c = s % 4); quarter q the 16 starting at e0 = 64 c + 16 q, which are one
// digit of 16 bytes of qs[0..31] (e0 < 160: digit e0 / 32 of bytes e0 % 32
// ..), one digit of qs[32..47] (e0 = 160 .. 224: digit (e0 - 160) / 16) or
// the four digits of qh[0..3] (e0 = 240).  The block is only 2-byte aligned,
// so the bytes are read as five aligned dwords (single-dword loads: one past
// the range reads zero and is never needed) and realigned with alignbyte; d
// is a 16-bit load.  Each weight is one of d * -1, d * 0, d * 1, exact in
// fp16: two weights' digits come from one packed 16-bit multiply and one
// byte permute picks their fp16 codes (as in the row materialisation).
struct Tq1Prefill {
  using T = _Float16;
  static constexpr bool kBf16 = false;
  static constexpr int kKMultiple = 256;
  static constexpr int kLoads = 3;
  struct Desc {
    __amdgpu_buffer_rsrc_t r;  // the tile's rows
    uint32_t row_bytes;
  };
  struct Raw {
    unsigned wd[5];
    unsigned short d;
    unsigned char sh;  // bytes to drop at the front of the window
  };
  static __device__ __forceinline__ Desc desc(const uint8_t* w, int, int k, int n0, int nv) {
    const uint32_t rb = (uint32_t)(k / 256 * 54);
    return Desc{make_rsrc(w + (int64_t)n0 * rb, (uint32_t)nv * rb), rb};
  }
  // first byte of quarter q's window within the block
  static __device__ __forceinline__ uint32_t window(int e0) {
    return e0 < 160 ? 16u * (uint32_t)((e0 >> 4) & 1) : e0 < 240 ? 32u : 48u;
  }
  static __device__ __forceinline__ Raw load(const Desc& d, int r, int s, int q, bool live) {
    const uint32_t blk = (uint32_t)r * d.row_bytes + (uint32_t)(s >> 2) * 54u;
    const uint32_t a = blk + window(64 * (s & 3) + 16 * q);
    const uint32_t al = a & ~3u;
    const uint32_t dead = live ? 0u : kPfDead;  // uniform
    Raw raw;
    // the 20 bytes from the dword below the window: one dwordx4 and one
    // dword load (dword-aligned, as multi-dword buffer loads require; the
    // range check is per dword, so the dwords of a qh window that lie past
    // the tile's last row read as zero, and only its first two are used)
    const u32x4 lo = ld128s(d.r, al, dead);
    raw.wd[0] = lo.x;
    raw.wd[1] = lo.y;
    raw.wd[2] = lo.z;
    raw.wd[3] = lo.w;
    raw.wd[4] = ld32s(d.r, al, dead + 16u);
    raw.d = ld16s(d.r, blk + 52u, dead);
    raw.sh = (unsigned char)(a & 3u);
    return raw;
  }
  // weights (2 pr, 2 pr + 1) from bytes bi, bi + 1 of the window, digit k
  static __device__ __forceinline__ unsigned pair(const unsigned (&q)[4], int bi, int k, unsigned vm, unsigned vp) {
    const unsigned word = q[bi >> 2];
    const unsigned b = (unsigned)(bi & 3);
    const unsigned pr = __builtin_amdgcn_perm(0u, word, 0x0C000C00u | b | ((b + 1u) << 16));
    const u16x2 dg = tq1_digits2(__builtin_bit_cast(u16x2, pr), pow3_u16(k));
    const u16x2 sel = dg * u16x2{0x0202, 0x0202} + u16x2{0x0100, 0x0100};
    return __builtin_amdgcn_perm(vp, vm, __builtin_bit_cast(unsigned, sel));
  }
  static __device__ __forceinline__ void make(const Raw& raw, int s, int qt, unsigned (&out)[8]) {
    unsigned q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = __builtin_amdgcn_alignbyte(raw.wd[j + 1], raw.wd[j], raw.sh);
    const float d = (float)__builtin_bit_cast(_Float16, raw.d);
    const unsigned vm = pf_pack2<T>(d * -1.f, d * 0.f);  // codes of d*(t-1), t = 0, 1
    const unsigned vp = pf_pack2<T>(d * 1.f, 0.f);        // and t = 2
    const int e0 = 64 * (s & 3) + 16 * qt;
    if (e0 < 240) {  // one digit of 16 consecutive bytes (lanes differ only in steps with c = 3)
      const int k = e0 < 160 ? e0 >> 5 : (e0 - 160) >> 4;
#pragma unroll
      for (int p = 0; p < 8; ++p) out[p] = pair(q, 2 * p, k, vm, vp);
    } else {  // element 240 + 4 k + m is digit k of qh[m]
#pragma unroll
      for (int p = 0; p < 8; ++p) out[p] = pair(q, (2 * p) & 3, p >> 1, vm, vp);
    }
  }
};

// ---- the kernel ---------------------------------------------------------------

constexpr int kPfWQ = 3;      // packed-weight register slots: loads run kPfWQ - 1 steps ahead of the decode
static_assert(kPfUnroll % kPfWQ == 0, "steps per loop iteration: a multiple of the weight register slots");

// Step s, with XS activation stages: the activations of step s + XS - 1 are
// copied into activation stage (s + XS - 1) % XS and the packed weights of
// step s + 3 are loaded into registers; the weights of step s + 1 (loaded
// during step s - 2) are decoded, the MFMAs consume activation stage s % XS
// and weight stage s % 2, and the decoded weights go to weight stage
// (s + 1) % 2.
// Before the step's barrier each wave waits for its own copy of step s + 1's
// activations (an LDS copy by one wave is read by all), so every copy has
// XS - 1 steps to land.  The stages are separate LDS arrays indexed at
// compile time (the loop runs kPfUnroll steps per iteration): the compiler
// then knows that the copies in flight into one stage never alias the
// fragment reads of another, and does not wait for them there.
// Where the partial sums of a tile split over K go.  With part == nullptr
// they are added into y with fp32 atomics (y cleared first).  Otherwise split
// z of tile `tile` stores its whole BT x 128 partial tile at part + (tile *
// nsplit + z) * BT * 128 (row-major, tile-local rows and columns), and
// prefill_reduce_kernel, launched after it on the same stream, adds the
// nsplit partials of every output in split order: the result does not vary
// from run to run, and no workgroup waits for another.
struct PfSplit {
  float* part;
  int tile;
  int nsplit;
};

// One workgroup's tile: tokens t0 .. t0 + BT - 1, weight rows n0 .. n0 + 127,
// K split z (steps [z * split_steps, ...)), with XS activation stages in the
// LDS arrays xs0..xs2 (at least BT * 128 bytes each, xs2 used when XS = 3)
// and the weight stages ws0, ws1; the partial sums go where `sp` says when
// `split` (a K split), they are stored otherwise.
template <typename F, int BT, int XS>
__device__ __forceinline__ void prefill_tile(const uint8_t* __restrict__ w, const uint16_t* __restrict__ x,
                                             float* __restrict__ y, int t_count, int n, int k, int split_steps,
                                             int t0, int n0, int z, bool split, PfSplit sp, unsigned char* xs0,
                                             unsigned char* xs1, unsigned char* xs2, unsigned char* ws0,
                                             unsigned char* ws1) {
  static_assert(BT == 256 || BT == 512, "256 or 512 tokens per tile");
  constexpr int kPfBT = BT;                       // tokens per workgroup tile
  constexpr int kPfXTile = BT * kPfRowB;          // 32 or 64 KiB of activations per stage
  constexpr int kPfXS = XS;                       // activation stages
  constexpr int kPfMI = BT / 128;                 // 32-token MFMA tiles per wave (waves are 4 x 2)
  constexpr int kPfCopies = BT / 64;              // 1 KiB activation copies per wave per step
  static_assert(XS == 2 || XS == 3, "two or three activation stages");
  static_assert(kPfXS * kPfXTile + 2 * kPfWTile <= 160 * 1024, "activation and weight stages fit the LDS");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // K split z: steps [z * split_steps, ...) of the K / 64 steps
  const int s_begin = z * split_steps;
  const int steps = min(split_steps, k / kPfKS - s_begin);
  const uint32_t xrow = (uint32_t)k * 2u;  // bytes per activation row

  // activations of the tile: rows t0.. (zero past T); weights: rows n0.. (zero past n)
  const int tv = min(kPfBT, t_count - t0), nv = min(kPfBN, n - n0);
  const auto xr = make_rsrc(x + (int64_t)t0 * k, (uint32_t)tv * xrow);
  const typename F::Desc wd = F::desc(w, n, k, n0, nv);

  // Activation copy: wave v copies tile rows 8C v .. 8C v + 8C - 1 of a step
  // in C = kPfCopies wave-wide loads of 8 rows; lane i of load j lands at LDS
  // row t = 8C v + 8 j + i / 8, position i % 8, which holds granule (i % 8) ^
  // ((t / 2) % 8) = (i % 8) ^ (i / 16) ^ (4 if j is odd) of the row.
  const uint32_t xrow_l = (uint32_t)(8 * kPfCopies * wave + (lane >> 3)) * xrow;
  const uint32_t xlane0 = xrow_l + 16u * (uint32_t)((lane & 7) ^ (lane >> 4));
  const uint32_t xlane1 = xrow_l + 16u * (uint32_t)((lane & 7) ^ (lane >> 4) ^ 4);
  auto copy_x = [&](unsigned char* stage, int s) {
    const uint32_t so = s < steps ? (uint32_t)(s_begin + s) * 128u : kPfDead;  // uniform
#pragma unroll
    for (int j = 0; j < kPfCopies; ++j)
      ld128_lds_s(xr, stage + (8 * kPfCopies * wave + 8 * j) * kPfRowB, j & 1 ? xlane1 : xlane0,
                  so + (uint32_t)j * 8u * xrow);
  };

  // Weight decode: thread i takes weights [16 dq, 16 dq + 16) of weight row
  // dr of each step.
  const int dr = tid >> 2, dq = tid & 3;
  auto store_w = [&](unsigned char* stage, const unsigned (&v)[8]) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
      *reinterpret_cast<u32x4*>(stage + pf_off(dr, 2 * dq + g)) = u32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
  };

  f32x16 acc[kPfMI][2];
#pragma unroll
  for (int i = 0; i < kPfMI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // wave sub-tile: tokens 32 MI (wave & 3) .., rows 64 (wave >> 2) ..
  const int wt = 32 * kPfMI * (wave & 3), wn = 64 * (wave >> 2);
  const int fl = lane & 31, fq = lane >> 5;  // fragment row / column and k-granule
  auto xstage = [&](int m) { return m % kPfXS == 0 ? xs0 : m % kPfXS == 1 ? xs1 : xs2; };

  // Loads return in issue order, and the wait counts below count the loads
  // issued after the one waited for: per step the activation copy (4), then
  // the weights (kLoads).
  constexpr int kStepLoads = kPfCopies + F::kLoads;
  // prologue: activations of steps 0 .. XS - 2, weights of steps 0 .. 2; step 0 decoded
  // Each group is fenced: the compiler may otherwise interleave independent
  // loads, and a weight load issued after a copy would let part of the copy
  // still be in flight when the count is reached.
  typename F::Raw wq[kPfWQ];
  copy_x(xs0, 0);
  compiler_fence();
  wq[0] = F::load(wd, dr, s_begin, dq, 0 < steps);
  compiler_fence();
  if constexpr (kPfXS == 3) {
    copy_x(xs1, 1);
    compiler_fence();
  }
  wq[1] = F::load(wd, dr, s_begin + 1, dq, 1 < steps);
  compiler_fence();
  wq[2] = F::load(wd, dr, s_begin + 2, dq, 2 < steps);
  compiler_fence();
  {
    unsigned v[8];
    F::make(wq[0], s_begin, dq, v);
    store_w(ws0, v);
  }
  // this wave's copy of step 0's activations (what may still be in flight:
  // the copy of step 1 and the weights of steps 1 and 2)
  wait_vm<(kPfXS == 3 ? kPfCopies : 0) + 2 * F::kLoads>();
  lds_barrier();

  // Every iteration runs kPfUnroll steps with no branch around their loads
  // (a branch around a step's loads makes the compiler's load-wait
  // bookkeeping merge paths and wait for every load in flight).  Steps past
  // `steps` load nothing and skip their arithmetic.
  for (int s0 = 0; s0 < steps; s0 += kPfUnroll) {
    static_for<0, kPfUnroll>([&](auto ic) {
      constexpr int I = decltype(ic)::value;  // = s % kPfUnroll
      const int s = s0 + I;
      unsigned char* const xa = xstage(I);              // consumed this step
      unsigned char* const xc = xstage(I + kPfXS - 1);  // filled for step s + XS - 1
      unsigned char* const wa = I % 2 ? ws1 : ws0;
      unsigned char* const wb = I % 2 ? ws0 : ws1;  // filled for step s + 1
      copy_x(xc, s + kPfXS - 1);
      compiler_fence();
      wq[I % kPfWQ] = F::load(wd, dr, s_begin + s + kPfWQ, dq, s + kPfWQ < steps);
      compiler_fence();
      // (no decode arithmetic above the loads: it would wait for step s + 1's
      // weights before this step's loads are even issued)
      __builtin_amdgcn_sched_barrier(0);
      // A step past the end (the last iteration's) skips its decode, MFMAs
      // and weight store; the branch holds no global load, so the load waits
      // stay exact.
      if (s < steps) {
      unsigned v[8];
      F::make(wq[(I + 1) % kPfWQ], s_begin + s + 1, dq, v);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {  // 16 weights of K per MFMA
        const int g = 2 * kc + fq;
        u32x4 af[kPfMI], bf[2];
#pragma unroll
        for (int i = 0; i < kPfMI; ++i) af[i] = *reinterpret_cast<const u32x4*>(xa + pf_off(wt + 32 * i + fl, g));
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = *reinterpret_cast<const u32x4*>(wa + pf_off(wn + 32 * j + fl, g));
#pragma unroll
        for (int i = 0; i < kPfMI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if constexpr (F::kBf16)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                                   __builtin_bit_cast(bf16x8, bf[j]), acc[i][j],
                                                                   0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, af[i]),
                                                                  __builtin_bit_cast(half8, bf[j]), acc[i][j], 0,
                                                                  0, 0);
          }
      }
      store_w(wb, v);
      }
      wait_vm<(kPfXS - 2) * kStepLoads + F::kLoads>();  // this wave's copy of step s + 1's activations
      lds_barrier();  // all reads of this step's stages and all writes of the next are done
    });
  }

  // D[m][n] of tile (i, j) sits at lane n + 32 ((m / 4) % 2), register
  // 4 (m / 8) + m % 4: register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4
  if (split && sp.part) {
    float* const mine = sp.part + ((int64_t)sp.tile * sp.nsplit + z) * ((int64_t)BT * kPfBN);
#pragma unroll
    for (int i = 0; i < kPfMI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          mine[(wt + 32 * i + 8 * (r >> 2) + 4 * fq + (r & 3)) * kPfBN + wn + 32 * j + fl] = acc[i][j][r];
    return;
  }
#pragma unroll
  for (int i = 0; i < kPfMI; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + wt + 32 * i + 8 * (r >> 2) + 4 * fq + (r & 3);
      if (t < t_count) {
        float* const yr = y + (int64_t)t * n;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn + 32 * j + fl;
          if (col < n) {
            if (!split)
              yr[col] = acc[i][j][r];
            else
              atomicAdd(yr + col, acc[i][j][r]);  // partial sum of one K split (y zeroed first)
          }
        }
      }
    }
}

template <typename F, int BT>
__global__ __launch_bounds__(64 * kPfWaves, 1) void prefill_kernel(const uint8_t* __restrict__ w,
                                                                  const uint16_t* __restrict__ x,
                                                                  float* __restrict__ y, int t_count, int n,
                                                                  int k, int split_steps, float* part) {
  constexpr int XS = BT == 512 ? 2 : 3;  // as many activation stages as fit the LDS
  __shared__ __attribute__((aligned(1024))) unsigned char xs0[BT * kPfRowB];
  __shared__ __attribute__((aligned(1024))) unsigned char xs1[BT * kPfRowB];
  __shared__ __attribute__((aligned(1024))) unsigned char xs2[XS == 3 ? BT * kPfRowB : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char ws0[kPfWTile];
  __shared__ __attribute__((aligned(1024))) unsigned char ws1[kPfWTile];
  const PfSplit sp{part, (int)(blockIdx.y * gridDim.x + blockIdx.x), (int)gridDim.z};
  prefill_tile<F, BT, XS>(w, x, y, t_count, n, k, split_steps, blockIdx.y * BT, blockIdx.x * kPfBN, blockIdx.z,
                          gridDim.z > 1, sp, xs0, xs1, xs2, ws0, ws1);
}

// 512-token tiles whose count leaves a last round at most a quarter full: the
// first n_full tiles (whole rounds of workgroups, in index order) run over
// all of K and store their sums; each remaining tile is split over K into
// tail_split parts of split_steps steps whose workgroups fill the last round
// together and add their partial sums into y with atomics (the rows of those
// tiles are zeroed first).
template <typename F>
__global__ __launch_bounds__(64 * kPfWaves, 1) void prefill_tail_kernel(const uint8_t* __restrict__ w,
                                                                       const uint16_t* __restrict__ x,
                                                                       float* __restrict__ y, int t_count, int n,
                                                                       int k, int row_tiles, int n_full,
                                                                       int tail_split, int split_steps,
                                                                       float* part) {
  __shared__ __attribute__((aligned(1024))) unsigned char xs0[512 * kPfRowB];
  __shared__ __attribute__((aligned(1024))) unsigned char xs1[512 * kPfRowB];
  __shared__ __attribute__((aligned(1024))) unsigned char xs2[16];
  __shared__ __attribute__((aligned(1024))) unsigned char ws0[kPfWTile];
  __shared__ __attribute__((aligned(1024))) unsigned char ws1[kPfWTile];
  const int b = blockIdx.x;
  int tile = b, z = 0, ss = k / kPfKS;
  if (b >= n_full) {
    tile = n_full + (b - n_full) / tail_split;
    z = (b - n_full) % tail_split;
    ss = split_steps;
  }
  const PfSplit sp{part, tile - n_full, tail_split};
  prefill_tile<F, 512, 2>(w, x, y, t_count, n, k, ss, (tile / row_tiles) * 512, (tile % row_tiles) * kPfBN, z,
                          b >= n_full, sp, xs0, xs1, xs2, ws0, ws1);
}

// Clears y[0 .. count): 16-byte stores from the first 16-byte boundary on,
// 1024 of them per workgroup (thread i stores the i-th of every 256, so each
// wave-wide store is contiguous), and the at most 3 + 3 loose floats before
// and after them one by one in workgroup 0 (y is only 4-byte aligned).
// Launched with count / 4096 + 1 workgroups of 256 threads.
__global__ __launch_bounds__(256) void prefill_zero_kernel(float* __restrict__ y, int64_t count) {
  const int64_t head = min(count, (int64_t)((16 - (reinterpret_cast<uintptr_t>(y) & 15)) & 15) / 4);
  const int64_t quads = (count - head) / 4;
  const int64_t q0 = (int64_t)blockIdx.x * 1024 + threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (q0 + 256 * j < quads) reinterpret_cast<u32x4*>(y + head)[q0 + 256 * j] = u32x4{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0) {
    const int64_t tail = head + 4 * quads;
    if (threadIdx.x < head) y[threadIdx.x] = 0.f;
    if (threadIdx.x < count - tail) y[tail + threadIdx.x] = 0.f;
  }
}

// Sums the nsplit partial tiles of the split tiles into y, in split order:
// partial tile p (p = 0 .. tiles - 1, bt x 128 outputs each) is output tile
// first + p of the launch, whose token rows start at ((first + p) /
// row_tiles) * bt and weight rows at ((first + p) % row_tiles) * 128.  A
// workgroup of 256 threads takes 8 rows x 128 columns of one tile (thread i:
// column i % 128, rows i / 128, + 2, + 4, + 6), so its loads and stores are
// contiguous across the wave.  Launched with tiles * bt / 8 workgroups.
__global__ __launch_bounds__(256) void prefill_reduce_kernel(const float* __restrict__ part, float* __restrict__ y,
                                                             int t_count, int n, int bt, int row_tiles, int first,
                                                             int nsplit) {
  const int per_tile = bt / 8;
  const int p = blockIdx.x / per_tile, r8 = (blockIdx.x % per_tile) * 8;
  const int tile = first + p;
  const int t0 = (tile / row_tiles) * bt, n0 = (tile % row_tiles) * kPfBN;
  const int c = threadIdx.x & 127;
  const int64_t tile_f = (int64_t)bt * kPfBN;
  const float* const src = part + (int64_t)p * nsplit * tile_f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = r8 + (threadIdx.x >> 7) + 2 * j;
    float v = 0.f;
    for (int z = 0; z < nsplit; ++z) v += src[z * tile_f + (int64_t)r * kPfBN + c];
    const int t = t0 + r, col = n0 + c;
    if (t < t_count && col < n) y[(int64_t)t * n + col] = v;
  }
}

// Tiles of 256 or 512 tokens x 128 rows, one workgroup per CU.  When there are
// fewer tiles than CUs, K is split as well (one round of workgroups, at
// least 8 steps per split); when 512-token tiles leave a last round at most a
// quarter full, only the tiles of that round are split (prefill_tail_kernel).
// The splits' partial sums either go to a workspace and a second kernel adds
// them in a fixed order (PfSplit), or, with no workspace, are added into y
// with fp32 atomics after a fill kernel clears y (a kernel, so that the
// sequence can be captured in a graph; the order of those few additions
// varies from run to run).
template <typename F>
static hipError_t launch_prefill(const void* w, const void* x, float* y, int64_t t, int64_t n, int64_t k,
                                 void* ws, hipStream_t s) {
  const PfPlan p = prefill_plan(t, n, k);
  float* const part = static_cast<float*>(ws);
  if (p.split > 1 && !part) {
    const int64_t count = t * n;
    hipLaunchKernelGGL(prefill_zero_kernel, dim3((unsigned)(count / 4096 + 1)), dim3(256), 0, s, y, count);
  }
  if (p.split == 1 && p.tail_split > 1) {
    if (!part) {
      const int64_t t_zero = p.n_full / p.row_tiles * 512;  // first token row of a split tile
      const int64_t count = (t - t_zero) * n;
      hipLaunchKernelGGL(prefill_zero_kernel, dim3((unsigned)(count / 4096 + 1)), dim3(256), 0, s, y + t_zero * n,
                         count);
    }
    hipLaunchKernelGGL((prefill_tail_kernel<F>), dim3((unsigned)(p.n_full + p.tail * p.tail_split)),
                       dim3(64 * kPfWaves), 0, s, (const uint8_t*)w, (const uint16_t*)x, y, (int)t, (int)n, (int)k,
                       (int)p.row_tiles, (int)p.n_full, (int)p.tail_split, (int)p.tail_steps, part);
    if (part)
      hipLaunchKernelGGL(prefill_reduce_kernel, dim3((unsigned)(p.tail * 512 / 8)), dim3(256), 0, s, part, y, (int)t,
                         (int)n, 512, (int)p.row_tiles, (int)p.n_full, (int)p.tail_split);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)p.row_tiles, (unsigned)((t + p.bt - 1) / p.bt), (unsigned)p.split);
  if (p.bt == 512)
    hipLaunchKernelGGL((prefill_kernel<F, 512>), grid, dim3(64 * kPfWaves), 0, s, (const uint8_t*)w,
                       (const uint16_t*)x, y, (int)t, (int)n, (int)k, (int)p.split_steps, part);
  else
    hipLaunchKernelGGL((prefill_kernel<F, 256>), grid, dim3(64 * kPfWaves), 0, s, (const uint8_t*)w,
                       (const uint16_t*)x, y, (int)t, (int)n, (int)k, (int)p.split_steps, part);
  if (p.split > 1 && part)
    hipLaunchKernelGGL(prefill_reduce_kernel, dim3((unsigned)(p.tiles * p.bt / 8)), dim3(256), 0, s, part, y, (int)t,
                       (int)n, p.bt, (int)p.row_tiles, 0, (int)p.split);
  return hipGetLastError();
}

hipError_t launch_q4k_prefill(const void* w, const void* x, float* y, int64_t t, int64_t n, int64_t k, void* ws,
                              hipStream_t s) {
  return launch_prefill<Q4kPrefill>(w, x, y, t, n, k, ws, s);
}
hipError_t launch_nvfp4_prefill(const void* w, const void* x, float* y, int64_t t, int64_t n, int64_t k, void* ws,
                                hipStream_t s) {
  return launch_prefill<Nvfp4Prefill>(w, x, y, t, n, k, ws, s);
}
hipError_t launch_tq1_prefill(const void* w, const void* x, float* y, int64_t t, int64_t n, int64_t k, void* ws,
                              hipStream_t s) {
  return launch_prefill<Tq1Prefill>(w, x, y, t, n, k, ws, s);
}

}  // namespace qgemv
