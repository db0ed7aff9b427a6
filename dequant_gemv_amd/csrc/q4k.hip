// Q4_K fused dequantise + GEMV and row materialisation for gfx950.
//
// Block format ("Writing a high performant GEMV + dequant for Metal", sections
// "What is a weight block?" and "Kernel code"): 144 bytes per 256 weights,
// fp16 d @0, fp16 dmin @2, 12 bytes of 6-bit scales/mins @4, 128 nibble bytes
// @16.  Weight i = d*s_g*q_i - dmin*m_g, g = i/32 (section "Compute").
//
// GEMV work split.  A wave owns one K-chunk of 8 blocks (2048 weights) for R
// consecutive rows.  Lane l takes block l/8 of the chunk and the 16-byte slice
// p = l%8 of its nibbles, so one dwordx4 per lane reads the 128 contiguous
// nibble bytes of 8 blocks: every load instruction is one contiguous 1 KiB run
// with 16-byte gaps, i.e. coalesced.  Nibble byte 16p+j sits at element
// 64c+16h+j (low nibble, group 2c) and 64c+32+16h+j (high nibble, group 2c+1)
// with c = p/2, h = p%2, so a lane touches exactly two groups per block.
//
// The dot product uses the page's factoring (section "Compute"): per group
// d*s_g*Q_g - dmin*m_g*X_g with Q_g = sum x_i q_i and X_g = sum x_i.  X_g over
// the lane's 16 elements is computed once per chunk and reused by all R rows,
// as are the lane's 32 activations, held in registers as fp16 pairs.  Q_g is
// built with v_dot2_f32_f16 straight on masked nibbles: a nibble masked in
// place is an fp16 subnormal q*2^-24 (low nibble) or 16q*2^-24 (high nibble),
// so no shift or integer->float conversion is spent per weight; the power of
// two is removed once per row (the shift-deferral of the page's Figures 7-8
// carried to the fp16 bit level).  Products are exact in fp32.
//
// Per row the lane's partial is reduced across the wave (R rows at once, see
// wave_reduce_rows) and across the K-chunk waves through LDS.
#include "device.hpp"
#include "launch.hpp"
#include "rows.hpp"
#include "stream.hpp"

namespace qgemv {

// Waves per workgroup of the K-split kernel (tuning).
#ifndef QGEMV_WG_WAVES
#define QGEMV_WG_WAVES 8
#endif

constexpr int kQ4kBytes = 144;

// 6-bit scale and min of the two consecutive groups (2c, 2c+1) a lane owns,
// packed as bytes 0 and 1.  h1, h2, h3 are scale bytes 0-3, 4-7, 8-11.  Groups
// 0-3 keep their 6 bits in the low bits of bytes 0-7; groups 4-7 take the low
// (scale) or high (min) nibble of bytes 8-11 and the top two bits of bytes
// 0-3 (scale) or 4-7 (min).
struct Q4kScaleSel {
  unsigned sh, shm, ma, mb;
  bool hi;
  __device__ __forceinline__ explicit Q4kScaleSel(int c) {
    hi = c >= 2;
    sh = 16u * (unsigned)(c & 1);
    shm = sh + (hi ? 4u : 0u);
    ma = hi ? 0x0F0Fu : 0x3F3Fu;
    mb = hi ? 0x3030u : 0u;
  }
  __device__ __forceinline__ unsigned scales(unsigned h1, unsigned h3) const {
    unsigned a = hi ? h3 : h1;
    return ((a >> sh) & ma) | ((h1 >> (sh + 2)) & mb);
  }
  __device__ __forceinline__ unsigned mins(unsigned h2, unsigned h3) const {
    unsigned a = hi ? h3 : h2;
    return ((a >> shm) & ma) | ((h2 >> (sh + 2)) & mb);
  }
};

// K-split GEMV (any K).  A wave owns one K-chunk of 8
// blocks for a batch of 8 rows: 8 x 1152 contiguous-per-row bytes = 9 KiB,
// read with nine dwordx4 loads of one 16-byte piece per lane.  Every load is
// one 1 KiB run starting on a 128-byte line (1152 = 9*128 and a row of a
// multiple of 8 blocks is a multiple of 1152 bytes).  Each piece is written to
// the wave's slice of LDS as it arrives and lanes read their 16-byte nibble
// slice and the block header back with ds_read_b128 (the header read is a
// broadcast among 8 lanes), a row at a time as soon as its pieces are in.
// Chunks beyond the wave's first are processed in turn through the same LDS.
constexpr int kQ4kBatchRows = 8;
constexpr int kQ4kStage = kQ4kBatchRows * 8 * kQ4kBytes;  // 9216 bytes per wave

template <typename Out>
__global__ __launch_bounds__(64 * QGEMV_WG_WAVES) void q4k_gemv_lds_kernel(const uint8_t* __restrict__ w,
                                                                          const uint16_t* __restrict__ x,
                                                                          Out out, int n, int nb,
                                                                          int kc, int kw, int rg) {
  __shared__ __attribute__((aligned(16))) unsigned char stage_all[QGEMV_WG_WAVES * kQ4kStage];
  __shared__ float red[QGEMV_WG_WAVES * kQ4kBatchRows];
  constexpr int R = kQ4kBatchRows;
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kwi = wave % kw;
  const int rgi = wave / kw;
  const int64_t row_bytes = (int64_t)nb * kQ4kBytes;
  const int row0 = blockIdx.x * rg * R + rgi * R;
  const int nrows = max(0, min(R, n - row0));
  const uint32_t range = (uint32_t)(nrows * row_bytes);
  const auto wr = make_rsrc(w + (int64_t)row0 * row_bytes, range);
  const auto xr = make_rsrc(x, (uint32_t)nb * 512u);
  unsigned char* stage = stage_all + wave * kQ4kStage;

  const int bl = lane >> 3, p = lane & 7, c = p >> 1, h = p & 1;
  const Q4kScaleSel sel(c);
  const unsigned kOnes = 0x3C003C00u;

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;

  for (int ch = kwi; ch < kc; ch += kw) {
    const int b = ch * 8 + bl;
    const int nbc = min(8, nb - ch * 8);  // blocks of this chunk inside the row
    // activations first: loads complete in issue order
    const uint32_t xo = (uint32_t)(b * 256 + 64 * c + 16 * h) * 2u;
    const u32x4 xa0 = ld128(xr, xo), xa1 = ld128(xr, xo + 16);
    const u32x4 xb0 = ld128(xr, xo + 64), xb1 = ld128(xr, xo + 80);
    // The batch: nine coalesced 1 KiB loads (one 16-byte piece per lane),
    // all in flight at once.
    u32x4 pc[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int piece = 64 * i + lane;         // 16-byte piece of the 8 x 1152-byte batch
      const int rr = piece / 72, within = piece % 72;
      const bool inside = within < nbc * 9;    // past the row's last block: read zeros
      const uint32_t off = inside ? (uint32_t)(rr * row_bytes + ch * 8 * kQ4kBytes + within * 16) : range;
      pc[i] = ld128w(wr, off);
    }
    const unsigned XA[8] = {xa0.x, xa0.y, xa0.z, xa0.w, xa1.x, xa1.y, xa1.z, xa1.w};
    const unsigned XB[8] = {xb0.x, xb0.y, xb0.z, xb0.w, xb1.x, xb1.y, xb1.z, xb1.w};
    unsigned pa02[4], pa13[4], pb02[4], pb13[4];
    float sxa = 0.f, sxb = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      pa02[t] = __builtin_amdgcn_perm(XA[2 * t + 1], XA[2 * t], 0x05040100u);
      pa13[t] = __builtin_amdgcn_perm(XA[2 * t + 1], XA[2 * t], 0x07060302u);
      pb02[t] = __builtin_amdgcn_perm(XB[2 * t + 1], XB[2 * t], 0x05040100u);
      pb13[t] = __builtin_amdgcn_perm(XB[2 * t + 1], XB[2 * t], 0x07060302u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sxa = dot2h(XA[i], kOnes, sxa);
      sxb = dot2h(XB[i], kOnes, sxb);
    }
    sxa *= 0x1p-24f;
    sxb *= 0x1p-24f;
    // the previous chunk's LDS reads are done before its slice is rewritten
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    int written = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // Row r lies in pieces 72r .. 72r+71, i.e. in loads 0 .. (72r+71)/64.
      // Each load is written to LDS right after it lands (loads complete in
      // issue order), so row r is consumed as soon as its two loads are in.
      const int need = (72 * r + 71) / 64;
#pragma unroll
      for (int i = 0; i < 9; ++i)
        if (i >= written && i <= need) *reinterpret_cast<u32x4*>(stage + 1024 * i + 16 * lane) = pc[i];
      written = need + 1;
      const unsigned char* blk = stage + r * 8 * kQ4kBytes + bl * kQ4kBytes;
      const u32x4 hdr = *reinterpret_cast<const u32x4*>(blk);
      const u32x4 qv = *reinterpret_cast<const u32x4*>(blk + 16 + 16 * p);
      const unsigned q[4] = {qv.x, qv.y, qv.z, qv.w};
      float qa = 0.f, qb = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const unsigned w0 = q[t], w8 = q[t] >> 8;
        qa = dot2h(w0 & 0x000F000Fu, pa02[t], qa);
        qa = dot2h(w8 & 0x000F000Fu, pa13[t], qa);
        qb = dot2h(w0 & 0x00F000F0u, pb02[t], qb);
        qb = dot2h(w8 & 0x00F000F0u, pb13[t], qb);
      }
      const unsigned sp = sel.scales(hdr.y, hdr.w);
      const unsigned mp = sel.mins(hdr.z, hdr.w);
      const float sa = (float)(sp & 0xFFu), sb = (float)((sp >> 8) & 0xFFu);
      const float ma = (float)(mp & 0xFFu), mb = (float)((mp >> 8) & 0xFFu);
      const float d = f16lo(hdr.x), dmin = f16hi(hdr.x);
      const float v = __builtin_fmaf(sb, qb * 0.0625f, sa * qa);
      const float mx = __builtin_fmaf(mb, sxb, ma * sxa);
      acc[r] = __builtin_fmaf(-dmin, mx, __builtin_fmaf(d, v, acc[r]));
    }
  }

  wave_reduce_rows<R>(acc);
  if ((lane & 7) == 0) red[(rgi * kw + kwi) * R + (lane >> 3)] = acc[0];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < rg * R) {
    const int g = t / R, r = t % R;
    float s = 0.f;
    for (int k = 0; k < kw; ++k) s += red[(g * kw + k) * R + r];
    const int row = blockIdx.x * rg * R + g * R + r;
    if (row < n) out.put(row, s * 0x1p24f);
  }
}


// Row-streaming variant: W waves per workgroup (one or two per SIMD), each
// wave owning R whole rows (all K) so no partial sum ever leaves the wave.
// Everything a wave reads is one contiguous run of R row records (at most
// 36 KiB), streamed with coalesced 1 KiB buffer loads that land straight in
// the wave's LDS stage (no VGPRs, no LDS writes).  A wave keeps only a few
// loads in flight ahead of the unit it is consuming and issues the next one
// as each unit is done: a CU's memory pipeline holds a bounded number of
// requests and a wave that tries to issue past that stalls at the load, so
// issuing everything up front would hold back the arithmetic (and the
// workgroup barrier below) until most of the data had already arrived.  The activations are
// read once per workgroup the same way into LDS, swizzled in 16-byte granules
// so that the per-lane reads below hit 8 distinct bank groups, and then held
// in registers for every K-chunk.
//
// Unit (r, ch) = the 8 blocks of chunk ch of row r (1152 bytes).  Lane l takes
// block l/8 and nibble slice l%8 of each unit exactly as the K-split kernel
// does, and consumes the unit as soon as the loads covering it are in (loads
// complete in issue order, so one vmcnt wait per unit).  The R row partials
// are summed across the wave with DPP (no LDS), and lanes 48..48+R-1 store
// one row each.
// Granule (16 bytes = 8 activations) swizzle of the activation copy in LDS.
// Granule g of a 512-byte block holds elements 8g..8g+7; a lane with chunk
// position c = (g >> 3) & 3 reads granules 8c + {0,1,4,5} + 2h, so XOR-ing bits
// 0 and 2 of g with c's two bits spreads the 8 lanes of a block over 8
// different 16-byte bank groups.  The map is its own inverse.
__device__ __forceinline__ constexpr int q4k_xswz(int g) {
  return g ^ (((g >> 3) & 1) | (((g >> 4) & 1) << 2));
}

#ifndef QGEMV_Q4K_AHEAD
#define QGEMV_Q4K_AHEAD 3  // weight loads in flight per wave beyond the unit being consumed
#endif
#ifndef QGEMV_Q4K_AHEAD0
#define QGEMV_Q4K_AHEAD0 QGEMV_Q4K_AHEAD  // weight loads issued before the activation barrier
#endif
#ifndef QGEMV_Q4K_FIRST
#define QGEMV_Q4K_FIRST QGEMV_Q4K_AHEAD0  // weight loads issued before the first unit
#endif

template <int KC, int R, int W>
struct Q4kRows {
  static constexpr int kUnitBytes = 8 * kQ4kBytes;  // 1152
  // Unit u = r*KC + ch; the schedule assumes the largest row record (8*KC
  // blocks), shorter records only end earlier.
  using S = StreamSchedule<kUnitBytes, R * KC, QGEMV_Q4K_AHEAD0, QGEMV_Q4K_AHEAD, QGEMV_Q4K_FIRST>;
  static constexpr int kXBytes = KC * 4096;  // activations in LDS
  static constexpr int kLds = W * S::kStage + kXBytes;
  static_assert(KC >= 1 && KC <= 8, "K-chunk count");
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};

template <int KC, int R, int W, typename Out>
__global__ __launch_bounds__(64 * W) void q4k_gemv_rows_kernel(const uint8_t* __restrict__ w,
                                                                      const uint16_t* __restrict__ x,
                                                                      Out out, int n, int nb) {
  using C = Q4kRows<KC, R, W>;
  using S = typename C::S;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::kLds];
  unsigned char* const xs = lds + W * S::kStage;
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned char* const stage = lds + wave * S::kStage;
  const int row_bytes = nb * kQ4kBytes;
  const int row0 = (blockIdx.x * W + wave) * R;
  const int nrows = max(0, min(R, n - row0));

  // Activations first (the workgroup's 4*KC one-KiB pieces, swizzled), then
  // the first weight loads of the wave's rows.
  load_shared_pieces<4 * KC, W>(make_rsrc(x, (uint32_t)nb * 512u), xs, wave, lane, [](int piece, int i) {
    return (uint32_t)(piece * 1024 + ((i & 32) + q4k_xswz(i & 31)) * 16);
  });
  const auto wr = make_rsrc(w + (int64_t)row0 * row_bytes, (uint32_t)(nrows * row_bytes));
  stream_loads<0, S::kUpFront, QGEMV_WLOAD_AUX>(wr, stage, lane);

  const int bl = lane >> 3, p = lane & 7, c = p >> 1, h = p & 1;
  const Q4kScaleSel sel(c);
  const unsigned kOnes = 0x3C003C00u;

  wait_vm<S::kUpFront>();  // this wave's activation pieces (issued before the weights) are in LDS
  __builtin_amdgcn_s_barrier();  // ... and every other wave's
  // the output stage's input for the wave's rows, after the barrier's wait
  // (the stream's later waits only get stricter by this one load)
  const auto pre = prefetch_rows(out, row0, nrows, lane);
  stream_loads<S::kUpFront, S::issued_before(0), QGEMV_WLOAD_AUX>(wr, stage, lane);

  // The lane's activations for every chunk, as fp16 pairs matching the masked
  // nibble layout, and their group sums (times 2^-24, see the K-split kernel).
  unsigned pa02[KC][4], pa13[KC][4], pb02[KC][4], pb13[KC][4];
  float sxa[KC], sxb[KC];
#pragma unroll
  for (int ch = 0; ch < KC; ++ch) {
    const unsigned char* xb = xs + (ch * 8 + bl) * 512;
    const int g0 = 8 * c + 2 * h;
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(xb + 16 * q4k_xswz(g0));
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(xb + 16 * q4k_xswz(g0 + 1));
    const u32x4 b0 = *reinterpret_cast<const u32x4*>(xb + 16 * q4k_xswz(g0 + 4));
    const u32x4 b1 = *reinterpret_cast<const u32x4*>(xb + 16 * q4k_xswz(g0 + 5));
    const unsigned XA[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const unsigned XB[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      pa02[ch][t] = __builtin_amdgcn_perm(XA[2 * t + 1], XA[2 * t], 0x05040100u);
      pa13[ch][t] = __builtin_amdgcn_perm(XA[2 * t + 1], XA[2 * t], 0x07060302u);
      pb02[ch][t] = __builtin_amdgcn_perm(XB[2 * t + 1], XB[2 * t], 0x05040100u);
      pb13[ch][t] = __builtin_amdgcn_perm(XB[2 * t + 1], XB[2 * t], 0x07060302u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sa = dot2h(XA[i], kOnes, sa);
      sb = dot2h(XB[i], kOnes, sb);
    }
    sxa[ch] = sa * 0x1p-24f;
    sxb[ch] = sb * 0x1p-24f;
  }

  // Lanes past the row's last block in a ragged last chunk see the next
  // record's bytes (or zeros); their share is dropped.
  const bool tail_ok = (KC - 1) * 8 + bl < nb;

  static_assert(R <= 16, "one row per lane of the last 16-lane row");
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  static_for<0, R * KC>([&](auto u) {
    constexpr int U = decltype(u)::value, r = U / KC, ch = U % KC;
    wait_vm<S::wait_count(U)>();
    // refill first: the stage holds the whole run, so the next loads never
    // overwrite unread bytes, and issuing them before this unit's arithmetic
    // keeps the arithmetic off the load path
    stream_loads<S::issued_before(U), S::issued_before(U + 1), QGEMV_WLOAD_AUX>(wr, stage, lane);
    const unsigned char* blk = stage + r * row_bytes + ch * C::kUnitBytes + bl * kQ4kBytes;
    const u32x4 hdr = *reinterpret_cast<const u32x4*>(blk);
    const u32x4 qv = *reinterpret_cast<const u32x4*>(blk + 16 + 16 * p);
    const unsigned q[4] = {qv.x, qv.y, qv.z, qv.w};
    float qa = 0.f, qb = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const unsigned w0 = q[t], w8 = q[t] >> 8;
      qa = dot2h(w0 & 0x000F000Fu, pa02[ch][t], qa);
      qa = dot2h(w8 & 0x000F000Fu, pa13[ch][t], qa);
      qb = dot2h(w0 & 0x00F000F0u, pb02[ch][t], qb);
      qb = dot2h(w8 & 0x00F000F0u, pb13[ch][t], qb);
    }
    const unsigned sp = sel.scales(hdr.y, hdr.w);
    const unsigned mp = sel.mins(hdr.z, hdr.w);
    const float sa = (float)(sp & 0xFFu), sb = (float)((sp >> 8) & 0xFFu);
    const float ma = (float)(mp & 0xFFu), mb = (float)((mp >> 8) & 0xFFu);
    const float d = f16lo(hdr.x), dmin = f16hi(hdr.x);
    const float v = __builtin_fmaf(sb, qb * 0.0625f, sa * qa);
    const float mx = __builtin_fmaf(mb, sxb[ch], ma * sxa[ch]);
    const float part = __builtin_fmaf(-dmin, mx, d * v);
    if constexpr (ch == KC - 1)
      acc[r] += tail_ok ? part : 0.f;
    else
      acc[r] += part;
  });
  store_rows<R>(acc, out, pre, row0, nrows, 0x1p24f, lane);
}

// Row materialisation.  Task t of an output row makes weights
// [E t, E t + E) (E = 8 or 4, all in one 32-weight group g of block b): the
// block header (d, dmin, packed scales) and E nibbles, low or high, of
// qs[32 c + l .. + E) with c = g / 2.  Each weight is the correctly rounded
// fp32 of d*s*q - dmin*m (both products are exact in fp32, so one fma rounds
// once), then converted to T.
#ifndef QGEMV_Q4K_ROWS_U
#define QGEMV_Q4K_ROWS_U 8  // row-materialisation tasks per thread
#endif

struct Q4kRowIn {
  u32x4 hdr;
  uint64_t q;
};

template <typename T, int U>
__global__ __launch_bounds__(256) void q4k_rows_kernel(const uint8_t* __restrict__ w, int n, int nb,
                                                       const int32_t* __restrict__ rows, T* __restrict__ out,
                                                       int bpr) {
  constexpr int E = kRowsE<T>;
  const int j = blockIdx.x / bpr;
  const int r = source_row(rows, j, n);
  // the source row as a buffer (32-bit offsets into it)
  const auto wr = make_rsrc(w + (int64_t)(r < 0 ? 0 : r) * nb * kQ4kBytes, (uint32_t)nb * kQ4kBytes);
  T* const orow = out + (int64_t)j * nb * 256;
  rows_thread<U, Q4kRowIn>(
      bpr, nb * (256 / E), r >= 0,
      [&](int t) {
        const int e0 = t * E, e = e0 & 255;
        const uint32_t blk = (uint32_t)(e0 >> 8) * kQ4kBytes;
        Q4kRowIn in;
        in.hdr = ld128s(wr, blk, 0u);
        const uint32_t qo = blk + 16u + (uint32_t)(32 * (e >> 6) + (e & 31));
        if constexpr (E == 8) {
          const u32x2 q = ld64s(wr, qo, 0u);
          in.q = (uint64_t)q.x | ((uint64_t)q.y << 32);
        } else {
          in.q = ld32s(wr, qo, 0u);
        }
        return in;
      },
      [&](int t, const Q4kRowIn& in) {
        const int e = (t * E) & 255;
        const int c = e >> 6, hi = (e >> 5) & 1;
        const Q4kScaleSel sel(c);
        const unsigned sh = 8u * (unsigned)hi;
        const unsigned sg = (sel.scales(in.hdr.y, in.hdr.w) >> sh) & 0xFFu;
        const unsigned mg = (sel.mins(in.hdr.z, in.hdr.w) >> sh) & 0xFFu;
        const float ds = f16lo(in.hdr.x) * (float)sg, dm = f16hi(in.hdr.x) * (float)mg;
        const unsigned nsh = 4u * (unsigned)hi;
        // the E nibbles as bytes 0..3 of one or two words (byte i -> weight i)
        unsigned m[2] = {((unsigned)in.q >> nsh) & 0x0F0F0F0Fu, ((unsigned)(in.q >> 32) >> nsh) & 0x0F0F0F0Fu};
        // opaque to the compiler, so that each byte converts with one
        // v_cvt_f32_ubyteN (with the masked bits known it shifts first)
        __asm__("" : "+v"(m[0]), "+v"(m[1]));
        float v[E];
#pragma unroll
        for (int i = 0; i < E; ++i) v[i] = __builtin_fmaf(ds, (float)((m[i >> 2] >> (8 * (i & 3))) & 0xFFu), -dm);
        store_e(orow + t * E, v);
      },
      [&](int t) { store_e_nan(orow + t * E); });
}

template <typename Out>
static hipError_t launch_q4k_lds(const void* w, const void* x, const Out& y, int64_t n, int64_t k,
                                 hipStream_t s) {
  const int nb = (int)(k / 256);
  const int kc = (nb + 7) / 8;
  const int kw = kc < QGEMV_WG_WAVES ? kc : QGEMV_WG_WAVES;
  const int rg = kw >= QGEMV_WG_WAVES ? 1 : QGEMV_WG_WAVES / kw;
  const int rows_per_wg = rg * kQ4kBatchRows;
  const int64_t grid = (n + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL(q4k_gemv_lds_kernel<Out>, dim3((unsigned)grid), dim3(64 * kw * rg), 0, s,
                     (const uint8_t*)w, (const uint16_t*)x, y, (int)n, nb, kc, kw, rg);
  return hipGetLastError();
}


// Row-streaming launch for the K-chunk counts it is instantiated for: R rows
// per wave chosen so the grid is about one wave per SIMD (one-shot), capped by
// the LDS stage; returns false when the shape has no instantiation.
template <int KC, int R, int W, typename Out>
static hipError_t launch_q4k_rows_r(const void* w, const void* x, const Out& y, int64_t n, int64_t k, hipStream_t s) {
  const int64_t rows_per_wg = (int64_t)W * R;
  const int64_t grid = (n + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((q4k_gemv_rows_kernel<KC, R, W, Out>), dim3((unsigned)grid), dim3(64 * W), 0, s,
                     (const uint8_t*)w, (const uint16_t*)x, y, (int)n, (int)(k / 256));
  return hipGetLastError();
}

template <int KC, typename Out>
static hipError_t launch_q4k_rows_kc(const void* w, const void* x, const Out& y, int64_t n, int64_t k, hipStream_t s) {
  constexpr int kRmax = largest_fitting_r([](int r) {
    return 8 * ((r * KC * 8 * kQ4kBytes + 1023) / 1024) * 1024 + KC * 4096 <= 160 * 1024;
  });
  return dispatch_rows<kRmax>(n, [&](auto rc, auto wc) {
    return launch_q4k_rows_r<KC, decltype(rc)::value, decltype(wc)::value, Out>(w, x, y, n, k, s);
  });
}

// Row streaming for K up to 16384 (at most 8 K-chunks of 2048); false when K
// is larger (the K-split kernel takes it).
template <typename Out>
static bool launch_q4k_rows(const void* w, const void* x, const Out& y, int64_t n, int64_t k, hipStream_t s,
                            hipError_t* err) {
  const int kc = (int)((k / 256 + 7) / 8);
  switch (kc) {
    case 1: *err = launch_q4k_rows_kc<1, Out>(w, x, y, n, k, s); return true;
    case 2: *err = launch_q4k_rows_kc<2, Out>(w, x, y, n, k, s); return true;
    case 3: *err = launch_q4k_rows_kc<3, Out>(w, x, y, n, k, s); return true;
    case 4: *err = launch_q4k_rows_kc<4, Out>(w, x, y, n, k, s); return true;
    case 5: *err = launch_q4k_rows_kc<5, Out>(w, x, y, n, k, s); return true;
    case 6: *err = launch_q4k_rows_kc<6, Out>(w, x, y, n, k, s); return true;
    case 7: *err = launch_q4k_rows_kc<7, Out>(w, x, y, n, k, s); return true;
    case 8: *err = launch_q4k_rows_kc<8, Out>(w, x, y, n, k, s); return true;
    default: return false;
  }
}

// 1: K-split kernel only, 2: row-streaming kernel for K <= 16384 (K-split beyond)
#ifndef QGEMV_Q4K_IMPL
#define QGEMV_Q4K_IMPL 2
#endif

template <typename Out>
static hipError_t launch_q4k_gemv_out(const void* w, const void* x, const Out& y, int64_t n, int64_t k,
                                      hipStream_t s) {
  if (QGEMV_Q4K_IMPL == 2) {
    hipError_t e = hipSuccess;
    if (launch_q4k_rows(w, x, y, n, k, s, &e)) return e;
  }
  return launch_q4k_lds(w, x, y, n, k, s);
}

hipError_t launch_q4k_gemv(const void* w, const void* x, const OutF32& y, int64_t n, int64_t k, hipStream_t s) {
  return launch_q4k_gemv_out(w, x, y, n, k, s);
}
hipError_t launch_q4k_gemv(const void* w, const void* x, const OutEx& y, int64_t n, int64_t k, hipStream_t s) {
  return launch_q4k_gemv_out(w, x, y, n, k, s);
}

template <typename T, int U>
static hipError_t launch_q4k_rows_u(const void* w, int64_t n, int64_t k, const int32_t* rows, int64_t nrows,
                                    void* out, hipStream_t s) {
  const RowsGeom g = rows_geom(k / kRowsE<T>, nrows, U);
  hipLaunchKernelGGL((q4k_rows_kernel<T, U>), dim3((unsigned)g.grid), dim3(g.block), 0, s, (const uint8_t*)w,
                     (int)n, (int)(k / 256), rows, (T*)out, g.bpr);
  return hipGetLastError();
}

// Small launches (a few hundred gathered rows) take one task per thread so
// that they still spread over the whole chip.
template <typename T>
static hipError_t launch_q4k_rows_t(const void* w, int64_t n, int64_t k, const int32_t* rows, int64_t nrows,
                                    void* out, hipStream_t s) {
  if (nrows * (k / kRowsE<T>) < kRowsSmallTasks) return launch_q4k_rows_u<T, 1>(w, n, k, rows, nrows, out, s);
  return launch_q4k_rows_u<T, QGEMV_Q4K_ROWS_U>(w, n, k, rows, nrows, out, s);
}

hipError_t launch_q4k_get_rows(const void* w, int64_t n, int64_t k, const int32_t* rows, int64_t nrows, void* out,
                               int dtype, hipStream_t s) {
  if (dtype == kF16) return launch_q4k_rows_t<_Float16>(w, n, k, rows, nrows, out, s);
  if (dtype == kBF16) return launch_q4k_rows_t<__bf16>(w, n, k, rows, nrows, out, s);
  return launch_q4k_rows_t<float>(w, n, k, rows, nrows, out, s);
}

}  // namespace qgemv
