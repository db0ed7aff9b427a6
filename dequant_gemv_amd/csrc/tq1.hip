// TQ1_0 fused dequantise + GEMV and row materialisation for gfx950.
//
// Format ("metal: TQ1_0 kernel performance", sections 1 and 2): 54 bytes per
// 256 weights, qs[48] (five base-3 digits per byte) | qh[4] (four digits per
// byte) | fp16 d.  Digit k of byte b is floor(3^(k+1) b / 256) - 3 floor(3^k b / 256);
// digit k of qs[j] feeds element 32k+j (j < 32) or 160+16k+(j-32) (j < 48),
// digit k < 4 of qh[m] feeds element 240+4k+m; weight = d*(digit-1).
//
// GEMV work split.  That page's flattened mat-vec treats qs and qh as one
// 52-byte payload; here the whole row is the payload stream.  A wave owns a
// segment of 16 blocks (864 bytes = 54 dwordx4, lanes 0..53, coalesced) for R
// rows.  Every byte pair (2i, 2i+1) of a lane's 16 bytes belongs to one block
// (blocks start at even offsets) and its two bytes feed activation pairs that
// are adjacent in x (elements e, e+1 for the same digit), so each lane keeps
// 8 pairs x 5 digits of fp16 activation pairs in registers, loaded once per
// segment; coefficients of non-elements (digit 4 of qh bytes, the d bytes)
// are zero, the zero-padding trick of the page's section 1, so all byte pairs
// run one code path.
//
// Digits in registers: with L_0 = b and L_{k+1} = 3 L_k mod 256 (the
// fractional part of 3^(k+1) b / 256, in 256ths), digit k is floor(3 L_k /
// 256), because 3^(k+1) b = 3 (256 floor(3^k b / 256) + L_k).  With B = (b0 |
// b1 << 16) both bytes go through one 32-bit multiply by 3 (each half stays
// below 768, so no carry crosses) and two masks per digit: 3 L & 0xFF00FF00
// holds digit << 8 in each half, 3 L & 0x00FF00FF the next L.  The 16-bit
// pattern digit << 8 is the fp16 subnormal digit * 2^-16 (exact), so
// v_dot2_f32_f16 consumes it directly against the activation pair: sum x*t =
// 2^16 * acc exactly up to fp32 accumulation.  No fp16 arithmetic touches the
// digits themselves (the page's "Not applicable" section shows why fp16
// floors fail).
//
// Each block's d sits in the lane whose 16 bytes hold bytes 52-53 of that
// block; lanes fetch the d of the (at most two) blocks they touch with
// ds_bpermute.  sum x*(t-1) = sum x*t - sum x, the second term precomputed.
//
// Digits from a table (the row-streaming kernel for K = 4096 and more than
// 1024 rows): a 256-entry LDS table gives the five values digit_k(b) - 1 of a
// byte as fp16 pairs, so a byte's five weights cost one 16-byte LDS read,
// one v_perm_b32 (the table address) and three v_dot2 instead of the
// arithmetic above (about 0.85 VALU instructions per weight instead of 2;
// the table is built per workgroup, 16 copies side by side so the lanes of a
// read never contend for a bank), and each lane takes a quarter block.
#include "device.hpp"
#include "launch.hpp"
#include "rows.hpp"
#include "stream.hpp"

namespace qgemv {

// Rows per wave and waves per workgroup (tuning).
#ifndef QGEMV_TQ1_R
#define QGEMV_TQ1_R 8
#endif
#ifndef QGEMV_WG_WAVES
#define QGEMV_WG_WAVES 8
#endif

constexpr int kTq1Bytes = 54;
constexpr int kTq1SegBlocks = 16;
constexpr int kTq1SegBytes = kTq1SegBlocks * kTq1Bytes;  // 864 = 54 * 16

// Element (0..255) fed by digit k of payload byte pos, or -1.
__device__ __forceinline__ int tq1_element(int pos, int k) {
  if (pos < 32) return 32 * k + pos;
  if (pos < 48) return 160 + 16 * k + (pos - 32);
  if (pos < 52) return k < 4 ? 240 + 4 * k + (pos - 48) : -1;
  return -1;
}


// Five fp16 pairs (digit_k(b0) * 2^-16, digit_k(b1) * 2^-16), k = 0..4, from
// B = b0 | b1 << 16 (32-bit operations, cheaper here than packed 16-bit ones).
__device__ __forceinline__ void tq1_digits(unsigned B, unsigned (&D)[5]) {
  unsigned L = B;
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const unsigned t = L * 3u;  // 3 L_k per half, < 768
    D[k] = t & 0xFF00FF00u;     // digit_k << 8 per half
    L = t & 0x00FF00FFu;        // L_{k+1}
  }
}

template <int R, typename Out>
__global__ __launch_bounds__(64 * QGEMV_WG_WAVES) void tq1_gemv_kernel(const uint8_t* __restrict__ w,
                                                       const uint16_t* __restrict__ x,
                                                       Out out, int n, int nb,
                                                       int kc, int kw, int rg) {
  __shared__ float red[16 * 16];
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: keeps the buffer descriptors in SGPRs
  const int kwi = wave % kw;
  const int rgi = wave / kw;
  const int64_t row_bytes = (int64_t)nb * kTq1Bytes;
  const int row0 = blockIdx.x * rg * R + rgi * R;
  const int nrows = max(0, min(R, n - row0));
  const auto wr = make_rsrc(w + (int64_t)row0 * row_bytes, (uint32_t)(nrows * row_bytes));
  const auto xr = make_rsrc(x, (uint32_t)nb * 512u);

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;

  const int o0 = 16 * lane;  // first byte of this lane inside a segment
  const int blk_first = o0 / kTq1Bytes;

  for (int ch = kwi; ch < kc; ch += kw) {
    const int nbs = min(kTq1SegBlocks, nb - ch * kTq1SegBlocks);  // blocks in this segment
    const bool active = lane < 54 && blk_first < nbs;

    // Per-lane activation pairs for 8 byte pairs x 5 digits, zero where the
    // digit feeds no element of a block inside this segment.  Loaded before
    // the weights: loads complete in issue order.
    unsigned xp[8][5];
    int bnd = 8;  // byte pairs that belong to the lane's first block
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int o = o0 + 2 * i;
      const int blk = o / kTq1Bytes;
      const int pos = o - blk * kTq1Bytes;
      const bool in = active && blk < nbs;
      if (blk != blk_first && bnd == 8) bnd = i;
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        const int e = tq1_element(pos, k);
        const int ge = (ch * kTq1SegBlocks + blk) * 256 + e;
        // an out-of-range offset reads as zero
        xp[i][k] = ld32(xr, (in && e >= 0) ? (uint32_t)ge * 2u : 0xFFFFFFF0u);
      }
    }
    // The d of a block sits in its bytes 52-53, inside exactly one lane's 16
    // bytes; that lane loads it with a 16-bit load (a wider load could cross
    // the end of the buffer and read as zero).
    int hold = -1;
    for (int bh = blk_first; bh <= blk_first + 1; ++bh) {
      const int dpos = bh * kTq1Bytes + 52 - o0;
      if (dpos >= 0 && dpos < 16 && bh < nbs && lane < 54) hold = bh * kTq1Bytes + 52;
    }
    u32x4 raw[R];
    unsigned short dbits[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t base = (uint32_t)(r * row_bytes + ch * kTq1SegBytes);
      raw[r] = ld128w(wr, base + o0);
      dbits[r] = ld16(wr, hold >= 0 ? base + (uint32_t)hold : 0xFFFFFFF0u);
    }

    float xs0 = 0.f, xs1 = 0.f;  // sum of x over the lane's elements, per block slot
    const unsigned kOnes = 0x3C003C00u;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        xs0 = dot2h(i < bnd ? xp[i][k] : 0u, kOnes, xs0);
        xs1 = dot2h(i < bnd ? 0u : xp[i][k], kOnes, xs1);
      }
    // A slot whose block lies outside the segment (or a lane past the
    // payload) gets d = 0 from a non-holding lane and zero coefficients, so
    // it adds exactly 0 without a branch.
    const int src0 = ((blk_first * kTq1Bytes + 52) / 16) << 2;
    const int src1 = (((blk_first + 1) * kTq1Bytes + 52) / 16) << 2;

#pragma unroll
    for (int r = 0; r < R; ++r) {
      const unsigned dw[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
      const float dh = (float)__builtin_bit_cast(_Float16, dbits[r]);
      const float d0 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src0, __builtin_bit_cast(int, dh)));
      const float d1 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src1, __builtin_bit_cast(int, dh)));

      float a = 0.f, snap = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned B = __builtin_amdgcn_perm(0u, dw[i >> 1], (i & 1) ? 0x0C030C02u : 0x0C010C00u);
        unsigned D[5];
        tq1_digits(B, D);
#pragma unroll
        for (int k = 0; k < 5; ++k) a = dot2h(D[k], xp[i][k], a);
        snap = (i == bnd - 1) ? a : snap;
      }
      float t = __builtin_fmaf(d0, __builtin_fmaf(snap, 65536.f, -xs0), acc[r]);
      acc[r] = __builtin_fmaf(d1, __builtin_fmaf(a - snap, 65536.f, -xs1), t);
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


// Row-streaming variant (K a multiple of 2048, up to 8192): a wave owns R
// whole rows, whose bytes are one contiguous run of R*KS segments of up to
// 864 bytes (16 blocks; the last segment of a row may hold 8) streamed into
// the wave's LDS stage with the shared lookahead schedule (a row of 8m blocks
// is 432m bytes, so every segment starts 16-byte aligned).
// Lane l < 54 takes bytes 16l..16l+15 of every segment, as in the K-split
// kernel; its 8 x 5 activation pairs and per-block-slot sums are read once
// per segment position from the workgroup's LDS copy of x and reused for all
// R rows.  The two d values a lane needs are read from the stage; slots whose
// block lies outside the segment, and lanes past the payload, use d = 0 and
// zero activations, so they add exactly 0.
#ifndef QGEMV_TQ1_AHEAD
#define QGEMV_TQ1_AHEAD 4
#endif
#ifndef QGEMV_TQ1_FIRST
#define QGEMV_TQ1_FIRST QGEMV_TQ1_AHEAD
#endif

template <int KS, int R, int W>
struct Tq1Rows {
  using S = StreamSchedule<kTq1SegBytes, R * KS, QGEMV_TQ1_AHEAD, QGEMV_TQ1_AHEAD, QGEMV_TQ1_FIRST>;
  static constexpr int kXBytes = KS * 8192;
  static constexpr int kLds = W * S::kStage + kXBytes + 16;  // + one zero dword: coefficient of a non-element
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};

template <int KS, int R, int W, typename Out>
__global__ __launch_bounds__(64 * W) void tq1_gemv_rows_kernel(const uint8_t* __restrict__ w,
                                                              const uint16_t* __restrict__ x,
                                                              Out out, int n, int nb) {
  using C = Tq1Rows<KS, R, W>;
  using S = typename C::S;  // assumes full segments; a short last segment only ends earlier
  const int kRowBytes = nb * kTq1Bytes;
  const int nbs_last = nb - (KS - 1) * kTq1SegBlocks;  // 8 or 16
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::kLds];
  unsigned char* const xs = lds + W * S::kStage;
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned char* const stage = lds + wave * S::kStage;
  const int row0 = (blockIdx.x * W + wave) * R;
  const int nrows = max(0, min(R, n - row0));

  load_shared_pieces<8 * KS, W>(make_rsrc(x, (uint32_t)nb * 512u), xs, wave, lane,
                                [](int piece, int i) { return (uint32_t)(piece * 1024 + 16 * i); });
  const auto wr = make_rsrc(w + (int64_t)row0 * kRowBytes, (uint32_t)(nrows * kRowBytes));
  stream_loads<0, S::kUpFront, QGEMV_WLOAD_AUX>(wr, stage, lane);

  // Lanes past the payload address byte 0 (their results are masked), so every
  // LDS access below stays inside the wave's own segment or the activations.
  const bool active = lane < 54;
  const int o0 = active ? 16 * lane : 0;
  const int blk0 = o0 / kTq1Bytes;  // the lane's first block in a segment
  int bnd = 8;                      // byte pairs in the first block
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if ((o0 + 2 * i) / kTq1Bytes != blk0 && bnd == 8) bnd = i;
  // per segment: the lane's first / second block slot holds a block of the segment
  auto slot0 = [&](int sg) { return active && blk0 < (sg == KS - 1 ? nbs_last : kTq1SegBlocks); };
  auto slot1 = [&](int sg) { return active && bnd < 8 && blk0 + 1 < (sg == KS - 1 ? nbs_last : kTq1SegBlocks); };
  const int dof0 = blk0 * kTq1Bytes + 52;
  const int dof1 = (bnd < 8 && blk0 + 1 < kTq1SegBlocks) ? (blk0 + 1) * kTq1Bytes + 52 : dof0;

  unsigned char* const zero = xs + C::kXBytes;
  if (wave == 0 && lane == 0) {
    *reinterpret_cast<unsigned*>(zero) = 0u;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the zero is in LDS before the barrier
  }
  wait_vm<S::kUpFront>();        // activations (issued first) are in LDS
  __builtin_amdgcn_s_barrier();  // ... every wave's pieces too
  // the output stage's input for the wave's rows, after the barrier's wait
  // (the stream's later waits only get stricter by this one load)
  const auto pre = prefetch_rows(out, row0, nrows, lane);
  stream_loads<S::kUpFront, S::issued_before(0), QGEMV_WLOAD_AUX>(wr, stage, lane);

  // Activation pairs of the lane's byte pairs: digit k of payload byte pos
  // feeds element base + k*stride of its block (qs[0..31]: pos, 32; qs[32..47]:
  // pos + 128, 16; qh: pos + 192, 4 with no fifth digit); byte pairs past the
  // payload (d) and lanes past it read the zero dword.  Sums per block slot
  // use the same snapshot as the units below.
  unsigned xp[KS][8][5];
  float xs0[KS], xs1[KS];
  const unsigned kOnes = 0x3C003C00u;
  bool last_of_first[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) last_of_first[i] = i == bnd - 1;
#pragma unroll
  for (int sg = 0; sg < KS; ++sg) {
    float a = 0.f, snap = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int o = o0 + 2 * i;
      const int blk = o / kTq1Bytes;
      const int pos = o - blk * kTq1Bytes;
      const int base = pos < 32 ? pos : pos < 48 ? pos + 128 : pos + 192;
      const int stride = pos < 32 ? 64 : pos < 48 ? 32 : 8;  // bytes
      const bool payload = slot0(sg) && pos < 52 && (blk == blk0 || slot1(sg));
      const unsigned char* p0 = payload ? xs + sg * 8192 + (blk * 256 + base) * 2 : zero;
      const int st = payload ? stride : 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) xp[sg][i][k] = *reinterpret_cast<const unsigned*>(p0 + k * st);
      xp[sg][i][4] = *reinterpret_cast<const unsigned*>(pos < 48 ? p0 + 4 * st : zero);
#pragma unroll
      for (int k = 0; k < 5; ++k) a = dot2h(xp[sg][i][k], kOnes, a);
      snap = last_of_first[i] ? a : snap;
    }
    xs0[sg] = snap;
    xs1[sg] = a - snap;
  }

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  static_for<0, R * KS>([&](auto uc) {
    constexpr int U = decltype(uc)::value, r = U / KS, sg = U % KS;
    wait_vm<S::wait_count(U)>();
    // refill first: the stage holds the whole run (no unread byte is
    // overwritten) and the arithmetic stays off the load path
    stream_loads<S::issued_before(U), S::issued_before(U + 1), QGEMV_WLOAD_AUX>(wr, stage, lane);
    const unsigned char* seg = stage + r * kRowBytes + sg * kTq1SegBytes;
    const u32x4 raw = *reinterpret_cast<const u32x4*>(seg + o0);
    const unsigned short db0 = *reinterpret_cast<const unsigned short*>(seg + dof0);
    const unsigned short db1 = *reinterpret_cast<const unsigned short*>(seg + dof1);
    const float d0 = slot0(sg) ? (float)__builtin_bit_cast(_Float16, db0) : 0.f;
    const float d1 = slot1(sg) ? (float)__builtin_bit_cast(_Float16, db1) : 0.f;
    const unsigned dw[4] = {raw.x, raw.y, raw.z, raw.w};
    float a = 0.f, snap = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned B = __builtin_amdgcn_perm(0u, dw[i >> 1], (i & 1) ? 0x0C030C02u : 0x0C010C00u);
      unsigned D[5];
      tq1_digits(B, D);
#pragma unroll
      for (int k = 0; k < 5; ++k) a = dot2h(D[k], xp[sg][i][k], a);
      snap = last_of_first[i] ? a : snap;
    }
    const float t = __builtin_fmaf(d0, __builtin_fmaf(snap, 65536.f, -xs0[sg]), acc[r]);
    acc[r] = __builtin_fmaf(d1, __builtin_fmaf(a - snap, 65536.f, -xs1[sg]), t);
  });
  store_rows<R>(acc, out, pre, row0, nrows, 1.f, lane);
}

// Table-driven row-streaming kernel (K = 4096, more than 1024 rows).  The
// digits come from a 256-entry table instead of arithmetic: entry b holds the
// fp16 values digit_k(b) - 1 (-1, 0 or +1, exact) as the pairs (k0, k1), (k2,
// k3), (k4, 0) and a zero dword, so one 16-byte LDS read and three
// v_dot2_f32_f16 against the activation pairs (x[e0], x[e1]), (x[e2], x[e3]),
// (x[e4], 0) (e_k the element digit k of the byte feeds) take a byte's five
// weights, and the sum of x (t - 1) needs no correction term.  The table is
// built per workgroup with LREP copies of each entry side by side and lane l
// reads copy l % LREP: for LREP = 16 any 16 consecutive lanes read 16
// different 16-byte bank groups whatever their bytes are.  The address is the
// byte moved to bit 8 over the lane's copy offset, one v_perm_b32.
//
// A wave streams its R rows through a ring of eight one-KiB LDS slots (the
// lookahead never reaches further), one 864-byte segment of 16 blocks per
// unit.  Lane l takes the 13 payload bytes 13 q .. 13 q + 12 (q = l % 4) of
// block l / 4 of the segment, so the 64 lanes cover the 16 blocks' 832
// payload bytes exactly, a lane's bytes all belong to one block (one d per
// unit) and no lane idles.  A lane's bytes start at segment offset
// 54 (l / 4) + 13 q, which is 4-byte but not 16-byte aligned: the lane reads
// the 16 bytes from the dword at or below it and byte-aligns them in
// registers (v_alignbyte_b32 by the lane's misalignment); the last byte's
// address takes one v_perm_b32 with a per-lane selector.  Per unit a lane
// reads 13 table entries and issues 39 v_dot2_f32_f16 in one chain
// (dependent v_dot2 issue back to back: more chains only cost the adds).
// The activation pairs of a lane's 13 bytes are built once per workgroup from
// its LDS copy of x and held in registers for all R rows.
#ifndef QGEMV_TQ1_RING
#define QGEMV_TQ1_RING 8  // stage slots (one KiB each) per wave of the table-driven kernel
#endif
constexpr int kTq1Ring = QGEMV_TQ1_RING;

template <int KS, int R, int W, int LREP>
struct Tq1TableRows {
  using S = StreamSchedule<kTq1SegBytes, R * KS, QGEMV_TQ1_AHEAD, QGEMV_TQ1_AHEAD, QGEMV_TQ1_FIRST, kTq1Ring>;
  static constexpr int kLutBytes = 256 * 16 * LREP;  // at LDS offset 0
  static constexpr int kXBytes = KS * 8192;
  static constexpr int kEntries = 13 * 64;  // activation pair entries (byte, lane) per segment
  static constexpr int kPairBytes = KS * kEntries * 16;
  static constexpr int kBuildersPerWave = KS * 16 * 7 / W;  // pair build tasks: 28 per block, 4 per builder
  static constexpr int kLds = kLutBytes + W * S::kStage + kXBytes + kPairBytes;
  static_assert(LREP == 8 || LREP == 16, "table copies");
  static_assert(W == 4 || W == 8, "waves per workgroup");
  static_assert((8 * KS) % W == 0 && kBuildersPerWave <= 64, "whole pieces of x per wave");
};

// LDS bytes of a table-driven launch (what the launcher checks against the
// 160 KiB of a workgroup).
constexpr int tq1_table_lds(int ks, int r, int w, int lrep) {
  const int loads = (r * ks * kTq1SegBytes + 1023) / 1024;
  return 256 * 16 * lrep + w * (loads < kTq1Ring ? loads : kTq1Ring) * 1024 + ks * 8192 + ks * 13 * 64 * 16;
}

// fp16 bits of digit_k(b) - 1 for k = 0..4 (same recurrence as tq1_digits on
// one byte: L_{k+1} = 3 L_k mod 256, digit_k = floor(3 L_k / 256)).
__device__ __forceinline__ void tq1_lut_codes(unsigned b, unsigned (&h)[5]) {
  unsigned L = b;
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const unsigned t = 3u * L;
    const unsigned digit = t >> 8;
    h[k] = digit == 0 ? 0xBC00u : digit == 1 ? 0u : 0x3C00u;
    L = t & 0xFFu;
  }
}

template <int KS, int R, int W, int LREP, typename Out>
__global__ __launch_bounds__(64 * W) void tq1_gemv_table_kernel(const uint8_t* __restrict__ w,
                                                                const uint16_t* __restrict__ x,
                                                                Out out, int n, int nb) {
  using C = Tq1TableRows<KS, R, W, LREP>;
  using S = typename C::S;
  constexpr int kRowBytes = KS * kTq1SegBytes;  // nb == 16 KS, checked by the launcher
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::kLds];
  unsigned char* const lut = lds;
  unsigned char* const xs = lds + C::kLutBytes + W * S::kStage;  // x
  unsigned char* const pairs = xs + C::kXBytes;
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned char* const stage = lds + C::kLutBytes + wave * S::kStage;
  const int row0 = (blockIdx.x * W + wave) * R;
  const int nrows = max(0, min(R, n - row0));

  // x into LDS in 1 KiB pieces (two blocks each): this wave copies pieces
  // i W + wave
  load_shared_pieces<8 * KS, W>(make_rsrc(x, (uint32_t)nb * 512u), xs, wave, lane,
                                [](int piece, int i) { return (uint32_t)(piece * 1024 + 16 * i); });
  const auto wr = make_rsrc(w + (int64_t)row0 * kRowBytes, (uint32_t)(nrows * kRowBytes));
  stream_loads<0, S::kUpFront, QGEMV_WLOAD_AUX, S::kRing>(wr, stage, lane);

  // The digit table: thread t computes entry b = t % 256; the H = 64W / 256
  // threads of an entry write LREP / H of its LREP copies each, copy
  // (b + H j + t / 256) % LREP on step j, so the 16 consecutive entries
  // written by 16 consecutive lanes land in 16 different bank groups.
  {
    constexpr int H = 64 * W / 256;
    const unsigned b = threadIdx.x & 255u;
    const int part = (int)(threadIdx.x >> 8);
    unsigned h[5];
    tq1_lut_codes(b, h);
    const u32x4 v = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4], 0u};
#pragma unroll
    for (int j = 0; j < LREP / H; ++j) {
      const int copy = ((int)b + H * j + part) & (LREP - 1);
      *reinterpret_cast<u32x4*>(lut + b * (16 * LREP) + copy * 16) = v;
    }
  }

  // the lane's 13 bytes: segment offset s = 54 (lane / 4) + 13 (lane % 4),
  // read from the dword at s - m (m = s % 4); its block's d at 54 (lane / 4) + 52
  const int s0 = 54 * (lane >> 2) + 13 * (lane & 3);
  const unsigned mis = (unsigned)(s0 & 3);
  const int a0 = s0 - (int)mis;
  const int dof = 54 * (lane >> 2) + 52;

  // Activation pairs of entry (byte i, lane l) of segment sg: lane l's byte
  // i is payload byte pos = 13 (l % 4) + i of block l / 4, whose digit k
  // feeds element e_k of the block: pos + 32 k for qs[0..31], pos + 128 +
  // 16 k for qs[32..47], pos + 192 + 4 k (k < 4, no fifth digit) for qh.
  // The entry (x[e0], x[e1]), (x[e2], x[e3]), (x[e4] or 0) sits in slot
  // (sg * 13 + i) * 64 + (l ^ 4 i), so a lane's reads of its 13 entries are
  // conflict-free.  A build task (block, g, j) makes the entries of payload
  // bytes 8 g + 2 j and 8 g + 2 j + 1 (g < 6, j < 4; for g = 6, bytes 48 +
  // 2 j and 48 + 2 j + 1, j < 2): digit k of the two bytes reads the two
  // halves of one dword of x, elements 2 j and 2 j + 1 of the run that
  // starts at 8 g + 32 k (g < 4), 128 + 8 g + 16 k (g = 4, 5) or 240 + 4 k
  // (g = 6).  The 28 tasks of a block run in the wave that copied the
  // block's piece of x, so that wave's own wait for its copy stands in for a
  // workgroup barrier: task t of the wave (lane t % 64 in round t / 64)
  // serves block 2 P + (t % 56) / 28 (counted over the segments) of piece
  // P = (t / 56) W + wave, g = (t % 28) / 4, j = t % 4.
  constexpr int kTasks = 4 * C::kBuildersPerWave, kRounds = (kTasks + 63) / 64;
  unsigned xof[kRounds][5];   // LDS offsets in x of the task's dwords
  unsigned slot[kRounds][2];  // and of its two entries
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int t = 64 * r + lane;
    const int bblk = 2 * ((t / 56) * W + wave) + (t % 56) / 28, g = (t % 28) / 4, j = t % 4;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int e = g < 4 ? 8 * g + 32 * k : g < 6 ? 128 + 8 * g + 16 * k : k < 4 ? 240 + 4 * k : 240;
      xof[r][k] = (unsigned)(bblk * 512 + 2 * (e + 2 * j));
      settle(xof[r][k]);  // computed while the copies are in flight
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int pos = 8 * g + 2 * j + h, q = pos / 13, i13 = pos - 13 * q;
      slot[r][h] = (unsigned)((((bblk >> 4) * 13 + i13) * 64 + (((bblk & 15) * 4 + q) ^ (4 * i13))) * 16);
      settle(slot[r][h]);
    }
  }

  wait_vm<S::kUpFront>();  // this wave's pieces of x (copied first) are in LDS
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int t = 64 * r + lane;
    const int g = (t % 28) / 4, j = t % 4;
    if (t < kTasks && (g < 6 || j < 2)) {
      unsigned d[5];
#pragma unroll
      for (int k = 0; k < 5; ++k) d[k] = *reinterpret_cast<const unsigned*>(xs + xof[r][k]);
      if (g == 6) d[4] = 0u;  // the qh bytes have no fifth digit
      // entry 2 j from the low halves, entry 2 j + 1 from the high ones
      const u32x4 lo = {__builtin_amdgcn_perm(d[1], d[0], 0x05040100u), __builtin_amdgcn_perm(d[3], d[2], 0x05040100u),
                        d[4] & 0xFFFFu, 0u};
      const u32x4 hi = {__builtin_amdgcn_perm(d[1], d[0], 0x07060302u), __builtin_amdgcn_perm(d[3], d[2], 0x07060302u),
                        d[4] >> 16, 0u};
      *reinterpret_cast<u32x4*>(pairs + slot[r][0]) = lo;
      *reinterpret_cast<u32x4*>(pairs + slot[r][1]) = hi;
    }
  }
  lds_barrier();  // the table and every pair entry are in LDS
  const auto pre = prefetch_rows(out, row0, nrows, lane);
  stream_loads<S::kUpFront, S::issued_before(0), QGEMV_WLOAD_AUX, S::kRing>(wr, stage, lane);

  unsigned xp[KS][13][3];
#pragma unroll
  for (int sg = 0; sg < KS; ++sg) {
#pragma unroll
    for (int i = 0; i < 13; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(pairs + ((sg * 13 + i) * 64 + (lane ^ (4 * i))) * 16);
      xp[sg][i][0] = v.x;
      xp[sg][i][1] = v.y;
      xp[sg][i][2] = v.z;
    }
  }
  // the lane's table copy, in the low byte of the perm source
  const unsigned colw = LREP == 16 ? (unsigned)(lane & 15) * 16u : (unsigned)(lane & 7) * 32u;
  // byte 12 sits in the fourth dword at byte mis: perm selector putting it
  // in byte 1 of the address, colw's byte 0 in byte 0
  const unsigned sel12 = 0x0C0C0000u | ((4u + mis) << 8);

  // One unit's table entries and d, read one unit ahead of its sums so that
  // the LDS latency of unit U + 1 hides behind the arithmetic of unit U.
  struct UnitIn {
    u32x4 t[13];
    float d;
  };
  auto fetch = [&](auto uc) {
    constexpr int U = decltype(uc)::value, r = U / KS, sg = U % KS;
    UnitIn in;
    wait_vm<S::wait_count(U)>();
    stream_loads<S::issued_before(U), S::issued_before(U + 1), QGEMV_WLOAD_AUX, S::kRing>(wr, stage, lane);
    constexpr int ub = S::slot_offset(r * kRowBytes + sg * kTq1SegBytes);
    unsigned dw[4];
    unsigned short db;
    if constexpr (ub + kTq1SegBytes <= S::kStage) {
      const unsigned* p = reinterpret_cast<const unsigned*>(stage + ub + a0);
#pragma unroll
      for (int j = 0; j < 4; ++j) dw[j] = p[j];
      db = *reinterpret_cast<const unsigned short*>(stage + ub + dof);
    } else {  // the unit wraps round the ring's end: every dword on its own
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int o = ub + a0 + 4 * j;
        dw[j] = *reinterpret_cast<const unsigned*>(stage + (o >= S::kStage ? o - S::kStage : o));
      }
      const int o = ub + dof;
      db = *reinterpret_cast<const unsigned short*>(stage + (o >= S::kStage ? o - S::kStage : o));
    }
    in.d = (float)__builtin_bit_cast(_Float16, db);
    // bytes 4j .. 4j + 3 of the lane's run
    const unsigned al[3] = {__builtin_amdgcn_alignbyte(dw[1], dw[0], mis),
                            __builtin_amdgcn_alignbyte(dw[2], dw[1], mis),
                            __builtin_amdgcn_alignbyte(dw[3], dw[2], mis)};
#pragma unroll
    for (int i = 0; i < 13; ++i) {
      unsigned addr = i < 12 ? __builtin_amdgcn_perm(al[i >> 2], colw, 0x0C0C0000u | ((4u + (i & 3)) << 8))
                             : __builtin_amdgcn_perm(dw[3], colw, sel12);
      if (LREP == 8) addr >>= 1;
      in.t[i] = *reinterpret_cast<const u32x4*>(lut + addr);
    }
    return in;
  };
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  auto consume = [&](auto uc, const UnitIn& in) {
    constexpr int U = decltype(uc)::value, r = U / KS, sg = U % KS;
    float c = 0.f;
#pragma unroll
    for (int i = 0; i < 13; ++i) {
      c = dot2h(in.t[i].x, xp[sg][i][0], c);
      c = dot2h(in.t[i].y, xp[sg][i][1], c);
      c = dot2h(in.t[i].z, xp[sg][i][2], c);
    }
    acc[r] = __builtin_fmaf(in.d, c, acc[r]);
    settle(acc[r]);  // this unit's sums end before the next unit's wait
  };
  constexpr int kUnits = R * KS;
  UnitIn cur = fetch(Int<0>{});
  static_for<0, kUnits>([&](auto uc) {
    constexpr int U = decltype(uc)::value;
    if constexpr (U + 1 < kUnits) {
      const UnitIn nxt = fetch(Int<U + 1>{});
      consume(uc, cur);
      cur = nxt;
    } else {
      consume(uc, cur);
    }
  });
  store_rows<R>(acc, out, pre, row0, nrows, 1.f, lane);
}

// Row materialisation.  Task t of an output row makes weights
// [E t, E t + E) (E = 8 or 4) of block b, in the section-2 element order of
// the TQ1_0 page: element 32 k + j (j < 32) is digit k of qs[j], element
// 160 + 16 k + i (i < 16) digit k of qs[32 + i], element 240 + 4 k + m digit
// k of qh[m].  So the E weights are one digit of E consecutive qs bytes, or
// (past element 240) E/4 digits of the four qh bytes.  Weight = d * (digit -
// 1), exact in fp32 (and in fp16).
//
// A weight can only be one of three values, d * -1, d * 0 and d * 1, so the
// thread computes those three once (with the same fp32 arithmetic, then the
// conversion to T) and each weight only selects one.  For 16-bit outputs two
// weights are done at once: their bytes sit in the two 16-bit halves of a
// register, packed 16-bit multiplies give digit = ((3^k * q) mod 256) * 3 >> 8
// ("Not applicable" section of the TQ1_0 page) for both, and one v_perm_b32
// picks each half's 2 output bytes out of the 6-byte table (-d, 0d, +d).

#ifndef QGEMV_TQ1_ROWS_U
#define QGEMV_TQ1_ROWS_U 8  // row-materialisation tasks per thread
#endif

struct Tq1RowIn {
  uint64_t bytes;
  unsigned short d;
};

template <typename T, int U>
__global__ __launch_bounds__(256) void tq1_rows_kernel(const uint8_t* __restrict__ w, int n, int nb,
                                                       const int32_t* __restrict__ rows, T* __restrict__ out,
                                                       int bpr) {
  constexpr int E = kRowsE<T>;
  const int j = blockIdx.x / bpr;
  const int r = source_row(rows, j, n);
  // the row's bytes (the row is the same for the whole workgroup)
  const auto wr = make_rsrc(w + (int64_t)(r < 0 ? 0 : r) * nb * kTq1Bytes, r < 0 ? 0u : (uint32_t)(nb * kTq1Bytes));
  T* const orow = out + (int64_t)j * nb * 256;
  auto pow3 = [](int k) { return pow3_u16(k); };
  rows_thread<U, Tq1RowIn>(
      bpr, nb * (256 / E), r >= 0,
      [&](int t) {
        const int e0 = t * E, e = e0 & 255;
        const uint32_t blk = (uint32_t)((e0 >> 8) * kTq1Bytes);
        // the run's qs bytes, or the qh dword (and the bytes after it, unused);
        // every lane issues the same loads, with no branch around them
        const uint32_t off = e < 160 ? (e & 31) : (e >= 240 ? 48 : 32 + ((e - 160) & 15));
        Tq1RowIn in;
        in.bytes = load_le_a2_dw<E>(wr, blk + off);
        in.d = ld16(wr, blk + 52);
        return in;
      },
      [&](int t, const Tq1RowIn& in) {
        const int e = (t * E) & 255;
        const bool qh = e >= 240;
        const int k0 = e < 160 ? (e >> 5) : (qh ? (e - 240) >> 2 : (e - 160) >> 4);
        const float d = (float)__builtin_bit_cast(_Float16, in.d);
        if constexpr (E == 8) {
          // the three possible outputs as 16-bit codes: table bytes 0-1, 2-3, 4-5
          const unsigned vm = pack2<T>(d * -1.f, d * 0.f);
          const unsigned vp = pack2<T>(d * 1.f, 0.f);
          unsigned res[4];
#pragma unroll
          for (int pr = 0; pr < 4; ++pr) {
            // elements 2pr, 2pr+1: bytes (2pr, 2pr+1) of the run, or of the qh dword
            const int b0 = qh ? (2 * pr) & 3 : 2 * pr;
            const unsigned short p = pow3(qh ? k0 + (pr >> 1) : k0);
            const unsigned word = (unsigned)(in.bytes >> (8 * (b0 & 4)));
            const unsigned pair =
                __builtin_amdgcn_perm(0u, word, 0x0C000C00u | (unsigned)(b0 & 3) | ((unsigned)((b0 & 3) + 1) << 16));
            const u16x2 dg = tq1_digits2(__builtin_bit_cast(u16x2, pair), p);
            const u16x2 sel = dg * u16x2{0x0202, 0x0202} + u16x2{0x0100, 0x0100};
            res[pr] = __builtin_amdgcn_perm(vp, vm, __builtin_bit_cast(unsigned, sel));
          }
          *reinterpret_cast<u32x4*>(orow + t * E) = u32x4{res[0], res[1], res[2], res[3]};
        } else {
          const float vals[3] = {d * -1.f, d * 0.f, d * 1.f};
          float v[E];
#pragma unroll
          for (int i = 0; i < E; ++i) {
            const int bi = qh ? (i & 3) : i;
            const unsigned q = (unsigned)(in.bytes >> (8 * bi)) & 0xFFu;
            const unsigned pq = (pow3(qh ? k0 + (i >> 2) : k0) * q) & 0xFFu;
            const unsigned digit = (3u * pq) >> 8;
            v[i] = digit == 0 ? vals[0] : digit == 1 ? vals[1] : vals[2];
          }
          store_e(orow + t * E, v);
        }
      },
      [&](int t) { store_e_nan(orow + t * E); });
}

template <int R, typename Out>
static hipError_t launch_tq1_r(const void* w, const void* x, const Out& y, int64_t n, int64_t k,
                               hipStream_t s) {
  const int nb = (int)(k / 256);
  const int kc = (nb + kTq1SegBlocks - 1) / kTq1SegBlocks;
  const int kw = kc < QGEMV_WG_WAVES ? kc : QGEMV_WG_WAVES;
  const int rg = kw >= QGEMV_WG_WAVES ? 1 : QGEMV_WG_WAVES / kw;
  const int rows_per_wg = rg * R;
  const int64_t grid = (n + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((tq1_gemv_kernel<R, Out>), dim3((unsigned)grid), dim3(64 * kw * rg), 0, s,
                     (const uint8_t*)w, (const uint16_t*)x, y, (int)n, nb, kc, kw, rg);
  return hipGetLastError();
}

template <int KS, int R, int W, typename Out>
static hipError_t launch_tq1_rows_r(const void* w, const void* x, const Out& y, int64_t n, int64_t k, hipStream_t s) {
  const int64_t rows_per_wg = (int64_t)W * R;
  const int64_t grid = (n + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((tq1_gemv_rows_kernel<KS, R, W, Out>), dim3((unsigned)grid), dim3(64 * W), 0, s,
                     (const uint8_t*)w, (const uint16_t*)x, y, (int)n, (int)(k / 256));
  return hipGetLastError();
}

template <int KS, typename Out>
static hipError_t launch_tq1_rows(const void* w, const void* x, const Out& y, int64_t n, int64_t k, hipStream_t s) {
  constexpr int kRmax = largest_fitting_r([](int r) {
    return 8 * ((r * KS * kTq1SegBytes + 1023) / 1024) * 1024 + KS * 8192 + 16 <= 160 * 1024;
  });
  return dispatch_rows<kRmax>(n, [&](auto rc, auto wc) {
    return launch_tq1_rows_r<KS, decltype(rc)::value, decltype(wc)::value, Out>(w, x, y, n, k, s);
  });
}

#ifndef QGEMV_TQ1_LREP
#define QGEMV_TQ1_LREP 16  // digit table copies when the stages leave room for 16, else 8
#endif

template <int KS, int R, int W, typename Out>
static hipError_t launch_tq1_table_r(const void* w, const void* x, const Out& y, int64_t n, int64_t k,
                                     hipStream_t s) {
  if (k != (int64_t)KS * 4096) return hipErrorInvalidValue;  // full 16-block segments only
  constexpr int kLrep = QGEMV_TQ1_LREP == 16 && tq1_table_lds(KS, R, W, 16) <= 160 * 1024 ? 16 : 8;
  static_assert(tq1_table_lds(KS, R, W, kLrep) <= 160 * 1024, "LDS per workgroup");
  const int64_t rows_per_wg = (int64_t)W * R;
  const int64_t grid = (n + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((tq1_gemv_table_kernel<KS, R, W, kLrep, Out>), dim3((unsigned)grid), dim3(64 * W), 0, s,
                     (const uint8_t*)w, (const uint16_t*)x, y, (int)n, (int)(k / 256));
  return hipGetLastError();
}

template <int KS, typename Out>
static hipError_t launch_tq1_table(const void* w, const void* x, const Out& y, int64_t n, int64_t k,
                                   hipStream_t s) {
  constexpr int kRmax = largest_fitting_r([](int r) { return tq1_table_lds(KS, r, 8, 8) <= 160 * 1024; });
  return dispatch_rows<kRmax>(n, [&](auto rc, auto wc) {
    return launch_tq1_table_r<KS, decltype(rc)::value, decltype(wc)::value, Out>(w, x, y, n, k, s);
  });
}

#ifndef QGEMV_TQ1_IMPL
#define QGEMV_TQ1_IMPL 2  // 1: K-split kernel only, 2: row-streaming for K % 2048 == 0, K <= 8192
                          // (table-driven for K = 4096 and more than 1024 rows)
#endif

template <typename Out>
static hipError_t launch_tq1_gemv_out(const void* w, const void* x, const Out& y, int64_t n, int64_t k,
                                      hipStream_t s) {
  if (QGEMV_TQ1_IMPL == 2 && k % 2048 == 0) {
    if (k <= 4096) {
      // K = 4096 over 1024 rows: the table-driven kernel; up to 1024 rows the
      // arithmetic kernel (one row per wave, four waves per workgroup) starts
      // faster than the table build pays off, and K = 2048 rows (half
      // segments) stay with it too
      if (k == 4096 && n > 1024) return launch_tq1_table<1, Out>(w, x, y, n, k, s);
      return launch_tq1_rows<1, Out>(w, x, y, n, k, s);
    }
    if (k <= 8192) return launch_tq1_rows<2, Out>(w, x, y, n, k, s);
  }
  return launch_tq1_r<QGEMV_TQ1_R, Out>(w, x, y, n, k, s);
}

hipError_t launch_tq1_gemv(const void* w, const void* x, const OutF32& y, int64_t n, int64_t k, hipStream_t s) {
  return launch_tq1_gemv_out(w, x, y, n, k, s);
}
hipError_t launch_tq1_gemv(const void* w, const void* x, const OutEx& y, int64_t n, int64_t k, hipStream_t s) {
  return launch_tq1_gemv_out(w, x, y, n, k, s);
}

template <typename T, int U>
static hipError_t launch_tq1_rows_u(const void* w, int64_t n, int64_t k, const int32_t* rows, int64_t nrows,
                                    void* out, hipStream_t s) {
  const RowsGeom g = rows_geom(k / kRowsE<T>, nrows, U);
  hipLaunchKernelGGL((tq1_rows_kernel<T, U>), dim3((unsigned)g.grid), dim3(g.block), 0, s, (const uint8_t*)w,
                     (int)n, (int)(k / 256), rows, (T*)out, g.bpr);
  return hipGetLastError();
}

// Small launches (a few hundred gathered rows) take one task per thread so
// that they still spread over the whole chip.
template <typename T>
static hipError_t launch_tq1_rows_t(const void* w, int64_t n, int64_t k, const int32_t* rows, int64_t nrows,
                                    void* out, hipStream_t s) {
  if (nrows * (k / kRowsE<T>) < kRowsSmallTasks) return launch_tq1_rows_u<T, 1>(w, n, k, rows, nrows, out, s);
  return launch_tq1_rows_u<T, QGEMV_TQ1_ROWS_U>(w, n, k, rows, nrows, out, s);
}

hipError_t launch_tq1_get_rows(const void* w, int64_t n, int64_t k, const int32_t* rows, int64_t nrows, void* out,
                               int dtype, hipStream_t s) {
  if (dtype == kF16) return launch_tq1_rows_t<_Float16>(w, n, k, rows, nrows, out, s);
  if (dtype == kBF16) return launch_tq1_rows_t<__bf16>(w, n, k, rows, nrows, out, s);
  return launch_tq1_rows_t<float>(w, n, k, rows, nrows, out, s);
}

}  // namespace qgemv
