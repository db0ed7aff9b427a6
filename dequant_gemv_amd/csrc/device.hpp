// Device helpers shared by the gfx950 kernels: range-checked buffer loads,
// packed-type aliases and wave64 reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qgemv {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int kWave = 64;

// Raw buffer descriptor over [base, base + bytes).  Loads whose byte range
// falls outside it return zero instead of touching memory, so ragged tails
// (last rows, last K-chunk) need no address clamping.  Offsets are 32-bit, so
// callers rebase `base` per workgroup and keep `bytes` below 2^31.
// Callers pass wave-uniform values; readfirstlane makes that explicit so the
// descriptor lives in SGPRs (a descriptor the compiler thinks divergent turns
// every load into a per-lane waterfall loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ u32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Cache policy of the read-once weight stream (buffer-load aux bits; on
// gfx950 bit 1 is the non-temporal hint).
#ifndef QGEMV_WLOAD_AUX
#define QGEMV_WLOAD_AUX 2  // nt: the weights are read once
#endif
__device__ __forceinline__ u32x4 ld128w(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, QGEMV_WLOAD_AUX);
}
__device__ __forceinline__ unsigned ld32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ unsigned short ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
// The same with a wave-uniform part of the offset in an SGPR (soff): the
// range check covers voff + soff, which must not exceed 2^32.
__device__ __forceinline__ u32x4 ld128s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)__builtin_amdgcn_readfirstlane(soff), 0);
}
__device__ __forceinline__ unsigned ld32s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)__builtin_amdgcn_readfirstlane(soff), 0);
}
__device__ __forceinline__ unsigned short ld16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)__builtin_amdgcn_readfirstlane(soff), 0);
}
__device__ __forceinline__ unsigned char ld8s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)__builtin_amdgcn_readfirstlane(soff), 0);
}
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
__device__ __forceinline__ u32x2 ld64s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)__builtin_amdgcn_readfirstlane(soff), 0);
}

__device__ __forceinline__ f16x2 as_h2(unsigned v) { return __builtin_bit_cast(f16x2, v); }

// Pins an fp32 value in a register, so that a following conversion to a
// 16-bit type rounds exactly this fp32 value.  Without it the compiler fuses
// the multiply or fma that produced the value with the conversion into one
// mixed-precision fma (v_fma_mixlo_f16): that rounds once from the exact
// result instead of twice, and a product fused with a +0 addend turns -0
// into +0.
__device__ __forceinline__ float pin_f32(float v) {
  __asm__("" : "+v"(v));
  return v;
}

// Makes v computed at this point of the program: a volatile asm keeps its
// place among the other volatile asm statements (the memory fences and
// counted waits), so arithmetic feeding v cannot sink past the next wait.
__device__ __forceinline__ void settle(float& v) { __asm__ __volatile__("" : "+v"(v)); }
__device__ __forceinline__ void settle(unsigned& v) { __asm__ __volatile__("" : "+v"(v)); }

// v_dot2_f32_f16: a.x*b.x + a.y*b.y + c with fp32 accumulation.
__device__ __forceinline__ float dot2h(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}
// v_dot2_f32_bf16
__device__ __forceinline__ float dot2bf(bf16x2 a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b), c, false);
}

// Two E2M1 codes (byte `sel` of v, low nibble first) -> exact bf16 / fp32 pair.
// The selector must be an immediate; the switch folds once `sel` is a constant.
__device__ __forceinline__ bf16x2 fp4x2_bf16(unsigned v, int sel) {
  switch (sel & 3) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 3);
  }
}
__device__ __forceinline__ f32x2 fp4x2_f32(unsigned v, int sel) {
  switch (sel & 3) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 3);
  }
}

// s_waitcnt vmcnt(n) for 0 <= n <= 15 (other counters untouched); the
// switch folds once n is a constant.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
  }
}

__device__ __forceinline__ float f16lo(unsigned v) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(v & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(unsigned v) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(v >> 16));
}

__device__ __forceinline__ float shfl_xor(float v, int m) {
  int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __builtin_bit_cast(int, v)));
}

// Reduce R (a power of two <= 64) per-lane partials across the 64 lanes of a
// wave.  Each halving step exchanges half of the values with the partner lane,
// so the whole reduction costs about R + log2(64/R) exchanges instead of
// 6 R.  On return v[0] of lane l holds the total of row l >> (6 - log2 R).
template <int R, int CNT = R, int S = 32>
__device__ __forceinline__ void wave_reduce_rows(float (&v)[R]) {
  static_assert(R >= 1 && R <= 64 && (R & (R - 1)) == 0, "R must be a power of two <= 64");
  if constexpr (CNT > 1) {
    constexpr int H = CNT / 2;
    const bool up = (__lane_id() & S) != 0;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      float send = up ? v[i] : v[i + H];
      float keep = up ? v[i + H] : v[i];
      v[i] = keep + shfl_xor(send, S);
    }
    wave_reduce_rows<R, H, S / 2>(v);
  } else if constexpr (S >= 1) {
    v[0] += shfl_xor(v[0], S);
    wave_reduce_rows<R, 1, S / 2>(v);
  }
}


// s_waitcnt vmcnt(N) for a compile-time 0 <= N <= 63 (gfx9 encoding: vmcnt
// bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima, i.e. no wait).
// Compiler-only memory fence (emits nothing): no load, store or LDS access
// is moved across it.  The kernels count their own loads for the vmcnt
// waits, which is only sound if loads are issued, and waits placed, exactly
// in source order; the compiler otherwise treats independent buffer loads
// (and loads around a wait) as free to reorder.
__device__ __forceinline__ void compiler_fence() { __asm__ __volatile__("" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  compiler_fence();
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  compiler_fence();
}

// Workgroup barrier that waits only for this wave's LDS accesses (lgkmcnt),
// not for its outstanding global loads: __syncthreads() also waits vmcnt(0),
// which would drain loads issued for later pipeline stages.
__device__ __forceinline__ void lds_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// Base-3 digit of two bytes at once (the 16-bit halves of q): digit k of a
// TQ1_0 byte b is ((3^k b) mod 256) * 3 >> 8 ("metal: TQ1_0 kernel
// performance", section "Not applicable"); p = 3^k.
__device__ __forceinline__ u16x2 tq1_digits2(u16x2 q, unsigned short p) {
  const u16x2 m = (q * u16x2{p, p}) & u16x2{0xFF, 0xFF};
  return (m * u16x2{3, 3}) >> u16x2{8, 8};
}

// 3^k for k = 0..4 without branches: 1, 3, 9, 27 are the bytes of one word.
__device__ __forceinline__ unsigned short pow3_u16(int k) {
  const unsigned lo = (0x1B090301u >> (8 * (k & 3))) & 0xFFu;
  return (unsigned short)(k >= 4 ? 81u : lo);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One wave-wide 16-byte-per-lane buffer load straight into LDS: lane i's
// bytes [voff, voff+16) of the descriptor land at lds + 16*i (the LDS base is
// wave-uniform).  Bytes outside the descriptor's range land as zeros.
// Completion is counted by vmcnt like any other buffer load.
template <int AUX = 0>
__device__ __forceinline__ void ld128_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, 0, 0, AUX);
}
// The same with a wave-uniform part of the offset in an SGPR (see ld128s).
__device__ __forceinline__ void ld128_lds_s(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, (int)__builtin_amdgcn_readfirstlane(soff), 0,
                                           0);
}

// Compile-time loop: calls f(Int<I>{}) for I = B .. E-1, so the body can use
// its index in constant expressions (wait counts, register array indices).
template <int V>
struct Int {
  static constexpr int value = V;
};
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(Int<B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ float dpp_ror8(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_ror4(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {  // quad_perm [2,3,0,1]
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor1(float v) {  // quad_perm [1,0,3,2]
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ float dpp_bcast15(float v) {  // rows 1, 3 read lane 15 of the row before
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
}
__device__ __forceinline__ float dpp_bcast31(float v) {  // rows 2, 3 read lane 31
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
}

// Sum each of R per-lane values over the 64 lanes of the wave with DPP only
// (no LDS round trip): rotations and quad permutes sum each 16-lane row into
// all of its lanes, then two row broadcasts carry rows 0-2 into row 3.  On
// return lanes 48-63 hold every total; the other lanes hold partial sums.
template <int R>
__device__ __forceinline__ void wave_reduce_dpp(float (&v)[R]) {
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float t = v[i];
    t += dpp_ror8(t);
    t += dpp_ror4(t);
    t += dpp_xor2(t);
    t += dpp_xor1(t);
    t += dpp_bcast15(t);
    t += dpp_bcast31(t);
    v[i] = t;
  }
}

template <int R>
__device__ __forceinline__ constexpr int log2i() {
  return R <= 1 ? 0 : 1 + log2i<R / 2>();
}

}  // namespace qgemv
