// Row-streaming skeleton shared by the GEMV kernels: a wave owns whole rows,
// their bytes are one contiguous run streamed into the wave's LDS stage with
// 1 KiB buffer loads (lane i of a load fetches bytes 16i..16i+15 of that KiB),
// the loads are issued on a compile-time schedule that keeps a bounded number
// in flight ahead of the unit being consumed, and the finished row partials
// are summed across the wave with DPP and stored by lanes 48.. .
#pragma once
#include "device.hpp"
#include "epilogue.hpp"

namespace qgemv {

// Schedule of a stream of UNITS units of UNIT_BYTES consecutive bytes (unit u
// covers bytes [u*UNIT_BYTES, (u+1)*UNIT_BYTES) of the run).  AHEAD0 loads are
// issued up front (before the kernel's activation barrier), FIRST - AHEAD0
// more right after it (they keep the memory pipe fed while the activations
// are unpacked), and after unit u enough to stay AHEAD loads past the last
// load unit u depends on.  A CU's memory pipeline holds a bounded number of
// requests and a wave issuing past that stalls at the load, holding back its
// own arithmetic (and the barrier): hence the bounds.
//
// With RING > 0 the stage is a ring of RING one-KiB slots (load i lands in
// slot i % RING) instead of the whole run; a unit's 16-byte granules never
// straddle the ring's end (units and slots are multiples of 16 bytes).  The
// ring must hold every load issued while a unit's bytes are still unread:
// the refill after unit u's wait reaches load issued_before(u + 1) - 1, unit
// u starts at load first_load(u).
template <int UNIT_BYTES, int UNITS, int AHEAD0, int AHEAD, int FIRST = AHEAD0, int RING = 0>
struct StreamSchedule {
  static constexpr int kLoads = (UNITS * UNIT_BYTES + 1023) / 1024;
  static constexpr int kRing = RING > 0 && RING < kLoads ? RING : kLoads;  // slots
  static constexpr int kStage = kRing * 1024;
  static_assert(AHEAD >= (UNIT_BYTES + 1023) / 1024 + 1, "lookahead below one unit's loads");
  static_assert(AHEAD0 >= 1 && FIRST >= AHEAD0 && FIRST < 60 && AHEAD < 60, "vmcnt holds at most 63 outstanding loads");
  static constexpr int kUpFront = AHEAD0 < kLoads ? AHEAD0 : kLoads;  // issued before the barrier
  static constexpr int last_load(int u) { return (u * UNIT_BYTES + UNIT_BYTES - 1) / 1024; }
  static constexpr int issued_before(int u) {
    int n = FIRST < kLoads ? FIRST : kLoads;
    for (int v = 0; v < u; ++v) {
      const int t = last_load(v) + 1 + AHEAD;
      n = t > n ? (t < kLoads ? t : kLoads) : n;
    }
    return n;
  }
  // vmcnt to wait for before consuming unit u (loads complete in issue order)
  static constexpr int wait_count(int u) { return issued_before(u) - 1 - last_load(u); }
  static constexpr int first_load(int u) { return u * UNIT_BYTES / 1024; }
  static constexpr bool ring_holds() {
    if (issued_before(0) > kRing) return false;
    for (int u = 0; u < UNITS; ++u)
      if (issued_before(u + 1) - 1 - first_load(u) >= kRing) return false;
    return true;
  }
  static_assert(ring_holds(), "the ring would overwrite bytes not yet read");
  // LDS offset in the stage of byte b of the run
  static constexpr int slot_offset(int b) { return b % kStage; }
};

// Issue loads [B, E) of a stream whose LDS stage starts at `stage` (a ring
// of SLOTS one-KiB slots when the run is longer).
// The group stays between the memory accesses before and after it (the
// counted waits depend on the issue order of groups).
template <int B, int E, int AUX, int SLOTS = (1 << 30)>
__device__ __forceinline__ void stream_loads(__amdgpu_buffer_rsrc_t r, unsigned char* stage, int lane) {
  compiler_fence();
  static_for<B, E>([&](auto i) {
    constexpr int I = decltype(i)::value;
    ld128_lds<AUX>(r, stage + (I % SLOTS) * 1024, (uint32_t)(I * 1024 + 16 * lane));
  });
  compiler_fence();
}

// The workgroup's copy of the activations: PIECES one-KiB pieces dealt to the
// W waves in turn; lane i of piece P fetches the 16-byte granule src(P, i)
// (a permutation inside the piece, e.g. a bank swizzle) and stores it at
// dst + 1024 P + 16 i.  Returns nothing; completion is counted by vmcnt.
template <int PIECES, int W, typename SrcFn>
__device__ __forceinline__ void load_shared_pieces(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int wave, int lane,
                                                   SrcFn src) {
  constexpr int kPer = (PIECES + W - 1) / W;
  compiler_fence();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int piece = i * W + wave;
    if (piece < PIECES) ld128_lds(r, dst + piece * 1024, src(piece, lane));
  }
  compiler_fence();
}

// What the output stage reads for the wave's rows, fetched early: lane
// 48 + j fetches for row row0 + j (j < nrows).  Loads complete in issue
// order, so the stream's vmcnt waits stay valid wherever this load sits: it
// is either older than the load being waited for, or one more load after it
// (the wait is then only stricter).
template <typename Out>
__device__ __forceinline__ typename Out::Pre prefetch_rows(const Out& out, int row0, int nrows, int lane) {
  compiler_fence();
  const auto p = out.prefetch(row0, lane & 15, lane >= 48 && (lane & 15) < nrows);
  compiler_fence();
  return p;
}

// Sum R per-lane row partials across the wave and hand row j (< nrows),
// times `scale`, to the output stage as row row0 + j from lane 48 + j.
template <int R, typename Out>
__device__ __forceinline__ void store_rows(float (&acc)[R], const Out& out, typename Out::Pre pre, int row0,
                                           int nrows, float scale, int lane) {
  static_assert(R >= 1 && R <= 16, "one row per lane of the last 16-lane row");
  wave_reduce_dpp<R>(acc);
  const int j = lane & 15;
  float t = acc[0];
#pragma unroll
  for (int s = 1; s < R; ++s) t = j == s ? acc[s] : t;
  if (lane >= 48 && j < nrows) out.put(row0 + j, t * scale, pre);
}

// Shape -> (R rows per wave, W waves per workgroup) of a row-streaming
// kernel: up to 1024 rows one row per wave and 4 waves per workgroup (up to
// one wave per SIMD); beyond, 8 waves (two per SIMD, so one wave's LDS
// latency hides behind the other's arithmetic) and R = ceil(N / 2048), i.e.
// about 256 workgroups that all run at once (R = 1 to 8, 10, 12, 14 or 16,
// the smallest that covers N in one round: a 6144-row matrix takes R = 3,
// not 4, which would leave a quarter of the CUs idle); past what RMAX (the largest R
// whose stage fits LDS at 8 waves) allows, R = min(4, RMAX) so that two
// workgroups can share a CU and one's loads overlap the other's tail.
// `launch(Int<R>{}, Int<W>{})` launches the instantiation.
template <int RMAX, typename Launch>
hipError_t dispatch_rows(int64_t n, Launch&& launch) {
  static_assert(RMAX >= 1, "no configuration fits");
  if (n <= 1024) return launch(Int<1>{}, Int<4>{});
  const int64_t r8 = (n + 2047) / 2048;
  if (RMAX < 2 || r8 <= 1) return launch(Int<1>{}, Int<8>{});
  if constexpr (RMAX >= 2) {
    if (RMAX < 3 || r8 <= 2) return launch(Int<2>{}, Int<8>{});
  }
  if constexpr (RMAX >= 3) {
    if (RMAX < 4 || r8 <= 3) return launch(Int<3>{}, Int<8>{});
  }
  if constexpr (RMAX >= 4) {
    if (RMAX < 5 || r8 <= 4) return launch(Int<4>{}, Int<8>{});
  }
  if constexpr (RMAX >= 5) {
    if (RMAX < 6 || r8 <= 5) return launch(Int<5>{}, Int<8>{});
  }
  if constexpr (RMAX >= 6) {
    if (RMAX < 7 || r8 <= 6) return launch(Int<6>{}, Int<8>{});
  }
  if constexpr (RMAX >= 7) {
    if (r8 <= 7) return launch(Int<7>{}, Int<8>{});
  }
  if constexpr (RMAX >= 8) {
    if (r8 <= 8) return launch(Int<8>{}, Int<8>{});
  }
  // still one round when the stages allow it (TQ1_0 rows are short: gate and
  // up of Llama-8B as one 28672-row matrix take 14 rows per wave)
  if constexpr (RMAX >= 10) {
    if (r8 <= 10) return launch(Int<10>{}, Int<8>{});
  }
  if constexpr (RMAX >= 12) {
    if (r8 <= 12) return launch(Int<12>{}, Int<8>{});
  }
  if constexpr (RMAX >= 14) {
    if (r8 <= 14) return launch(Int<14>{}, Int<8>{});
  }
  if constexpr (RMAX >= 16) {
    if (r8 <= 16) return launch(Int<16>{}, Int<8>{});
  }
  return launch(Int<(RMAX >= 4 ? 4 : RMAX >= 2 ? 2 : 1)>{}, Int<8>{});
}

// Largest R <= 16 for which FITS(R) holds (FITS: a constexpr predicate).
template <typename Fits>
constexpr int largest_fitting_r(Fits fits) {
  int best = 0;
  for (int r = 1; r <= 16; ++r)
    if (fits(r)) best = r;
  return best;
}

}  // namespace qgemv
