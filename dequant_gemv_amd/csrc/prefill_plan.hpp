// The launch plan of a prefill (many activation rows, matrix cores): tile
// shape, K split and the workspace the splits need.  Plain host code, shared
// by the launcher and by the C ABI's argument validation.
#pragma once
#include <stdint.h>

#include <algorithm>

namespace qgemv {

constexpr int kPfBN = 128;    // weight rows per workgroup tile
constexpr int kPfKS = 64;     // weights per K step
constexpr int kPfUnroll = 6;  // steps per loop iteration (a multiple of XS, 2 and kPfWQ): indices are compile-time

// The launch a T x N x K prefill takes: tile size, K split of every tile
// (split > 1) or of the last round's tiles (tail_split > 1), and the fp32
// partial tiles a workspace for the splits holds.
struct PfPlan {
  int bt;
  int64_t row_tiles, tiles, steps;
  int64_t split, split_steps;
  int64_t n_full, tail, tail_split, tail_steps;
  int64_t part_floats;
};

inline PfPlan prefill_plan(int64_t t, int64_t n, int64_t k) {
  PfPlan p{};
  p.bt = 256;
  p.split = p.tail_split = 1;
  if (t <= 0 || n <= 0 || k < kPfKS) return p;  // nothing to launch
  // 512-token tiles decode each weight half as often and feed more MFMAs per
  // fragment read, but one takes about 1.7 times as long as a 256-token tile
  // (measured): they are used when they fill at least two rounds of
  // workgroups, or when 256-token tiles need more than one round and the
  // 512-token rounds take fewer tile-times (1024 tokens x 14336 rows: one
  // round of 224 tiles, against two rounds of 448)
  p.row_tiles = (n + kPfBN - 1) / kPfBN;
  const int64_t tiles512 = p.row_tiles * ((t + 511) / 512), tiles256 = p.row_tiles * ((t + 255) / 256);
  const bool use512 =
      tiles512 >= 512 || (tiles256 > 256 && 17 * ((tiles512 + 255) / 256) < 10 * ((tiles256 + 255) / 256));
  p.bt = use512 ? 512 : 256;
  p.tiles = p.row_tiles * ((t + p.bt - 1) / p.bt);
  p.steps = k / kPfKS;
  int64_t split = 1;
  if (p.tiles < 256) split = std::max(int64_t(1), 256 / p.tiles);  // fewer tiles than CUs
  split = std::min(split, std::max(int64_t(1), p.steps / 8));
  split = std::min(split, int64_t(16));
  // a whole number of loop iterations per split (only the last split ends
  // early): a step past the end skips its arithmetic but still waits for the
  // loads in flight, and measured nearly as slow as a full one
  p.split_steps = ((p.steps + split - 1) / split + kPfUnroll - 1) / kPfUnroll * kPfUnroll;
  p.split = (p.steps + p.split_steps - 1) / p.split_steps;
  p.tail_split = 1;
  if (p.split > 1) {
    p.part_floats = p.tiles * p.split * p.bt * kPfBN;
  } else if (p.bt == 512 && p.tiles % 256 != 0 && p.tiles % 256 <= 64 && p.tiles < (int64_t(1) << 28) &&
             n < (int64_t(1) << 24)) {
    // the last round would be at most a quarter full: split its tiles over K
    // so that it takes about 1 / tail_split of a round.  (A half-full last
    // round is left alone: splitting it measured 2 % slower at 4096 tokens x
    // 14336 rows, the clock of the power-limited chip being higher while
    // half of it idles, and the clear and atomics costing extra.)
    // (the one-dimensional grid and the clear stay well inside 32-bit counts)
    p.tail = p.tiles % 256;
    p.n_full = p.tiles - p.tail;
    int64_t tail_split = std::min(256 / p.tail, int64_t(4));
    tail_split = std::min(tail_split, std::max(int64_t(1), p.steps / 12));
    p.tail_steps = ((p.steps + tail_split - 1) / tail_split + kPfUnroll - 1) / kPfUnroll * kPfUnroll;
    p.tail_split = (p.steps + p.tail_steps - 1) / p.tail_steps;
    if (p.tail_split > 1) p.part_floats = p.tail * p.tail_split * 512 * kPfBN;
  }
  return p;
}

inline int64_t prefill_workspace_bytes(int64_t t, int64_t n, int64_t k) {
  const PfPlan p = prefill_plan(t, n, k);
  return 4 * p.part_floats;
}

}  // namespace qgemv
