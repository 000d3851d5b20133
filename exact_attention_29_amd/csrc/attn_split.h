// Split launches of the forward kernel: how the query tiles left after the
// whole rounds of workgroups are cut into ranges of (tile, 64-key tile)
// iterations, which pieces of which tiles a range holds, where their
// partial results go, and when a call is split at all.  Integer arithmetic
// only, usable on the host (launch planning, and a host-side check of the
// decomposition) and on the device.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace attn_detail {

// A split partial: per wave, 8 chunks x 64 lanes of 4 floats (the O^T
// accumulators) and 64 lanes of (m, l).
constexpr int kSplitAccFloats = 8 * 8 * 64 * 4;
constexpr int kSplitSlotFloats = kSplitAccFloats + 8 * 64 * 2;

// One piece of work of a split launch: key tiles [kt_a, kt_b) of query tile
// `logical`; `parts` pieces cover that tile (1: the whole tile, no merge),
// this is piece `part`; slot_first / ord0 locate the partial slots of the
// tile's pieces, `counter` its arrival counter.
struct Piece {
  int logical, kt_a, kt_b, parts, part, slot_first, ord0, counter;
};

// The leftover of a split launch.  XCD x (the hardware deals workgroups to
// the 8 XCDs in turn, and xcd_remap gives XCD x the logical tiles [start,
// start + cnt)) owns the rem = cnt - R*C tiles past its R = sk_rounds whole
// rounds of C = sk_cus: rem * n_kt (tile, key tile) iterations, cut into C
// contiguous ranges of equal length (within one), one per workgroup: range
// jj, id 8*jj + x, is workgroup dp_blocks + id, which lands on XCD x.  The
// range [it0, it1) is at most n_kt long (rem < C), so it touches one or two
// tiles: `count` pieces, the first in tile it0 / n_kt, done one after the
// other by the same workgroup (so every CU of the last round gets about
// rem * n_kt / C key tiles, whichever order the hardware starts them in).
// Piece slots: range jj's pieces use slots 2*(x*C + jj) + 0 and + 1.  (All
// products stay below 2^31: the host splits only when C * C * n_kt does.)
struct SplitRange {
  int x, jj, c, start, base;
  unsigned nkt, len, it0, it1;
  int count;
};

// Args: anything with total_tiles, sk_rounds, sk_cus and n_kt.
template <class Args>
__host__ __device__ inline SplitRange split_range(const Args& a, int id) {
  SplitRange r;
  r.c = a.sk_cus;
  r.x = id & 7;
  r.jj = id >> 3;
  const int per = a.total_tiles >> 3, r8 = a.total_tiles & 7;
  const int cnt = per + (r.x < r8 ? 1 : 0);
  r.start = r.x * per + (r.x < r8 ? r.x : r8);
  r.base = a.sk_rounds * r.c;
  r.nkt = (unsigned)a.n_kt;
  r.len = (unsigned)(cnt - r.base) * r.nkt;
  r.it0 = (unsigned)r.jj * r.len / (unsigned)r.c;
  r.it1 = (unsigned)(r.jj + 1) * r.len / (unsigned)r.c;
  r.count = 0;
  if (r.it1 > r.it0) r.count = (r.it1 - 1) / r.nkt == r.it0 / r.nkt ? 1 : 2;
  return r;
}

// Piece pc (0 or 1) of range r.
__host__ __device__ inline Piece split_piece(const SplitRange& r, int pc) {
  const unsigned nkt = r.nkt, c = (unsigned)r.c;
  const unsigned s = r.it0 / nkt + (unsigned)pc;  // the tile, local to the XCD's leftover
  const unsigned lo = r.it0 > s * nkt ? r.it0 : s * nkt;
  const unsigned hi = r.it1 < (s + 1) * nkt ? r.it1 : (s + 1) * nkt;
  // the range that holds iteration q: the largest j with
  // floor(j * len / C) <= q, i.e. ((q + 1) * C - 1) / len
  const int first = (int)(((s * nkt + 1) * c - 1) / r.len);
  const int last = (int)(((s + 1) * nkt * c - 1) / r.len);
  Piece p;
  p.logical = r.start + r.base + (int)s;
  p.kt_a = (int)(lo - s * nkt);
  p.kt_b = (int)(hi - s * nkt);
  p.parts = last - first + 1;
  p.part = r.jj - first;
  p.slot_first = 2 * (r.x * r.c + first);
  p.ord0 = (unsigned)first * r.len / c < s * nkt ? 1 : 0;  // the tile is the second of `first`'s range
  p.counter = r.x * r.c + (int)s;
  return p;
}

// Workspace of a split launch on a device with `cus` compute units: the
// arrival counters (one per query tile a round can leave over: 8 * C ints,
// C = cus / 8 workgroups per XCD, padded to 256 bytes), then two partial
// slots per range of the last round.
__host__ __device__ inline int split_cus_per_xcd(int cus) { return cus >= 16 ? cus / 8 : 1; }
__host__ __device__ inline size_t split_count_bytes(int cus) {
  return ((size_t)8 * split_cus_per_xcd(cus) * sizeof(int) + 255) / 256 * 256;
}
__host__ __device__ inline size_t split_workspace_bytes(int cus) {
  return split_count_bytes(cus) + (size_t)2 * 8 * split_cus_per_xcd(cus) * kSplitSlotFloats * sizeof(float);
}

// Whether a non-causal dense call splits its last round, and how.  T query
// tiles of 256 rows go to the 8 XCDs in contiguous blocks of T/8 (+1 for
// the first T%8); an XCD runs C at a time.  After R = floor((T/8) / C)
// whole rounds, XCD x has rem_x tiles left.  `valid`: the decomposition
// applies (no XCD's leftover is a whole round, rem_x < C; some leftover;
// every leftover tile has at least C key tiles, so each range is at least
// one key tile long; C * C * n_kt < 2^31 for the device's 32-bit range
// arithmetic; C <= 64, i.e. up to 512 CUs and a workspace of at most 72 MB).
// `on`: valid and worth it --
//   * the leftover fills at most half of a round (sum rem_x <= 4C).  The
//     part is power-limited: with a few CUs idle the busy ones clock higher
//     and make up most of the idle time, so a nearly full last round (3 MP
//     patches at 16 heads: 7/8) gains nothing from the split, while a
//     mostly empty one (1/8 .. 3/8) gains 20-60% of its time;
//   * there is a whole round before it, or the rows are long (at least 160
//     key tiles): with no whole round the plain launch uses 4-wave
//     workgroups, which already spread short rows over every CU.
struct SplitPlan {
  bool on, valid;
  int rounds, cus_per_xcd;
};
__host__ __device__ inline SplitPlan plan_split(long long tiles, int n_kt, int cus) {
  SplitPlan p = {false, false, 0, split_cus_per_xcd(cus)};
  const int c = p.cus_per_xcd;
  const long long per = tiles / 8;
  const long long r8 = tiles % 8;
  p.rounds = (int)(per / c);
  const long long rem_max = per + (r8 ? 1 : 0) - (long long)p.rounds * c;
  const long long left = tiles - 8LL * p.rounds * c;  // leftover tiles, all XCDs
  p.valid = rem_max > 0 && rem_max < c && n_kt >= c && (long long)c * c * n_kt < (1LL << 31) && c <= 64;
  p.on = p.valid && 2 * left <= 8LL * c && (p.rounds >= 1 || n_kt >= 160);
  return p;
}

}  // namespace attn_detail
