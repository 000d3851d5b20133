// Host-side check of the split decomposition in attn_split.h (no GPU
// needed; only host code runs).
//
//   split_plan_check            check every valid plan over a grid of tile
//                               counts, key-tile counts and CU counts:
//                               whole-round tiles and leftover pieces cover
//                               every (query tile, key tile) exactly once;
//                               each leftover tile's pieces are numbered
//                               0 .. parts-1, share one arrival counter and
//                               no other tile's; every piece's slot is the
//                               slot its range writes and no two pieces share
//                               one; prints "ok <plans checked>"
//   split_plan_check B H N CUS  print the plan of a B x H x N call on CUS
//                               compute units: "<on> <rounds> <C>"
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <utility>
#include <vector>

#include "attn_common.h"
#include "attn_split.h"

using namespace attn_detail;

struct Args {
  int total_tiles, sk_rounds, sk_cus, n_kt;
};

static int fail(const char* what, long long t, int nkt, int cus) {
  std::printf("FAIL %s: tiles=%lld n_kt=%d cus=%d\n", what, t, nkt, cus);
  return 1;
}

static int check(int tiles, int nkt, int cus, const SplitPlan& p) {
  const int c = p.cus_per_xcd;
  const Args a = {tiles, p.rounds, c, nkt};
  std::vector<char> whole(tiles, 0);
  for (int w = 0; w < 8 * p.rounds * c; ++w) {
    const int t = xcd_remap(w, tiles);
    if (t < 0 || t >= tiles || whole[t]) return fail("whole-round tiles", tiles, nkt, cus);
    whole[t] = 1;
  }
  std::map<int, std::vector<std::pair<int, int>>> spans;  // tile -> (kt_a, kt_b)
  std::map<int, std::set<int>> parts_seen;
  std::map<int, std::pair<int, int>> tile_info;  // tile -> (parts, counter)
  std::set<int> slots, counters;
  for (int id = 0; id < 8 * c; ++id) {
    const SplitRange r = split_range(a, id);
    if (r.count < 0 || r.count > 2) return fail("piece count", tiles, nkt, cus);
    for (int pc = 0; pc < r.count; ++pc) {
      const Piece q = split_piece(r, pc);
      if (q.logical < 0 || q.logical >= tiles || whole[q.logical]) return fail("piece tile", tiles, nkt, cus);
      if (!(0 <= q.kt_a && q.kt_a < q.kt_b && q.kt_b <= nkt)) return fail("key range", tiles, nkt, cus);
      if (q.parts < 1 || q.part < 0 || q.part >= q.parts) return fail("part index", tiles, nkt, cus);
      const int own = 2 * (r.x * c + r.jj) + pc;
      const int named = q.slot_first + 2 * q.part + (q.part == 0 ? q.ord0 : 0);
      if (own != named || own < 0 || own >= 16 * c || !slots.insert(own).second)
        return fail("slot", tiles, nkt, cus);
      if (q.counter < 0 || q.counter >= 8 * c) return fail("counter range", tiles, nkt, cus);
      auto it = tile_info.find(q.logical);
      if (it == tile_info.end()) {
        if (!counters.insert(q.counter).second) return fail("counter shared", tiles, nkt, cus);
        tile_info[q.logical] = {q.parts, q.counter};
      } else if (it->second != std::make_pair(q.parts, q.counter)) {
        return fail("parts/counter of a tile", tiles, nkt, cus);
      }
      if (!parts_seen[q.logical].insert(q.part).second) return fail("part twice", tiles, nkt, cus);
      spans[q.logical].push_back({q.kt_a, q.kt_b});
    }
  }
  for (int t = 0; t < tiles; ++t) {
    if (whole[t]) {
      if (spans.count(t)) return fail("whole tile also split", tiles, nkt, cus);
      continue;
    }
    auto it = spans.find(t);
    if (it == spans.end()) return fail("tile not covered", tiles, nkt, cus);
    std::vector<std::pair<int, int>> v = it->second;
    std::sort(v.begin(), v.end());
    int at = 0;
    for (auto& s : v) {
      if (s.first != at) return fail("key tiles not covered exactly once", tiles, nkt, cus);
      at = s.second;
    }
    if (at != nkt) return fail("key tiles short", tiles, nkt, cus);
    if ((int)parts_seen[t].size() != tile_info[t].first) return fail("parts missing", tiles, nkt, cus);
  }
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 5) {
    const long long B = std::atoll(argv[1]), H = std::atoll(argv[2]), N = std::atoll(argv[3]);
    const int cus = std::atoi(argv[4]);
    const SplitPlan p = plan_split(B * H * ((N + 255) / 256), (int)((N + 63) / 64), cus);
    std::printf("%d %d %d\n", p.on ? 1 : 0, p.rounds, p.cus_per_xcd);
    return 0;
  }
  const int cus_list[] = {256, 304, 228, 80, 64, 16, 8};
  const int nkt_list[] = {1, 2, 8, 31, 32, 33, 36, 44, 47, 64, 100, 160, 161, 182, 188, 600, 4096};
  long long checked = 0;
  for (int cus : cus_list)
    for (int nkt : nkt_list)
      for (int tiles = 1; tiles <= 1300; ++tiles) {
        const SplitPlan p = plan_split(tiles, nkt, cus);
        if (!p.valid) continue;
        if (check(tiles, nkt, cus, p)) return 1;
        ++checked;
      }
  std::printf("ok %lld\n", checked);
  return 0;
}
