// Host check of the prefill score kernel's tile enumeration (prefill_grid / prefill_tile in
// clsa_internal.h): for calls starting at many positions pos0 with many row counts, the tiles
// 0 .. tiles-1 map to distinct (row block, column block) pairs, and those pairs are exactly the
// 128 x 128 tiles that hold a visible entry (some row i of the block sees column j: j <= pos0 + i).
#include <cstdio>
#include <set>
#include <utility>

#include "../../cross_layer_token_amd/csrc/clsa_internal.h"

int main() {
  using clsa::kPfTile;
  const int pos0s[] = {0, 1, 50, 127, 128, 129, 3000, 8191, 65536, 100003};
  const int rows[] = {1, 2, 127, 128, 129, 200, 255, 256, 257, 1000, 1024, 4097, 8192};
  long checked = 0;
  for (int pos0 : pos0s)
    for (int n : rows) {
      const clsa::PrefillGrid g = clsa::prefill_grid(pos0, n);
      std::set<std::pair<int, int>> seen;
      for (int64_t t = 0; t < g.tiles; ++t) {
        int rb, cb;
        clsa::prefill_tile(g, t, &rb, &cb);
        const int last_row = (rb + 1) * kPfTile - 1 < n - 1 ? (rb + 1) * kPfTile - 1 : n - 1;
        if (rb < 0 || rb > g.last_rb || cb < 0 || (int64_t)cb * kPfTile > pos0 + last_row ||
            !seen.insert({rb, cb}).second) {
          std::printf("pos0=%d n=%d tile %lld -> (%d, %d) invalid or repeated\n", pos0, n, (long long)t, rb, cb);
          return 1;
        }
      }
      int64_t want = 0;  // every causal tile
      for (int rb = 0; rb * kPfTile < n; ++rb) {
        const int last_row = (rb + 1) * kPfTile - 1 < n - 1 ? (rb + 1) * kPfTile - 1 : n - 1;
        want += (pos0 + last_row) / kPfTile + 1;
      }
      if (want != g.tiles || (int64_t)seen.size() != want) {
        std::printf("pos0=%d n=%d: %lld tiles, want %lld\n", pos0, n, (long long)g.tiles, (long long)want);
        return 1;
      }
      checked += g.tiles;
    }
  // a large call: spot-check the mapping's ends (2^24 rows of 128-row blocks)
  const clsa::PrefillGrid g = clsa::prefill_grid(0, 1 << 24);
  int rb, cb;
  clsa::prefill_tile(g, g.tiles - 1, &rb, &cb);
  if (rb != g.last_rb || cb != g.last_rb) {
    std::printf("2^24 rows: last tile -> (%d, %d)\n", rb, cb);
    return 1;
  }
  for (int64_t t : {(int64_t)0, (int64_t)1, g.tiles / 2, g.tiles - 2}) {
    clsa::prefill_tile(g, t, &rb, &cb);
    if (cb > rb || clsa::pf_prefix(rb, g.c0) + cb != t) {
      std::printf("2^24 rows: tile %lld -> (%d, %d)\n", (long long)t, rb, cb);
      return 1;
    }
  }
  std::printf("ok %ld\n", checked);
  return 0;
}
