// Host check of the distillation KL pass's tile enumeration (kl_tile_count / kl_tile in
// clsa_internal.h): for calls starting at many positions pos0 with many row counts, the tiles
// 0 .. count-1 map to distinct (row block, key block) pairs, and those pairs are exactly the
// 32-position x 256-key tiles that hold a visible (position, key) pair: key j <= pos0 + i.
#include <cstdio>
#include <set>
#include <utility>

#include "../../cross_layer_token_amd/csrc/clsa_internal.h"

int main() {
  using clsa::kDistillKeyBlock;
  using clsa::kDistillRowBlock;
  const int pos0s[] = {0, 1, 7, 31, 32, 33, 50, 224, 255, 256, 257, 3000, 8191, 65536, 100003};
  const int rows[] = {1, 2, 31, 32, 33, 63, 64, 200, 255, 256, 257, 500, 600, 1000, 1024, 4097, 8192};
  long checked = 0;
  for (int pos0 : pos0s)
    for (int n : rows) {
      const int64_t tiles = clsa::kl_tile_count(pos0, n);
      std::set<std::pair<int, int>> seen;
      for (int64_t t = 0; t < tiles; ++t) {
        int rb, kb;
        clsa::kl_tile(pos0, n, t, &rb, &kb);
        const int first = rb * kDistillRowBlock;
        const int last = first + kDistillRowBlock - 1 < n - 1 ? first + kDistillRowBlock - 1 : n - 1;
        if (rb < 0 || first >= n || kb < 0 || (int64_t)kb * kDistillKeyBlock > (int64_t)pos0 + last ||
            !seen.insert({rb, kb}).second) {
          std::printf("pos0=%d n=%d tile %lld -> (%d, %d) invalid or repeated\n", pos0, n, (long long)t, rb, kb);
          return 1;
        }
      }
      int64_t want = 0;  // every tile with a visible pair
      for (int rb = 0; rb * kDistillRowBlock < n; ++rb) {
        const int last = (rb + 1) * kDistillRowBlock - 1 < n - 1 ? (rb + 1) * kDistillRowBlock - 1 : n - 1;
        want += ((int64_t)pos0 + last) / kDistillKeyBlock + 1;
      }
      if (want != tiles || (int64_t)seen.size() != want) {
        std::printf("pos0=%d n=%d: %lld tiles, want %lld\n", pos0, n, (long long)tiles, (long long)want);
        return 1;
      }
      checked += tiles;
    }
  // the largest call (2^24 positions): more tiles than one grid row holds; spot-check the ends
  const int n = 1 << 24;
  const int64_t tiles = clsa::kl_tile_count(0, n);
  int rb, kb;
  clsa::kl_tile(0, n, tiles - 1, &rb, &kb);
  if (tiles <= (int64_t)1 << 23 || rb != n / kDistillRowBlock - 1 || kb != (n - 1) / kDistillKeyBlock) {
    std::printf("2^24 rows: %lld tiles, last -> (%d, %d)\n", (long long)tiles, rb, kb);
    return 1;
  }
  for (int64_t t : {(int64_t)0, (int64_t)1, tiles / 3, tiles / 2, tiles - 2}) {
    clsa::kl_tile(0, n, t, &rb, &kb);
    const int64_t row_last = (int64_t)rb * kDistillRowBlock + kDistillRowBlock - 1;
    if (kb > row_last / kDistillKeyBlock || clsa::kl_prefix(0, rb) + kb != t) {
      std::printf("2^24 rows: tile %lld -> (%d, %d)\n", (long long)t, rb, kb);
      return 1;
    }
  }
  std::printf("ok %ld\n", checked);
  return 0;
}
