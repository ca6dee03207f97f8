// Host check of split_key_range (clsa_internal.h), the rule every attention workgroup uses to find
// the selection positions its split reads: for any count a caller passes (negative, zero, above k),
// any k and any split layout, every position read lies in [0, k), and the splits of a row cover
// exactly the first min(max(count, 0), k) positions once.  Prints "ok" or the first failure.
#include <cstdio>

#include "../../cross_layer_token_amd/csrc/clsa_internal.h"

int main() {
  const int counts[] = {-100000, -7, -1, 0, 1, 2, 63, 64, 65, 99, 100, 101, 2047, 2048, 2049, 4096, 65536, 1 << 30};
  const int ks[] = {1, 7, 64, 100, 256, 2048, 2049, 65536};
  long checked = 0;
  for (int k : ks)
    for (int kps = 64; kps <= 8192; kps *= 2) {
      const int splits = (k + kps - 1) / kps;
      for (int count : counts) {
        const int want = count < 0 ? 0 : (count > k ? k : count);
        int covered = 0;
        for (int s = 0; s < splits; ++s) {
          int b, e;
          clsa::split_key_range(count, k, s, kps, &b, &e);
          if (e > k || (e > b && b < 0) || e - b > kps) {
            std::printf("bad range k=%d kps=%d count=%d split=%d: [%d, %d)\n", k, kps, count, s, b, e);
            return 1;
          }
          if (e > b) covered += e - b;
          ++checked;
        }
        if (covered != want) {
          std::printf("coverage k=%d kps=%d count=%d: %d positions, want %d\n", k, kps, count, covered, want);
          return 1;
        }
      }
    }
  std::printf("ok %ld\n", checked);
  return 0;
}
