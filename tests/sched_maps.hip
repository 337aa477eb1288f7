// Host-side check of the workgroup -> job maps of fa_device.h (built for the host only and run
// by test_schedule_maps.py): for every grid size and head length tried, xcd_remap and
// xcd_remap_interleaved are permutations of the jobs, the interleaved map gives every XCD the
// same jobs as the plain one, and causal_tile permutes a head's tiles.
#include <cstdio>
#include <vector>

#include "../exact_attention_fa_amd/csrc/fa_device.h"

int main() {
  long checked = 0;
  for (int nblk = 1; nblk <= 2304; ++nblk) {
    std::vector<int> a(nblk, 0);
    for (int b = 0; b < nblk; ++b) {
      const int j = fa::xcd_remap(b, nblk);
      if (j < 0 || j >= nblk || a[j]++) { printf("xcd_remap not a permutation: nblk %d\n", nblk); return 1; }
    }
    for (int per_head = 1; per_head <= 72; ++per_head) {
      if (nblk % per_head) continue;
      std::vector<int> c(nblk, 0);
      for (int b = 0; b < nblk; ++b) {
        const int j = fa::xcd_remap_interleaved(b, nblk, per_head);
        if (j < 0 || j >= nblk || c[j]++) {
          printf("xcd_remap_interleaved not a permutation: nblk %d per_head %d\n", nblk, per_head);
          return 1;
        }
        // same XCD range as the plain map: both lie in the jobs xcd_remap gives XCD b % 8
        const int q = nblk / 8, r = nblk % 8, x = b % 8;
        const int lo = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q, len = x < r ? q + 1 : q;
        if (j < lo || j >= lo + len) {
          printf("xcd_remap_interleaved moved a job across XCDs: nblk %d per_head %d\n", nblk, per_head);
          return 1;
        }
      }
      ++checked;
    }
  }
  for (int n = 1; n <= 300; ++n)
    for (int snake = 0; snake < 2; ++snake)
      for (int head = 0; head < 3; ++head) {
        std::vector<int> t(n, 0);
        for (int i = 0; i < n; ++i) {
          const int k = fa::causal_tile(i, head, n, snake);
          if (k < 0 || k >= n || t[k]++) { printf("causal_tile not a permutation: n %d\n", n); return 1; }
        }
      }
  printf("ok %ld\n", checked);
  return 0;
}
