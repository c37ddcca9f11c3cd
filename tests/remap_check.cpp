// Host-side check of the workgroup -> work-item maps of sla_tiles.hpp: xcd_remap is a
// bijection, and xcd_chunk_map sends the valid workgroups of an xcd_chunk_grid grid one to one
// onto every (head, item) with every XCD holding the same share (within one item) of every head.
// Built and run on the CPU by tests/test_remap.py.
#include <cstdio>
#include <vector>

#include "sla_tiles.hpp"

int main() {
  int bad = 0;
  for (int total = 1; total <= 5000 && !bad; total += 7) {
    std::vector<int> seen(total, 0);
    for (int wg = 0; wg < total; ++wg) {
      const int it = sla::xcd_remap(wg, total);
      if (it < 0 || it >= total || seen[it]++) {
        std::printf("xcd_remap not a bijection: total %d wg %d\n", total, wg);
        bad = 1;
        break;
      }
    }
  }
  for (int heads = 1; heads <= 41 && !bad; heads += 4) {
    for (int per = 1; per <= 700 && !bad; per += (per < 40 ? 1 : 37)) {
      const int grid = sla::xcd_chunk_grid(heads, per);
      std::vector<int> seen(heads * per, 0);
      std::vector<int> share(8 * heads, 0);
      int valid = 0;
      for (int wg = 0; wg < grid; ++wg) {
        int h, it;
        if (!sla::xcd_chunk_map(wg, per, &h, &it)) continue;
        ++valid;
        if (h < 0 || h >= heads || it < 0 || it >= per || seen[h * per + it]++) {
          std::printf("xcd_chunk_map: heads %d per %d wg %d -> (%d, %d) out of range or repeated\n", heads, per, wg, h, it);
          bad = 1;
          break;
        }
        share[(wg % 8) * heads + h]++;
      }
      if (!bad && valid != heads * per) {
        std::printf("xcd_chunk_map: heads %d per %d covers %d of %d items\n", heads, per, valid, heads * per);
        bad = 1;
      }
      for (int h = 0; h < heads && !bad; ++h) {
        int mn = 1 << 30, mx = 0;
        for (int x = 0; x < 8; ++x) {
          const int v = share[x * heads + h];
          mn = v < mn ? v : mn;
          mx = v > mx ? v : mx;
        }
        if (mx - mn > 1) {
          std::printf("unbalanced: heads %d per %d head %d: %d..%d\n", heads, per, h, mn, mx);
          bad = 1;
        }
      }
    }
  }
  std::printf(bad ? "FAIL\n" : "OK\n");
  return bad;
}
