// Host-side check of the workgroup -> work-item maps of sla_tiles.hpp: xcd_remap is a
// bijection, and xcd_chunk_map sends the valid workgroups of an xcd_chunk_grid grid one to one
// onto every (head, item) with every XCD holding the same share (within one item) of every head;
// xcd_chunk_id inverts it.  xcd_group_map<XG> does the same over xcd_group_grid<XG> with each
// head on the XG XCDs of its group only (group h % (8 / XG)), balanced within one item over
// them, and xcd_group_id<XG> inverts it.  The quantiser's transposed staging of sla_quant.hpp:
// v8_pos permutes the 64 keys, qz_tr_at places every byte of a channel row once inside that
// row, the flush's qz_tr_word finds each 4-byte word again, and the 16 channel groups writing
// one key position hit 16 different banks.  Built and run on the CPU by tests/test_remap.py.
#include <cstdio>
#include <vector>

#include "sla_quant.hpp"
#include "sla_tiles.hpp"

template <int XG>
int check_group(int heads, int per) {
  constexpr int G = 8 / XG;
  const int grid = sla::xcd_group_grid<XG>(heads, per);
  std::vector<int> seen(heads * per, 0), share(8 * heads, 0);
  int valid = 0;
  for (int wg = 0; wg < grid; ++wg) {
    int h, it;
    if (!sla::xcd_group_map<XG>(wg, heads, per, &h, &it)) continue;
    ++valid;
    if (h < 0 || h >= heads || it < 0 || it >= per || seen[h * per + it]++) {
      std::printf("xcd_group_map<%d>: heads %d per %d wg %d -> (%d, %d) out of range or repeated\n", XG, heads,
                  per, wg, h, it);
      return 1;
    }
    if ((wg % 8) / XG != h % G) {
      std::printf("xcd_group_map<%d>: head %d on XCD %d outside its group\n", XG, h, wg % 8);
      return 1;
    }
    if (sla::xcd_group_id<XG>(h, it, per) != wg) {
      std::printf("xcd_group_id<%d>: (%d, %d) -> %d, expected %d\n", XG, h, it,
                  sla::xcd_group_id<XG>(h, it, per), wg);
      return 1;
    }
    share[(wg % 8) * heads + h]++;
  }
  if (valid != heads * per) {
    std::printf("xcd_group_map<%d>: heads %d per %d covers %d of %d items\n", XG, heads, per, valid, heads * per);
    return 1;
  }
  for (int h = 0; h < heads; ++h) {
    int mn = 1 << 30, mx = 0;
    for (int x = (h % G) * XG; x < (h % G + 1) * XG; ++x) {
      const int v = share[x * heads + h];
      mn = v < mn ? v : mn;
      mx = v > mx ? v : mx;
    }
    if (mx - mn > 1) {
      std::printf("xcd_group_map<%d> unbalanced: heads %d per %d head %d: %d..%d\n", XG, heads, per, h, mn, mx);
      return 1;
    }
  }
  return 0;
}

int check_quant_staging() {
  constexpr int D = 128;
  std::vector<int> hit(64, 0);
  for (int n = 0; n < 64; ++n) {
    const int p = sla::v8_pos(n);
    if (p < 0 || p >= 64 || hit[p]++) {
      std::printf("v8_pos: key %d -> %d out of range or repeated\n", n, p);
      return 1;
    }
  }
  for (int c = 0; c < D; ++c) {
    std::vector<int> row(64, 0);
    for (int pos = 0; pos < 64; ++pos) {
      const int a = sla::qz_tr_at(c, pos) - c * 64;
      if (a < 0 || a >= 64 || row[a]++) {
        std::printf("qz_tr_at: channel %d byte %d -> %d outside its row or repeated\n", c, pos, a);
        return 1;
      }
      if (sla::qz_tr_word(c, pos >> 2) * 4 + (pos & 3) != a) {
        std::printf("qz_tr_word: channel %d byte %d not found again by the flush\n", c, pos);
        return 1;
      }
    }
  }
  for (int e = 0; e < 8; ++e)
    for (int pos = 0; pos < 64; ++pos) {
      std::vector<int> bank(64, 0);
      for (int ch = 0; ch < 16; ++ch)
        if (bank[(sla::qz_tr_at(8 * ch + e, pos) / 4) % 64]++) {
          std::printf("qz_tr_at: channel groups share a bank at e %d byte %d\n", e, pos);
          return 1;
        }
    }
  return 0;
}

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
        if (sla::xcd_chunk_id(h, it, per) != wg) {
          std::printf("xcd_chunk_id: (%d, %d) -> %d, expected %d\n", h, it, sla::xcd_chunk_id(h, it, per), wg);
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
  for (int heads = 1; heads <= 41 && !bad; heads += 2)
    for (int per = 1; per <= 1024 && !bad; per += (per < 40 ? 1 : 53))
      bad = check_group<8>(heads, per) || check_group<4>(heads, per) || check_group<2>(heads, per) ||
            check_group<1>(heads, per);
  if (!bad) bad = check_quant_staging();
  std::printf(bad ? "FAIL\n" : "OK\n");
  return bad;
}
