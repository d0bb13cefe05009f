// Host-side check of the persistent launches' tile lists (queue_decode in
// csrc/common.h): for many geometries, the eight XCD lists together hand out
// every (unit, level, document) tile exactly once, list x only units
// u = x (mod 8); within a list the level groups come in order (every tile of
// group g before any of group g + 1) and, within a group, a unit's tiles are
// contiguous, document by document, each document's levels in order; and the
// first tiles handed out by workgroup
// index and the counter's claims together cover each list once. Built for the
// host only and run by
// tests/test_tile_queue_cpu.py.
#include <cstdio>
#include <set>
#include <tuple>

#include "common.h"

using namespace uly;

int main() {
  int bad = 0, cases = 0;
  const int units_v[] = {1, 2, 3, 7, 8, 9, 13, 16, 32, 64, 65};
  const int nslots_v[] = {1, 2, 3, 4, 5, 7, 16, 33, 512};
  const int ndoc_v[] = {1, 2, 4, 13};
  for (int units : units_v)
    for (int nslots : nslots_v)
      for (int ndoc : ndoc_v) {
        ++cases;
        std::set<std::tuple<int, int, int>> seen;
        const int lg = (nslots + kLevelGroups - 1) / kLevelGroups;
        for (int x = 0; x < kUnitGroup; ++x) {
          const int n = queue_list_len(x, units, nslots, ndoc);
          int prev_grp = -1, prev_unit = -1, prev_lvl = -1, prev_doc = -1;
          std::set<std::pair<int, int>> units_done;  // (group, unit) finished
          for (int i = 0; i < n; ++i) {
            const TileId t = queue_decode(x, i, units, nslots, ndoc);
            const int grp = t.lvl / lg;
            const int g0 = grp * lg, g1 = (grp + 1) * lg < nslots ? (grp + 1) * lg : nslots;
            if (t.unit < 0 || t.unit >= units || t.unit % kUnitGroup != x) ++bad;
            if (t.lvl < 0 || t.lvl >= nslots || t.doc < 0 || t.doc >= ndoc) ++bad;
            if (!seen.insert({t.unit, t.lvl, t.doc}).second) ++bad;
            if (grp < prev_grp) ++bad;  // groups in order
            if (grp == prev_grp && t.unit != prev_unit) {
              if (units_done.count({grp, t.unit})) ++bad;  // a unit's part is contiguous
              units_done.insert({grp, prev_unit});
            }
            if (grp == prev_grp && t.unit == prev_unit) {
              // the next tile of the unit's part: the document's next level, or
              // the next document's first level of the group
              const bool next_lvl = t.doc == prev_doc && t.lvl == prev_lvl + 1;
              const bool next_doc = t.doc == prev_doc + 1 && prev_lvl == g1 - 1 && t.lvl == g0;
              if (!next_lvl && !next_doc) ++bad;
            } else if (t.doc != 0 || t.lvl != g0) {
              ++bad;  // a unit's part starts with its first document's first level
            }
            prev_grp = grp;
            prev_unit = t.unit;
            prev_lvl = t.lvl;
            prev_doc = t.doc;
          }
        }
        if ((int)seen.size() != units * nslots * ndoc) ++bad;
      }
  // First tiles by workgroup index: for every grid size, the workgroups
  // b = x (mod 8) take tiles b / 8 of list x, exactly the first
  // queue_static_count(x, grid, n) of them, and the counter's claims
  // (static count + 0, 1, ...) hand out the rest, each once.
  for (int grid = 1; grid <= 300; ++grid)
    for (int n : {0, 1, 5, 31, 32, 33, 64, 100, 1000}) {
      ++cases;
      for (int x = 0; x < kUnitGroup; ++x) {
        std::set<int> got;
        for (int b = x; b < grid; b += kUnitGroup)
          if (b / kUnitGroup < n && !got.insert(b / kUnitGroup).second) ++bad;
        const int nst = queue_static_count(x, grid, n);
        if ((int)got.size() != nst) ++bad;
        for (int c = 0; nst + c < n; ++c)
          if (!got.insert(nst + c).second) ++bad;
        if ((int)got.size() != n) ++bad;
        if (!got.empty() && (*got.begin() != 0 || *got.rbegin() != n - 1)) ++bad;
      }
    }
  std::printf("tile queue geometries %d, mismatches %d\n", cases, bad);
  return bad != 0;
}
