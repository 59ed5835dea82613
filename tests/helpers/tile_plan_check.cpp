// Host-side check of the grouped GEMM's tile schedule (csrc/tile_plan.h), built with the host
// compiler by tests/test_tile_plan_cpu.py. Prints "ok" and exits 0, or prints the first
// violation and exits 1.
//
// For every launch size n (tiles), K depth (steps of 32) and split limit it checks:
//   * every workgroup with work has bid < the host grid (grid_bound);
//   * every tile is covered exactly once when unsplit, or by parts 0..P-1 exactly once each;
//   * side slots are unique, below kSideSlots and (kMaxParts - 1) n (the side buffer's size),
//     -1 exactly for part 0, and the fixup kernel's
//     enumeration (split_tiles, split_tile) names every split tile once with the same slots;
//   * the XCDs' work (workgroups with a unit, bid mod 8) differs by at most one bundle;
//   * K parts tile [0, nk) in order; with an even nk (the bf16 MFMA path) each part starts on
//     an even step and has an even length, at least 4 steps when split (so a pair load never
//     reaches past its part);
//   * tile_in_expert is a bijection onto the tm x tn tiles of an expert, and inside the whole
//     blocks of kColBlock column tiles each run of kColBlock consecutive tiles is one row tile
//     over consecutive column tiles.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tile_plan.h"

using namespace moe::plan;

static int fail(const char* what, int a, int b, int c, int d) {
  std::printf("FAIL %s (%d %d %d %d)\n", what, a, b, c, d);
  return 1;
}

static int check_launch(int n, int nk, int max_parts) {
  const int grid = grid_bound(n, max_parts);
  std::vector<int> seen(static_cast<size_t>(n) * kMaxParts, 0);
  std::vector<int> parts_of(n, 0);
  std::vector<int> side_used(kSideSlots, 0);
  std::vector<int> side_tile(kSideSlots, -1), side_part(kSideSlots, -1);
  for (int bid = 0; bid < grid + 64 * kXcds; ++bid) {
    Unit u;
    if (!unit_of(bid, n, nk, max_parts, u)) continue;
    if (bid >= grid) return fail("work past the grid", n, nk, max_parts, bid);
    if (u.tile < 0 || u.tile >= n) return fail("tile out of range", n, nk, max_parts, u.tile);
    if (u.parts < 1 || u.parts > kMaxParts || u.kpart < 0 || u.kpart >= u.parts)
      return fail("bad part", n, nk, u.kpart, u.parts);
    if (u.parts > 1 && (max_parts <= 1 || u.parts > max_parts || u.parts > nk / 4))
      return fail("split beyond its limits", n, nk, max_parts, u.parts);
    if (parts_of[u.tile] != 0 && parts_of[u.tile] != u.parts) return fail("mixed parts", n, nk, u.tile, u.parts);
    parts_of[u.tile] = u.parts;
    if (seen[static_cast<size_t>(u.tile) * kMaxParts + u.kpart]++) return fail("unit twice", n, nk, u.tile, u.kpart);
    if ((u.kpart == 0) != (u.side < 0)) return fail("side slot of part 0", n, nk, u.tile, u.side);
    if (u.side >= 0) {
      if (u.side >= kSideSlots || u.side >= (kMaxParts - 1) * n) return fail("side slot too large", n, nk, u.tile, u.side);
      if (side_used[u.side]++) return fail("side slot twice", n, nk, u.tile, u.side);
      side_tile[u.side] = u.tile;
      side_part[u.side] = u.kpart;
    }
    int kf = 0, kl = 0;
    part_range(nk, u.kpart, u.parts, kf, kl);
    if (kl - kf < 1) return fail("empty part", n, nk, u.kpart, u.parts);
    if (nk % 2 == 0 && ((kf & 1) || ((kl - kf) & 1))) return fail("odd part with an even K", n, nk, kf, kl);
    if (u.parts > 1 && kl - kf < 4) return fail("part under 4 steps", n, nk, kf, kl);
  }
  for (int t = 0; t < n; ++t) {
    if (parts_of[t] == 0) return fail("tile not covered", n, nk, max_parts, t);
    for (int p = 0; p < parts_of[t]; ++p)
      if (seen[static_cast<size_t>(t) * kMaxParts + p] != 1) return fail("part not covered", n, nk, t, p);
  }
  // the fixup kernel's enumeration of the split tiles names every split tile once, with the
  // side slots its parts wrote
  const int n_split = split_tiles(n, nk, max_parts);
  int split_seen = 0;
  for (int t = 0; t < n; ++t) split_seen += parts_of[t] > 1;
  if (n_split != split_seen) return fail("split tile count", n, nk, n_split, split_seen);
  std::vector<int> listed(n, 0);
  for (int s = 0; s < n_split; ++s) {
    int tile = -1, P = 0, side0 = -1;
    split_tile(s, n, nk, max_parts, tile, P, side0);
    if (tile < 0 || tile >= n || listed[tile]++) return fail("fixup tile", n, nk, s, tile);
    if (parts_of[tile] != P) return fail("fixup parts", n, nk, tile, P);
    for (int p = 1; p < P; ++p)
      if (side_tile[side0 + p - 1] != tile || side_part[side0 + p - 1] != p) return fail("fixup slot", n, nk, tile, p);
  }
  int lo = 1 << 30, hi = 0;
  for (int x = 0; x < kXcds; ++x) {
    int units = 0;
    for (int bid = x; bid < grid; bid += kXcds) {
      Unit u;
      units += unit_of(bid, n, nk, max_parts, u) ? 1 : 0;
    }
    lo = units < lo ? units : lo;
    hi = units > hi ? units : hi;
  }
  if (hi - lo > kBundle) return fail("unbalanced XCDs", n, nk, lo, hi);
  // part ranges tile [0, nk) in order
  for (int P = 1; P <= kMaxParts && P <= (nk >= 4 ? nk / 4 : 1); ++P) {
    int prev = 0;
    for (int p = 0; p < P; ++p) {
      int kf = 0, kl = 0;
      part_range(nk, p, P, kf, kl);
      if (kf != prev || kl <= kf) return fail("part ranges", nk, P, p, kf);
      prev = kl;
    }
    if (prev != nk) return fail("part ranges end", nk, P, prev, 0);
  }
  return 0;
}

int main() {
  const int nks[] = {1, 2, 3, 4, 6, 8, 12, 17, 32, 64, 128, 130, 256, 448};
  for (int n = 1; n <= 2100; n += (n < 600 ? 1 : 7))
    for (int nk : nks)
      for (int mp : {1, 8})
        if (check_launch(n, nk, mp)) return 1;
  for (int tm = 1; tm <= 60; ++tm)
    for (int tn = 1; tn <= 70; ++tn) {
      std::vector<int> hit(static_cast<size_t>(tm) * tn, 0);
      for (int t = 0; t < tm * tn; ++t) {
        int mt = -1, nt = -1;
        tile_in_expert(t, tm, tn, mt, nt);
        if (mt < 0 || mt >= tm || nt < 0 || nt >= tn) return fail("tile_in_expert range", tm, tn, t, mt);
        if (hit[static_cast<size_t>(mt) * tn + nt]++) return fail("tile_in_expert twice", tm, tn, mt, nt);
        if (t < tn / kColBlock * kColBlock * tm && t % kColBlock > 0) {
          int mp = -1, np = -1;
          tile_in_expert(t - 1, tm, tn, mp, np);
          if (mp != mt || np + 1 != nt) return fail("tile_in_expert block", tm, tn, t, mt);
        }
      }
    }
  std::printf("ok\n");
  return 0;
}
