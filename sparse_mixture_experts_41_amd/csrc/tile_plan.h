// Tile schedule of the bf16 grouped GEMM: which (expert, row tile, column tile, K part) each
// workgroup of a launch takes. Plain integer arithmetic with no HIP dependence, compiled into
// the kernels and, on the host, into the CPU test that enumerates it.
//
// Order. Experts come in order; within an expert, the column tiles form blocks of kColBlock
// (the last block may be narrower), blocks come in order, and inside a block the row tiles are
// outer and its column tiles inner. A bundle of kBundle = 16 consecutive tiles then covers 4 row
// tiles x 4 column tiles: 4 row panels and 4 weight panels for 16 tiles, where column tiles
// outermost (16 row tiles of one weight panel) needed 17. Measured on MI355X against that order:
// the GEMMs' L2 misses (FETCH_SIZE) fell from 8.0 / 8.6 GB to 4.8 / 4.8 GB per launch on the
// long-tail layer (65536 tokens, d 2048, d_ffn 8192), and its GEMM1 and GEMM2 ran 2.2% and 2.7%
// faster (Mixtral-like layer unchanged, switch-style -1%); blocks of 2 columns timed the same
// and blocks of 8 about 1% slower.
//
// Placement. The hardware hands workgroup b to XCD (b mod 8). Workgroups are renumbered so that
// each XCD takes bundles of kBundle consecutive tiles (tiles that share an expert's operand
// panels, so they meet in that XCD's L2), and bundles go round-robin over the 8 XCDs, so every
// XCD gets the same mix of full and partial tiles. (Measured against giving each XCD one
// contiguous eighth of the tiles, ordered in blocks of 4 row x 8 column tiles for L2 reuse:
// that cut the re-reads but left the XCDs unevenly loaded, because an expert's partial last
// row tile is far cheaper than a full one, and was 2-3% slower on the Mixtral-like layer and
// 13% slower on the switch-style one.)
//
// Tail split. The tiles of the whole rounds of 256 workgroups run unsplit; the L tiles of the
// last, partial round are split along K into P = min(256 / L, max_parts, K steps / 4) parts,
// so the launch ends after about full/256 + 1/P rounds instead of a whole extra round. Part 0
// writes the output (with the bias); parts 1..P-1 write dense 256 x 256 float tiles to a side
// buffer, and a fixup kernel adds them in part order.
#pragma once

#if defined(__HIPCC__)
#define MOE_PLAN_FN __host__ __device__ __forceinline__
#else
#define MOE_PLAN_FN inline
#endif

namespace moe {
namespace plan {

constexpr int kXcds = 8;
constexpr int kBundle = 16;
constexpr int kRound = 256;       // workgroups resident at once: one per CU
constexpr int kMaxParts = 8;
constexpr int kSideSlots = 255;   // side tiles a split tail can need: L (P - 1) < 256

MOE_PLAN_FN int imin(int a, int b) { return a < b ? a : b; }

// Tile t (0 <= t < tm * tn) of one expert with tm row tiles and tn column tiles -> (mt, nt).
constexpr int kColBlock = 4;

MOE_PLAN_FN void tile_in_expert(int t, int tm, int tn, int& mt, int& nt) {
  const int full = tn / kColBlock * kColBlock;     // column tiles in whole blocks
  const int span = tm * kColBlock;                 // tiles of one whole block
  if (t < full * tm) {
    const int cb = t / span, r = t - cb * span;
    mt = r / kColBlock;
    nt = cb * kColBlock + (r - mt * kColBlock);
  } else {                                         // the last block: tn - full columns
    const int rest = tn - full, r = t - full * tm;
    mt = r / rest;
    nt = full + (r - mt * rest);
  }
}

// Workgroup b -> its position in the tile order (bundles of kBundle, round-robin over XCDs).
MOE_PLAN_FN int bundle_order(int bid) {
  const int x = bid % kXcds, j = bid / kXcds;
  return ((j / kBundle) * kXcds + x) * kBundle + j % kBundle;
}

struct TailPlan {
  int full;   // tiles run whole
  int L;      // split tiles after them (0: none)
  int P;      // parts per split tile
};

MOE_PLAN_FN TailPlan tail_plan(int n_tiles, int nk_total, int max_parts) {
  const int rem = n_tiles % kRound;
  int P = rem > 0 ? kRound / rem : 1;
  P = imin(P, max_parts);
  P = imin(P, nk_total / 4);
  TailPlan p;
  if (max_parts <= 1 || rem == 0 || P < 2) {
    p.full = n_tiles;
    p.L = 0;
    p.P = 1;
  } else {
    p.full = n_tiles - rem;
    p.L = rem;
    p.P = P;
  }
  return p;
}

// Workgroups that cover every launch of at most n_max tiles: the units (tiles and the split
// tail's extra parts, fewer than kRound) rounded up to whole bundles on every XCD.
MOE_PLAN_FN int grid_bound(int n_max, int max_parts) {
  const int n = n_max + (max_parts > 1 ? kRound : 0);
  const int g = kXcds * kBundle;
  return (n + g - 1) / g * g;
}

struct Unit {
  int tile;    // position in the tile order
  int kpart;   // K part of a split tile (0 otherwise)
  int parts;   // parts of the tile (1: not split)
  int side;    // side-buffer slot of a part > 0, else -1
};

// Workgroup `bid` of a launch over n_tiles tiles -> its unit; false when it has no work.
MOE_PLAN_FN bool unit_of(int bid, int n_tiles, int nk_total, int max_parts, Unit& u) {
  const int unit = bundle_order(bid);
  const TailPlan p = tail_plan(n_tiles, nk_total, max_parts);
  if (unit >= p.full + p.L * p.P) return false;
  if (unit < p.full) {
    u.tile = unit;
    u.kpart = 0;
    u.parts = 1;
    u.side = -1;
    return true;
  }
  const int v = unit - p.full, s = v / p.P;
  u.tile = p.full + s;
  u.kpart = v - s * p.P;
  u.parts = p.P;
  u.side = u.kpart > 0 ? s * (p.P - 1) + u.kpart - 1 : -1;
  return true;
}

// Split tiles of a launch: how many there are, and split tile s -> its tile, its number of
// parts and the side-buffer slot of its part 1 (part p > 0 is at side0 + p - 1).
MOE_PLAN_FN int split_tiles(int n_tiles, int nk_total, int max_parts) {
  return tail_plan(n_tiles, nk_total, max_parts).L;
}

MOE_PLAN_FN void split_tile(int s, int n_tiles, int nk_total, int max_parts, int& tile, int& P, int& side0) {
  const TailPlan p = tail_plan(n_tiles, nk_total, max_parts);
  tile = p.full + s;
  P = p.P;
  side0 = s * (p.P - 1);
}

// K steps [k_first, k_last) of part kpart of parts. A pair-staged operand loads two K steps at
// a time, so when nk_total is even (always on the bf16 MFMA path: K is a multiple of 64) the
// part boundaries fall on even steps, and no pair load reaches past its part's last step. The
// boundaries do not depend on the staging, so every operand layout sums the same K ranges in
// the same order (bit-identical results).
MOE_PLAN_FN void part_range(int nk_total, int kpart, int parts, int& k_first, int& k_last) {
  if (nk_total % 2 == 0) {
    const int np = nk_total / 2;
    k_first = 2 * (np * kpart / parts);
    k_last = kpart + 1 == parts ? nk_total : 2 * (np * (kpart + 1) / parts);
  } else {
    k_first = nk_total * kpart / parts;
    k_last = nk_total * (kpart + 1) / parts;
  }
}

}  // namespace plan
}  // namespace moe
