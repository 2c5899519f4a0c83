// Tile order of the grouped GEMMs: the integer arithmetic that maps a launch's work items to
// tiles, shared by grouped_gemm_bf16_kernel, grouped_gemm_packed_kernel and
// splitk_reduce_kernel (which must agree on it: the split-K tail is the same tiles in all of
// them).
//
// Each expert owns ceil(rows / BMt) * NT tiles, n-tile major, m-tile minor. Experts fall into
// two classes: "wide" ones, and "small" ones whose rows fit in kSmallRows (one m-tile: their
// tiles stream the expert's weights for few rows, while a wide expert's tiles are MFMA-bound
// and share weight panels across m-tiles through L2). The tile list holds the wide experts'
// tiles first (experts in index order), then the small ones'. A launch takes its tiles in
// rounds of the grid, XCD x the x-th run of `run` tiles of each round, one tile per block;
// merged_tile gives, while both classes last, XCD x the wide class in rounds r with r + x
// even and the small class in the others. So in every round half the XCDs stream weights
// while the others run MFMAs, and every block takes both classes in turn (a fixed class per
// XCD left half the chip idle at the end). With no small expert (or no wide one) the merged
// order is the list order.
//
// Paired ragged ends (`pairs`; GEMM 1 with SwiGLU on packed weights): an expert whose last
// m-tile holds at most kSmallRows rows gives that m-tile one tile per PAIR of n-tiles,
// kSmallRows rows by both n-tiles' columns. In a wide expert that is the MFMAs of a full
// tile, so it ends with the blocks that share its weight panels, where a half-height tile
// per n-tile ended early and pulled its block out of step with them. A small expert's
// m-tile is its ragged end too: its pair tiles stream two weight panels at once, twice the
// weight bytes in flight per k-step of a half-height tile, which waits on memory. Within
// the expert, n-tile pair q holds the full-height m-tiles of n-tile 2q, those of 2q + 1
// (none in a small expert), then the pair tile; an odd last n-tile keeps a tile of its own.
//
// Plain constexpr C++ (implicitly host and device functions under hipcc): a host compiler
// runs the same code in the CPU tests.
#pragma once

namespace moe {

constexpr int kXcds = 8;          // XCDs of the chip, each with its own L2
constexpr int kSmallRows = 128;   // rows of a small expert / of a pairable ragged end

// Tiles of one expert of m rows: one per m-tile and n-tile, except for a paired ragged end.
constexpr int expert_tiles(int m, int NT, int BMt, bool pairs) {
  if (!pairs || m <= 0) return ((m + BMt - 1) / BMt) * NT;
  const int rem = m % BMt;
  const int mw = m / BMt + (rem > kSmallRows ? 1 : 0);   // full-height m-tiles
  return mw * NT + (rem > 0 && rem <= kSmallRows ? (NT + 1) / 2 : 0);
}

// List index of merged position p. Runs of `run` tiles, kXcds runs per round: for rounds
// r < R the run of XCD x is the (4 r + x / 2)-th run of the wide part [0, nw) if r + x is
// even, else that run of the small part [nw, total); R = the whole rounds both parts can
// fill. Then the rest of the wide part, then the rest of the small part.
constexpr int merged_tile(int p, int nw, int total, int run) {
  constexpr int kHalf = kXcds / 2;
  const int rw = nw / (kHalf * run), rs = (total - nw) / (kHalf * run);
  const int R = rw < rs ? rw : rs;
  if (p < kXcds * run * R) {
    const int c = p / run, o = p - c * run;
    const int r = c / kXcds, x = c - r * kXcds;
    const int idx = (kHalf * r + (x >> 1)) * run + o;
    return ((r + x) & 1) ? nw + idx : idx;
  }
  const int q = p - kXcds * run * R, rest_w = nw - kHalf * run * R;
  return q < rest_w ? kHalf * run * R + q : nw + kHalf * run * R + (q - rest_w);
}

// Largest slot in [0, E) with s_start[slot] <= tile (experts without tiles have equal starts).
constexpr int find_expert(const int* s_start, int E, int tile) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Tile `rem` of an expert of m_e > 0 rows: its n-tile, m-tile and whether it is a pair tile
// (n-tiles n_t and n_t + 1).
struct TileInExpert {
  int n_t, m_t, pair;
};
constexpr TileInExpert tile_in_expert(int m_e, int rem, int NT, int BMt, bool pairs) {
  TileInExpert t{0, 0, 0};
  const int ragged = m_e % BMt;
  if (!pairs || ragged == 0 || ragged > kSmallRows) {
    const int mt_e = (m_e + BMt - 1) / BMt;
    t.n_t = rem / mt_e;
    t.m_t = rem - t.n_t * mt_e;
    return t;
  }
  // full-height m-tiles (0 in a small expert; then o < 2 mw never holds, so no division by
  // zero below); the ragged end is m-tile mw
  const int mw = m_e / BMt;
  const int blk = 2 * mw + 1;          // tiles of one n-tile pair
  const int q = rem / blk, o = rem - q * blk;
  if (q < NT / 2) {
    t.n_t = 2 * q + (o < 2 * mw ? o / mw : 0);
    t.m_t = o < 2 * mw ? o % mw : mw;
    t.pair = o >= 2 * mw;
  } else {                             // the odd last n-tile: its m-tiles, then its end
    t.n_t = NT - 1;
    t.m_t = o;
  }
  return t;
}

}  // namespace moe
