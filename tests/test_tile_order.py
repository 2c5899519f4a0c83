"""The grouped GEMMs' tile order (csrc/tile_order.h: the two expert classes and their merged
order, the paired ragged ends) checked on the CPU: the same header the kernels compile,
built with g++ into a checker that walks every launch position of many expert-size mixes
and requires every output block (expert, m-tile, n-tile) to be covered by exactly one tile,
pair tiles to hold at most 128 rows and two existing n-tiles, and the merged order to be a
permutation of the list. A planted mistake in the pair decoding or in the merged order
fails it."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "mixture_experts_layer_37_amd", "csrc", "tile_order.h")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")

# The list as the kernels build it (build_tile_starts): with classes, the experts of
# 1 .. kSmallRows rows go after the others, each part in expert order; the starts are the
# prefix sums of expert_tiles. Then every merged position is decoded as decode_tile does.
CHECKER = r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "tile_order.h"
using namespace moe;

static unsigned long long rng = 88172645463325252ull;
static int rnd(int n) { rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17; return (int)(rng % (unsigned)n); }

static int fail(const char* what, int E, int NT, int run, int pairs, int classes) {
  std::printf("FAIL %s E=%d NT=%d run=%d pairs=%d classes=%d\n", what, E, NT, run, pairs, classes);
  return 1;
}

int main() {
  const int BMt = 256;
  for (int iter = 0; iter < 4000; ++iter) {
    const int E = 1 + rnd(iter % 4 == 0 ? 256 : 24);
    const int NT = 1 + rnd(20);
    const int runs[] = {1, 2, 8, 32, 64};
    const int run = runs[rnd(5)];
    const bool pairs = rnd(4) != 0, classes = rnd(4) != 0;
    std::vector<int> m(E);
    for (int e = 0; e < E; ++e) {
      switch (rnd(7)) {
        case 0: m[e] = 0; break;
        case 1: m[e] = 1 + rnd(64); break;
        case 2: m[e] = 65 + rnd(64); break;                  // 65 .. 128
        case 3: m[e] = 129 + rnd(127); break;                // one ragged m-tile > 128
        case 4: m[e] = 256 * (1 + rnd(8)) + 1 + rnd(128); break;   // a pairable ragged end
        case 5: m[e] = 256 * (1 + rnd(8)) + 129 + rnd(127); break;
        default: m[e] = 256 * (1 + rnd(8)); break;
      }
    }
    std::vector<int> perm, start(E + 1);
    for (int e = 0; e < E; ++e) if (!(classes && m[e] > 0 && m[e] <= kSmallRows)) perm.push_back(e);
    const int n_wide_experts = (int)perm.size();
    for (int e = 0; e < E; ++e) if (classes && m[e] > 0 && m[e] <= kSmallRows) perm.push_back(e);
    start[0] = 0;
    for (int s = 0; s < E; ++s) start[s + 1] = start[s] + expert_tiles(m[perm[s]], NT, BMt, pairs);
    const int total = start[E], nw = start[n_wide_experts];
    std::vector<int> seen(total, 0);
    // covered[e][mtile][n]
    std::vector<std::vector<int>> cov(E);
    for (int e = 0; e < E; ++e) cov[e].assign(((m[e] + BMt - 1) / BMt) * NT, 0);
    for (int p = 0; p < total; ++p) {
      const int tile = merged_tile(p, nw, total, run);
      if (tile < 0 || tile >= total || seen[tile]++) return fail("merged order not a permutation", E, NT, run, pairs, classes);
      const int slot = find_expert(start.data(), E, tile);
      const int e = perm[slot];
      if (tile < start[slot] || tile >= start[slot + 1] || m[e] <= 0) return fail("find_expert", E, NT, run, pairs, classes);
      const TileInExpert t = tile_in_expert(m[e], tile - start[slot], NT, BMt, pairs);
      const int mrows = m[e] - t.m_t * BMt < BMt ? m[e] - t.m_t * BMt : BMt;
      if (t.n_t < 0 || t.n_t >= NT || t.m_t < 0 || mrows <= 0) return fail("tile outside the expert", E, NT, run, pairs, classes);
      if (t.pair && (t.n_t + 1 >= NT || mrows > kSmallRows || !pairs)) return fail("bad pair tile", E, NT, run, pairs, classes);
      const int mt_e = (m[e] + BMt - 1) / BMt;
      for (int h = 0; h <= t.pair; ++h)
        if (cov[e][(t.n_t + h) * mt_e + t.m_t]++) return fail("block covered twice", E, NT, run, pairs, classes);
    }
    for (int e = 0; e < E; ++e)
      for (int v : cov[e]) if (v != 1) return fail("block not covered", E, NT, run, pairs, classes);
    // the interleave: while both parts fill whole rounds, XCD x of round r takes the wide
    // part iff r + x is even
    const int R = (nw / (4 * run)) < ((total - nw) / (4 * run)) ? nw / (4 * run) : (total - nw) / (4 * run);
    for (int p = 0; p < 8 * run * R; ++p) {
      const int c = p / run, r = c / 8, x = c % 8;
      if ((merged_tile(p, nw, total, run) < nw) != ((r + x) % 2 == 0)) return fail("interleave", E, NT, run, pairs, classes);
    }
  }
  std::printf("ok\n");
  return 0;
}
"""


def _run(header_text: str):
    with tempfile.TemporaryDirectory() as d:
        with open(os.path.join(d, "tile_order.h"), "w") as f:
            f.write(header_text)
        src = os.path.join(d, "check.cpp")
        with open(src, "w") as f:
            f.write(CHECKER)
        exe = os.path.join(d, "check")
        r = subprocess.run(["g++", "-std=c++17", "-O1", "-I", d, src, "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        return r.returncode, r.stdout


def _header():
    with open(HEADER) as f:
        return f.read()


def test_tile_order_covers_every_block_once():
    rc, out = _run(_header())
    assert rc == 0 and out.strip() == "ok", out


PLANTED = {
    # a pair block one tile too long: each n-tile pair's tiles drift into the next pair's
    # (one tile short instead divides by zero for a small expert, whose block is one tile)
    "pair_block_size": ("const int blk = 2 * mw + 1;", "const int blk = 2 * mw + 2;"),
    # the odd last n-tile's ragged end counted as a pair tile
    "odd_tail_pair": ("    t.n_t = NT - 1;\n    t.m_t = o;", "    t.n_t = NT - 1;\n    t.m_t = o;\n    t.pair = o == mw;"),
    # the interleave gives the same class to both XCD parities
    "interleave_parity": ("return ((r + x) & 1) ? nw + idx : idx;", "return (r & 1) ? nw + idx : idx;"),
    # a ragged end of exactly kSmallRows rows left out of the pairs (and of the tile count)
    "boundary_rows": ("return mw * NT + (rem > 0 && rem <= kSmallRows ? (NT + 1) / 2 : 0);",
                      "return mw * NT + (rem > 0 && rem < kSmallRows ? (NT + 1) / 2 : 0);"),
}


@pytest.mark.parametrize("name", list(PLANTED))
def test_planted_mistakes_fail(name):
    old, new = PLANTED[name]
    text = _header()
    assert old in text, name
    rc, out = _run(text.replace(old, new))
    assert rc != 0 and out.startswith("FAIL"), (name, out)
