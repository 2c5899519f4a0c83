// Issue-order model of the packed GEMMs' k-loop, and the wait counts derived from it.
//
// The k-loop (packed_kloop.h, shared by grouped_gemm_packed_kernel and
// grouped_wgrad_packed_kernel) issues its global loads as inline asm, so the compiler tracks
// none of them and the loop waits with explicit `s_waitcnt vmcnt(N)` counts. Vector memory
// loads of one wave complete in issue order (the global->LDS DMA ones included), so a wait
// for a given load must allow exactly the number of this wave's loads issued after it. A
// count one too high lets the wait pass while the load is in flight, and the compiler, which
// sees the asm output as ready, may hand the destination registers to another value that the
// landing load then overwrites (a memory-safety bug, not only a wrong result); one too low
// only waits longer.
//
// The loop executes the op lists below (kPrologue, which only issues a tile's first loads;
// kStart, which waits for its first stage; kStep once per k-step), and every count it uses
// comes from wait_count() / start_count(), which simulate the steady state: the previous
// k-step's loads, then this one's up to the wait. tile_mismatches() then replays whole tiles
// of 2 to 10 k-steps from their prologue, with each step's own predicates (a next k-step
// exists, a refill of the current stage exists), and the static_asserts at the bottom
// require every wait of every step to equal the load count that replay finds. A change to
// the op lists re-derives the counts; a count that no longer matches the replay fails the
// build. Global stores issued between tiles (the previous tile's epilogue) can only make the
// waits stricter, never let one pass early, since loads complete in order among themselves.
//
// Plain constexpr C++ (no HIP): it also compiles with a host compiler.
#pragma once

namespace moe {
namespace kloop {

// Every function below takes kLA, the A DMA instructions per k-step and wave, and kLB, the
// B loads per 16-wide k slice (one 1 KB block per weight fragment: 4 in the 2 x 2 wave
// layout, 2 in the 1 x 4 one).

enum Kind : int {
  // prologue (issue only) and start
  kDmaA,        // A DMA of k-step kb + arg into stage arg
  kLoadB,       // B slice arg (0..3) of k-step kb into ring slot arg
  kWaitA0,      // wait for A(kb) (and this wave's LDS operations)
  kReadA0,      // LDS reads of A slice 0 of stage 0
  // k-step kt on stage `cur` (its B slices in ring slots sb .. sb + 3)
  kLgkm0,       // wait for this wave's LDS reads
  kWaitB,       // wait for B slice 4 kt + arg
  kReadA,       // LDS reads of A slice arg of `cur` (into fragment arg & 1)
  kLoadBNext,   // if a next k-step exists: B slice 4 (kt + 1) + arg into slot sb + 4 + arg
  kMfma,        // the 16 MFMAs of slice arg (fragment arg & 1, slot sb + arg)
  kWaitANext,   // next exists: wait for A(kt + 1) and the LDS reads; else wait for everything
  kBarrier,     // workgroup barrier: publishes the next stage, frees `cur`
  kDmaA2,       // if a refill exists (kt + 2 < ke): A(kt + 2) into `cur`
  kReadANext,   // if a next k-step exists: LDS reads of A slice 0 of the next stage
};

struct Op {
  Kind kind;
  int arg;
};

// Once per tile, issue only: A(kb), B slices 0..2 of kb, A(kb + 1), B slice 3, in this
// order (a k-step's own load order, so the first k-step's waits are the steady state's);
// the k-steps below then find their loads one k-step ahead.
constexpr Op kPrologue[] = {
    {kDmaA, 0}, {kLoadB, 0}, {kLoadB, 1}, {kLoadB, 2}, {kDmaA, 1}, {kLoadB, 3},
};
constexpr int kPrologueOps = sizeof(kPrologue) / sizeof(kPrologue[0]);
// Then the first stage lands and is published.
constexpr Op kStart[] = {{kWaitA0, 0}, {kBarrier, 0}, {kReadA0, 0}};
constexpr int kStartOps = sizeof(kStart) / sizeof(kStart[0]);

// One k-step: three slices, each waiting for its B fragments, issuing the next slice's A
// reads and (one k-step ahead) the B loads of slice s + 4, then running its MFMAs; then the
// wait for the next stage, the barrier, the refill DMA of this stage, the first A reads of
// the next stage and the last slice.
constexpr Op kStep[] = {
    {kLgkm0, 0}, {kWaitB, 0}, {kReadA, 1}, {kLoadBNext, 0}, {kMfma, 0},
    {kLgkm0, 0}, {kWaitB, 1}, {kReadA, 2}, {kLoadBNext, 1}, {kMfma, 1},
    {kLgkm0, 0}, {kWaitB, 2}, {kReadA, 3}, {kLoadBNext, 2}, {kMfma, 2},
    {kWaitANext, 0}, {kBarrier, 0},
    {kWaitB, 3}, {kDmaA2, 0}, {kReadANext, 0}, {kLoadBNext, 3}, {kMfma, 3},
};
constexpr int kStepOps = sizeof(kStep) / sizeof(kStep[0]);

// A load of one wave as the model sees it: an A k-step (kLA DMA instructions) or a B slice
// (kLB loads), by absolute index within the tile.
struct Load {
  bool is_a;
  int id;
};

// Loads (counted in instructions) issued after `want` in seq[0, n); -1 if it was never issued.
template <int kLA, int kLB>
constexpr int loads_after(const Load* seq, int n, Load want) {
  int after = 0;
  for (int i = n - 1; i >= 0; --i) {
    if (seq[i].is_a == want.is_a && seq[i].id == want.id) return after;
    after += seq[i].is_a ? kLA : kLB;
  }
  return -1;
}

// The loads k-step kt issues when op i runs (relative to the tile's first k-step).
constexpr int issue(const Op& op, int kt, bool next, bool refill, Load* out) {
  if (op.kind == kLoadBNext && next) {
    out[0] = Load{false, 4 * (kt + 1) + op.arg};
    return 1;
  }
  if (op.kind == kDmaA2 && refill) {
    out[0] = Load{true, kt + 2};
    return 1;
  }
  return 0;
}

// The load a wait op of k-step kt needs; returns false for a wait that needs everything (or
// for an op that is not a vector-memory wait).
constexpr bool awaited(const Op& op, int kt, bool next, Load& want) {
  if (op.kind == kWaitB) {
    want = Load{false, 4 * kt + op.arg};
    return true;
  }
  if (op.kind == kWaitANext && next) {
    want = Load{true, kt + 1};
    return true;
  }
  return false;
}

// The count the loop uses at op i of a k-step with these predicates, from the steady state:
// the previous k-step (which always had a next one, and had a refill exactly when this one
// has a next) followed by this step's ops before i. -1 for a wait-for-everything op.
template <int kLA, int kLB>
constexpr int wait_count(int i, bool next, bool refill) {
  Load seq[2 * kStepOps] = {};
  int n = 0;
  for (int j = 0; j < kStepOps; ++j) n += issue(kStep[j], -1, true, next, seq + n);
  for (int j = 0; j < i; ++j) n += issue(kStep[j], 0, next, refill, seq + n);
  Load want{false, 0};
  if (!awaited(kStep[i], 0, next, want)) return -1;
  return loads_after<kLA, kLB>(seq, n, want);
}

// The prologue's loads in issue order; returns their number.
constexpr int prologue_loads(Load* seq) {
  int n = 0;
  for (int j = 0; j < kPrologueOps; ++j) {
    const Op& op = kPrologue[j];
    if (op.kind == kDmaA) seq[n++] = Load{true, op.arg};
    if (op.kind == kLoadB) seq[n++] = Load{false, op.arg};
  }
  return n;
}

// The count of kWaitA0: the loads the prologue issues after A(kb).
template <int kLA, int kLB>
constexpr int start_count() {
  Load seq[kPrologueOps] = {};
  const int n = prologue_loads(seq);
  return loads_after<kLA, kLB>(seq, n, Load{true, 0});
}

// Replay of whole tiles of 2 .. 10 k-steps (the real predicates of every step, the real
// prologue and start): the number of waits whose count differs from what the replay finds.
template <int kLA, int kLB>
constexpr int tile_mismatches() {
  int bad = 0;
  for (int nsteps = 2; nsteps <= 10; nsteps += 2) {
    Load seq[kPrologueOps + 10 * kStepOps] = {};
    int n = prologue_loads(seq);
    for (int j = 0; j < kStartOps; ++j) {
      if (kStart[j].kind == kWaitA0) {
        const int need = loads_after<kLA, kLB>(seq, n, Load{true, 0});
        if (need < 0 || need != start_count<kLA, kLB>()) ++bad;
      }
    }
    for (int kt = 0; kt < nsteps; ++kt) {
      const bool next = kt + 1 < nsteps, refill = kt + 2 < nsteps;
      for (int i = 0; i < kStepOps; ++i) {
        const Op& op = kStep[i];
        Load want{false, 0};
        if (awaited(op, kt, next, want)) {
          const int need = loads_after<kLA, kLB>(seq, n, want);
          if (need < 0 || need != wait_count<kLA, kLB>(i, next, refill)) ++bad;
        } else if (op.kind == kWaitANext) {
          if (wait_count<kLA, kLB>(i, next, refill) != -1) ++bad;   // the last step waits for all
        }
        n += issue(op, kt, next, refill, seq + n);
      }
    }
  }
  return bad;
}

// vmcnt is a 6-bit field: every count the loop can use must fit.
template <int kLA, int kLB>
constexpr bool counts_fit() {
  if (start_count<kLA, kLB>() > 63) return false;
  for (int i = 0; i < kStepOps; ++i)
    for (int m = 0; m < 4; ++m) {
      const int c = wait_count<kLA, kLB>(i, m & 1, m & 2);
      if (c > 63) return false;
    }
  return true;
}

// The loop's schedule, as data the loop executes: pairs of steady k-steps while at least two
// more remain, then the last two. Each entry is {offset from the pair's first k-step, ring
// base, k-steps left counting this one (capped at 3, the steady state: a next k-step for
// 2 or more, a refill for 3 or more)}. The B slices of k-step kt sit in ring slots
// (4 kt + s) mod kRingSlots, so a pair's bases are the constants 0 and 4.
constexpr int kRingSlots = 8;
struct StepSlot {
  int off, sb, r;
};
// The slot a k-step on ring base sb waits on for its slice s, and the slot it loads slice s
// of the next k-step into; the loop indexes its ring with these, and the replay below
// checks them.
constexpr int wait_slot(int sb, int s) { return (sb + s) % kRingSlots; }
constexpr int next_slot(int sb, int s) { return (sb + 4 + s) % kRingSlots; }
constexpr StepSlot kSteadyPair[] = {{0, 0, 3}, {1, 4, 3}};
constexpr StepSlot kLastPair[] = {{0, 0, 2}, {1, 4, 1}};
constexpr int kPairSteps = 2;

// Replay of the schedule over tiles of 2 .. 40 k-steps with the ring's slots: every k-step
// runs once, in order, with the predicates of its position; every wait for slice s of
// k-step kt finds that slice in its slot; no load overwrites a slice not yet read; and every
// slice loaded is read. (A slot loaded and never read would leave an asm output unused, and
// the compiler may give its registers to another value while the load is in flight.)
// Returns the number of violations.
constexpr int schedule_mismatches() {
  int bad = 0;
  for (int n = 2; n <= 40; n += 2) {
    int slot_kt[kRingSlots] = {}, slot_s[kRingSlots] = {};
    bool unread[kRingSlots] = {}, filled[kRingSlots] = {};
    auto load = [&](int slot, int kt, int sl) {
      if (unread[slot]) ++bad;
      slot_kt[slot] = kt;
      slot_s[slot] = sl;
      unread[slot] = true;
      filled[slot] = true;
    };
    for (int j = 0; j < kPrologueOps; ++j)
      if (kPrologue[j].kind == kLoadB) load(kPrologue[j].arg % kRingSlots, 0, kPrologue[j].arg);
    int expect = 0;
    auto run = [&](const StepSlot* t, int kt0) {
      for (int e = 0; e < kPairSteps; ++e) {
        const int kt = kt0 + t[e].off, left = n - kt;
        if (kt != expect++) ++bad;
        if (t[e].r != (left < 3 ? left : 3)) ++bad;
        if (t[e].sb != (4 * kt) % kRingSlots) ++bad;
        for (int sl = 0; sl < 4; ++sl) {
          const int slot = wait_slot(t[e].sb, sl);
          if (!filled[slot] || slot_kt[slot] != kt || slot_s[slot] != sl) ++bad;
          unread[slot] = false;
          if (t[e].r >= 2) load(next_slot(t[e].sb, sl), kt + 1, sl);
        }
      }
    };
    int kt = 0;
    for (; kt + 2 < n; kt += kPairSteps) run(kSteadyPair, kt);
    run(kLastPair, kt);
    if (expect != n) ++bad;
    for (int q = 0; q < kRingSlots; ++q)
      if (unread[q]) ++bad;
  }
  return bad;
}
static_assert(schedule_mismatches() == 0,
              "the loop's schedule breaks the ring (a slice read before its load, overwritten "
              "unread, or loaded and never read) or the k-steps' order or predicates");

// The counts in numbers, for kLA = 8 A DMA instructions per k-step (both kernels) and kLB
// = 4 B loads per slice (the 2 x 2 wave layout): 3 kLB + kLA = 20 before slice 0's MFMAs,
// 2 kLB + kLA + kLB = 20 before slice 1's and kLB + kLA + 2 kLB = 20 before slice 2's when a
// next k-step exists (12, 8 and 4 in the last step), 4 kLB = 16 for the next stage before
// the barrier and 3 kLB = 12 for slice 3 after it (0 in the last step); 3 kLB + kLA + kLB =
// 24 loads follow A(kb) in the prologue. With kLB = 2 (the 1 x 4 layout) the same formulas
// give 14, 14, 14 (6, 4, 2), 8, 6 (0) and 16.
static_assert(tile_mismatches<8, 4>() == 0, "k-loop wait counts disagree with the issue order");
static_assert(counts_fit<8, 4>(), "k-loop wait count exceeds the 6-bit vmcnt field");
static_assert(wait_count<8, 4>(1, true, true) == 20 && wait_count<8, 4>(6, true, true) == 20 &&
                  wait_count<8, 4>(11, true, true) == 20 && wait_count<8, 4>(15, true, true) == 16 &&
                  wait_count<8, 4>(17, true, true) == 12 && wait_count<8, 4>(1, false, false) == 12 &&
                  wait_count<8, 4>(6, false, false) == 8 && wait_count<8, 4>(11, false, false) == 4 &&
                  wait_count<8, 4>(15, false, false) == -1 && wait_count<8, 4>(17, false, false) == 0 &&
                  start_count<8, 4>() == 24,
              "the documented k-loop wait counts");
static_assert(tile_mismatches<8, 2>() == 0 && counts_fit<8, 2>(),
              "k-loop wait counts disagree with the issue order (1 x 4 layout)");
static_assert(wait_count<8, 2>(1, true, true) == 14 && wait_count<8, 2>(6, true, true) == 14 &&
                  wait_count<8, 2>(11, true, true) == 14 && wait_count<8, 2>(15, true, true) == 8 &&
                  wait_count<8, 2>(17, true, true) == 6 && wait_count<8, 2>(1, false, false) == 6 &&
                  wait_count<8, 2>(6, false, false) == 4 && wait_count<8, 2>(11, false, false) == 2 &&
                  wait_count<8, 2>(17, false, false) == 0 && start_count<8, 2>() == 16,
              "the documented k-loop wait counts (1 x 4 layout)");

}  // namespace kloop
}  // namespace moe
