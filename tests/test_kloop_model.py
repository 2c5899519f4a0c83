"""The packed k-loop's wait counts are checked at compile time (csrc/kloop_model.h): the
header compiles as it is, and a count moved by one, or an issue order changed without the
counts following, fails the build. The model is plain constexpr C++, so a host compiler
checks it; the HIP build compiles the same header into both packed GEMM kernels."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "mixture_experts_layer_37_amd", "csrc", "kloop_model.h")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")


def _compile(text: str):
    with tempfile.TemporaryDirectory() as d:
        with open(os.path.join(d, "kloop_model.h"), "w") as f:
            f.write(text)
        src = os.path.join(d, "t.cpp")
        with open(src, "w") as f:
            f.write('#include "kloop_model.h"\nint main() { return 0; }\n')
        r = subprocess.run(["g++", "-std=c++17", "-fsyntax-only", src], capture_output=True,
                           text=True)
        return r.returncode, r.stderr


def _header():
    with open(HEADER) as f:
        return f.read()


def test_model_compiles():
    rc, err = _compile(_header())
    assert rc == 0, err


COUNT_LINE = "  return loads_after<kLA, kLB>(seq, n, want);\n}"

PERTURBATIONS = {
    # every count the loop uses one too high (a wait that passes with its load in flight)
    "count_plus_one": (COUNT_LINE, "  return loads_after<kLA, kLB>(seq, n, want) + 1;\n}"),
    # one too low
    "count_minus_one": (COUNT_LINE, "  return loads_after<kLA, kLB>(seq, n, want) - 1;\n}"),
    # only the counts of the step before the last (next k-step, no refill) one too high
    "second_last_step_plus_one": (
        COUNT_LINE, "  return loads_after<kLA, kLB>(seq, n, want) + (next && !refill ? 1 : 0);\n}"),
    # the prologue issues B slice 3 before A(kb + 1): the steady-state counts no longer hold
    # for the first k-step (its wait for A(kb + 1) would pass with that stage in flight)
    "prologue_order": ("{kLoadB, 2}, {kDmaA, 1}, {kLoadB, 3},",
                       "{kLoadB, 2}, {kLoadB, 3}, {kDmaA, 1},"),
    # the first stage's wait counted one load too many
    "start_plus_one": ("  return loads_after<kLA, kLB>(seq, n, Load{true, 0});\n}",
                       "  return loads_after<kLA, kLB>(seq, n, Load{true, 0}) + 1;\n}"),
    # a k-step that issues the next B slice before waiting for its own: the derived counts
    # change, and the documented numbers no longer match
    "step_order": ("{kLgkm0, 0}, {kWaitB, 0}, {kReadA, 1}, {kLoadBNext, 0}, {kMfma, 0},",
                   "{kLgkm0, 0}, {kLoadBNext, 0}, {kWaitB, 0}, {kReadA, 1}, {kMfma, 0},"),
    # a ring of 16 slots under the pair schedule: the second step of a pair loads slots
    # 8..11, which no later step reads (asm outputs left unused while their loads are in
    # flight), and the next pair reads stale slots
    "ring_slots": ("constexpr int kRingSlots = 8;", "constexpr int kRingSlots = 16;"),
    # the next k-step's slices loaded two k-steps' worth of slots ahead: the waits then read
    # slots never loaded
    "next_slot": ("constexpr int next_slot(int sb, int s) { return (sb + 4 + s) % kRingSlots; }",
                  "constexpr int next_slot(int sb, int s) { return (sb + 8 + s) % kRingSlots; }"),
    # the second step of a steady pair on the first one's ring base
    "steady_ring_base": ("constexpr StepSlot kSteadyPair[] = {{0, 0, 3}, {1, 4, 3}};",
                         "constexpr StepSlot kSteadyPair[] = {{0, 0, 3}, {1, 0, 3}};"),
    # the step before the last run as a steady one: it would refill a stage past the tile
    "last_pair_remaining": ("constexpr StepSlot kLastPair[] = {{0, 0, 2}, {1, 4, 1}};",
                            "constexpr StepSlot kLastPair[] = {{0, 0, 3}, {1, 4, 1}};"),
}


@pytest.mark.parametrize("name", list(PERTURBATIONS))
def test_perturbed_model_fails_to_build(name):
    old, new = PERTURBATIONS[name]
    text = _header()
    assert text.count(old) == 1, name
    rc, err = _compile(text.replace(old, new))
    assert rc != 0 and "static assert" in err, (name, err[-2000:])
