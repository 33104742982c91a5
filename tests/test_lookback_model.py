"""The look-back protocol of the single-pass kernels checked on the CPU under
adversarial schedules (tests/c/lookback_model.cpp): workgroups as
coroutines stepped one shared-memory action at a time, descriptor words as
relaxed atomics whose loads may return any value not older than the last
one seen ("Single-Pass Prefix Scan with Decoupled Look-Back", sections
"Three states in a per-block descriptor", "Why the work stays linear" and
"Where the algorithm meets the hardware"; "GPUPrefixSums", section
"Decoupled Fallback"; "Parallel Prefix Sum (Scan), in depth", section
"Scanning a whole array: three grid strategies").

With ticket-ordered tiles every schedule terminates with every exclusive
prefix exact, for one-word and two-word descriptors, PARTIAL jumps,
fallbacks racing the owners' own stores, words left by earlier calls, and
the closing step in which a workgroup resolves its last three tiles.
With tiles in a fixed order and fewer resident slots than workgroups,
dispatched highest index first, every schedule deadlocks unless the
fallback is on.  Each rule of the protocol, broken on purpose in the model,
is caught."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("lookback_model") / "lookback_model")
    subprocess.run(["g++", "-O2", "-std=c++20", "-Wall", "-Wextra", "-Werror",
                    "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(ROOT, "device_wide_prefix_chained_amd", "csrc"),
                    os.path.join(ROOT, "tests", "c", "lookback_model.cpp"), "-o", exe], check=True)
    return exe


def run(model, *args):
    r = subprocess.run([model, *args], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    line = [x for x in r.stdout.splitlines() if x.startswith("schedules")][-1]
    # the "name value" pairs of the summary line
    counts = {name.strip(): int(value) for name, value in re.findall(r"([a-zA-Z][a-zA-Z ]*?) (\d+)", line)}
    return r.returncode, counts


ONE = ["words=1", "op=affine16"]
TWO = ["words=2", "op=affine32", "pair=0"]  # the two-word kernels publish no pairs
SEG = ["words=1", "op=segmented", "pair=0"]


def test_one_word_exact_under_every_schedule(model):
    rc, c = run(model, *ONE, "seeds=40")
    assert rc == 0 and c["ok"] == 40 and c["violation"] == 0
    # the cases the rules are for were reached
    assert c["stale"] > 0 and c["words of earlier calls"] > 0
    assert c["PARTIAL published"] > 0 and c["PARTIAL jumps"] > 0 and c["stalls"] > 0


def test_one_word_fallbacks_race_the_owners(model):
    rc, c = run(model, *ONE, "seeds=40", "fallback=2", "p_fresh=0.3")
    assert rc == 0 and c["ok"] == 40
    # installs that won, that lost to the owner (or another fallback), and
    # that found the word already published
    assert c["installs won"] > 0 and c["lost"] > 0 and c["skipped"] > 0


def test_withheld_aggregates_resolve_through_fallbacks(model):
    # owners publish no AGGREGATE: every stall ends in a fallback
    rc, c = run(model, *ONE, "seeds=30", "fallback=1", "withhold=1")
    assert rc == 0 and c["ok"] == 30 and c["fallbacks"] == c["stalls"] > 0


def test_two_word_descriptors(model):
    rc, c = run(model, *TWO, "seeds=40", "fallback=2", "p_fresh=0.2")
    assert rc == 0 and c["ok"] == 40 and c["violation"] == 0
    # half-published descriptors were read and refused; halves of two
    # publications of one state word (an install racing the owner) were
    # accepted, and held one value
    assert c["torn reads"] > 0 and c["mixed reads"] > 0 and c["lost"] > 0


def test_two_word_without_fallback(model):
    rc, c = run(model, *TWO, "seeds=30")
    assert rc == 0 and c["ok"] == 30 and c["torn reads"] > 0


def test_segmented_form(model):
    for extra in ([], ["fallback=1", "withhold=1"]):
        rc, c = run(model, *SEG, "seeds=30", *extra)
        assert rc == 0 and c["ok"] == 30, extra


def test_kernel_window_width(model):
    # the kernels' window (64 lanes x 2 words) over a call of thousands of tiles
    rc, c = run(model, *ONE, "win=128", "tiles=3000", "wgs=64", "resident=64", "seeds=4", "fallback=2")
    assert rc == 0 and c["ok"] == 4


def test_fixed_order_deadlocks_without_fallback(model):
    # one group per workgroup in index order, 8 resident slots, the highest
    # indices dispatched first: they wait on tiles no running workgroup owns
    rc, c = run(model, *ONE, "persistent=0", "tickets=0", "wgs=150", "resident=8", "order=desc", "seeds=5",
                "expect=deadlock")
    assert rc == 0 and c["deadlock"] == 5


def test_fixed_order_with_fallback_terminates(model):
    rc, c = run(model, *ONE, "persistent=0", "tickets=0", "wgs=150", "resident=8", "order=desc", "seeds=5",
                "fallback=2")
    assert rc == 0 and c["ok"] == 5 and c["fallbacks"] > 0


def test_tickets_terminate_with_few_slots(model):
    # the same dispatch order, no fallback: a tile's predecessors always
    # belong to workgroups that started earlier
    rc, c = run(model, *ONE, "persistent=0", "tickets=1", "wgs=150", "resident=8", "order=desc", "seeds=5")
    assert rc == 0 and c["ok"] == 5 and c["fallbacks"] == 0


@pytest.mark.parametrize("base", [ONE, TWO, ["words=1", "op=affine16", "pair=0"]])
def test_closing_step_keeps_prefixes_exact(model, base):
    # the closing phase of the three-phase kernels (flat scans with and
    # without pair prefixes, two-word descriptors, compaction): a workgroup
    # with nothing left to scan resolves prev2, prev and cur in one step,
    # the look-backs of prev and cur earlier than in the steady state
    for extra in ([], ["fallback=1", "withhold=1"]):
        rc, c = run(model, *base, "close=1", "seeds=20", *extra)
        assert rc == 0 and c["ok"] == 20 and c["violation"] == 0, extra
        assert c["closing steps"] > 0 and c["closing lookbacks"] > 0


def test_closing_step_order_is_checked(model):
    # resolving cur before prev in the closing step hands a group's second
    # tile the prefix of the wrong tile: caught
    rc, c = run(model, *ONE, "close=1", "seeds=20", "broken=close_order", "expect=violation")
    assert rc == 0 and c["violation"] > 0


@pytest.mark.parametrize("broken,base", [("torn", TWO), ("no_tag", ONE), ("partial_distance", ONE),
                                         ("skip_invalid", ONE)])
def test_broken_rules_are_caught(model, broken, base):
    # two-word agreement, the call tag, the PARTIAL distance, waiting on
    # an unpublished word nearer than the stopper
    rc, c = run(model, *base, "seeds=20", "fallback=2", "broken=" + broken, "expect=violation")
    assert rc == 0 and c["violation"] > 0, broken
