"""The workspace hand-over rules (device_wide_prefix_chained_amd/csrc/
ws_state.hpp, the functions the kernels call at the start and the end of a
single-pass call) checked on the CPU: tests/c/ws_model.cpp runs them over a
long random sequence of calls of every kind against a model of the
descriptor words and asserts that every word a call uses reads as
unpublished under the call's tag once the call has cleaned what it must
("Single-Pass Prefix Scan with Decoupled Look-Back", section "Three states
in a per-block descriptor": a slot starts out invalid).  The same model run
with the tag-wrap rule left out must find a violation, which shows that the
sequence reaches the case the rule is for."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("ws_model") / "ws_model")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-Werror",
                    "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(ROOT, "device_wide_prefix_chained_amd", "csrc"),
                    os.path.join(ROOT, "tests", "c", "ws_model.cpp"), "-o", exe], check=True)
    return exe


def test_rules_keep_every_used_word_unpublished(model):
    r = subprocess.run([model], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 violations" in r.stdout
    wraps = int(r.stdout.split(" tag wraps")[0].split(",")[-1])
    assert wraps >= 100


def test_model_finds_a_missing_wrap_rule(model):
    r = subprocess.run([model, "broken"], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
