"""Host logic of bench.py that runs without a GPU: the hash that ties a
counter summary under profiles/ to the kernel code it was taken on, the
workload-to-source map behind it, how a summary is accepted, and the
refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

WORKLOADS = ("u32x", "u32x-ragged", "u32i", "u32s", "u32s-single-pass", "u64x", "f32", "f32max", "linrec",
             "linrec-h", "segmented", "compact", "compact-staged", "copy", "read", "write")


def test_code_text_drops_comments_only():
    a = 'int a = 1; // one\n/* block\n comment */ const char *s = "x // y /* z */";\n'
    b = 'int a = 1;\nconst char *s = "x // y /* z */";'
    assert bench._code_text(a) == bench._code_text(b)
    # a change of code, or of a string literal, is a change
    assert bench._code_text(a) != bench._code_text(a.replace("a = 1", "a = 2"))
    assert bench._code_text(a) != bench._code_text(a.replace("x // y", "x / y"))
    # an escaped quote does not end the literal
    c = 'const char *t = "a\\" // b"; int z;'
    assert "// b" in bench._code_text(c) and bench._code_text(c).endswith("int z;")


@pytest.mark.parametrize("workload", WORKLOADS)
def test_every_workload_has_its_sources(workload):
    files = bench.kernel_sources(workload)
    assert all(os.path.exists(f) for f in files)
    hip = [os.path.basename(f) for f in files if f.endswith(".hip")]
    assert len(hip) == 1
    expected = {"segmented": "segscan.hip", "compact": "compact.hip", "copy": "common.hip",
                "read": "common.hip", "write": "common.hip"}.get(workload, "scan.hip")
    assert hip[0] == expected
    assert any(f.endswith("dwps.h") for f in files) and any(f.endswith("dwps_device.hpp") for f in files)


def test_kernels_in_different_files_hash_apart():
    h = {w: bench.kernel_source_hash(w) for w in ("u32x", "f32", "segmented", "compact", "copy")}
    assert h["u32x"] == h["f32"]  # one source file
    assert len({h["u32x"], h["segmented"], h["compact"], h["copy"]}) == 4


def test_traffic_summary_accepted_only_on_its_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.load_traffic("u32x", 1.0) is None  # no summary
    summary = {"kernel_source_sha256_16": bench.kernel_source_hash("u32x"), "hbm_bytes_per_launch": 2154235404}
    (tmp_path / "traffic_u32x.json").write_text(json.dumps(summary))
    assert bench.load_traffic("u32x", 1.0) == 2154235404.0
    # taken on other code: refused
    summary["kernel_source_sha256_16"] = "0" * 16
    (tmp_path / "traffic_u32x.json").write_text(json.dumps(summary))
    assert bench.load_traffic("u32x", 1.0) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
