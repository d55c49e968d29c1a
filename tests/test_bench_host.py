"""Host-side logic of bench.py (CPU only): the one-GPU refusal and the
whole-step roofline arithmetic, against counts worked out by hand."""

import subprocess
import sys
import os

import bench
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_step_roofline_of_the_13b_step():
    # one chunk: 3 frames x 1560 tokens x 12 heads; 49834 merged and 6326
    # inserted tokens; 66804 live slots at attend; a 0.343 ms step
    w = WORKLOADS["dit1.3b"]
    r = bench._step_roofline(w, 49834, 6326, 66804, 0.343)
    nb = r["algorithmic_bytes"]
    assert nb["hash"] == 56160 * 272                        # bf16 row + 4 codes
    assert nb["match"] == 56160 * 536                       # row, codes, one candidate, decision
    assert nb["apply"] == 49834 * 3104 + 6326 * 2080
    assert nb["index"] == 3 * (66804 * 4 * 12 + 12 * 4 * 2049 * 4)   # 2048 buckets at 8192 slots
    assert nb["attend"] == 12 * 4680 * 512 + 66804 * 516
    # attend is bound by 4 * 4680 * 66804 * 128 flops at 2.5 PFLOP/s
    assert abs(r["bound_us"]["attend"] - 160073072640 / 2.5e15 * 1e6) < 0.01
    # the HBM-bound kernels by their bytes at 8 TB/s
    assert abs(r["bound_us"]["apply"] - (49834 * 3104 + 6326 * 2080) / 8e12 * 1e6) < 0.01
    total = sum(r["bound_us"].values())
    assert abs(r["bound_us_total"] - total) < 0.02
    assert abs(r["frac"] - r["bound_us_total"] / 343.0) < 1e-3


def test_traffic_record_survives_comment_edits_only(tmp_path, monkeypatch):
    """The attention source hash that keys a traffic record ignores // comments
    and blank lines, and changes with any code edit."""
    src = tmp_path / "attend.hip"
    monkeypatch.setattr(bench, "ATTEND_SRC", str(src))
    src.write_text("int f(int x) {\n  return x + 1;  // add one\n}\n")
    h0 = bench._attend_src_hash()
    src.write_text("// a new header line\nint f(int x) {\n\n  return x + 1;  // plus one\n}\n")
    assert bench._attend_src_hash() == h0
    src.write_text("int f(int x) {\n  return x + 2;  // add one\n}\n")
    assert bench._attend_src_hash() != h0
