"""Host-side checks of bench.py's measurement arithmetic and its refusal of several GPUs
(no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_algorithmic_bytes_and_flops_of_the_bench_workload():
    """B=4, H=16, T=4096, dk=dv=128, bf16 inputs, fp32 initial and final states.

    Per token-head: q, k, log_alpha (128 each), v, gate (128 each), beta and o (128), two bytes
    each: 2 (5*128 + 1 + 128) = 1538 bytes.  Per (sequence, head): the initial and the final
    state, 128 x 128 fp32 each.  Flops per token-head: 6*128*128 + 6*16*128 + 4*16*128."""
    b, f = bench.prefill_algorithmic([4096] * 4, 16, 128, 128, 2, True)
    token_heads = 4 * 4096 * 16
    assert b == token_heads * 1538 + 4 * 16 * 2 * 128 * 128 * 4 == 411_566_080
    assert f == token_heads * (6 * 128 * 128 + 6 * 16 * 128 + 4 * 16 * 128) == 31_138_512_896
    # without an initial state only the final one is written
    b0, _ = bench.prefill_algorithmic([4096] * 4, 16, 128, 128, 2, False)
    assert b - b0 == 4 * 16 * 128 * 128 * 4


def test_several_gpus_are_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_stored_summaries_are_ignored_when_stale(tmp_path):
    """A counter summary is used only for its workload and for the kernel source it was
    measured on."""
    good = {"workload": "w", "kernel_source_sha256": "abc", "traffic_bytes_per_step": 5}
    p = tmp_path / "s.json"
    p.write_text(json.dumps(good))
    assert bench.stored_summary(str(p), "w", "abc")["traffic_bytes_per_step"] == 5
    assert bench.stored_summary(str(p), "other", "abc") is None
    assert bench.stored_summary(str(p), "w", "def") is None
    assert bench.stored_summary(str(tmp_path / "missing.json"), "w", "abc") is None
    p.write_text("{not json")
    assert bench.stored_summary(str(p), "w", "abc") is None


@pytest.mark.parametrize("path", [bench.TRAFFIC_FILE, bench.MFMA_FILE, bench.DECODE_TRAFFIC_FILE])
def test_committed_summaries_name_their_workload_and_command(path):
    t = json.load(open(path))
    assert t["workload"] in ("prefill_b4_h16_t4096", "decode_n256_h32")
    assert len(t["kernel_source_sha256"]) == 64
    cmds = t.get("commands") or [t["command"]]
    assert all("rocprofv3 --pmc" in c and "bench.py" in c for c in cmds)
