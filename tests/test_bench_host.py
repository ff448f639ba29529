"""Host-side checks of bench.py's measurement arithmetic and its refusal of several GPUs
(no GPU needed)."""
import glob
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


SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json")) +
                   glob.glob(os.path.join(ROOT, "profiles", "*_mfma_counters.json")))


@pytest.mark.parametrize("path", SUMMARIES, ids=os.path.basename)
def test_committed_summaries_name_their_workload_and_command(path):
    """Every committed counter summary names a workload of kda_inputs, the kernel source it
    was measured on, and the rocprofv3 commands (over bench.py) that produced it."""
    import kda_inputs as ki
    t = json.load(open(path))
    assert t["workload"] in ki.WORKLOADS
    assert os.path.basename(path).startswith(t["workload"])
    assert len(t["kernel_source_sha256"]) == 64
    cmds = t.get("commands") or [t["command"]]
    assert any("rocprofv3 --pmc" in c and "bench.py" in c for c in cmds)


def test_varlen_sample_covers_every_length_class_with_distinct_pairs():
    import kda_inputs as ki
    w = ki.WORKLOADS[bench.HEADLINE]
    pairs = bench.varlen_sample(w.lengths, w.H, 16)
    assert len(pairs) == 16 * len(set(w.lengths)) == len(set(pairs))
    for L in set(w.lengths):
        assert sum(1 for n, _ in pairs if w.lengths[n] == L) == 16


def test_headline_workload_is_the_packed_varlen_batch():
    """The headline is the largest single-GPU workload: 64 packed sequences (3,768,320
    tokens), H=32, d=128; its algorithmic bytes per launch are 1538 per token-head plus
    the per-sequence initial and final states."""
    import kda_inputs as ki
    w = ki.WORKLOADS[bench.HEADLINE]
    assert sum(w.lengths) == 3_768_320 and len(w.lengths) == 64 and w.H == 32
    b, f = bench.prefill_algorithmic(w.lengths, w.H, w.dk, w.dv, 2, True)
    assert b == 3_768_320 * 32 * 1538 + 64 * 32 * 2 * 128 * 128 * 4
    assert f == 3_768_320 * 32 * 118_784


def test_counter_steps_sum_the_kernels_between_flushes(tmp_path):
    """The counter summaries take one entry per timed step: the library's dispatches between
    two cache flushes (other kernels) are summed, however many kernels a step launches."""
    import csv
    names = ["flush", "kda::a", "kda::b", "flush", "kda::a", "kda::c", "kda::b", "flush", "kda::a"]
    with open(tmp_path / "x_counter_collection.csv", "w") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i, n in enumerate(names):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": n, "Counter_Name": "FETCH_SIZE",
                        "Counter_Value": i + 1, "Start_Timestamp": 0, "End_Timestamp": 1000})
    out, dur, nm = bench._read_steps([str(tmp_path)], "kda::")
    assert out == {"FETCH_SIZE": [2 + 3, 5 + 6 + 7, 9]}
    assert dur == [2.0, 3.0, 1.0]
    assert nm == ["kda::a + kda::b", "kda::a + kda::c + kda::b", "kda::a"]
