"""GPU parity of kda_chunk_prefill against the fp64 oracle."""
import os

import numpy as np
import pytest
import torch

import kda_inputs as ki
import linear_attention_sequence_chunked_amd as kda
from parity import assert_close, host, log, oracle_full, oracle_pairs

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def run(x, **kw):
    o, S = kda.chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate,
                             cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_seqlens_host,
                             initial_state=x.initial_state, **kw)
    torch.cuda.synchronize()
    return o, S


def check_full(x, dtype, **kw):
    o, S = run(x, **kw)
    ro, rS = oracle_full(x, floor=kw.get("log_alpha_floor", -0.3), scale=kw.get("scale", 1.0))
    if x.total_tokens:
        assert_close("o", host(o), ro, DT[dtype])
    assert_close("S_T", host(S), rS, DT[dtype])
    return o, S


def test_tiny_f32_workload():
    """B=1, H=2, T=256, d=64, fp32 tensors, zero initial state."""
    w = ki.WORKLOADS["tiny_f32"]
    log("prefill tiny_f32")
    check_full(ki.make_workload_inputs(w, seed=0, device="cuda"), "f32")


@pytest.mark.parametrize("T", [1, 15, 16, 17, 100])
def test_lengths_bf16_d128(T):
    log(f"prefill bf16 d=128 T={T}")
    x = ki.make_prefill_inputs((T,), 2, 128, 128, "bf16", 0.02, seed=T, device="cuda")
    check_full(x, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_varlen_shapes(dtype, dk, dv):
    """Packed varlen with a zero-length sequence, partial chunks, per-sequence S0."""
    log(f"prefill varlen dtype={dtype} dk={dk} dv={dv}")
    x = ki.make_prefill_inputs((37, 0, 16, 1, 50), 3, dk, dv, dtype, 0.3, seed=dk + dv,
                               device="cuda")
    check_full(x, dtype, scale=0.9, log_alpha_floor=-0.5)


@pytest.mark.parametrize("nv", [16, 32, 64, 128])
def test_value_slicing_is_bitwise_invariant(nv, monkeypatch):
    """Every dv-slice width gives bit-identical results (columns are independent)."""
    log(f"prefill slice width nv={nv}")
    x = ki.make_prefill_inputs((70, 33), 2, 128, 128, "bf16", 0.02, seed=3, device="cuda")
    monkeypatch.setenv("KDA_PREFILL_NV", "128")
    o_ref, S_ref = run(x)
    monkeypatch.setenv("KDA_PREFILL_NV", str(nv))
    o, S = run(x)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    ro, rS = oracle_full(x)
    assert_close("o", host(o), ro, torch.bfloat16)


def test_final_state_aliases_initial_state():
    log("prefill in-place state")
    x = ki.make_prefill_inputs((40, 9, 64), 2, 128, 64, "bf16", 0.1, seed=4, device="cuda")
    ref_o, ref_S = run(x)
    st = x.initial_state.clone()
    o, S = kda.chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate,
                             cu_seqlens=x.cu_seqlens, initial_state=st, final_state=st)
    torch.cuda.synchronize()
    assert S.data_ptr() == st.data_ptr()
    assert torch.equal(o, ref_o) and torch.equal(st, ref_S)


def test_all_sequences_empty():
    log("prefill empty batch")
    x = ki.make_prefill_inputs((0, 0), 2, 64, 64, "bf16", 0.5, seed=5, device="cuda")
    o, S = run(x)
    assert o.shape[0] == 0
    assert torch.equal(S, x.initial_state)


def test_guards_nan_poison_and_determinism():
    """Every output element is written, nothing outside the outputs is, and two runs
    are bit-identical (no atomics, fixed reduction order)."""
    log("prefill guards / determinism")
    x = ki.make_prefill_inputs((33, 64, 5), 4, 128, 128, "bf16", 0.05, seed=6, device="cuda")
    T, H, d, N = x.total_tokens, 4, 128, 3
    guard = 8192
    runs = []
    for _ in range(2):
        obuf = torch.full((T * H * d + 2 * guard,), float("nan"), dtype=torch.bfloat16,
                          device="cuda")
        sbuf = torch.full((N * H * d * d + 2 * guard,), -3.5, dtype=torch.float32,
                          device="cuda")
        o = obuf[guard:guard + T * H * d].view(T, H, d)
        S = sbuf[guard:guard + N * H * d * d].view(N, H, d, d)
        S.fill_(float("nan"))
        run(x, out=o, final_state=S)
        assert torch.isnan(obuf[:guard].float()).all() and torch.isnan(obuf[-guard:].float()).all()
        assert torch.all(sbuf[:guard] == -3.5) and torch.all(sbuf[-guard:] == -3.5)
        assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
        runs.append((o.clone(), S.clone()))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])


def sampled_check(x, pairs, o, S, dtype=torch.bfloat16):
    ref = oracle_pairs(x, pairs)
    got_o = np.concatenate([host(o[x.cu_seqlens_host[n]:x.cu_seqlens_host[n + 1], h])
                            for n, h in pairs])
    ref_o = np.concatenate([ref[p][0] for p in pairs])
    assert_close("o (sampled)", got_o, ref_o, dtype)
    assert_close("S_T (sampled)", np.stack([host(S[n, h]) for n, h in pairs]),
                 np.stack([ref[p][1] for p in pairs]), dtype)


def test_workload_b4_h16_t4096_sampled():
    """B=4, H=16, T=4096, d=128, bf16, S0 ~ N(0, 0.02^2): the benchmark's workload and
    launch configuration; sampled (sequence, head) pairs against the oracle."""
    w = ki.WORKLOADS["prefill_b4_h16_t4096"]
    log("prefill workload b4_h16_t4096")
    x = ki.make_workload_inputs(w, seed=1, device="cuda")
    o, S = run(x)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    sampled_check(x, [(0, 0), (1, 7), (2, 15), (3, 3)], o, S)


def test_workload_b1_h32_t131072_sampled():
    """Long context: B=1, H=32, T=131072, d=128, bf16, zero S0; three heads checked."""
    w = ki.WORKLOADS["prefill_b1_h32_t131072"]
    log("prefill workload b1_h32_t131072")
    x = ki.make_workload_inputs(w, seed=2, device="cuda")
    o, S = run(x)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    sampled_check(x, [(0, 0), (0, 13), (0, 31)], o, S)


@pytest.mark.skipif(os.environ.get("KDA_SKIP_HUGE") == "1", reason="KDA_SKIP_HUGE=1")
def test_workload_varlen_n64_h32_sampled():
    """64 packed sequences, lengths 40% 8K / 42% 32K / 15% 128K / 3% 256K (3.77M tokens,
    ~185 GB of device tensors), H=32, d=128, per-sequence S0."""
    w = ki.WORKLOADS["varlen_n64_h32"]
    log(f"prefill workload varlen_n64_h32 T_total={sum(w.lengths)}")
    x = ki.make_workload_inputs(w, seed=4, device="cuda")
    o, S = run(x)
    lens = w.lengths
    short = lens.index(8192)
    mid = lens.index(32768)
    longest = lens.index(max(lens))
    assert torch.isfinite(S).all()
    sampled_check(x, [(short, 0), (mid, 31), (longest, 17)], o, S)
    del x, o, S
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strongest_decay_floor(dtype):
    """The lowest accepted floor (-5): log-decays drawn down to -5, so a chunk's cumulative
    decay reaches tens of nats and e^(G_C - G), e^-G span ~e^80 -- the range the lower
    bound on the log-decay exists to keep finite."""
    log(f"prefill floor=-5 dtype={dtype}")
    x = ki.make_prefill_inputs((40, 64, 17), 2, 128, 128, dtype, 0.3, seed=55, device="cuda",
                               log_alpha_min=-5.0)
    check_full(x, dtype, log_alpha_floor=-5.0)
