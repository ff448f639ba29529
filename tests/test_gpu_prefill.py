"""GPU parity of kda_chunk_prefill against the fp64 oracle."""
import os

import numpy as np
import pytest
import torch

import kda_inputs as ki
import linear_attention_sequence_chunked_amd as kda
from parity import assert_close, check_pairs, host, log, oracle_full

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


def test_workload_b4_h16_t4096_every_pair():
    """B=4, H=16, T=4096, d=128, bf16, S0 ~ N(0, 0.02^2): the whole workload (all 64
    (sequence, head) pairs, every output row and final state) against the oracle, in the
    launch configuration the benchmark times."""
    w = ki.WORKLOADS["prefill_b4_h16_t4096"]
    log("prefill workload b4_h16_t4096, every pair")
    x = ki.make_workload_inputs(w, seed=1, device="cuda")
    o, S = run(x)
    ro, rS = oracle_full(x)
    assert_close("o", host(o), ro, torch.bfloat16)
    assert_close("S_T", host(S), rS, torch.bfloat16)


def test_workload_b1_h32_t131072_every_head():
    """Long context: B=1, H=32, T=131072, d=128, bf16, zero S0: every head against the
    oracle, downloaded and checked eight heads at a time."""
    w = ki.WORKLOADS["prefill_b1_h32_t131072"]
    log("prefill workload b1_h32_t131072, every head")
    x = ki.make_workload_inputs(w, seed=2, device="cuda")
    o, S = run(x)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    for h0 in range(0, w.H, 8):
        check_pairs(x, [(0, h) for h in range(h0, h0 + 8)], o, S,
                    label=f"heads {h0}..{h0 + 7}")


def varlen_pairs(lengths, H, per_class=16):
    """per_class (sequence, head) pairs from every length class of the varlen mix,
    spread over the class's sequences and over the heads."""
    classes = sorted(set(lengths))
    out = {}
    for c in classes:
        seqs = [n for n, L in enumerate(lengths) if L == c]
        out[c] = [(seqs[j % len(seqs)], (5 * j + c // 8192) % H)
                  for j in range(per_class)]
        assert len(set(out[c])) == per_class
    return out


@pytest.mark.skipif(os.environ.get("KDA_SKIP_HUGE") == "1", reason="KDA_SKIP_HUGE=1")
def test_workload_varlen_n64_h32_every_length_class():
    """64 packed sequences, lengths 40% 8K / 42% 32K / 15% 128K / 3% 256K (3.77M tokens,
    ~185 GB of device tensors), H=32, d=128, per-sequence S0: 16 (sequence, head) pairs
    of every length class (64 pairs, 6.9M token-heads) against the oracle."""
    w = ki.WORKLOADS["varlen_n64_h32"]
    log(f"prefill workload varlen_n64_h32 T_total={sum(w.lengths)}")
    x = ki.make_workload_inputs(w, seed=4, device="cuda")
    o, S = run(x)
    assert torch.isfinite(S).all()
    for L, pairs in varlen_pairs(w.lengths, w.H).items():
        check_pairs(x, pairs, o, S, label=f"length {L}")
    del x, o, S
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("floor", [-0.3, -0.5])
def test_log_decay_below_floor(dtype, floor):
    """Log-decays drawn down to -2 with the floor at -0.3 / -0.5, so most of them are
    clamped: a kernel that skipped the clamp (or clamped elsewhere) fails."""
    log(f"prefill below-floor decays dtype={dtype} floor={floor}")
    x = ki.make_prefill_inputs((37, 0, 16, 1, 50, 200), 3, 128, 128, dtype, 0.3,
                               seed=77, device="cuda", log_alpha_min=-2.0)
    assert float(x.log_alpha.float().min()) < floor - 1.0
    check_full(x, dtype, log_alpha_floor=floor, scale=0.9)
    # the same inputs with the clamp applied beforehand give the same result
    xc = ki.KdaInputs(x.q, x.k, x.v, torch.clamp(x.log_alpha, min=floor), x.beta, x.gate,
                      x.cu_seqlens, x.cu_seqlens_host, x.initial_state)
    o, S = run(x, log_alpha_floor=floor, scale=0.9)
    oc, Sc = run(xc, log_alpha_floor=floor, scale=0.9)
    assert torch.equal(o, oc) and torch.equal(S, Sc)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strongest_decay_floor(dtype):
    """The lowest accepted floor (-5): log-decays drawn down to -5, so a chunk's cumulative
    decay reaches tens of nats and e^(G_C - G), e^-G span ~e^80 -- the range the lower
    bound on the log-decay exists to keep finite."""
    log(f"prefill floor=-5 dtype={dtype}")
    x = ki.make_prefill_inputs((40, 64, 17), 2, 128, 128, dtype, 0.3, seed=55, device="cuda",
                               log_alpha_min=-5.0)
    check_full(x, dtype, log_alpha_floor=-5.0)


@pytest.mark.parametrize("half", ["1", "0"])
def test_both_precision_forms(half, monkeypatch):
    """At floors >= -0.5 the bf16-input prefill takes single fp16 operands; KDA_PREFILL_HALF=0
    forces the bf16 hi/lo pairs instead.  Both forms against the oracle on varlen input with
    ragged chunks and clamped decays, at the full and a quarter slice width."""
    log(f"prefill precision form half={half}")
    monkeypatch.setenv("KDA_PREFILL_HALF", half)
    x = ki.make_prefill_inputs((300, 0, 17, 1024, 48), 4, 128, 128, "bf16", 0.05, seed=91,
                               device="cuda", log_alpha_min=-1.0)
    for nv in ("128", "32"):
        monkeypatch.setenv("KDA_PREFILL_NV", nv)
        check_full(x, "bf16", log_alpha_floor=-0.4)


def test_half_form_at_its_range_edge():
    """The fp16 form's range: with every log-decay clamped at the floor -0.5, the decay-folded
    query rows reach e^{7.5} ~ 1808 times q; q is a one-hot of size 20 per token (entries up
    to 20, ~36,000 after folding, inside fp16's 65504), k unit-norm."""
    log("prefill fp16 range edge: |q| = 20 one-hot, all decays at the floor -0.5")
    x = ki.make_prefill_inputs((160, 37), 2, 128, 128, "bf16", 0.05, seed=92, device="cuda")
    T, H, d = x.total_tokens, 2, 128
    idx = torch.arange(T * H, device="cuda") % d
    q = torch.zeros(T * H, d, device="cuda")
    q[torch.arange(T * H, device="cuda"), idx] = 20.0
    la = torch.full_like(x.log_alpha, -3.0)
    xe = ki.KdaInputs(q.view(T, H, d).to(torch.bfloat16), x.k, x.v, la, x.beta, x.gate,
                      x.cu_seqlens, x.cu_seqlens_host, x.initial_state)
    o, S = check_full(xe, "bf16", log_alpha_floor=-0.5)
    assert torch.isfinite(o.float()).all()
