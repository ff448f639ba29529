"""GPU parity of speculative verify / commit (digest of "Kimi K3: Open Frontier
Intelligence", section "基础设施": drafts' inputs kept, accepted prefix replayed on chip,
no per-draft state stored).

Verify outputs are checked against the oracle's token loop over the K drafts from the
stored state; commit is checked for every accepted length 0..K (and clamped values)
against the oracle's state after that many drafts.  Commit is also compared bit for bit
with the same number of kda_decode_step calls, which compute each step in the same order,
and so is verify where it runs step by step (fp32 drafts, floors below -0.5, or
KDA_PREFILL_HALF=0); bf16 drafts at floors >= -0.5 are verified in chunk form on the
matrix core, which sums in another order."""
import os

import numpy as np
import pytest
import torch

import kda_inputs as ki
import linear_attention_sequence_chunked_amd as kda
import oracle
from parity import assert_close, host, log

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def drafts(N, K, H, dk, dv, dtype, seed, log_alpha_min=-0.3):
    """N sequences of K drafts, packed sequence-major ([N*K, H, .]), plus states."""
    x = ki.make_prefill_inputs((K,) * N, H, dk, dv, dtype, 0.3, seed=seed, device="cuda",
                               log_alpha_min=log_alpha_min)
    return x


def oracle_after(x, K, a, floor, scale):
    """Oracle outputs [N*K, H, dv] over all K drafts and states after the first a[n]."""
    hs = lambda t: host(t)
    out, _, _ = oracle.run(hs(x.q), hs(x.k), hs(x.v), hs(x.log_alpha), hs(x.beta), hs(x.gate),
                           x.cu_seqlens_host, hs(x.initial_state), floor, scale)
    N = len(x.cu_seqlens_host) - 1
    states = []
    for n in range(N):
        an = min(max(int(a[n]), 0), K)
        sl = lambda t: hs(t[n * K:n * K + an])
        _, Sf, _ = oracle.run(sl(x.q), sl(x.k), sl(x.v), sl(x.log_alpha), sl(x.beta),
                              sl(x.gate), [0, an], hs(x.initial_state[n:n + 1]), floor, scale)
        states.append(Sf[0])
    return out, np.stack(states)


def decode_steps(x, N, K, a, floor, scale):
    """a[n] kda_decode_step calls per sequence on a copy of the states (drafts as the
    per-step tokens); returns (outputs of all K steps [N*K, H, dv], states after a[n])."""
    H, dv = x.v.shape[1], x.v.shape[2]
    st = x.initial_state.clone()
    outs = torch.empty_like(x.v)
    res = torch.empty_like(st)
    per = lambda t, j: t.view(N, K, *t.shape[1:])[:, j].contiguous()
    for j in range(K + 1):
        for n in range(N):
            if min(max(int(a[n]), 0), K) == j:
                res[n] = st[n]
        if j == K:
            break
        o = kda.decode_step(per(x.q, j), per(x.k, j), per(x.v, j), per(x.log_alpha, j),
                            per(x.beta, j), per(x.gate, j), st, log_alpha_floor=floor,
                            scale=scale)
        outs.view(N, K, H, dv)[:, j] = o
    return outs, res


def verify_and_commit_case(dtype, dk, dv, K, floor, log_alpha_min):
    N, H = K + 3, 2
    x = drafts(N, K, H, dk, dv, dtype, seed=100 + K + dk, log_alpha_min=log_alpha_min)
    scale = 0.9
    # every length 0..K once, then values past both ends (clamped)
    a = list(range(K + 1)) + [K + 5, -2]
    assert len(a) == N
    acc = torch.tensor(a, dtype=torch.int32, device="cuda")
    state = x.initial_state.clone()
    o = kda.spec_verify(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, state,
                        log_alpha_floor=floor, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(state, x.initial_state), "verify wrote the state"
    kda.spec_commit(x.k, x.v, x.log_alpha, x.beta, state, acc, log_alpha_floor=floor)
    torch.cuda.synchronize()
    ro, rS = oracle_after(x, K, a, floor, scale)
    assert_close("o (verify)", host(o), ro, DT[dtype])
    assert_close("S (commit)", host(state), rS, DT[dtype])
    assert torch.equal(state[0], x.initial_state[0]), "accepted = 0 changed the state"
    assert torch.equal(state[N - 1], x.initial_state[N - 1]), "accepted < 0 changed the state"
    do, dS = decode_steps(x, N, K, a, floor, scale)
    torch.cuda.synchronize()
    chunk_form = dtype == "bf16" and floor >= -0.5 and os.environ.get("KDA_PREFILL_HALF") != "0"
    if not chunk_form:
        assert torch.equal(o, do), "verify differs from consecutive decode steps"
    assert torch.equal(state, dS), "commit differs from consecutive decode steps"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("K", [1, 4, 16])
def test_verify_and_every_accepted_length(dtype, dk, dv, K):
    log(f"spec dtype={dtype} dk={dk} dv={dv} K={K}")
    verify_and_commit_case(dtype, dk, dv, K, floor=-0.4, log_alpha_min=-0.3)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("floor", [-0.3, -0.5])
@pytest.mark.parametrize("K", [4, 16])
def test_log_decay_below_floor(dtype, floor, K):
    """Draft log-decays drawn down to -2 with the floor at -0.3 / -0.5."""
    log(f"spec below-floor decays dtype={dtype} floor={floor} K={K}")
    verify_and_commit_case(dtype, 128, 128, K, floor=floor, log_alpha_min=-2.0)


@pytest.mark.parametrize("K", [1, 4, 16])
def test_step_by_step_verify_when_forced(K, monkeypatch):
    """KDA_PREFILL_HALF=0 keeps bf16 verify on the step-by-step kernel: oracle parity and
    bit-for-bit agreement with consecutive decode steps."""
    log(f"spec bf16 step-by-step verify K={K}")
    monkeypatch.setenv("KDA_PREFILL_HALF", "0")
    verify_and_commit_case("bf16", 128, 128, K, floor=-0.3, log_alpha_min=-2.0)


def test_decode_workload_with_four_drafts():
    """The decode workload's states (256 sequences x 32 heads, d=128, fp32) with K = 4
    bf16 drafts and random accepted lengths: sampled heads against the oracle."""
    N, H, d, K = 256, 32, 128, 4
    log("spec on decode_n256_h32, K=4")
    x = drafts(N, K, H, d, d, "bf16", seed=5)
    g = torch.Generator().manual_seed(5)
    a = torch.randint(0, K + 1, (N,), generator=g).tolist()
    acc = torch.tensor(a, dtype=torch.int32, device="cuda")
    state = x.initial_state.clone()
    o = kda.spec_verify(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, state)
    kda.spec_commit(x.k, x.v, x.log_alpha, x.beta, state, acc)
    torch.cuda.synchronize()
    for n in (0, 77, 255):
        for h in (0, 31):
            sl = lambda t: host(t[n * K:(n + 1) * K, h:h + 1])
            ro, _, _ = oracle.run(sl(x.q), sl(x.k), sl(x.v), sl(x.log_alpha), sl(x.beta),
                                  sl(x.gate), [0, K], host(x.initial_state[n:n + 1, h:h + 1]))
            assert_close(f"o n={n} h={h}", host(o[n * K:(n + 1) * K, h:h + 1]), ro,
                         torch.bfloat16)
            sa = lambda t: host(t[n * K:n * K + a[n], h:h + 1])
            _, rS, _ = oracle.run(sa(x.q), sa(x.k), sa(x.v), sa(x.log_alpha), sa(x.beta),
                                  sa(x.gate), [0, a[n]], host(x.initial_state[n:n + 1, h:h + 1]))
            assert_close(f"S n={n} h={h} a={a[n]}", host(state[n, h:h + 1]), rS[0],
                         torch.bfloat16)


def test_chunk_form_verify_at_its_range_edge():
    """Verify in chunk form with every draft decay at the floor -0.5 and q entries of 20
    (one-hot rows): the operands that meet the state are bounded by q and k, and k e^{-G}
    stays below e^8 times k; outputs against the oracle."""
    N, K, H, d = 6, 16, 2, 128
    log("spec chunk-form verify at the fp16 range edge")
    x = drafts(N, K, H, d, d, "bf16", seed=31, log_alpha_min=-3.0)
    T = N * K
    q = torch.zeros(T * H, d, device="cuda")
    q[torch.arange(T * H, device="cuda"), torch.arange(T * H, device="cuda") % d] = 20.0
    xe = ki.KdaInputs(q.view(T, H, d).to(torch.bfloat16), x.k, x.v,
                      torch.full_like(x.log_alpha, -3.0), x.beta, x.gate, x.cu_seqlens,
                      x.cu_seqlens_host, x.initial_state)
    state = xe.initial_state.clone()
    o = kda.spec_verify(xe.q, xe.k, xe.v, xe.log_alpha, xe.beta, xe.gate, state,
                        log_alpha_floor=-0.5)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    ro, _ = oracle_after(xe, K, [0] * N, -0.5, 1.0)
    assert_close("o (verify, range edge)", host(o), ro, torch.bfloat16)
