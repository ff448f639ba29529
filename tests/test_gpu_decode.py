"""GPU parity of kda_decode_step against the fp64 oracle."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import linear_attention_sequence_chunked_amd as kda
import oracle
from parity import assert_close, host, log

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def decode_oracle(steps_in, S0, pairs, floor=-0.3, scale=1.0):
    """Run the oracle over the decode steps of selected (n, h) pairs as one sequence each.
    steps_in tensors are [steps, N, H, d]; returns out [steps, P, dv], S [P, dk, dv]."""
    steps = steps_in["q"].shape[0]
    sel = lambda t: np.stack([host(t[:, n, h]) for n, h in pairs], axis=0)  # [P, steps, ...]
    q, k, v, la, g = (sel(steps_in[x]) for x in ("q", "k", "v", "log_alpha", "gate"))
    b = sel(steps_in["beta"])
    P = len(pairs)
    flat = lambda a: a.reshape(P * steps, 1, *a.shape[2:]) if a.ndim > 2 else a.reshape(
        P * steps, 1)
    S0p = np.stack([host(S0[n, h]) for n, h in pairs])[:, None]
    out, Sf, _ = oracle.run(flat(q), flat(k), flat(v), flat(la), flat(b), flat(g),
                            [i * steps for i in range(P + 1)], S0p, floor, scale)
    return out.reshape(P, steps, -1).transpose(1, 0, 2), Sf[:, 0]


def run_steps(inp, state, steps, **kw):
    outs = []
    for s in range(steps):
        outs.append(kda.decode_step(inp["q"][s], inp["k"][s], inp["v"][s],
                                    inp["log_alpha"][s], inp["beta"][s], inp["gate"][s],
                                    state, **kw))
    torch.cuda.synchronize()
    return torch.stack(outs)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_decode_small(dtype, dk, dv):
    N, H, steps = 5, 3, 4
    log(f"decode small dtype={dtype} dk={dk} dv={dv}")
    inp = ki.make_decode_inputs(steps, N, H, dk, dv, dtype, seed=100 + dk + dv,
                                device="cuda")
    S0 = ki.make_state(N, H, dk, dv, 0.5, seed=7, device="cuda")
    state = S0.clone()
    out = run_steps(inp, state, steps, scale=0.8)
    pairs = [(n, h) for n in range(N) for h in range(H)]
    ro, rS = decode_oracle(inp, S0, pairs, scale=0.8)
    got_o = host(out).reshape(steps, N * H, dv)
    assert_close("o", got_o, ro, DT[dtype])
    assert_close("S", host(state).reshape(N * H, dk, dv), rS, DT[dtype])


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_decode_256_steps_match_prefill_oracle(dtype, d):
    """256 consecutive decode steps of one sequence (H=2) equal the oracle's prefill."""
    log(f"decode 256 steps dtype={dtype} d={d}")
    x = ki.make_prefill_inputs((256,), 2, d, d, dtype, 0.0, seed=31, device="cuda")
    state = torch.zeros((1, 2, d, d), dtype=torch.float32, device="cuda")
    outs = []
    for t in range(256):
        outs.append(kda.decode_step(x.q[t:t + 1], x.k[t:t + 1], x.v[t:t + 1],
                                    x.log_alpha[t:t + 1], x.beta[t:t + 1], x.gate[t:t + 1],
                                    state))
    torch.cuda.synchronize()
    o = torch.cat(outs)
    ref_o, ref_S, _ = oracle.run(host(x.q), host(x.k), host(x.v), host(x.log_alpha),
                                 host(x.beta), host(x.gate), x.cu_seqlens_host, None)
    assert_close("o", host(o), ref_o, DT[dtype])
    assert_close("S", host(state), ref_S, DT[dtype])


def test_decode_workload_1000_steps_every_pair():
    """The decode workload as specified: 256 sequences x 32 heads, 128x128 fp32 states
    (537 MB), 1000 consecutive bf16 tokens each, the state read-modify-written in place.
    Every (sequence, head) pair is traced through the oracle over all 1000 steps (32
    sequences at a time): each step's outputs, graded per step and over all steps, and
    the states after the last step."""
    N, H, d, steps = 256, 32, 128, 1000
    log("decode workload 256x32 d=128 bf16, 1000 steps, every pair")
    inp = ki.make_decode_inputs(steps, N, H, d, d, "bf16", seed=5, device="cuda")
    S0 = ki.make_state(N, H, d, d, 0.02, seed=5, device="cuda")
    state = S0.clone()
    out = torch.empty((steps, N, H, d), dtype=torch.bfloat16, device="cuda")
    for s in range(steps):
        kda.decode_step(inp["q"][s], inp["k"][s], inp["v"][s], inp["log_alpha"][s],
                        inp["beta"][s], inp["gate"][s], state, out=out[s])
    torch.cuda.synchronize()
    assert torch.isfinite(state).all() and torch.isfinite(out.float()).all()
    nb = 32
    ref_o = np.empty((steps, N, H, d), dtype=np.float32)
    for n0 in range(0, N, nb):
        # the steps of sequences n0 .. n0+nb-1 as nb sequences of `steps` tokens each
        seq = lambda t: host(t[:, n0:n0 + nb].transpose(0, 1).reshape(nb * steps, *t.shape[2:]))
        ro, rS, _ = oracle.run(seq(inp["q"]), seq(inp["k"]), seq(inp["v"]),
                               seq(inp["log_alpha"]), seq(inp["beta"]), seq(inp["gate"]),
                               [i * steps for i in range(nb + 1)], host(S0[n0:n0 + nb]))
        ref_o[:, n0:n0 + nb] = ro.reshape(nb, steps, H, d).transpose(1, 0, 2, 3)
        assert_close(f"S after {steps} steps, sequences {n0}..{n0 + nb - 1}",
                     host(state[n0:n0 + nb]), rS, torch.bfloat16)
    # graded one step at a time (each step against its own RMS), then over all steps
    # (the largest excess over the rounding bound against the RMS of every output)
    excess, sumsq, per_step = np.empty(steps), np.empty(steps), np.empty(steps)
    for s in range(steps):
        got, ref = host(out[s]).astype(np.float64), ref_o[s].astype(np.float64)
        excess[s] = np.max(np.abs(got - ref) - 2.0 ** -8 * np.abs(ref))
        sumsq[s] = np.sum(ref * ref)
        per_step[s] = max(excess[s], 0.0) / np.sqrt(sumsq[s] / ref.size)
    worst = int(np.argmax(per_step))
    total = max(float(np.max(excess)), 0.0) / np.sqrt(np.sum(sumsq) / ref_o.size)
    log(f"  o over all {steps} steps: max(|err| - 2^-8|ref|)/RMS = {total:.3e}; worst "
        f"single step {worst}: {per_step[worst]:.3e} (tol 2e-2)")
    assert total <= 2e-2 and per_step[worst] <= 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("floor", [-0.3, -0.5])
def test_decode_log_decay_below_floor(dtype, floor):
    """Log-decays drawn down to -2, floor -0.3 / -0.5: most decays are clamped."""
    N, H, d, steps = 6, 4, 128, 8
    log(f"decode below-floor decays dtype={dtype} floor={floor}")
    inp = ki.make_decode_inputs(steps, N, H, d, d, dtype, seed=41, device="cuda",
                                log_alpha_min=-2.0)
    assert float(inp["log_alpha"].float().min()) < floor - 1.0
    S0 = ki.make_state(N, H, d, d, 0.5, seed=41, device="cuda")
    state = S0.clone()
    out = run_steps(inp, state, steps, log_alpha_floor=floor, scale=0.9)
    pairs = [(n, h) for n in range(N) for h in range(H)]
    ro, rS = decode_oracle(inp, S0, pairs, floor=floor, scale=0.9)
    assert_close("o", host(out).reshape(steps, N * H, d), ro, DT[dtype])
    assert_close("S", host(state).reshape(N * H, d, d), rS, DT[dtype])


def test_decode_deterministic_and_no_stray_writes():
    N, H, d = 7, 4, 128
    log("decode determinism / guards")
    inp = ki.make_decode_inputs(1, N, H, d, d, "bf16", seed=9, device="cuda")
    S0 = ki.make_state(N, H, d, d, 0.1, seed=9, device="cuda")
    guard = 4096
    results = []
    for _ in range(2):
        buf = torch.full((N * H * d * d + 2 * guard,), 7.25, dtype=torch.float32,
                         device="cuda")
        st = buf[guard:guard + N * H * d * d].view(N, H, d, d)
        st.copy_(S0)
        obuf = torch.full((N * H * d + 2 * guard,), float("nan"), dtype=torch.bfloat16,
                          device="cuda")
        o = obuf[guard:guard + N * H * d].view(N, H, d)
        kda.decode_step(inp["q"][0], inp["k"][0], inp["v"][0], inp["log_alpha"][0],
                        inp["beta"][0], inp["gate"][0], st, out=o)
        torch.cuda.synchronize()
        assert torch.all(buf[:guard] == 7.25) and torch.all(buf[-guard:] == 7.25)
        assert torch.isnan(obuf[:guard].float()).all() and torch.isnan(obuf[-guard:].float()).all()
        assert torch.isfinite(o.float()).all()
        results.append((st.clone(), o.clone()))
    assert torch.equal(results[0][0], results[1][0])
    assert torch.equal(results[0][1], results[1][1])
