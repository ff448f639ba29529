"""GPU parity of kda_prefill_backward against the oracle's reverse-mode gradients
(oracle/reference.py recurrent_backward, pinned by finite differences in
tests/test_oracle_backward.py), per (sequence, head), on the same rounded inputs.

The GPU walks the recurrence in fp32 whatever the input dtype, so one tolerance applies:
max|err| <= 1e-3 * RMS(ref) per gradient tensor."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import linear_attention_sequence_chunked_amd as kda
from oracle import reference as ref
from parity import host, log

pytestmark = pytest.mark.gpu
TOL = 1e-3


def check(name, got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    rms = float(np.sqrt(np.mean(want * want)))
    err = float(np.max(np.abs(got - want))) / max(rms, 1e-30)
    log(f"  {name}: max|err|/RMS = {err:.2e}")
    assert err <= TOL, f"{name}: {err:.3e} > {TOL}"


def run_case(x, do, dSf, floor, scale, pairs=None):
    g = kda.prefill_backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, do,
                             cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_seqlens_host,
                             initial_state=x.initial_state, d_final_state=dSf,
                             log_alpha_floor=floor, scale=scale)
    torch.cuda.synchronize()
    cu = x.cu_seqlens_host
    H = x.q.shape[1]
    N = len(cu) - 1
    pairs = pairs or [(n, h) for n in range(N) for h in range(H)]
    want = {k: [] for k in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dgate", "dS0")}
    got = {k: [] for k in want}
    for n, h in pairs:
        a, e = cu[n], cu[n + 1]
        sl = lambda t: host(t[a:e, h])
        r = ref.recurrent_backward(sl(x.q), sl(x.k), sl(x.v), sl(x.log_alpha), sl(x.beta),
                                   sl(x.gate), sl(do),
                                   None if dSf is None else host(dSf[n, h]),
                                   None if x.initial_state is None else host(x.initial_state[n, h]),
                                   floor=floor, scale=scale)
        for key, gk in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dlog_alpha", "dlog_alpha"),
                        ("dbeta", "dbeta"), ("dgate", "dgate")):
            want[key].append(r[key].reshape(-1))
            got[key].append(host(g[gk][a:e, h]).reshape(-1))
        want["dS0"].append(r["dS0"].reshape(-1))
        got["dS0"].append(host(g["d_initial_state"][n, h]).reshape(-1))
    for key in want:
        check(key, np.concatenate(got[key]), np.concatenate(want[key]))
    return g


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_backward_varlen(dtype, dk, dv):
    lengths = (37, 0, 16, 1, 50)
    log(f"backward dtype={dtype} dk={dk} dv={dv}")
    x = ki.make_prefill_inputs(lengths, 2, dk, dv, dtype, 0.3, seed=dk + 2 * dv,
                               device="cuda", log_alpha_min=-0.6)
    g = torch.Generator().manual_seed(dk + dv)
    do = (torch.randn(x.v.shape, generator=g) * 0.5).to(x.v.dtype).cuda()
    dSf = (torch.randn(x.initial_state.shape, generator=g) * 0.1).cuda()
    # floor -0.4: part of the log-decays (drawn down to -0.6) are clamped
    run_case(x, do, dSf, floor=-0.4, scale=0.8)


def test_backward_no_initial_state_no_state_gradient():
    x = ki.make_prefill_inputs((70, 33), 2, 64, 64, "bf16", 0.0, seed=9, device="cuda")
    assert x.initial_state is None
    g = torch.Generator().manual_seed(9)
    do = torch.randn(x.v.shape, generator=g).to(x.v.dtype).cuda()
    run_case(x, do, None, floor=-0.3, scale=1.0)


def test_backward_bench_workload_sampled():
    """B=4, H=16, T=4096, d=128, bf16: two (sequence, head) pairs against the oracle."""
    w = ki.WORKLOADS["prefill_b4_h16_t4096"]
    log("backward on prefill_b4_h16_t4096 (sampled)")
    x = ki.make_workload_inputs(w, seed=1, device="cuda")
    g = torch.Generator().manual_seed(1)
    do = torch.randn(x.v.shape, generator=g).to(x.v.dtype).cuda()
    run_case(x, do, None, floor=-0.3, scale=1.0, pairs=[(0, 3), (3, 12)])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_strongest_decay_floor(dtype):
    """Floor -5 with log-decays drawn down to -5: decay-folded operands span ~e^80 within a
    chunk (finite in fp32 and in bf16 hi/lo pairs)."""
    log(f"backward floor=-5 dtype={dtype}")
    x = ki.make_prefill_inputs((40, 64, 17), 2, 128, 128, dtype, 0.3, seed=56, device="cuda",
                               log_alpha_min=-5.0)
    g = torch.Generator().manual_seed(56)
    do = torch.randn(x.v.shape, generator=g).to(x.v.dtype).cuda()
    dSf = (torch.randn(x.initial_state.shape, generator=g) * 0.1).cuda()
    run_case(x, do, dSf, floor=-5.0, scale=1.0)
