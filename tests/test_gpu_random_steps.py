"""GPU parity of the token-step paths on seeded random cases: decode, speculative verify and
commit (digest of "Kimi K3: Open Frontier Intelligence", section "基础设施": the state is
updated in place while decoding; the drafts' inputs are kept and the accepted prefix is
replayed on chip).

Each case draws, from its own seed: the input dtype, dk and dv (64 or 128), heads, the number
of sequences, the draft count K (1 to 16, around the kernels' draft buckets 4, 8 and 16), the
floor (-0.3, -0.5, -1 or -5) with log-decays down to it or 1.5 nats below it, the scale, and
each sequence's accepted count (including values below 0 and above K, which clamp).  Verify's
outputs, the outputs of K consecutive decode steps and commit's states are graded against
the fp64 oracle; commit must equal the same number of decode steps bit for bit, and so must
verify where it runs step by step."""
import os

import numpy as np
import pytest
import torch

import test_gpu_spec as spec
from parity import assert_close, host, log

import linear_attention_sequence_chunked_amd as kda

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def draw(seed: int) -> dict:
    rng = np.random.default_rng(20_000 + seed)
    K = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 12, 15, 16]))
    N = int(rng.integers(1, 9))
    floor = float(rng.choice([-0.3, -0.5, -1.0, -5.0]))
    return dict(dtype=("bf16", "f32")[seed % 2], dk=int(rng.choice([64, 128])),
                dv=int(rng.choice([64, 128])), H=int(rng.integers(1, 4)), N=N, K=K,
                floor=floor, la_min=float(rng.choice([floor, max(floor - 1.5, -5.0)])),
                scale=float(rng.uniform(0.5, 1.2)),
                accepted=[int(a) for a in rng.integers(-1, K + 3, size=N)])


@pytest.mark.parametrize("seed", range(32))
def test_random_decode_verify_commit(seed):
    c = draw(seed)
    log(f"random steps seed={seed}: {c}")
    N, K, floor, scale = c["N"], c["K"], c["floor"], c["scale"]
    x = spec.drafts(N, K, c["H"], c["dk"], c["dv"], c["dtype"], seed=700 + seed,
                    log_alpha_min=c["la_min"])
    dt = DT[c["dtype"]]
    a = c["accepted"]
    state = x.initial_state.clone()
    o = kda.spec_verify(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, state,
                        log_alpha_floor=floor, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(state, x.initial_state), "verify wrote the state"
    acc = torch.tensor(a, dtype=torch.int32, device="cuda")
    kda.spec_commit(x.k, x.v, x.log_alpha, x.beta, state, acc, log_alpha_floor=floor)
    torch.cuda.synchronize()
    ro, rS = spec.oracle_after(x, K, a, floor, scale)
    assert_close("o (verify)", host(o), ro, dt)
    assert_close("S (commit)", host(state), rS, dt)
    do, dS = spec.decode_steps(x, N, K, a, floor, scale)
    torch.cuda.synchronize()
    assert_close("o (decode steps)", host(do), ro, dt)
    assert torch.equal(state, dS), "commit differs from consecutive decode steps"
    chunk_form = c["dtype"] == "bf16" and floor >= -0.5 and os.environ.get("KDA_PREFILL_HALF") != "0"
    if not chunk_form:
        assert torch.equal(o, do), "verify differs from consecutive decode steps"
