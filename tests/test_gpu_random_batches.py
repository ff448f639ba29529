"""GPU parity on seeded random varlen batches, through every prefill entry point.

Each case draws, from its own seed: the input dtype, dk and dv (64 or 128), the head count,
one to six sequence lengths (chunk-boundary lengths 0, 1, 15, 16, 17, 31, 33, ... mixed with
lengths up to 600), the decay floor (-0.3, -0.5, -1 or -5; the floor is the lower bound on
the per-step log-decay of the digest of "Kimi K3: Open Frontier Intelligence", section
"KDA：百万上下文先要过「数值 算子」这一关", Fig. 3(a)), log-decays drawn down to the floor or
1.5 nats below it, an initial state (none, std 0.02 or 0.3) and a scale.  The same batch then
runs through the plain prefill, the segmented schedule with a short forced segment length,
and the snapshot variant; each is graded against the fp64 oracle with the bars of
tests/parity.py, and the snapshot variant's outputs must equal the plain prefill's bit for
bit."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import linear_attention_sequence_chunked_amd as kda
import oracle
from parity import assert_close, host, log, oracle_full

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}
EDGE_LENGTHS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 47, 129]


def draw(seed: int) -> dict:
    rng = np.random.default_rng(10_000 + seed)
    n = int(rng.integers(1, 7))
    lengths = [int(rng.choice(EDGE_LENGTHS)) if rng.random() < 0.5 else int(rng.integers(1, 601))
               for _ in range(n)]
    floor = float(rng.choice([-0.3, -0.5, -1.0, -5.0]))
    return dict(dtype=("bf16", "f32")[seed % 2], dk=int(rng.choice([64, 128])),
                dv=int(rng.choice([64, 128])), H=int(rng.integers(1, 4)), lengths=lengths,
                floor=floor, la_min=float(rng.choice([floor, max(floor - 1.5, -5.0)])),
                s0=float(rng.choice([0.0, 0.02, 0.3])), scale=float(rng.uniform(0.5, 1.2)),
                seg=16 * int(rng.integers(1, 9)), m=16 * int(rng.integers(1, 5)))


@pytest.mark.parametrize("seed", range(48))
def test_random_batch_every_prefill_entry_point(seed):
    c = draw(seed)
    log(f"random batch seed={seed}: {c}")
    x = ki.make_prefill_inputs(c["lengths"], c["H"], c["dk"], c["dv"], c["dtype"], c["s0"],
                               seed=500 + seed, device="cuda", log_alpha_min=c["la_min"])
    kw = dict(log_alpha_floor=c["floor"], scale=c["scale"])
    ro, rS = oracle_full(x, floor=c["floor"], scale=c["scale"])
    dt = DT[c["dtype"]]
    args = (x.q, x.k, x.v, x.log_alpha, x.beta, x.gate)

    # plain schedule
    o, S = kda.chunk_prefill(*args, cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_seqlens_host,
                             initial_state=x.initial_state, segment_len=0, **kw)
    torch.cuda.synchronize()
    if x.total_tokens:
        assert_close("o (plain)", host(o), ro, dt)
    assert_close("S_T (plain)", host(S), rS, dt)

    # segmented schedule, forced short segments
    so, sS = kda.chunk_prefill_segmented(*args, x.cu_seqlens_host, c["seg"],
                                         initial_state=x.initial_state, **kw)
    torch.cuda.synchronize()
    if x.total_tokens:
        assert_close(f"o (segments of {c['seg']})", host(so), ro, dt)
    assert_close(f"S_T (segments of {c['seg']})", host(sS), rS, dt)

    # snapshot variant: the same outputs bit for bit, and every snapshot a prefix state
    m = c["m"]
    ck = torch.full((x.total_tokens // m, c["H"], c["dk"], c["dv"]), float("nan"), device="cuda")
    co, cS, _ = kda.chunk_prefill(*args, cu_seqlens=x.cu_seqlens,
                                  cu_seqlens_host=x.cu_seqlens_host,
                                  initial_state=x.initial_state, checkpoint_every=m,
                                  checkpoints=ck, segment_len=0, **kw)
    torch.cuda.synchronize()
    assert torch.equal(co, o) and torch.equal(cS, S), "snapshot variant differs from the plain one"
    cu = x.cu_seqlens_host
    for n, T_n in enumerate(c["lengths"]):
        for j in range(1, T_n // m + 1):
            a = cu[n]
            sl = lambda t: host(t[a:a + j * m])
            S0 = None if x.initial_state is None else host(x.initial_state[n:n + 1])
            _, ref, _ = oracle.run(sl(x.q), sl(x.k), sl(x.v), sl(x.log_alpha), sl(x.beta),
                                   sl(x.gate), [0, j * m], S0, c["floor"], c["scale"])
            assert_close(f"snapshot n={n} t={j * m}", host(ck[kda.checkpoint_slot(cu, n, j, m)]),
                         ref[0], dt)
