"""GPU parity of kda_prefill_backward on seeded random varlen batches, against the oracle's
reverse-mode gradients (oracle/reference.py recurrent_backward, pinned by finite differences)
with the tolerance of tests/test_gpu_backward.py (32 * 2^-16 of RMS per gradient tensor).

Each case draws, from its own seed: the input dtype, dk and dv (64 or 128), heads, one to four
sequence lengths (chunk-edge lengths mixed with lengths up to 300, so that chunk pairs with and
without a second chunk occur), the floor (-0.3 to -5) with log-decays down to it or below it,
the scale, and whether an initial state and a final-state gradient are given."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import test_gpu_backward as bw
from parity import log

pytestmark = pytest.mark.gpu
EDGE_LENGTHS = [0, 1, 15, 16, 17, 32, 33, 48]


def draw(seed: int) -> dict:
    rng = np.random.default_rng(30_000 + seed)
    n = int(rng.integers(1, 5))
    lengths = [int(rng.choice(EDGE_LENGTHS)) if rng.random() < 0.5 else int(rng.integers(1, 301))
               for _ in range(n)]
    floor = float(rng.choice([-0.3, -0.4, -0.5, -1.0, -5.0]))
    return dict(dtype=("bf16", "f32")[seed % 2], dk=int(rng.choice([64, 128])),
                dv=int(rng.choice([64, 128])), H=int(rng.integers(1, 4)), lengths=lengths,
                floor=floor, la_min=float(rng.choice([floor, max(floor - 1.0, -5.0)])),
                scale=float(rng.uniform(0.5, 1.2)), s0=bool(rng.random() < 0.7),
                dsf=bool(rng.random() < 0.7))


@pytest.mark.parametrize("seed", range(16))
def test_random_backward(seed):
    c = draw(seed)
    log(f"random backward seed={seed}: {c}")
    x = ki.make_prefill_inputs(c["lengths"], c["H"], c["dk"], c["dv"], c["dtype"],
                               0.3 if c["s0"] else 0.0, seed=900 + seed, device="cuda",
                               log_alpha_min=c["la_min"])
    g = torch.Generator().manual_seed(900 + seed)
    do = (torch.randn(x.v.shape, generator=g) * 0.5).to(x.v.dtype).cuda()
    N = len(c["lengths"])
    dSf = None
    if c["dsf"]:
        dSf = (torch.randn((N, c["H"], c["dk"], c["dv"]), generator=g) * 0.1).cuda()
    bw.run_case(x, do, dSf, floor=c["floor"], scale=c["scale"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("lengths,s0,dsf", [((1,), False, False), ((1, 1), False, False),
                                            ((0,), True, False), ((0,), False, True),
                                            ((0, 1), False, True)])
def test_backward_degenerate_batches(dtype, lengths, s0, dsf):
    """Batches whose oracle gradients vanish or are empty: one-token sequences without S0 and
    dS_final (no decay gradient: the decay multiplies a zero state), and empty sequences (no
    token gradients; dS0 is dS_final passed through, or zero)."""
    log(f"backward degenerate dtype={dtype} lengths={lengths} s0={s0} dsf={dsf}")
    x = ki.make_prefill_inputs(lengths, 2, 64, 64, dtype, 0.3 if s0 else 0.0, seed=41,
                               device="cuda", log_alpha_min=-0.5)
    g = torch.Generator().manual_seed(41)
    do = (torch.randn(x.v.shape, generator=g) * 0.5).to(x.v.dtype).cuda()
    dSf = (torch.randn((len(lengths), 2, 64, 64), generator=g) * 0.1).cuda() if dsf else None
    bw.run_case(x, do, dSf, floor=-0.5, scale=0.9)
