"""The two precision forms of the bf16-input prefill, emulated on the CPU against the oracle
(tests/rounding_emulation.py): both meet the tolerance the GPU tests apply, and the half
form's decay-folded tiles stay inside fp16's range at the floors it is used for."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from rounding_emulation import prefill


def _head(T, seed, floor, log_alpha_min=-0.3):
    x = ki.make_prefill_inputs((T,), 1, 128, 128, "bf16", 0.02, seed=seed, device="cpu",
                               log_alpha_min=log_alpha_min)
    f = lambda t: t.float().numpy().astype(np.float64)
    args = [f(t)[:, 0] for t in (x.q, x.k, x.v, x.log_alpha, x.beta, x.gate)]
    S0 = f(x.initial_state)[0, 0]
    ro, rS, _ = oracle.run(*[a[:, None] if a.ndim == 1 else a[:, None, :] for a in args],
                           [0, T], S0[None, None], floor, 1.0)
    return args, S0, ro[:, 0], rS[0, 0]


def _errors(o, S, ro, rS):
    rms = np.sqrt(np.mean(ro ** 2))
    out = max(float(np.max(np.abs(o - ro) - 2.0 ** -8 * np.abs(ro))), 0.0) / rms
    st = float(np.max(np.abs(S - rS))) / np.sqrt(np.mean(rS ** 2))
    return out, st


@pytest.mark.parametrize("floor,log_alpha_min", [(-0.3, -0.3), (-0.5, -2.0)])
def test_both_forms_meet_the_tolerance(floor, log_alpha_min):
    args, S0, ro, rS = _head(4096, seed=11, floor=floor, log_alpha_min=log_alpha_min)
    for form in ("half", "split"):
        o, S = prefill(*args, S0, floor=floor, form=form)
        e_o, e_S = _errors(o, S, ro, rS)
        print(f"{form} floor={floor}: outputs {e_o:.2e}, final state {e_S:.2e} of RMS")
        # the GPU bar is 2e-2; the emulation must leave at least a 2x margin
        assert e_o <= 1e-2 and e_S <= 1e-2


def test_half_form_range_at_its_lowest_floor():
    """Every decay at the floor -0.5: row 0 of a chunk is scaled by e^{7.5} ~ 1808, so the
    fp16 Qt of a q entry of 20 stays finite (36,155 < 65504)."""
    F = np.exp(15 * 0.5)
    assert 20 * F < 65504 < 40 * F
    with np.errstate(over="ignore"):
        assert np.isfinite(np.float16(20 * F)) and not np.isfinite(np.float16(40 * F))
