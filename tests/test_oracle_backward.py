"""Pins for the oracle's backward pass (oracle/reference.py recurrent_backward).

The gradients are checked against central finite differences of the pinned forward
recurrence in fp64 (an independent derivative: no shared algebra with the reverse-mode
code), on several tiny configurations, including log-decays below the floor (where the
clamp passes no gradient).  Deliberately broken copies of the reverse code (mutants)
must each fail that check."""
import inspect

import numpy as np
import pytest

from oracle import reference as ref

pytestmark = pytest.mark.filterwarnings("ignore")


def _inputs(seed, T=6, dk=4, dv=3, below_floor=False):
    rng = np.random.default_rng(seed)
    x = dict(q=rng.standard_normal((T, dk)), k=rng.standard_normal((T, dk)) / 2,
             v=rng.standard_normal((T, dv)), log_alpha=-rng.random((T, dk)) * 0.25 - 0.01,
             beta=rng.random(T), gate=rng.random((T, dv)), S0=rng.standard_normal((dk, dv)))
    if below_floor:  # a third of the entries sit well below the floor
        mask = rng.random((T, dk)) < 0.33
        x["log_alpha"] = np.where(mask, -0.8, x["log_alpha"])
    do = rng.standard_normal((T, dv))
    dS_T = rng.standard_normal((dk, dv))
    return x, do, dS_T


def _loss(x, do, dS_T, floor, scale):
    o, S = ref.recurrent(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["gate"], x["S0"],
                         floor=floor, scale=scale)
    return float(np.sum(do * o) + np.sum(dS_T * S))


def _fd_error(bwd, x, do, dS_T, floor, scale, h=1e-6):
    g = bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["gate"], do, dS_T, x["S0"],
            floor=floor, scale=scale)
    worst = 0.0
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_alpha", "dlog_alpha"),
                      ("beta", "dbeta"), ("gate", "dgate"), ("S0", "dS0")):
        num = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp, xm = dict(x), dict(x)
            xp[name] = x[name].copy(); xp[name][idx] += h
            xm[name] = x[name].copy(); xm[name][idx] -= h
            num[idx] = (_loss(xp, do, dS_T, floor, scale) - _loss(xm, do, dS_T, floor, scale)) / (2 * h)
        err = np.max(np.abs(num - g[key])) / max(np.max(np.abs(num)), 1e-12)
        worst = max(worst, err)
    return worst


@pytest.mark.parametrize("seed,floor,scale,below", [(0, -0.3, 1.0, False), (1, -0.3, 0.7, False),
                                                   (2, -0.5, 1.3, True), (3, -0.05, 1.0, True)])
def test_backward_matches_finite_differences(seed, floor, scale, below):
    x, do, dS_T = _inputs(seed, below_floor=below)
    assert _fd_error(ref.recurrent_backward, x, do, dS_T, floor, scale) < 1e-7


def test_backward_without_state_gradient_or_initial_state():
    x, do, _ = _inputs(7)
    x["S0"] = np.zeros_like(x["S0"])
    assert _fd_error(ref.recurrent_backward, x, do, np.zeros((4, 3)), -0.3, 1.0) < 1e-7


def test_clamped_decay_passes_no_gradient():
    x, do, dS_T = _inputs(5, below_floor=True)
    g = ref.recurrent_backward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["gate"], do,
                               dS_T, x["S0"], floor=-0.3)
    assert np.all(g["dlog_alpha"][x["log_alpha"] < -0.3] == 0)
    assert np.any(g["dlog_alpha"][x["log_alpha"] > -0.3] != 0)


MUTANTS = {
    "state gradient not decayed": ("dS = a[:, None] * dSp", "dS = dSp"),
    "erase gradient sign": ("dw = -beta[t] * du", "dw = beta[t] * du"),
    "clamp mask dropped": ("out[\"dlog_alpha\"][t] = da * a * (la[t] > floor)",
                           "out[\"dlog_alpha\"][t] = da * a"),
    "key gradient from the undecayed state": ("dkt = dkt + Sp @ dw", "dkt = dkt + Sprev @ dw"),
    "readout gradient misses the gate": ("dy = do[t] * g[t]", "dy = do[t]"),
    "beta gradient from v only": ("out[\"dbeta\"][t] = du @ (v[t] - w)", "out[\"dbeta\"][t] = du @ v[t]"),
}


@pytest.mark.parametrize("kind", sorted(MUTANTS))
def test_finite_differences_catch_backward_mutant(kind):
    old, new = MUTANTS[kind]
    src = inspect.getsource(ref.recurrent_backward)
    assert old in src, kind
    ns = dict(np=np, _as64=ref._as64)
    exec(src.replace(old, new), ns)
    x, do, dS_T = _inputs(11, below_floor=True)
    assert _fd_error(ns["recurrent_backward"], x, do, dS_T, -0.3, 0.9) > 1e-3, kind
