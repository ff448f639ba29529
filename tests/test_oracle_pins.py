"""Pins for the oracle: checks against facts that the pages and the mathematics fix.

Every pin is written as a function of an implementation `impl(q, k, v, la, beta, g, S0,
floor, scale) -> (o, S_T)` for ONE (sequence, head), so the same pins run against the C
fp64 oracle, the numpy token loop, and deliberately broken variants (mutants) that must
each fail at least one pin.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import reference as ref

HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------------------- impls
def c_impl(q, k, v, la, beta, g, S0=None, floor=-0.3, scale=1.0):
    """The C oracle on one (sequence, head)."""
    T, dk = np.shape(q)
    dv = np.shape(v)[1]
    out, Sf, _ = oracle.run(np.reshape(q, (T, 1, dk)), np.reshape(k, (T, 1, dk)),
                            np.reshape(v, (T, 1, dv)), np.reshape(la, (T, 1, dk)),
                            np.reshape(beta, (T, 1)), np.reshape(g, (T, 1, dv)), [0, T],
                            None if S0 is None else np.reshape(S0, (1, 1, dk, dv)),
                            floor, scale, nthreads=1)
    return out[:, 0], Sf[0, 0]


def np_impl(q, k, v, la, beta, g, S0=None, floor=-0.3, scale=1.0):
    return ref.recurrent(q, k, v, la, beta, g, S0, floor, scale)


IMPLS = {"c_oracle": c_impl, "numpy_loop": np_impl}


# ----------------------------------------------------------------------------- data
def rand_case(T, dk, dv, seed, unit_keys=True, floor_hits=True, s0=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, dk))
    k = r.standard_normal((T, dk))
    if unit_keys:
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((T, dv))
    beta = 1 / (1 + np.exp(-r.standard_normal(T)))
    la = -np.log1p(np.exp(r.standard_normal((T, dk))))  # -softplus
    if not floor_hits:
        la = np.maximum(la, -0.3)
    g = 1 / (1 + np.exp(-r.standard_normal((T, dv))))
    S0 = 0.5 * r.standard_normal((dk, dv)) if s0 else None
    # values exactly representable in float32 (the C oracle takes float32 inputs)
    f = lambda x: None if x is None else np.asarray(x, np.float32).astype(np.float64)
    return [f(x) for x in (q, k, v, la, beta, g, S0)]


# ----------------------------------------------------------------------------- pins
def pin_golden_onehot(impl):
    """Worked instance of the beta=0.7 update figure (hand-computed fixture)."""
    d = json.load(open(os.path.join(HERE, "golden", "onehot_beta07.json")))
    o, S = impl(np.array([d["q"]]), np.array([d["k"]]), np.array([d["v"]]),
                np.array([d["log_alpha"]]), np.array([d["beta"]]), np.array([d["gate"]]),
                np.array(d["S0"]), -0.3, 1.0)
    np.testing.assert_allclose(S, np.array(d["expected_S1"]), rtol=0, atol=1e-6)
    np.testing.assert_allclose(o[0], np.array(d["expected_o"]), rtol=0, atol=1e-6)


def pin_single_token_from_zero(impl):
    """From S0 = 0, one token: S_1 = beta k v^T and o_1 = g * (beta (k.q) v)."""
    q, k, v, la, beta, g, _ = rand_case(1, 5, 4, seed=11)
    o, S = impl(q, k, v, la, beta, g, None, -0.3, 1.0)
    np.testing.assert_allclose(S, beta[0] * np.outer(k[0], v[0]), atol=1e-6)
    np.testing.assert_allclose(o[0], g[0] * beta[0] * (k[0] @ q[0]) * v[0], atol=1e-6)


def pin_pure_decay(impl):
    """beta = 0: S_t = Diag(exp(sum_{s<=t} max(lambda_s, floor))) S0, o_t = g_t*(S_t^T q_t)."""
    q, k, v, la, beta, g, S0 = rand_case(9, 6, 5, seed=12)
    beta = np.zeros_like(beta)
    floor = -0.4
    o, S = impl(q, k, v, la, beta, g, S0, floor, 1.0)
    cum = np.cumsum(np.maximum(la, floor), axis=0)          # [T, dk]
    for t in range(len(q)):
        St = np.exp(cum[t])[:, None] * S0
        np.testing.assert_allclose(o[t], g[t] * (q[t] @ St), rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(S, np.exp(cum[-1])[:, None] * S0, rtol=1e-7, atol=1e-9)


def pin_identity_gemm(impl):
    """alpha = 1, beta = 0 (dk != dv): the state never changes and o = g * (scale Q S0)."""
    q, k, v, la, beta, g, S0 = rand_case(7, 6, 3, seed=13)
    la = np.zeros_like(la)
    beta = np.zeros_like(beta)
    o, S = impl(q, k, v, la, beta, g, S0, -0.3, 0.75)
    np.testing.assert_allclose(S, S0, atol=0)
    np.testing.assert_allclose(o, g * (0.75 * q @ S0), rtol=1e-12, atol=1e-12)


def pin_unit_key_recall(impl):
    """alpha = 1, beta = 1, |k| = 1: after each write, S_t^T k_t = v_t."""
    q, k, v, la, beta, g, S0 = rand_case(6, 8, 4, seed=14)
    la = np.zeros_like(la)
    beta = np.ones_like(beta)
    k = k / np.linalg.norm(k, axis=1, keepdims=True)
    for t in range(1, len(q) + 1):
        _, S = impl(q[:t], k[:t], v[:t], la[:t], beta[:t], g[:t], S0, -0.3, 1.0)
        np.testing.assert_allclose(S.T @ k[t - 1], v[t - 1], atol=1e-6)


def pin_orthonormal_keys(impl):
    """alpha = 1, beta = 1, orthonormal keys: S = (I - sum k k^T) S0 + sum k v^T."""
    r = np.random.default_rng(15)
    dk, dv, m = 7, 3, 4
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    k = Qm[:, :m].T.copy()
    q = r.standard_normal((m, dk))
    v = r.standard_normal((m, dv))
    g = np.ones((m, dv))
    S0 = r.standard_normal((dk, dv))
    _, S = impl(q, k, v, np.zeros((m, dk)), np.ones(m), g, S0, -0.3, 1.0)
    expect = (np.eye(dk) - k.T @ k) @ S0 + k.T @ v
    np.testing.assert_allclose(S, expect, atol=1e-6)


def pin_dplr_brute_force(impl):
    """Dense Diagonal-Plus-Low-Rank products multiplied out equal the recurrence."""
    q, k, v, la, beta, g, S0 = rand_case(7, 4, 3, seed=16)
    o, S = impl(q, k, v, la, beta, g, S0, -0.7, 1.3)
    o2, S2 = ref.dplr_unrolled(q, k, v, la, beta, g, S0, -0.7, 1.3)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, S2, rtol=0, atol=1e-12)


def pin_split_resume(impl):
    """Running [0,B) then [B,T) from the carried state equals one run over [0,T)."""
    q, k, v, la, beta, g, S0 = rand_case(40, 6, 5, seed=17)
    o, S = impl(q, k, v, la, beta, g, S0, -0.3, 1.0)
    for B in (1, 15, 16, 17):
        o1, S1 = impl(q[:B], k[:B], v[:B], la[:B], beta[:B], g[:B], S0, -0.3, 1.0)
        o2, S2 = impl(q[B:], k[B:], v[B:], la[B:], beta[B:], g[B:], S1, -0.3, 1.0)
        # the C oracle takes float32 inputs, so the carried state is rounded to float32
        np.testing.assert_allclose(np.concatenate([o1, o2]), o, atol=1e-6)
        np.testing.assert_allclose(S2, S, atol=1e-6)


def pin_channel_permutation(impl):
    """Permuting key channels (q, k, lambda columns, S0 rows) permutes S rows, keeps o."""
    q, k, v, la, beta, g, S0 = rand_case(11, 6, 4, seed=18)
    p = np.random.default_rng(5).permutation(6)
    o, S = impl(q, k, v, la, beta, g, S0, -0.3, 1.0)
    o2, S2 = impl(q[:, p], k[:, p], v, la[:, p], beta, g, S0[p], -0.3, 1.0)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(S2, S[p], atol=1e-12)


def pin_floor_clamps(impl):
    """A log-decay below the floor acts exactly like the floor itself."""
    q, k, v, la, beta, g, S0 = rand_case(10, 5, 4, seed=19)
    la_low = la.copy()
    la_low[::2, ::2] = -9.0
    la_at = la.copy()
    la_at[::2, ::2] = -0.3
    a = impl(q, k, v, la_low, beta, g, S0, -0.3, 1.0)
    b = impl(q, k, v, la_at, beta, g, S0, -0.3, 1.0)
    np.testing.assert_allclose(a[0], b[0], atol=0)
    np.testing.assert_allclose(a[1], b[1], atol=0)
    # and a floor below every input leaves the decay untouched (differs from -0.3)
    c = impl(q, k, v, la_low, beta, g, S0, -20.0, 1.0)
    assert np.max(np.abs(c[1] - a[1])) > 1e-3


def pin_non_expansive(impl):
    """|k| = 1, beta in [0, 2], alpha <= 1: ||S_t||_2 <= ||S0||_2 + sum_s beta_s ||v_s||."""
    q, k, v, la, beta, g, S0 = rand_case(30, 6, 5, seed=20)
    beta = 2.0 * beta
    bound = np.linalg.norm(S0, 2)
    for t in range(1, 31):
        _, S = impl(q[:t], k[:t], v[:t], la[:t], beta[:t], g[:t], S0, -0.3, 1.0)
        bound += beta[t - 1] * np.linalg.norm(v[t - 1])
        assert np.linalg.norm(S, 2) <= bound * (1 + 1e-12)


PINS = [pin_golden_onehot, pin_single_token_from_zero, pin_pure_decay, pin_identity_gemm,
        pin_unit_key_recall, pin_orthonormal_keys, pin_dplr_brute_force, pin_split_resume,
        pin_channel_permutation, pin_floor_clamps, pin_non_expansive]


@pytest.mark.parametrize("impl_name", sorted(IMPLS))
@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(impl_name, pin):
    pin(IMPLS[impl_name])


# ----------------------------------------------------------------------------- cross
def test_c_oracle_matches_numpy_packed_varlen():
    """Packed varlen batch with a zero-length sequence; per-sequence initial states."""
    r = np.random.default_rng(21)
    lens = [5, 0, 17, 33, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = int(cu[-1]), 3, 8, 6
    f32 = lambda x: np.asarray(x, np.float32)
    q = f32(r.standard_normal((T, H, dk)))
    k = f32(r.standard_normal((T, H, dk)) / np.sqrt(dk))
    v = f32(r.standard_normal((T, H, dv)))
    la = f32(-np.log1p(np.exp(r.standard_normal((T, H, dk)))))
    b = f32(1 / (1 + np.exp(-r.standard_normal((T, H)))))
    g = f32(r.random((T, H, dv)))
    S0 = f32(r.standard_normal((len(lens), H, dk, dv)))
    out, Sf, _ = oracle.run(q, k, v, la, b, g, cu, S0, -0.3, 0.9, nthreads=3)
    out2, Sf2 = ref.run_packed(ref.recurrent, q, k, v, la, b, g, cu, S0, floor=-0.3,
                               scale=0.9)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Sf, Sf2, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(Sf[:, :][1], S0[1])  # zero-length: S_T = S0


def test_c_oracle_pair_subset():
    """Computing only some (sequence, head) pairs gives the same values for those."""
    r = np.random.default_rng(22)
    cu = [0, 9, 20]
    T, H, dk, dv = 20, 4, 5, 3
    xs = [np.asarray(r.standard_normal(s), np.float32) * 0.3 for s in
          ((T, H, dk), (T, H, dk), (T, H, dv), (T, H, dk), (T, H), (T, H, dv))]
    out, Sf, _ = oracle.run(*xs, cu, None)
    out2, Sf2, _ = oracle.run(*xs, cu, None, pairs=[1 * H + 2, 0 * H + 3])
    np.testing.assert_array_equal(out2[9:20, 2], out[9:20, 2])
    np.testing.assert_array_equal(Sf2[0, 3], Sf[0, 3])
    assert np.isnan(out2[0:9, 0]).all()


@pytest.mark.parametrize("chunk", [1, 4, 16, 37])
@pytest.mark.parametrize("d", [(8, 8), (16, 6)])
def test_chunked_algebra_equals_recurrence(chunk, d):
    """The 16-token chunk algebra (and other chunk sizes, with a partial last chunk)
    reproduces the token loop to rounding."""
    dk, dv = d
    q, k, v, la, beta, g, S0 = rand_case(37, dk, dv, seed=23)
    o, S = ref.recurrent(q, k, v, la, beta, g, S0, -0.3, 1.1)
    o2, S2 = ref.chunked(q, k, v, la, beta, g, S0, -0.3, 1.1, chunk=chunk)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-11)
    np.testing.assert_allclose(S2, S, rtol=0, atol=1e-11)


# ----------------------------------------------------------------------------- mutants
def _mutant(kind):
    def impl(q, k, v, la, beta, g, S0=None, floor=-0.3, scale=1.0):
        q, k, v, la, beta, g = (np.asarray(x, np.float64) for x in (q, k, v, la, beta, g))
        T, dk = q.shape
        dv = v.shape[1]
        S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)
        o = np.zeros((T, dv))
        for t in range(T):
            lam = la[t] if kind == "no_floor" else np.maximum(la[t], floor)
            a = np.exp(lam)
            if kind != "no_decay" and kind != "decay_after_write":
                S = a[:, None] * S
            if kind == "readout_before_write":
                o[t] = g[t] * (S.T @ (scale * q[t]))
            w = S.T @ k[t]
            sgn = 1.0 if kind == "wrong_sign" else -1.0
            bb = 1.0 if kind == "beta_ignored" else beta[t]
            S = S + bb * np.outer(k[t], v[t] + sgn * w)
            if kind == "decay_after_write":
                S = a[:, None] * S
            if kind == "transposed_readout":
                o[t] = g[t] * (S[:dv, :dv] @ (scale * q[t][:dv]))
            elif kind == "no_gate":
                o[t] = S.T @ (scale * q[t])
            elif kind != "readout_before_write":
                o[t] = g[t] * (S.T @ (scale * q[t]))
        return o, S
    return impl


MUTANTS = ["no_floor", "no_decay", "decay_after_write", "readout_before_write",
           "wrong_sign", "beta_ignored", "transposed_readout", "no_gate"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_mutant(kind):
    """Each plausible mistake planted in a copy of the token loop fails some pin."""
    impl = _mutant(kind)
    failed = []
    for pin in PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every pin"
