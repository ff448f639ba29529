"""Shared helpers for GPU-vs-oracle parity tests.

Tolerances, per tensor (outputs and final states checked separately), tol = 2e-2 for
bf16 inputs and 1e-4 for fp32 inputs; the oracle runs in fp64 on the exact
(bf16-rounded) inputs the GPU saw:

  fp32 tensors (states, fp32 outputs):  max|x - ref| <= tol * RMS(ref)
  bf16-stored outputs:                  |x - ref| <= tol * RMS(ref) + 2^-8 * |ref|,
                                        element by element

The second term of the bf16 bound is exactly the rounding of the stored value and
nothing more: round-to-nearest-even to bf16 (8 significant bits) moves a value by at
most half an ulp, and for |x| in [2^e, 2^(e+1)) half an ulp is 2^(e-8) <= 2^-8 |x|.
The literal "max|err| <= tol * RMS" cannot hold for a bf16-stored tensor whose largest
elements exceed tol / 2^-8 = 5.12 x RMS: the exact result rounded to bf16 already
misses it there (these workloads' outputs reach ~20 x RMS).  So the arithmetic error
of the kernel gets exactly tol * RMS, as for the fp32 tensors, and the rounding of
the stored result gets its own exact bound.  Both the literal max|err|/RMS of the GPU
result and that of the exactly rounded oracle result are logged next to it.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
BF16_HALF_ULP = 2.0 ** -8  # max |bf16(x) - x| / |x| under round-to-nearest-even


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def rms(ref) -> float:
    ref = _f64(ref)
    return float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0


def rel_max_err(got, ref) -> float:
    """max|got - ref| / RMS(ref) (the literal form; fp32 tensors)."""
    got, ref = _f64(got), _f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    r = rms(ref)
    if r == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / r)


def bf16_arith_err(got, ref) -> float:
    """max over elements of (|got - ref| - 2^-8 |ref|) / RMS(ref), floored at 0: the
    error left once the rounding of the stored bf16 value is taken out.  A bf16-stored
    tensor passes when this is <= tol (see the module docstring)."""
    got, ref = _f64(got), _f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    if not ref.size:
        return 0.0
    r = rms(ref)
    excess = np.abs(got - ref) - BF16_HALF_ULP * np.abs(ref)
    m = float(np.max(excess))
    if m <= 0.0:
        return 0.0
    return m / r if r > 0.0 else float("inf")


def bf16_rounded_literal(ref) -> float:
    """max|bf16(ref) - ref| / RMS(ref): the literal figure of the exact result rounded
    to bf16 (round-to-nearest-even)."""
    ref = _f64(ref)
    if not ref.size:
        return 0.0
    rounded = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).double().numpy()
    r = rms(ref)
    return float(np.max(np.abs(rounded - ref)) / r) if r > 0.0 else 0.0


def check_close(name, got, ref, dtype, stored_bf16=None) -> float:
    """Assert parity of one tensor; returns the graded error (<= TOL[dtype]).

    stored_bf16: the tensor is kept in bf16 (outputs of the bf16 path); defaults to
    False for names starting with 'S' (fp32 states) and to dtype == bf16 otherwise."""
    if stored_bf16 is None:
        stored_bf16 = dtype == torch.bfloat16 and not name.startswith("S")
    lit = rel_max_err(got, ref)
    tol = TOL[dtype]
    if stored_bf16:
        e = bf16_arith_err(got, ref)
        log(f"  {name}: max(|err| - 2^-8|ref|)/RMS = {e:.3e} (tol {tol:.0e}, margin "
            f"{tol / max(e, 1e-30):.1f}x); literal max|err|/RMS = {lit:.3e} "
            f"(oracle rounded to bf16: {bf16_rounded_literal(ref):.3e})")
    else:
        e = lit
        log(f"  {name}: max|err|/RMS = {e:.3e} (tol {tol:.0e}, margin "
            f"{tol / max(e, 1e-30):.1f}x)")
    assert e <= tol, f"{name}: error {e:.3e} > {tol}"
    return e


assert_close = check_close


def host(x):
    return None if x is None else x.detach().to("cpu", torch.float32).numpy()


def oracle_full(x, floor=-0.3, scale=1.0, initial_state=None):
    """Oracle on every (sequence, head) of a KdaInputs batch."""
    S0 = x.initial_state if initial_state is None else initial_state
    out, Sf, _ = oracle.run(host(x.q), host(x.k), host(x.v), host(x.log_alpha),
                            host(x.beta), host(x.gate), x.cu_seqlens_host, host(S0), floor,
                            scale)
    return out, Sf


def oracle_pairs(x, pairs, floor=-0.3, scale=1.0):
    """Oracle on selected (sequence n, head h) pairs, downloading only their rows.

    Returns {(n, h): (o [T_n, dv], S_T [dk, dv])}."""
    qs, ks, vs, las, bs, gs, s0s, cu = [], [], [], [], [], [], [], [0]
    for n, h in pairs:
        a, e = x.cu_seqlens_host[n], x.cu_seqlens_host[n + 1]
        qs.append(host(x.q[a:e, h:h + 1]))
        ks.append(host(x.k[a:e, h:h + 1]))
        vs.append(host(x.v[a:e, h:h + 1]))
        las.append(host(x.log_alpha[a:e, h:h + 1]))
        bs.append(host(x.beta[a:e, h:h + 1]))
        gs.append(host(x.gate[a:e, h:h + 1]))
        if x.initial_state is not None:
            s0s.append(host(x.initial_state[n, h:h + 1]))
        cu.append(cu[-1] + (e - a))
    cat = lambda xs: np.concatenate(xs, axis=0)
    S0 = None if x.initial_state is None else np.stack(s0s)  # [P, 1, dk, dv]
    out, Sf, _ = oracle.run(cat(qs), cat(ks), cat(vs), cat(las), cat(bs), cat(gs), cu, S0,
                            floor, scale)
    res = {}
    for i, (n, h) in enumerate(pairs):
        res[(n, h)] = (out[cu[i]:cu[i + 1], 0], Sf[i, 0])
    return res


def check_pairs(x, pairs, o, S, dtype=torch.bfloat16, floor=-0.3, scale=1.0, label=""):
    """Oracle on the given (sequence, head) pairs against the GPU's o and S (all pairs'
    outputs graded as one tensor, and all their final states as another)."""
    ref = oracle_pairs(x, pairs, floor, scale)
    cu = x.cu_seqlens_host
    got_o = np.concatenate([host(o[cu[n]:cu[n + 1], h]) for n, h in pairs])
    ref_o = np.concatenate([ref[p][0] for p in pairs])
    eo = check_close(f"o {label}".strip(), got_o, ref_o, dtype)
    eS = check_close(f"S_T {label}".strip(), np.stack([host(S[n, h]) for n, h in pairs]),
                     np.stack([ref[p][1] for p in pairs]), dtype)
    return eo, eS
