"""ctypes front end of the C fp64 oracle (kda_oracle.c).  Test infrastructure only."""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build

_lib = None


def library_path() -> str:
    return _build.LIB


def ensure_built() -> str:
    if not os.path.exists(_build.LIB) or (
            os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
        _build.build()
    return _build.LIB


def _load():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(ensure_built())
        f = _lib.kda_oracle_run
        P = ctypes.c_void_p
        f.argtypes = [ctypes.c_int64, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                      P, P, P, P, P, P, P, ctypes.c_double, ctypes.c_double, P, P, P,
                      ctypes.c_int64, ctypes.c_int]
        f.restype = ctypes.c_int
    return _lib


def _f32(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor -> exact float32 copy on the host
        import torch
        x = x.detach().to("cpu", torch.float32).numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a) -> Optional[int]:
    return None if a is None else a.ctypes.data


def run(q, k, v, log_alpha, beta, gate, cu_seqlens: Sequence[int], initial_state=None,
        log_alpha_floor: float = -0.3, scale: float = 1.0, want_out: bool = True,
        pairs: Optional[Sequence[int]] = None, nthreads: int = 0):
    """Run the fp64 token loop.

    q/k/log_alpha: [T_total, H, dk]; v/gate: [T_total, H, dv]; beta: [T_total, H];
    initial_state: [N, H, dk, dv] or None.  pairs: optional subset of n*H+h to compute
    (other outputs stay NaN).  Returns (out fp64 [T_total,H,dv] or None,
    S_final fp64 [N,H,dk,dv], threads_used).
    """
    lib = _load()
    q, k, v, la, b, g = (_f32(x) for x in (q, k, v, log_alpha, beta, gate))
    S0 = _f32(initial_state)
    T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and la.shape == q.shape and b.shape == (T, H)
    assert v.shape == (T, H, dv) and g.shape == v.shape
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    if S0 is not None:
        assert S0.shape == (N, H, dk, dv)
    out = np.full((T, H, dv), np.nan) if want_out else None
    Sf = np.full((N, H, dk, dv), np.nan)
    pr = None if pairs is None else np.ascontiguousarray(np.asarray(pairs, dtype=np.int64))
    if nthreads <= 0:
        nthreads = len(os.sched_getaffinity(0))
    used = lib.kda_oracle_run(N, _ptr(cu), H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(la),
                              _ptr(b), _ptr(g), _ptr(S0), float(log_alpha_floor),
                              float(scale), _ptr(out), _ptr(Sf), _ptr(pr),
                              0 if pr is None else len(pr), int(nthreads))
    if used < 0:
        raise ValueError("kda_oracle_run rejected its arguments")
    return out, Sf, used
