"""CPU emulation of the roundings of the bf16-input chunked prefill, in its two precision forms.

TEST INFRASTRUCTURE ONLY: it supports the choice between the forms (the kernel is checked
against the oracle on the GPU; this shows on the CPU why both forms meet the tolerance and
what each product's operands carry).  It follows the chunk algebra of the prefill kernel,
with every operand rounded as the kernel rounds it and every sum taken in fp64 and rounded
to fp32 (the matrix core accumulates in fp32):

  per 16-token chunk, G = inclusive cumsum of max(lambda, floor) (fp32), GC = G[last],
  Qt, Kt = (q, k) e^{G - GC}, Kb = k e^{GC - G}, gamma = e^{GC}, S' = gamma * S
  A = strict_lower(Diag(beta) Kt Kb^T), T = (I + A)^-1 Diag(beta) (nilpotent product)
  P = lower_incl(Qt Kb^T), Wt = T Kt, U = T V - Wt S', O = Qt S' + P U, S <- S' + Kb^T U

  split form: x = hi + lo in bf16 for Qt and Kb (P, the readout, the update), S' (readout)
              and U; one bf16 copy of Kt, Wt, T and of S' in Wt S'
  half form:  one fp16 copy of every operand

Sources: the chunk algebra is the one the oracle's chunked() writes in fp64 (digest of
"Kimi K3: Open Frontier Intelligence", section "KDA：百万上下文先要过「数值 算子」这一关",
Fig. 3: the floor on the log-decay keeps the decay-folded block products bounded).
"""
from __future__ import annotations

import numpy as np
import torch


def _round(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)
    return t.float().numpy().astype(np.float64)


def bf16(x):
    return _round(x, torch.bfloat16)


def f16(x):
    return _round(x, torch.float16)


def f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def split(x):
    """x = hi + lo, both bf16, lo the bf16 rounding of the exact fp32 residual."""
    hi = bf16(x)
    return hi, bf16(f32(x) - hi)


def _inverse(A, r):
    """(I + A)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8) for strictly lower A (A^16 = 0),
    each product of operands rounded by r."""
    A2 = f32(r(A) @ r(A))
    A4 = f32(r(A2) @ r(A2))
    A8 = f32(r(A4) @ r(A4))
    X = np.eye(A.shape[0]) + A8
    X = X + f32(r(X) @ r(A4))
    X = X + f32(r(X) @ r(A2))
    return X - f32(r(X) @ r(A))


def prefill(q, k, v, log_alpha, beta, gate, S0, floor=-0.3, form="half"):
    """One (sequence, head): inputs already bf16-valued ([T, d] arrays), S0 fp32 [dk, dv].
    Returns (o [T, dv] rounded to bf16, final state)."""
    T, dk = q.shape
    dv = v.shape[1]
    S = f32(S0)
    o = np.zeros((T, dv))
    for c0 in range(0, T, 16):
        n = min(16, T - c0)
        Q, K, L = (np.zeros((16, dk)) for _ in range(3))
        V, Gt = np.zeros((16, dv)), np.zeros((16, dv))
        B = np.zeros(16)
        sl = slice(c0, c0 + n)
        Q[:n], K[:n], L[:n], V[:n], Gt[:n], B[:n] = q[sl], k[sl], log_alpha[sl], v[sl], gate[sl], beta[sl]
        lam = np.maximum(L, floor)
        lam[n:] = 0.0                                  # identity rows past the end
        G = f32(np.cumsum(f32(lam), axis=0))
        GC = G[-1]
        F, Fi, gam = f32(np.exp(G - GC)), f32(np.exp(GC - G)), f32(np.exp(GC))
        Qt, Kt, Kb = f32(Q * F), f32(K * F), f32(K * Fi)
        Sp = f32(gam[:, None] * S)
        if form == "half":
            q16, kt16, kb16 = f16(Qt), f16(Kt), f16(Kb)
            A = np.tril(B[:, None] * f32(kt16 @ kb16.T), -1)
            T16 = f16(_inverse(A, f16) * B[None, :])
            P16 = f16(np.tril(f32(q16 @ kb16.T)))
            W16 = f16(f32(T16 @ kt16))
            s16 = f16(Sp)
            U = f32(T16 @ f16(V) - W16 @ s16)
            u16 = f16(U)
            O = f32(q16 @ s16 + P16 @ u16)
            S = f32(Sp + kb16.T @ u16)
        elif form == "split":
            qh, ql = split(Qt)
            kbh, kbl = split(Kb)
            kt = bf16(Kt)
            A = np.tril(B[:, None] * f32(kt @ kbh.T), -1)
            Tm = bf16(_inverse(A, bf16) * B[None, :])
            ph, pl = split(np.tril(f32(qh @ kbh.T + ql @ kbh.T + qh @ kbl.T)))
            sh, sl_ = split(Sp)
            U = f32(Tm @ V - bf16(f32(Tm @ kt)) @ sh)
            uh, ul = split(U)
            O = f32(qh @ sh + ql @ sh + qh @ sl_ + ph @ uh + pl @ uh + ph @ ul)
            S = f32(Sp + kbh.T @ uh + kbl.T @ uh + kbh.T @ ul)
        else:
            raise ValueError(form)
        o[sl] = bf16(f32(Gt * O))[:n]
    return o, S
