"""numpy fp64 references for one (sequence, head) of the KDA recurrence.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Shapes for one recurrence: q, k, log_alpha [T, dk]; v, gate [T, dv]; beta [T];
S0 [dk, dv] (rows = key channels).  All arithmetic is float64.

Sources (page title, section/figure):
  * "Kimi-K3 为什么这么强？", §① KDA part ②, "一次 KDA 更新" figure caption -- per-row
    decay, then the key's row keeps (1-beta) of its value, then beta of the new value
    is written (interpolation of old and new).
  * "Kimi K3 深度拆解", 突破一 -- per-channel diagonal decay; Diagonal-Plus-Low-Rank
    transition matrix.
  * Digest of "Kimi K3: Open Frontier Intelligence", section "KDA：百万上下文先要过
    「数值 算子」这一关" and Fig. 3 -- per-step log-decay has a lower bound so that the
    cumulative decay inside a 16-token block stays representable, which lets the whole
    causal diagonal block run as dense matrix products; output gate is a channel-wise
    switch on the recurrence output.
"""
from __future__ import annotations

import numpy as np


def _as64(*xs):
    return [None if x is None else np.asarray(x, dtype=np.float64) for x in xs]


def recurrent(q, k, v, log_alpha, beta, gate, S0=None, floor=-0.3, scale=1.0,
              return_states=False):
    """Token-by-token recurrence (the definition).

    For each token: a = exp(max(lambda, floor)); S <- Diag(a) S; w = S^T k;
    S <- S + beta k (v - w)^T; o = gate * (S^T (scale q)).
    Returns (o [T, dv], S_T [dk, dv]) and, if asked, the list of states after each token.
    """
    q, k, v, la, beta, g, S0 = _as64(q, k, v, log_alpha, beta, gate, S0)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else S0.copy()
    o = np.zeros((T, dv))
    states = []
    for t in range(T):
        a = np.exp(np.maximum(la[t], floor))
        S = a[:, None] * S                      # each key-channel row decays at its rate
        w = S.T @ k[t]                           # value currently stored along k
        S = S + beta[t] * np.outer(k[t], v[t] - w)  # erase (1-beta kept) and write
        o[t] = g[t] * (S.T @ (scale * q[t]))     # gated readout of the updated state
        if return_states:
            states.append(S.copy())
    if return_states:
        return o, S, states
    return o, S


def transition_matrices(k, log_alpha, beta, floor=-0.3):
    """Explicit per-token transitions A_t = (I - beta_t k_t k_t^T) Diag(alpha_t) (dk x dk)."""
    k, la, beta = _as64(k, log_alpha, beta)
    T, dk = k.shape
    I = np.eye(dk)
    return [(I - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(np.maximum(la[t], floor)))
            for t in range(T)]


def dplr_unrolled(q, k, v, log_alpha, beta, gate, S0=None, floor=-0.3, scale=1.0):
    """Closed form of the recurrence from dense DPLR matrices.

    With A_t = (I - beta_t k_t k_t^T) Diag(alpha_t) and B_t = beta_t k_t v_t^T:
        S_t = (A_t ... A_1) S0 + sum_{s<=t} (A_t ... A_{s+1}) B_s.
    Every product is formed explicitly (O(T^2 dk^3)); meant for tiny inputs.
    """
    q, k, v, la, beta, g, S0 = _as64(q, k, v, log_alpha, beta, gate, S0)
    T, dk = q.shape
    dv = v.shape[1]
    if S0 is None:
        S0 = np.zeros((dk, dv))
    A = transition_matrices(k, la, beta, floor)
    B = [beta[t] * np.outer(k[t], v[t]) for t in range(T)]
    o = np.zeros((T, dv))
    S_t = S0
    for t in range(T):
        prod = np.eye(dk)
        for s in range(t, -1, -1):     # prod = A_t ... A_s after this iteration
            prod = prod @ A[s]
        S_t = prod @ S0
        for s in range(t + 1):
            tail = np.eye(dk)
            for j in range(t, s, -1):  # A_t ... A_{s+1}
                tail = tail @ A[j]
            S_t = S_t + tail @ B[s]
        o[t] = g[t] * (S_t.T @ (scale * q[t]))
    return o, S_t


def chunked(q, k, v, log_alpha, beta, gate, S0=None, floor=-0.3, scale=1.0, chunk=16):
    """The chunked (WY / UT-transform) form, in fp64.

    A derivation check for the chunk algebra, not the oracle.  Per chunk of C' <= chunk
    rows, with G_r = sum_{s<=r} max(lambda_s, floor) (inclusive) and G_C = G_{C'}:
        Qh = (scale q) e^G,  Kh = k e^G,  Kc = k e^-G,  Kb = k e^(G_C - G)
        A  = strict_lower(Diag(beta) Kh Kc^T),  T = (I + A)^-1 Diag(beta)
        W  = T Kh,  Ut = T V,  U = Ut - W S
        O  = Qh S + lower_incl_diag(Qh Kc^T) U
        S <- Diag(e^G_C) S + Kb^T U
        o  = gate * O
    """
    q, k, v, la, beta, g, S0 = _as64(q, k, v, log_alpha, beta, gate, S0)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else S0.copy()
    o = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        n = c1 - c0
        G = np.cumsum(np.maximum(la[c0:c1], floor), axis=0)
        GC = G[-1]
        Qh = scale * q[c0:c1] * np.exp(G)
        Kh = k[c0:c1] * np.exp(G)
        Kc = k[c0:c1] * np.exp(-G)
        Kb = k[c0:c1] * np.exp(GC - G)
        A = np.tril(beta[c0:c1, None] * (Kh @ Kc.T), -1)
        Tm = np.linalg.solve(np.eye(n) + A, np.diag(beta[c0:c1]))
        W = Tm @ Kh
        U = Tm @ v[c0:c1] - W @ S
        O = Qh @ S + np.tril(Qh @ Kc.T) @ U
        S = np.exp(GC)[:, None] * S + Kb.T @ U
        o[c0:c1] = g[c0:c1] * O
    return o, S


def run_packed(fn, q, k, v, log_alpha, beta, gate, cu_seqlens, S0=None, **kw):
    """Apply a one-head reference to a packed [T_total, H, d] batch."""
    q, k, v, la, b, g = (np.asarray(x, dtype=np.float64) for x in
                         (q, k, v, log_alpha, beta, gate))
    T, H, dk = q.shape
    dv = v.shape[-1]
    N = len(cu_seqlens) - 1
    out = np.zeros((T, H, dv))
    Sf = np.zeros((N, H, dk, dv))
    for n in range(N):
        a, e = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        for h in range(H):
            s0 = None if S0 is None else np.asarray(S0, dtype=np.float64)[n, h]
            o, S = fn(q[a:e, h], k[a:e, h], v[a:e, h], la[a:e, h], b[a:e, h], g[a:e, h],
                      s0, **kw)
            out[a:e, h] = o
            Sf[n, h] = S
    return out, Sf


def recurrent_backward(q, k, v, log_alpha, beta, gate, do, dS_T=None, S0=None, floor=-0.3,
                       scale=1.0):
    """Gradients of the token recurrence (reverse mode, written out step by step).

    The loss is sum(do * o) + sum(dS_T * S_T).  Forward step t (see recurrent()):
        a = exp(max(lambda_t, floor)); S' = Diag(a) S_{t-1}; w = S'^T k_t;
        u = beta_t (v_t - w); S_t = S' + k_t u^T; y = S_t^T (scale q_t); o_t = gate_t * y.
    Going back through the same steps, with dS the gradient of S_t:
        dgate = do * y;  dy = do * gate;  dS += (scale q) dy^T;  dq = scale S_t dy
        dk = dS u;  du = dS^T k;  dbeta = du . (v - w);  dv = beta du;  dw = -beta du
        dS' = dS + k dw^T;  dk += S' dw
        da = rowsum(dS' * S_{t-1});  dlambda = da * a * [lambda > floor];  dS = Diag(a) dS'
    and dS0 is the dS left after the first token.  max(lambda, floor) passes the
    gradient only where lambda > floor (zero at a tie).
    Returns a dict with dq, dk, dv, dlog_alpha [T, d], dbeta [T], dgate [T, dv], dS0.
    """
    q, k, v, la, beta, g, do, dS_T, S0 = _as64(q, k, v, log_alpha, beta, gate, do, dS_T, S0)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else S0.copy()
    prev, decay, ws = [], [], []
    for t in range(T):                       # forward, keeping what the reverse needs
        a = np.exp(np.maximum(la[t], floor))
        prev.append(S)
        Sp = a[:, None] * S
        w = Sp.T @ k[t]
        S = Sp + beta[t] * np.outer(k[t], v[t] - w)
        decay.append(a)
        ws.append(w)
    out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v),
                                            ("dlog_alpha", la), ("dgate", g))}
    out["dbeta"] = np.zeros(T)
    dS = np.zeros((dk, dv)) if dS_T is None else dS_T.copy()
    for t in range(T - 1, -1, -1):
        a, w, Sprev = decay[t], ws[t], prev[t]
        Sp = a[:, None] * Sprev
        u = beta[t] * (v[t] - w)
        St = Sp + np.outer(k[t], u)
        y = St.T @ (scale * q[t])
        out["dgate"][t] = do[t] * y
        dy = do[t] * g[t]
        dS = dS + np.outer(scale * q[t], dy)
        out["dq"][t] = scale * (St @ dy)
        dkt = dS @ u
        du = dS.T @ k[t]
        out["dbeta"][t] = du @ (v[t] - w)
        out["dv"][t] = beta[t] * du
        dw = -beta[t] * du
        dSp = dS + np.outer(k[t], dw)
        dkt = dkt + Sp @ dw
        out["dk"][t] = dkt
        da = np.sum(dSp * Sprev, axis=1)
        out["dlog_alpha"][t] = da * a * (la[t] > floor)
        dS = a[:, None] * dSp
    out["dS0"] = dS
    return out
