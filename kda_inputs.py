"""Seeded synthetic inputs for the KDA operator.

This module only draws random tensors with the distributions of the five workloads
(there is no dataset: every input is synthetic).  It holds none of the operator's
arithmetic and is the one module that both the oracle-side tests and the GPU path's
tests/benchmark use.

Distributions (all draws in float32 from a seeded torch.Generator, then rounded to the
tensor dtype with round-to-nearest-even):
  q, k        ~ N(0, 1), then L2-normalised over the channel axis per (token, head)
  v           ~ N(0, 1)
  beta        = sigmoid(N(0, 1))                       one per (token, head)
  log_alpha   = max(-softplus(N(0, 1)), -0.3)          per key channel
  gate        = sigmoid(N(0, 1))                       per value channel
  S0          = zeros, or N(0, std^2) in float32       [N, H, dk, dv]

Layout: packed tokens.  q/k/log_alpha are [T_total, H, dk], v/gate are
[T_total, H, dv], beta is [T_total, H]; sequence n owns rows cu_seqlens[n] ..
cu_seqlens[n+1]-1.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "WORKLOADS",
    "Workload",
    "KdaInputs",
    "make_prefill_inputs",
    "make_decode_inputs",
    "varlen_lengths",
    "uniform_cu_seqlens",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    lengths: tuple          # per-sequence token counts
    H: int
    dk: int
    dv: int
    dtype: str              # "bf16" | "f32"
    s0_std: float           # 0 -> zero initial state
    steps: int = 0          # decode steps (decode workload only)


def varlen_lengths(seed: int = 4, n: int = 64) -> tuple:
    """Length mix 40% 8K / 42% 32K / 15% 128K / 3% 1M (capped to 256K)."""
    rng = np.random.default_rng(seed)
    draw = rng.choice([8192, 32768, 131072, 262144], n, p=[0.40, 0.42, 0.15, 0.03])
    return tuple(int(x) for x in draw)


WORKLOADS = {
    # tiny fp32 prefill: B=1, H=2, T=256, d=64, zero initial state
    "tiny_f32": Workload("tiny_f32", (256,), 2, 64, 64, "f32", 0.0),
    # chunked prefill, bf16 inputs / fp32 state: B=4, H=16, T=4096, d=128, S0~N(0,0.02^2)
    "prefill_b4_h16_t4096": Workload("prefill_b4_h16_t4096", (4096,) * 4, 16, 128, 128,
                                     "bf16", 0.02),
    # long-context prefill: B=1, H=32, T=131072, d=128, zero initial state
    "prefill_b1_h32_t131072": Workload("prefill_b1_h32_t131072", (131072,), 32, 128, 128,
                                       "bf16", 0.0),
    # decode: 256 sequences x 32 heads, 128x128 fp32 state, 1000 steps
    "decode_n256_h32": Workload("decode_n256_h32", (1,) * 256, 32, 128, 128, "bf16", 0.02,
                                steps=1000),
    # varlen packed prefill: 64 sequences, H=32, d=128, per-sequence S0
    "varlen_n64_h32": Workload("varlen_n64_h32", varlen_lengths(), 32, 128, 128, "bf16",
                               0.02),
    # few heads, long context (the segmented prefill's case): B=1, H=4, T=524288, d=128
    "prefill_b1_h4_t524288": Workload("prefill_b1_h4_t524288", (524288,), 4, 128, 128,
                                      "bf16", 0.0),
}


@dataclasses.dataclass
class KdaInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    log_alpha: torch.Tensor
    beta: torch.Tensor
    gate: torch.Tensor
    cu_seqlens: torch.Tensor        # int32, on the same device
    cu_seqlens_host: list           # python ints
    initial_state: Optional[torch.Tensor]

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens_host[-1])


def uniform_cu_seqlens(batch: int, seqlen: int) -> list:
    return [i * seqlen for i in range(batch + 1)]


def _torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _gen(seed: Sequence[int], device) -> torch.Generator:
    # fold the seed tuple into one 63-bit integer, deterministically
    s = np.random.SeedSequence(list(seed)).generate_state(2, dtype=np.uint32)
    g = torch.Generator(device=device)
    g.manual_seed(int(s[0]) << 31 ^ int(s[1]))
    return g


def _randn(shape, seed, device) -> torch.Tensor:
    return torch.randn(*shape, generator=_gen(seed, device), device=device,
                       dtype=torch.float32)


def _l2norm(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def make_prefill_inputs(lengths: Sequence[int], H: int, dk: int, dv: int, dtype: str,
                        s0_std: float, seed: int, device="cpu",
                        log_alpha_min: float = -0.3) -> KdaInputs:
    """Draw one packed varlen batch.  Every (sequence, tensor) pair has its own seeded
    stream (seed, tensor_id, sequence), so a sequence's values do not depend on the
    other lengths in the batch and temporaries stay one sequence in size."""
    dt = _torch_dtype(dtype)
    T = int(sum(lengths))
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    q = torch.empty((T, H, dk), dtype=dt, device=device)
    k = torch.empty((T, H, dk), dtype=dt, device=device)
    v = torch.empty((T, H, dv), dtype=dt, device=device)
    la = torch.empty((T, H, dk), dtype=dt, device=device)
    beta = torch.empty((T, H), dtype=dt, device=device)
    gate = torch.empty((T, H, dv), dtype=dt, device=device)
    sp = torch.nn.functional.softplus
    for n, L in enumerate(lengths):
        a, e = cu[n], cu[n + 1]
        if L == 0:
            continue
        q[a:e] = _l2norm(_randn((L, H, dk), (seed, 0, n), device)).to(dt)
        k[a:e] = _l2norm(_randn((L, H, dk), (seed, 1, n), device)).to(dt)
        v[a:e] = _randn((L, H, dv), (seed, 2, n), device).to(dt)
        la[a:e] = torch.clamp(-sp(_randn((L, H, dk), (seed, 3, n), device)),
                              min=log_alpha_min).to(dt)
        beta[a:e] = torch.sigmoid(_randn((L, H), (seed, 4, n), device)).to(dt)
        gate[a:e] = torch.sigmoid(_randn((L, H, dv), (seed, 5, n), device)).to(dt)
    S0 = None
    if s0_std > 0:
        S0 = (_randn((len(lengths), H, dk, dv), (seed, 6), device) * s0_std).contiguous()
    return KdaInputs(q, k, v, la, beta, gate,
                     torch.tensor(cu, dtype=torch.int32, device=device), cu, S0)


def make_workload_inputs(w: Workload, seed: int, device="cpu",
                         lengths: Optional[Sequence[int]] = None) -> KdaInputs:
    return make_prefill_inputs(lengths if lengths is not None else w.lengths, w.H, w.dk,
                               w.dv, w.dtype, w.s0_std, seed, device)


def make_decode_inputs(steps: int, N: int, H: int, dk: int, dv: int, dtype: str, seed: int,
                       device="cpu", log_alpha_min: float = -0.3) -> dict:
    """Fresh tokens for `steps` consecutive decode steps, one per sequence per step.

    Returns a dict of tensors shaped [steps, N, H, d] ([steps, N, H] for beta); step s
    feeds row s.  Same distributions as the prefill inputs."""
    dt = _torch_dtype(dtype)
    sp = torch.nn.functional.softplus
    return dict(
        q=_l2norm(_randn((steps, N, H, dk), (seed, 10), device)).to(dt),
        k=_l2norm(_randn((steps, N, H, dk), (seed, 11), device)).to(dt),
        v=_randn((steps, N, H, dv), (seed, 12), device).to(dt),
        log_alpha=torch.clamp(-sp(_randn((steps, N, H, dk), (seed, 13), device)),
                              min=log_alpha_min).to(dt),
        beta=torch.sigmoid(_randn((steps, N, H), (seed, 14), device)).to(dt),
        gate=torch.sigmoid(_randn((steps, N, H, dv), (seed, 15), device)).to(dt),
    )


def make_state(N: int, H: int, dk: int, dv: int, std: float, seed: int,
               device="cpu") -> torch.Tensor:
    return (_randn((N, H, dk, dv), (seed, 7), device) * std).contiguous()
