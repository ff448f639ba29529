"""GPU parity of kda_chunk_prefill_checkpointed: prefix-cache state snapshots every m
tokens (digest of "Kimi K3: Open Frontier Intelligence", section "基础设施", Fig. 12).

Each snapshot is checked against the oracle's final state on that prefix (the oracle's
final state is pinned by the CPU suite), slots no snapshot maps to must stay untouched,
the outputs must be bit-identical to the plain entry point's, and resuming from a snapshot
must reproduce the uninterrupted run bit for bit."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import linear_attention_sequence_chunked_amd as kda
import oracle
from parity import assert_close, host, log

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def prefix_state(x, n, L, heads, floor, scale):
    """Oracle state of sequence n after its first L tokens, for the given heads."""
    a = x.cu_seqlens_host[n]
    sl = lambda t: host(t[a:a + L, heads[0]:heads[-1] + 1])
    S0 = None if x.initial_state is None else host(x.initial_state[n:n + 1, heads[0]:heads[-1] + 1])
    _, Sf, _ = oracle.run(sl(x.q), sl(x.k), sl(x.v), sl(x.log_alpha), sl(x.beta), sl(x.gate),
                          [0, L], S0, floor, scale)
    return Sf[0]


def plain_and_checkpointed(x, m, **kw):
    args = (x.q, x.k, x.v, x.log_alpha, x.beta, x.gate)
    common = dict(cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_seqlens_host,
                  initial_state=x.initial_state, **kw)
    o0, S0 = kda.chunk_prefill(*args, **common)
    H, dk, dv = x.q.shape[1], x.q.shape[2], x.v.shape[2]
    ck = torch.full((x.total_tokens // m, H, dk, dv), float("nan"), device="cuda")
    o1, S1, ck1 = kda.chunk_prefill(*args, checkpoint_every=m, checkpoints=ck, **common)
    torch.cuda.synchronize()
    assert ck1.data_ptr() == ck.data_ptr()
    assert torch.equal(o0, o1), "outputs differ from the plain entry point"
    assert torch.equal(S0, S1), "final states differ from the plain entry point"
    return o1, S1, ck


def snapshot_case(dtype, dk, dv, m, floor, log_alpha_min):
    lengths = (100, 0, 48, 129, 31, 64)
    x = ki.make_prefill_inputs(lengths, 2, dk, dv, dtype, 0.3, seed=7 * m + dk, device="cuda",
                               log_alpha_min=log_alpha_min)
    scale = 0.8
    _, _, ck = plain_and_checkpointed(x, m, log_alpha_floor=floor, scale=scale)
    used = set()
    cu = x.cu_seqlens_host
    for n, T_n in enumerate(lengths):
        for j in range(1, T_n // m + 1):
            slot = kda.checkpoint_slot(cu, n, j, m)
            assert 0 <= slot < ck.shape[0] and slot not in used
            used.add(slot)
            ref = prefix_state(x, n, j * m, [0, 1], floor, scale)
            assert_close(f"S(n={n}, t={j * m})", host(ck[slot]), ref, DT[dtype])
    for slot in range(ck.shape[0]):
        if slot not in used:
            assert torch.isnan(ck[slot]).all(), f"slot {slot} was written"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
@pytest.mark.parametrize("m", [16, 48, 64])
def test_snapshots_match_oracle_prefix_states(dtype, dk, dv, m):
    log(f"checkpoints dtype={dtype} dk={dk} dv={dv} m={m}")
    snapshot_case(dtype, dk, dv, m, floor=-0.4, log_alpha_min=-0.3)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("floor", [-0.3, -0.5])
def test_snapshots_log_decay_below_floor(dtype, floor):
    """Log-decays drawn down to -2 with the floor at -0.3 / -0.5."""
    log(f"checkpoints below-floor decays dtype={dtype} floor={floor}")
    snapshot_case(dtype, 128, 128, 48, floor=floor, log_alpha_min=-2.0)


def test_fewer_tokens_than_one_interval():
    x = ki.make_prefill_inputs((20, 9), 2, 64, 64, "bf16", 0.3, seed=3, device="cuda")
    o, S, ck = kda.chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate,
                                 cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_seqlens_host,
                                 initial_state=x.initial_state, checkpoint_every=32)
    torch.cuda.synchronize()
    assert ck.shape[0] == 0
    o0, S0 = kda.chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate,
                               cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_seqlens_host,
                               initial_state=x.initial_state)
    assert torch.equal(o, o0) and torch.equal(S, S0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_resume_from_snapshot_is_bitwise(dtype):
    """A prefix-cache hit at B = 2560 tokens (the pages' Fig. 12 example) with 512-token
    snapshots: prefill of the remaining tokens from the snapshot equals the uninterrupted
    run's rows and final state bit for bit."""
    B, m, T = 2560, 512, 3260
    log(f"resume dtype={dtype} B={B} m={m} T={T}")
    x = ki.make_prefill_inputs((T,), 4, 128, 128, dtype, 0.02, seed=11, device="cuda")
    o, S, ck = plain_and_checkpointed(x, m)
    slot = kda.checkpoint_slot(x.cu_seqlens_host, 0, B // m, m)
    rest = lambda t: t[B:].contiguous()
    o2, S2 = kda.chunk_prefill(rest(x.q), rest(x.k), rest(x.v), rest(x.log_alpha),
                               rest(x.beta), rest(x.gate), cu_seqlens=[0, T - B],
                               initial_state=ck[slot:slot + 1].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o2, o[B:]), "resumed outputs differ"
    assert torch.equal(S2, S), "resumed final state differs"


def test_bench_workload_snapshots_sampled():
    """B=4, H=16, T=4096, d=128, bf16 with 512-token snapshots (8 per sequence): outputs
    bit-identical to the plain call; sampled snapshots against the oracle."""
    w = ki.WORKLOADS["prefill_b4_h16_t4096"]
    log("checkpoints on prefill_b4_h16_t4096, m=512")
    x = ki.make_workload_inputs(w, seed=1, device="cuda")
    m = 512
    _, _, ck = plain_and_checkpointed(x, m)
    assert ck.shape[0] == 4 * 4096 // m
    assert torch.isfinite(ck).all()
    for n, h, j in [(0, 0, 1), (1, 9, 4), (3, 15, 8)]:
        slot = kda.checkpoint_slot(x.cu_seqlens_host, n, j, m)
        ref = prefix_state(x, n, j * m, [h], -0.3, 1.0)
        assert_close(f"S(n={n}, h={h}, t={j * m})", host(ck[slot, h:h + 1]), ref, torch.bfloat16)
