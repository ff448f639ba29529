"""GPU parity of kda_chunk_prefill_segmented (segments of one sequence run side by side
and are joined by a scan over their states; digest of "Kimi K3: Open Frontier
Intelligence", section "基础设施", KDA context parallelism).

The inputs use slow decays (per-step log-decay >= -0.02) so that a segment's transition
keeps a large part of the incoming state and the join is exercised; with the usual
-0.3 the incoming state would fade within a few chunks."""
import pytest
import torch

import kda_inputs as ki
import linear_attention_sequence_chunked_amd as kda
from parity import assert_close, host, log, oracle_full, oracle_pairs

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def segmented(x, L, **kw):
    o, S = kda.chunk_prefill_segmented(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate,
                                       x.cu_seqlens_host, L, initial_state=x.initial_state,
                                       **kw)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("L", [16, 64, 256])
def test_segmented_matches_oracle(dtype, dk, dv, L):
    lengths = (300, 0, 17, 1000, 64)
    log(f"segmented dtype={dtype} dk={dk} dv={dv} L={L}")
    x = ki.make_prefill_inputs(lengths, 2, dk, dv, dtype, 0.3, seed=L + dk + dv,
                               device="cuda", log_alpha_min=-0.02)
    o, S = segmented(x, L, scale=0.9, log_alpha_floor=-0.5)
    ro, rS = oracle_full(x, floor=-0.5, scale=0.9)
    assert_close("o", host(o), ro, DT[dtype])
    assert_close("S_T", host(S), rS, DT[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("floor", [-0.3, -0.5])
def test_segmented_log_decay_below_floor(dtype, floor):
    """Log-decays drawn from [-2, 0] with the floor at -0.3 / -0.5: the clamp acts in the
    segment states, the segment transitions and the output pass alike."""
    lengths = (300, 17, 1000)
    log(f"segmented below-floor decays dtype={dtype} floor={floor}")
    x = ki.make_prefill_inputs(lengths, 2, 128, 128, dtype, 0.3, seed=91, device="cuda",
                               log_alpha_min=-2.0)
    assert float(x.log_alpha.float().min()) < floor - 1.0
    o, S = segmented(x, 64, scale=0.9, log_alpha_floor=floor)
    ro, rS = oracle_full(x, floor=floor, scale=0.9)
    assert_close("o", host(o), ro, DT[dtype])
    assert_close("S_T", host(S), rS, DT[dtype])


def test_segmented_in_place_state_and_empty_batch():
    x = ki.make_prefill_inputs((0, 0), 2, 64, 64, "bf16", 0.3, seed=1, device="cuda")
    st = x.initial_state.clone()
    o, S = segmented(x, 32, final_state=st)
    assert o.shape[0] == 0 and torch.equal(st, x.initial_state)
    x = ki.make_prefill_inputs((100, 37), 2, 64, 64, "bf16", 0.3, seed=2, device="cuda",
                               log_alpha_min=-0.02)
    ref_o, ref_S = oracle_full(x)
    st = x.initial_state.clone()
    o, S = kda.chunk_prefill_segmented(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate,
                                       x.cu_seqlens_host, 32, initial_state=st,
                                       final_state=st)
    torch.cuda.synchronize()
    assert_close("o", host(o), ref_o, torch.bfloat16)
    assert_close("S_T (in place)", host(st), ref_S, torch.bfloat16)


def test_few_heads_long_sequence():
    """B=1, H=2, T=65536, d=128, bf16, 2048-token segments (32 per sequence): sampled
    against the oracle, and against the unsegmented kernel."""
    log("segmented few heads, T=65536, L=2048")
    x = ki.make_prefill_inputs((65536,), 2, 128, 128, "bf16", 0.02, seed=3, device="cuda",
                               log_alpha_min=-0.01)
    o, S = segmented(x, 2048)
    ref = oracle_pairs(x, [(0, 0), (0, 1)])
    for (n, h), (ro, rS) in ref.items():
        assert_close(f"o h={h}", host(o[:, h]), ro, torch.bfloat16)
        assert_close(f"S_T h={h}", host(S[n, h]), rS, torch.bfloat16)
    o2, S2 = kda.chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate,
                               cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_seqlens_host,
                               initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("S_T vs unsegmented", host(S), host(S2), torch.bfloat16)


def test_long_context_workload_segmented_sampled():
    """B=1, H=32, T=131072, d=128, bf16 (the long-context workload), 8192-token segments."""
    w = ki.WORKLOADS["prefill_b1_h32_t131072"]
    log("segmented prefill_b1_h32_t131072, L=8192")
    x = ki.make_workload_inputs(w, seed=2, device="cuda")
    o, S = segmented(x, 8192)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    ref = oracle_pairs(x, [(0, 5), (0, 30)])
    for (n, h), (ro, rS) in ref.items():
        assert_close(f"o h={h}", host(o[:, h]), ro, torch.bfloat16)
        assert_close(f"S_T h={h}", host(S[n, h]), rS, torch.bfloat16)
