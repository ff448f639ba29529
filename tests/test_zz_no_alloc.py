"""GPU test of kda_chunk_prefill_segmented_noalloc (the entry point that allocates
nothing and keeps its workspace in the library's fixed device buffer), called through
the C ABI: two calls in a row, the second on a smaller problem, each bit-identical to
kda_chunk_prefill_segmented with a caller-provided workspace on the same inputs (the
same kernels run in the same order), and within the operator's tolerance of the oracle."""
import ctypes

import pytest
import torch

import kda_inputs as ki
from linear_attention_sequence_chunked_amd import _lib
from parity import assert_close, host, log, oracle_full

pytestmark = pytest.mark.gpu


def call(x, L, floor, scale, noalloc, ws=None):
    lib = _lib.load()
    H, dk, dv = x.q.shape[1], x.q.shape[2], x.v.shape[2]
    N = len(x.cu_seqlens_host) - 1
    dt = _lib.KDA_DTYPE_BF16 if x.q.dtype == torch.bfloat16 else _lib.KDA_DTYPE_F32
    p = _lib.params(dt, H, dk, dv, floor, scale)
    cu_h = (ctypes.c_int32 * (N + 1))(*x.cu_seqlens_host)
    out = torch.full(x.v.shape, float("nan"), dtype=x.v.dtype, device="cuda")
    Sf = torch.full((N, H, dk, dv), float("nan"), dtype=torch.float32, device="cuda")
    ptr = lambda t: None if t is None else t.data_ptr()
    args = [ctypes.byref(p), ptr(x.q), ptr(x.k), ptr(x.v), ptr(x.log_alpha), ptr(x.beta),
            ptr(x.gate), cu_h, N, ptr(x.initial_state), ptr(Sf), ptr(out), L]
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = lib.kda_chunk_prefill_segmented_noalloc(*args, stream)
    else:
        need = lib.kda_prefill_segmented_workspace(ctypes.byref(p), cu_h, N, L)
        assert need > 0
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        st = lib.kda_chunk_prefill_segmented(*args, ptr(ws), need, stream)
    assert st == _lib.KDA_OK, lib.kda_last_error().decode()
    torch.cuda.synchronize()
    return out, Sf


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point_twice(dtype):
    cases = [((3000, 0, 1000, 17), 4, 256, 11), ((300, 50), 2, 64, 12)]
    for lengths, H, L, seed in cases:  # a large problem, then a smaller one
        log(f"no-alloc segmented dtype={dtype} lengths={lengths} H={H} L={L}")
        x = ki.make_prefill_inputs(lengths, H, 128, 128, dtype, 0.3, seed=seed, device="cuda",
                                   log_alpha_min=-0.05)
        o_ws, S_ws = call(x, L, -0.5, 0.9, noalloc=False)
        o_na, S_na = call(x, L, -0.5, 0.9, noalloc=True)
        assert torch.equal(o_na, o_ws), "outputs differ from the workspace entry point"
        assert torch.equal(S_na, S_ws), "final states differ from the workspace entry point"
        ro, rS = oracle_full(x, floor=-0.5, scale=0.9)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        assert_close("o", host(o_na), ro, tdt)
        assert_close("S_T", host(S_na), rS, tdt)
