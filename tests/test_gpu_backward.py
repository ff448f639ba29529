"""GPU parity of kda_prefill_backward against the oracle's reverse-mode gradients
(oracle/reference.py recurrent_backward, pinned by finite differences in
tests/test_oracle_backward.py), per (sequence, head), on the same rounded inputs.

Tolerance, per gradient tensor: max|err| <= TOL * RMS(ref), TOL = 32 * 2^-16 (~4.9e-4),
the same for bf16 and fp32 inputs because the backward computes the same way for both (the
inputs are exact in fp32; the state, its gradient and every sum are fp32).  Where it comes
from: the two walks form every product of the chunk recurrence from split-bf16 operands,
x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), and drop the lo*lo term, so each
product carries a relative error of at most ~3 * 2^-16 (each half rounds to within 2^-8
of what it represents); a sum of 128 such products over the key channels can grow that by
up to sqrt(128) ~ 11 relative to its own size where its terms cancel; and the transition
of a chunk is non-expansive, so the errors carried along the recurrence add up to a
bounded multiple (about 3x on these inputs) of one chunk's.  The gradient kernel itself
runs fp32 products (2^-24).  Measured errors are 1e-5 to 1.5e-4 of RMS."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import linear_attention_sequence_chunked_amd as kda
from oracle import reference as ref
from parity import host, log

pytestmark = pytest.mark.gpu
TOL = 32 * 2.0 ** -16


def check(name, got, want, zero_scale=0.0):
    """max|err| <= TOL * RMS(want).  Where the oracle's tensor is identically zero (a
    one-token sequence without S0 and dS_final has no decay gradient: the decay multiplies
    a zero state), the relative form divides by zero; the bar is then TOL * zero_scale in
    absolute terms, zero_scale being the size of the products that cancel to form it
    (exactly zero when none is given).  Empty tensors (no tokens) pass only if both are."""
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    if want.size == 0:
        log(f"  {name}: empty")
        return
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    rms = float(np.sqrt(np.mean(want * want)))
    if rms == 0.0:
        err = float(np.max(np.abs(got)))
        log(f"  {name}: the oracle's tensor is zero; max|got| = {err:.2e} "
            f"(bar {TOL * zero_scale:.2e})")
        assert err <= TOL * zero_scale, f"{name}: {err:.3e} > {TOL * zero_scale:.3e}"
        return
    err = float(np.max(np.abs(got - want))) / max(rms, 1e-30)
    log(f"  {name}: max|err|/RMS = {err:.2e} (tol {TOL:.2e}, margin {TOL / max(err, 1e-30):.1f}x)")
    assert err <= TOL, f"{name}: {err:.3e} > {TOL}"


def run_case(x, do, dSf, floor, scale, pairs=None):
    g = kda.prefill_backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, do,
                             cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_seqlens_host,
                             initial_state=x.initial_state, d_final_state=dSf,
                             log_alpha_floor=floor, scale=scale)
    torch.cuda.synchronize()
    cu = x.cu_seqlens_host
    H = x.q.shape[1]
    N = len(cu) - 1
    pairs = pairs or [(n, h) for n in range(N) for h in range(H)]
    want = {k: [] for k in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dgate", "dS0")}
    got = {k: [] for k in want}
    for n, h in pairs:
        a, e = cu[n], cu[n + 1]
        sl = lambda t: host(t[a:e, h])
        r = ref.recurrent_backward(sl(x.q), sl(x.k), sl(x.v), sl(x.log_alpha), sl(x.beta),
                                   sl(x.gate), sl(do),
                                   None if dSf is None else host(dSf[n, h]),
                                   None if x.initial_state is None else host(x.initial_state[n, h]),
                                   floor=floor, scale=scale)
        for key, gk in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dlog_alpha", "dlog_alpha"),
                        ("dbeta", "dbeta"), ("dgate", "dgate")):
            want[key].append(r[key].reshape(-1))
            got[key].append(host(g[gk][a:e, h]).reshape(-1))
        want["dS0"].append(r["dS0"].reshape(-1))
        got["dS0"].append(host(g["d_initial_state"][n, h]).reshape(-1))
    # the decay gradient sums products of q with dq and of k with dk (the terms of the
    # decay-folded operands' gradients), which cancel exactly where it vanishes
    rms = lambda a: float(np.sqrt(np.mean(a * a))) if a.size else 0.0
    qk = [(host(x.q[cu[n]:cu[n + 1], h]).reshape(-1), host(x.k[cu[n]:cu[n + 1], h]).reshape(-1))
          for n, h in pairs]
    qdq = np.concatenate([q * d for (q, _), d in zip(qk, want["dq"])])
    kdk = np.concatenate([k * d for (_, k), d in zip(qk, want["dk"])])
    for key in want:
        check(key, np.concatenate(got[key]), np.concatenate(want[key]),
              zero_scale=rms(qdq) + rms(kdk) if key == "dlog_alpha" else 0.0)
    return g


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_backward_varlen(dtype, dk, dv):
    lengths = (37, 0, 16, 1, 50)
    log(f"backward dtype={dtype} dk={dk} dv={dv}")
    x = ki.make_prefill_inputs(lengths, 2, dk, dv, dtype, 0.3, seed=dk + 2 * dv,
                               device="cuda", log_alpha_min=-0.6)
    g = torch.Generator().manual_seed(dk + dv)
    do = (torch.randn(x.v.shape, generator=g) * 0.5).to(x.v.dtype).cuda()
    dSf = (torch.randn(x.initial_state.shape, generator=g) * 0.1).cuda()
    # floor -0.4: part of the log-decays (drawn down to -0.6) are clamped
    run_case(x, do, dSf, floor=-0.4, scale=0.8)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_chunk_pairs(dtype):
    """Sequences of 7, 3, 4, 2, 0 and 3 chunks: pairs of chunks with and without a second
    chunk, ragged last chunks, and pairs whose state and gradient are both re-formed from the
    stored ones (the gradient kernel takes two chunks per workgroup)."""
    lengths = (100, 33, 64, 17, 0, 48)
    log(f"backward chunk pairs dtype={dtype} lengths={lengths}")
    x = ki.make_prefill_inputs(lengths, 3, 128, 128, dtype, 0.3, seed=71, device="cuda",
                               log_alpha_min=-0.6)
    g = torch.Generator().manual_seed(71)
    do = (torch.randn(x.v.shape, generator=g) * 0.5).to(x.v.dtype).cuda()
    dSf = (torch.randn(x.initial_state.shape, generator=g) * 0.1).cuda()
    run_case(x, do, dSf, floor=-0.4, scale=0.9)


def test_backward_no_initial_state_no_state_gradient():
    x = ki.make_prefill_inputs((70, 33), 2, 64, 64, "bf16", 0.0, seed=9, device="cuda")
    assert x.initial_state is None
    g = torch.Generator().manual_seed(9)
    do = torch.randn(x.v.shape, generator=g).to(x.v.dtype).cuda()
    run_case(x, do, None, floor=-0.3, scale=1.0)


def test_backward_bench_workload_sampled():
    """B=4, H=16, T=4096, d=128, bf16: two (sequence, head) pairs against the oracle."""
    w = ki.WORKLOADS["prefill_b4_h16_t4096"]
    log("backward on prefill_b4_h16_t4096 (sampled)")
    x = ki.make_workload_inputs(w, seed=1, device="cuda")
    g = torch.Generator().manual_seed(1)
    do = torch.randn(x.v.shape, generator=g).to(x.v.dtype).cuda()
    run_case(x, do, None, floor=-0.3, scale=1.0, pairs=[(0, 3), (3, 12)])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_many_items_per_workgroup(dtype):
    """More (pair of chunks, head) items than compute units (538 at H=8): each persistent
    gradient workgroup takes several in turn, loading the next one's operands while it
    finishes the current one.  Every (sequence, head) against the oracle."""
    lengths = (700, 513, 250, 31, 0, 480)
    log(f"backward many items per workgroup dtype={dtype} lengths={lengths} H=8")
    x = ki.make_prefill_inputs(lengths, 8, 128, 128, dtype, 0.3, seed=81, device="cuda",
                               log_alpha_min=-0.6)
    g = torch.Generator().manual_seed(81)
    do = torch.randn(x.v.shape, generator=g).to(x.v.dtype).cuda()
    dSf = (torch.randn(x.initial_state.shape, generator=g) * 0.1).cuda()
    run_case(x, do, dSf, floor=-0.4, scale=0.9)


@pytest.mark.parametrize("n_seq", [100, 300])
def test_backward_many_sequences(n_seq):
    """Batches of 100 and 300 sequences of 0..40 tokens: the gradient kernel finds an item's
    sequence among bounds held in registers (fewer than 256 sequences) or by a search of
    cu_seqlens in memory (more)."""
    rng = np.random.default_rng(n_seq)
    lengths = tuple(int(v) for v in rng.integers(0, 41, n_seq))
    log(f"backward {n_seq} sequences, {sum(lengths)} tokens")
    x = ki.make_prefill_inputs(lengths, 1, 64, 64, "bf16", 0.3, seed=n_seq, device="cuda")
    g = torch.Generator().manual_seed(n_seq)
    do = torch.randn(x.v.shape, generator=g).to(x.v.dtype).cuda()
    dSf = (torch.randn(x.initial_state.shape, generator=g) * 0.1).cuda()
    run_case(x, do, dSf, floor=-0.3, scale=1.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_strongest_decay_floor(dtype):
    """Floor -5 with log-decays drawn down to -5: decay-folded operands span ~e^80 within a
    chunk (finite in fp32 and in bf16 hi/lo pairs)."""
    log(f"backward floor=-5 dtype={dtype}")
    x = ki.make_prefill_inputs((40, 64, 17), 2, 128, 128, dtype, 0.3, seed=56, device="cuda",
                               log_alpha_min=-5.0)
    g = torch.Generator().manual_seed(56)
    do = torch.randn(x.v.shape, generator=g).to(x.v.dtype).cuda()
    dSf = (torch.randn(x.initial_state.shape, generator=g) * 0.1).cuda()
    run_case(x, do, dSf, floor=-5.0, scale=1.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_workspace_groups(dtype):
    """A workspace short of the batch's need: the library runs groups of consecutive
    sequences, one after another.  Every gradient equals the single-launch result bit for bit
    (each chunk's arithmetic is the same), for a workspace of one sequence's need and one of
    about half the batch's."""
    lengths = (100, 33, 64, 17, 0, 48)
    log(f"backward workspace groups dtype={dtype}")
    x = ki.make_prefill_inputs(lengths, 3, 128, 128, dtype, 0.3, seed=73, device="cuda",
                               log_alpha_min=-0.6)
    g = torch.Generator().manual_seed(73)
    do = (torch.randn(x.v.shape, generator=g) * 0.5).to(x.v.dtype).cuda()
    dSf = (torch.randn(x.initial_state.shape, generator=g) * 0.1).cuda()
    kw = dict(cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_seqlens_host,
              initial_state=x.initial_state, d_final_state=dSf, log_alpha_floor=-0.4, scale=0.9)
    full = kda.prefill_backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, do, **kw)
    lib = kda.load_library()
    import ctypes
    from linear_attention_sequence_chunked_amd import _lib as klib
    p = klib.params(klib.KDA_DTYPE_BF16 if dtype == "bf16" else klib.KDA_DTYPE_F32, 3, 128, 128,
                    -0.4, 0.9)
    cu = x.cu_seqlens_host
    need = lib.kda_prefill_backward_workspace(ctypes.byref(p), (ctypes.c_int32 * len(cu))(*cu),
                                              len(lengths))
    one = max(lib.kda_prefill_backward_workspace(ctypes.byref(p), (ctypes.c_int32 * 2)(0, L), 1)
              for L in lengths)
    assert one < need
    for size in (one, (need + one) // 2):
        part = kda.prefill_backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, do,
                                    max_workspace_bytes=size, **kw)
        torch.cuda.synchronize()
        for key in full:
            assert torch.equal(full[key], part[key]), f"{key} differs with a {size}-byte workspace"
    log(f"  groups equal to the single launch (workspace {one} and {(need + one) // 2} of {need} bytes)")


def test_backward_writes_every_element_and_is_deterministic():
    """Through the C ABI with NaN-poisoned outputs inside guard bands: every gradient element is
    written (no NaN left), nothing outside the outputs is (guards intact), and two runs agree
    bit for bit (no atomics)."""
    import ctypes
    from linear_attention_sequence_chunked_amd import _lib as klib
    lengths, H, d = (100, 33, 64, 17, 0, 48), 3, 128
    log("backward guards / NaN poison / determinism")
    x = ki.make_prefill_inputs(lengths, H, d, d, "bf16", 0.3, seed=79, device="cuda")
    g = torch.Generator().manual_seed(79)
    do = torch.randn(x.v.shape, generator=g).to(torch.bfloat16).cuda()
    T, N = x.total_tokens, len(lengths)
    lib = kda.load_library()
    p = klib.params(klib.KDA_DTYPE_BF16, H, d, d)
    cu = x.cu_seqlens_host
    cu_h = (ctypes.c_int32 * len(cu))(*cu)
    need = lib.kda_prefill_backward_workspace(ctypes.byref(p), cu_h, N)
    guard = 4096
    sizes = dict(dq=T * H * d, dk=T * H * d, dv=T * H * d, dla=T * H * d, dbeta=T * H,
                 dgate=T * H * d, ds0=N * H * d * d)
    runs = []
    for _ in range(2):
        bufs = {k: torch.full((n + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
                for k, n in sizes.items()}
        for b in bufs.values():
            b[:guard] = -7.5
            b[-guard:] = -7.5
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ptr = lambda k: bufs[k][guard:].data_ptr()
        st = lib.kda_prefill_backward(
            ctypes.byref(p), x.q.data_ptr(), x.k.data_ptr(), x.v.data_ptr(),
            x.log_alpha.data_ptr(), x.beta.data_ptr(), x.gate.data_ptr(), x.cu_seqlens.data_ptr(),
            cu_h, N, x.initial_state.data_ptr(), do.data_ptr(), None, ptr("dq"), ptr("dk"),
            ptr("dv"), ptr("dla"), ptr("dbeta"), ptr("dgate"), ptr("ds0"), ws.data_ptr(), need,
            torch.cuda.current_stream().cuda_stream)
        assert st == 0, lib.kda_last_error().decode()
        torch.cuda.synchronize()
        for k, b in bufs.items():
            body = b[guard:guard + sizes[k]]
            assert torch.isfinite(body).all(), f"{k}: elements left unwritten"
            assert torch.all(b[:guard] == -7.5) and torch.all(b[-guard:] == -7.5), f"{k}: guard"
        runs.append({k: b[guard:guard + sizes[k]].clone() for k, b in bufs.items()})
    for k in sizes:
        assert torch.equal(runs[0][k], runs[1][k]), f"{k} differs between runs"
