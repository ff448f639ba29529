"""Host-side validation of the torch wrappers (ops.py): every size, shape, dtype and
device mismatch that would make a kernel read or write outside its buffers is refused
with a ValueError before anything is launched.

These run without a GPU: the wrappers' GPU-residency test is redirected so that CPU
tensors stand in for device tensors, and the library is replaced by a stub that fails
the test if any entry point is reached."""
import pytest
import torch

import kda_inputs as ki
from linear_attention_sequence_chunked_amd import _lib, ops


class _NoLaunch:
    def __getattr__(self, name):
        raise AssertionError(f"{name} reached: validation should have refused the call")


@pytest.fixture(autouse=True)
def cpu_stands_in_for_gpu(monkeypatch):
    monkeypatch.setattr(ops, "_on_gpu", lambda t: True)
    monkeypatch.setattr(_lib, "load", lambda: _NoLaunch())


def inputs(lengths=(20, 0, 33), H=2, d=64, dtype="bf16", s0=0.1):
    return ki.make_prefill_inputs(lengths, H, d, d, dtype, s0, seed=1)


def prefill(x, **kw):
    args = dict(cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_seqlens_host,
                initial_state=x.initial_state)
    args.update(kw)
    return ops.chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, **args)


@pytest.mark.parametrize("cu,msg", [
    ([0, 20, 20], "inputs hold 53 tokens"),      # last entry short of T_total
    ([0, 20, 20, 60], "inputs hold 53 tokens"),  # past T_total
    ([1, 20, 20, 53], "must be 0"),
    ([0, 30, 20, 53], "decreases"),
    ([0], "at least two"),
])
def test_prefill_rejects_bad_cu_seqlens_host(cu, msg):
    x = inputs()
    with pytest.raises(ValueError, match=msg):
        prefill(x, cu_seqlens=torch.tensor(cu, dtype=torch.int32), cu_seqlens_host=cu)


def test_prefill_rejects_device_cu_seqlens_differing_from_host():
    x = inputs()
    dev = torch.tensor([0, 20, 21, 53], dtype=torch.int32)
    with pytest.raises(ValueError, match="differs from cu_seqlens_host"):
        prefill(x, cu_seqlens=dev)
    with pytest.raises(ValueError, match="shape"):
        prefill(x, cu_seqlens=torch.tensor([0, 20, 53], dtype=torch.int32))
    with pytest.raises(ValueError, match="int32"):
        prefill(x, cu_seqlens=x.cu_seqlens.to(torch.int64))


def test_device_cu_seqlens_rechecked_after_in_place_change():
    x = inputs()
    cu = x.cu_seqlens.clone()
    ops._check_cu_device(cu, x.cu_seqlens_host)  # passes and is remembered
    cu[1] = 19                                   # bumps the version counter
    with pytest.raises(ValueError, match="differs"):
        ops._check_cu_device(cu, x.cu_seqlens_host)


@pytest.mark.parametrize("name,shape,dtype", [
    ("out", (53, 2, 32), torch.bfloat16),
    ("out", (52, 2, 64), torch.bfloat16),
    ("out", (53, 2, 64), torch.float32),
    ("final_state", (3, 2, 64, 32), torch.float32),
    ("final_state", (2, 2, 64, 64), torch.float32),
    ("final_state", (3, 2, 64, 64), torch.bfloat16),
    ("initial_state", (3, 2, 32, 64), torch.float32),
    ("initial_state", (4, 2, 64, 64), torch.float32),
])
def test_prefill_rejects_mis_sized_buffers(name, shape, dtype):
    x = inputs()
    with pytest.raises(ValueError, match=name):
        prefill(x, **{name: torch.zeros(shape, dtype=dtype)})


def test_prefill_rejects_non_contiguous_buffers():
    x = inputs()
    out = torch.zeros((53, 2, 128), dtype=torch.bfloat16)[..., ::2]
    with pytest.raises(ValueError, match="out must be contiguous"):
        prefill(x, out=out)


def test_prefill_rejects_bad_checkpoint_buffer():
    x = inputs()
    with pytest.raises(ValueError, match="checkpoints"):
        prefill(x, checkpoint_every=16, checkpoints=torch.zeros((2, 2, 64, 64)))
    with pytest.raises(ValueError, match="positive multiple"):
        prefill(x, checkpoint_every=0, checkpoints=torch.zeros((0, 2, 64, 64)))


def test_decode_rejects_mis_sized_buffers():
    d = ki.make_decode_inputs(1, 3, 2, 64, 64, "bf16", seed=2)
    q, k, v, la, b, g = (d[n][0] for n in ("q", "k", "v", "log_alpha", "beta", "gate"))
    st = ki.make_state(3, 2, 64, 64, 0.1, seed=2)
    with pytest.raises(ValueError, match="out"):
        ops.decode_step(q, k, v, la, b, g, st, out=torch.zeros((3, 2, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out"):
        ops.decode_step(q, k, v, la, b, g, st, out=torch.zeros((3, 2, 64)))
    with pytest.raises(ValueError, match="state"):
        ops.decode_step(q, k, v, la, b, g, st[:2].contiguous())
    with pytest.raises(ValueError, match="beta"):
        ops.decode_step(q, k, v, la, b[:, :1].contiguous(), g, st)


def test_spec_rejects_mis_sized_buffers():
    x = ki.make_prefill_inputs((4,) * 3, 2, 64, 64, "bf16", 0.1, seed=3)
    with pytest.raises(ValueError, match="out"):
        ops.spec_verify(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, x.initial_state,
                        out=torch.zeros((11, 2, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="accepted"):
        ops.spec_commit(x.k, x.v, x.log_alpha, x.beta, x.initial_state,
                        torch.zeros((2,), dtype=torch.int32))


def test_segmented_rejects_bad_sizes():
    x = inputs()
    run = lambda **kw: ops.chunk_prefill_segmented(
        x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, kw.pop("cu", x.cu_seqlens_host), 32,
        initial_state=x.initial_state, **kw)
    with pytest.raises(ValueError, match="inputs hold 53 tokens"):
        run(cu=[0, 20, 20, 50])
    with pytest.raises(ValueError, match="final_state"):
        run(final_state=torch.zeros((3, 2, 64, 32)))
    with pytest.raises(ValueError, match="out"):
        run(out=torch.zeros((50, 2, 64), dtype=torch.bfloat16))


def test_backward_rejects_bad_sizes():
    x = inputs()
    do = torch.zeros_like(x.v)
    run = lambda **kw: ops.prefill_backward(
        x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, kw.pop("d_out", do),
        cu_seqlens=kw.pop("cu", x.cu_seqlens), initial_state=x.initial_state, **kw)
    with pytest.raises(ValueError, match="d_out"):
        run(d_out=do[:50].contiguous())
    with pytest.raises(ValueError, match="d_final_state"):
        run(d_final_state=torch.zeros((3, 2, 64, 32)))
    with pytest.raises(ValueError, match="differs"):
        run(cu=torch.tensor([0, 21, 21, 53], dtype=torch.int32),
            cu_seqlens_host=x.cu_seqlens_host)
