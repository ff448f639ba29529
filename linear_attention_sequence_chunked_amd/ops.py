"""torch-facing wrappers over the C ABI: shape checks, output allocation, the current
stream.  Every step of the operator runs in the HIP kernels of libkda.so; there is no
CPU or PyTorch fallback."""
from __future__ import annotations

import ctypes
import weakref
from typing import Optional, Sequence, Union

import torch

from . import _lib

_DT = {torch.bfloat16: _lib.KDA_DTYPE_BF16, torch.float32: _lib.KDA_DTYPE_F32}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _on_gpu(t: torch.Tensor) -> bool:
    return t.is_cuda


def _check_dev(name, t, dtype=None):
    if not _on_gpu(t):
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check_out(name, t, shape, dtype, device):
    """A caller-supplied output buffer: the kernels write exactly `shape` elements of
    `dtype` at its address, so anything else is refused before the launch."""
    _check_dev(name, t, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")


def _check_cu_host(cu_host: Sequence[int], Ttot: int) -> None:
    if len(cu_host) < 2:
        raise ValueError("cu_seqlens needs at least two entries (N + 1, N >= 1)")
    if cu_host[0] != 0:
        raise ValueError(f"cu_seqlens[0] = {cu_host[0]}, must be 0")
    for i in range(1, len(cu_host)):
        if cu_host[i] < cu_host[i - 1]:
            raise ValueError(f"cu_seqlens decreases at index {i}")
    if cu_host[-1] != Ttot:
        raise ValueError(f"cu_seqlens[-1] = {cu_host[-1]} but the inputs hold {Ttot} tokens")


# device cu_seqlens tensors already compared with their host copy: id -> (weak reference,
# version, host tuple).  A tensor whose version counter is unchanged has not been written
# through torch since, so the comparison (a device-to-host copy and a synchronisation)
# runs once per tensor and content, not per call.
_cu_checked: dict = {}


def _check_cu_device(cu_dev: torch.Tensor, cu_host: Sequence[int]) -> None:
    hit = _cu_checked.get(id(cu_dev))
    if hit is not None and hit[0]() is cu_dev and hit[1:] == (cu_dev._version, tuple(cu_host)):
        return
    if cu_dev.dim() != 1 or cu_dev.numel() != len(cu_host):
        raise ValueError(f"cu_seqlens has shape {tuple(cu_dev.shape)}, expected "
                         f"({len(cu_host)},)")
    if [int(v) for v in cu_dev.tolist()] != [int(v) for v in cu_host]:
        raise ValueError("cu_seqlens (device) differs from cu_seqlens_host")
    if len(_cu_checked) > 64:
        for key in [k for k, v in _cu_checked.items() if v[0]() is None]:
            del _cu_checked[key]
    _cu_checked[id(cu_dev)] = (weakref.ref(cu_dev), cu_dev._version, tuple(cu_host))


def _device_cu(cu_seqlens, cu_host, dev) -> torch.Tensor:
    """The device copy of cu_seqlens the kernels read, equal to cu_host."""
    if isinstance(cu_seqlens, torch.Tensor) and _on_gpu(cu_seqlens):
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
            raise ValueError("a device cu_seqlens must be a contiguous int32 tensor")
        if cu_seqlens.device != dev:
            raise ValueError(f"cu_seqlens is on {cu_seqlens.device}, the inputs on {dev}")
        _check_cu_device(cu_seqlens, cu_host)
        return cu_seqlens
    return torch.tensor(cu_host, dtype=torch.int32, device=dev)


def chunk_prefill(q, k, v, log_alpha, beta, gate, cu_seqlens=None, initial_state=None,
                  output_final_state: bool = True, log_alpha_floor: float = -0.3,
                  scale: float = 1.0, cu_seqlens_host: Optional[Sequence[int]] = None,
                  out: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None,
                  checkpoint_every: Optional[int] = None,
                  checkpoints: Optional[torch.Tensor] = None,
                  segment_len: Optional[int] = None):
    """KDA chunked prefill.

    Fixed length: q/k/log_alpha [B, T, H, dk], v/gate [B, T, H, dv], beta [B, T, H].
    Varlen: the same tensors packed as [T_total, H, .] with cu_seqlens (int32 tensor
    or list, N+1 entries).  initial_state: fp32 [N, H, dk, dv] or None.
    Returns (o, final_state or None); o has v's shape and dtype.

    checkpoint_every=m (a multiple of 16) also writes the state after every m tokens of
    each sequence (prefix-cache snapshots) and returns (o, final_state, checkpoints),
    checkpoints fp32 [T_total // m, H, dk, dv]: sequence n's snapshot after j*m tokens is
    at slot checkpoint_slot(cu_seqlens, n, j, m); slots no snapshot maps to keep their
    contents (uninitialised when the tensor is allocated here).

    segment_len: None lets the library choose the schedule (kda_prefill_segment_plan): for
    batches with too few (sequence, head) chains to fill the GPU, each sequence is cut into
    segments that run side by side (kda_chunk_prefill_segmented, with a workspace allocated
    here); 0 forces the plain schedule, a positive multiple of 16 that segment length.
    """
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    if q.dim() == 4:
        B, T, H, dk = q.shape
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens is for packed [T_total, H, d] inputs")
        cu_host = [i * T for i in range(B + 1)]
        flat = lambda x: x.reshape(B * T, *x.shape[2:])
        qf, kf, vf, laf, bf, gf = (flat(x) for x in (q, k, v, log_alpha, beta, gate))
    elif q.dim() == 3:
        if cu_seqlens is None:
            raise ValueError("packed [T_total, H, d] inputs need cu_seqlens")
        qf, kf, vf, laf, bf, gf = q, k, v, log_alpha, beta, gate
        if cu_seqlens_host is not None:
            cu_host = [int(x) for x in cu_seqlens_host]
        elif isinstance(cu_seqlens, torch.Tensor):
            cu_host = [int(x) for x in cu_seqlens.tolist()]
        else:
            cu_host = [int(x) for x in cu_seqlens]
    else:
        raise ValueError("q must be [B, T, H, dk] or [T_total, H, dk]")
    Ttot, H, dk = qf.shape
    dv = vf.shape[-1]
    N = len(cu_host) - 1
    for name, t, shp in (("q", qf, (Ttot, H, dk)), ("k", kf, (Ttot, H, dk)),
                         ("v", vf, (Ttot, H, dv)), ("log_alpha", laf, (Ttot, H, dk)),
                         ("beta", bf, (Ttot, H)), ("gate", gf, (Ttot, H, dv))):
        _check_dev(name, t, dt)
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    dev = qf.device
    for name, t in (("k", kf), ("v", vf), ("log_alpha", laf), ("beta", bf), ("gate", gf)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")
    _check_cu_host(cu_host, Ttot)
    cu_dev = _device_cu(cu_seqlens, cu_host, dev)
    cu_h = (ctypes.c_int32 * len(cu_host))(*cu_host)
    if initial_state is not None:
        _check_out("initial_state", initial_state, (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((Ttot, H, dv), dtype=dt, device=dev)
    else:  # [T_total, H, dv], or v's [B, T, H, dv]
        _check_out("out", out, v.shape if q.dim() == 4 else (Ttot, H, dv), dt, dev)
        out = out.reshape(Ttot, H, dv)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check_out("final_state", final_state, (N, H, dk, dv), torch.float32, dev)
    p = _lib.params(_DT[dt], H, dk, dv, log_alpha_floor, scale)
    lib = _lib.load()
    if checkpoint_every is None:
        seg = segment_len
        if seg is None:
            seg = lib.kda_prefill_segment_plan(ctypes.byref(p), cu_h, N)
            if seg < 0:
                raise _lib.KdaError(_lib.KDA_ERR_INVALID_ARGUMENT, lib.kda_last_error().decode())
        if seg > 0:
            need = lib.kda_prefill_segmented_workspace(ctypes.byref(p), cu_h, N, int(seg))
            if need < 0:
                raise _lib.KdaError(_lib.KDA_ERR_INVALID_ARGUMENT, lib.kda_last_error().decode())
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
            st = lib.kda_chunk_prefill_segmented(
                ctypes.byref(p), _ptr(qf), _ptr(kf), _ptr(vf), _ptr(laf), _ptr(bf), _ptr(gf), cu_h,
                N, _ptr(initial_state), _ptr(final_state), _ptr(out), int(seg), _ptr(ws),
                ws.numel(), _stream())
            _lib.check(st)
            o = out.reshape(v.shape) if q.dim() == 4 else out
            return o, final_state
        st = lib.kda_chunk_prefill(ctypes.byref(p), _ptr(qf), _ptr(kf), _ptr(vf), _ptr(laf),
                                   _ptr(bf), _ptr(gf), _ptr(cu_dev), cu_h, N,
                                   _ptr(initial_state), _ptr(final_state), _ptr(out),
                                   _stream())
        _lib.check(st)
        o = out.reshape(v.shape) if q.dim() == 4 else out
        return o, final_state
    m = int(checkpoint_every)
    if checkpoints is None:
        checkpoints = torch.empty((Ttot // m if m > 0 else 0, H, dk, dv), dtype=torch.float32,
                                  device=dev)
    else:
        if m <= 0:
            raise ValueError(f"checkpoint_every {m} must be a positive multiple of 16")
        _check_out("checkpoints", checkpoints, (Ttot // m, H, dk, dv), torch.float32, dev)
    st = lib.kda_chunk_prefill_checkpointed(
        ctypes.byref(p), _ptr(qf), _ptr(kf), _ptr(vf), _ptr(laf), _ptr(bf), _ptr(gf),
        _ptr(cu_dev), cu_h, N, _ptr(initial_state), _ptr(final_state), _ptr(out), m,
        _ptr(checkpoints) if checkpoints.numel() else None, _stream())
    _lib.check(st)
    o = out.reshape(v.shape) if q.dim() == 4 else out
    return o, final_state, checkpoints


def checkpoint_slot(cu_seqlens: Sequence[int], n: int, j: int, m: int) -> int:
    """Slot of sequence n's snapshot after its first j*m tokens (1 <= j, j*m <= T_n)."""
    return (int(cu_seqlens[n]) + j * m) // m - 1


def decode_step(q, k, v, log_alpha, beta, gate, state, log_alpha_floor: float = -0.3,
                scale: float = 1.0, out: Optional[torch.Tensor] = None):
    """One token per sequence; `state` (fp32 [N, H, dk, dv]) is updated in place.
    q/k/log_alpha [N, H, dk], v/gate [N, H, dv], beta [N, H].  Returns o [N, H, dv]."""
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    N, H, dk = q.shape
    dv = v.shape[-1]
    for name, t, shp in (("q", q, (N, H, dk)), ("k", k, (N, H, dk)), ("v", v, (N, H, dv)),
                         ("log_alpha", log_alpha, (N, H, dk)), ("beta", beta, (N, H)),
                         ("gate", gate, (N, H, dv))):
        _check_dev(name, t, dt)
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    _check_out("state", state, (N, H, dk, dv), torch.float32, q.device)
    if out is None:
        out = torch.empty((N, H, dv), dtype=dt, device=q.device)
    else:
        _check_out("out", out, (N, H, dv), dt, q.device)
    p = _lib.params(_DT[dt], H, dk, dv, log_alpha_floor, scale)
    st = _lib.load().kda_decode_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(log_alpha), _ptr(beta), _ptr(gate), N,
                                     _ptr(state), _ptr(out), _stream())
    _lib.check(st)
    return out


def _drafts(name, t, dt, N, K, H, d):
    _check_dev(name, t, dt)
    shp = (N, K, H, d) if d else (N, K, H)
    if t.dim() == len(shp) and tuple(t.shape) == shp:
        return t
    if tuple(t.shape) == (N * K,) + shp[2:]:
        return t
    raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp} or "
                     f"{(N * K,) + shp[2:]}")


def spec_verify(q, k, v, log_alpha, beta, gate, state, log_alpha_floor: float = -0.3,
                scale: float = 1.0, out: Optional[torch.Tensor] = None):
    """Outputs of K draft tokens per sequence from `state` (fp32 [N, H, dk, dv], only
    read).  q/k/log_alpha [N, K, H, dk], v/gate [N, K, H, dv], beta [N, K, H] (or the same
    packed as [N*K, H, .]).  Returns o shaped like v."""
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    _check_dev("state", state, torch.float32)
    N, H, dk, dv = state.shape
    K = q.shape[1] if q.dim() == 4 else q.shape[0] // max(N, 1)
    for name, t, d in (("q", q, dk), ("k", k, dk), ("v", v, dv), ("log_alpha", log_alpha, dk),
                       ("beta", beta, 0), ("gate", gate, dv)):
        _drafts(name, t, dt, N, K, H, d)
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta),
                    ("gate", gate)):
        if t.device != state.device:
            raise ValueError(f"{name} is on {t.device}, state on {state.device}")
    if out is None:
        out = torch.empty(v.shape, dtype=dt, device=q.device)
    else:
        _check_out("out", out, v.shape, dt, q.device)
    p = _lib.params(_DT[dt], H, dk, dv, log_alpha_floor, scale)
    st = _lib.load().kda_spec_verify(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(log_alpha), _ptr(beta), _ptr(gate), N, K,
                                     _ptr(state), _ptr(out), _stream())
    _lib.check(st)
    return out


def spec_commit(k, v, log_alpha, beta, state, accepted, log_alpha_floor: float = -0.3):
    """Advance state (fp32 [N, H, dk, dv], in place) over the first accepted[n] of the K
    drafts of sequence n; accepted is an int32 GPU tensor [N] (clamped to [0, K])."""
    dt = k.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    _check_dev("state", state, torch.float32)
    _check_dev("accepted", accepted, torch.int32)
    N, H, dk, dv = state.shape
    if tuple(accepted.shape) != (N,):
        raise ValueError("accepted must be [N]")
    K = k.shape[1] if k.dim() == 4 else k.shape[0] // max(N, 1)
    for name, t, d in (("k", k, dk), ("v", v, dv), ("log_alpha", log_alpha, dk),
                       ("beta", beta, 0)):
        _drafts(name, t, dt, N, K, H, d)
        if t.device != state.device:
            raise ValueError(f"{name} is on {t.device}, state on {state.device}")
    if accepted.device != state.device:
        raise ValueError(f"accepted is on {accepted.device}, state on {state.device}")
    p = _lib.params(_DT[dt], H, dk, dv, log_alpha_floor, 1.0)
    st = _lib.load().kda_spec_commit(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(log_alpha),
                                     _ptr(beta), N, K, _ptr(accepted), _ptr(state),
                                     _stream())
    _lib.check(st)
    return state


def chunk_prefill_segmented(q, k, v, log_alpha, beta, gate, cu_seqlens, segment_len: int,
                            initial_state=None, output_final_state: bool = True,
                            log_alpha_floor: float = -0.3, scale: float = 1.0,
                            out: Optional[torch.Tensor] = None,
                            final_state: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None):
    """chunk_prefill for long sequences with few heads: each sequence is cut into
    segments of segment_len tokens (a multiple of 16) that run side by side and are
    joined by a scan over the segment states.  Packed [T_total, H, .] inputs with
    cu_seqlens (list, or tensor copied to the host).  Returns (o, final_state or None)."""
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    cu_host = [int(x) for x in (cu_seqlens.tolist() if isinstance(cu_seqlens, torch.Tensor)
                                else cu_seqlens)]
    Ttot, H, dk = q.shape
    dv = v.shape[-1]
    N = len(cu_host) - 1
    for name, t, shp in (("q", q, (Ttot, H, dk)), ("k", k, (Ttot, H, dk)),
                         ("v", v, (Ttot, H, dv)), ("log_alpha", log_alpha, (Ttot, H, dk)),
                         ("beta", beta, (Ttot, H)), ("gate", gate, (Ttot, H, dv))):
        _check_dev(name, t, dt)
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    _check_cu_host(cu_host, Ttot)
    if initial_state is not None:
        _check_out("initial_state", initial_state, (N, H, dk, dv), torch.float32, q.device)
    if out is not None:
        _check_out("out", out, (Ttot, H, dv), dt, q.device)
    if final_state is not None:
        _check_out("final_state", final_state, (N, H, dk, dv), torch.float32, q.device)
    if workspace is not None:
        _check_dev("workspace", workspace, torch.uint8)
        if workspace.device != q.device:
            raise ValueError(f"workspace is on {workspace.device}, q on {q.device}")
    cu_h = (ctypes.c_int32 * len(cu_host))(*cu_host)
    p = _lib.params(_DT[dt], H, dk, dv, log_alpha_floor, scale)
    lib = _lib.load()
    need = lib.kda_prefill_segmented_workspace(ctypes.byref(p), cu_h, N, int(segment_len))
    if need < 0:
        raise _lib.KdaError(_lib.KDA_ERR_INVALID_ARGUMENT, lib.kda_last_error().decode())
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((Ttot, H, dv), dtype=dt, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    st = lib.kda_chunk_prefill_segmented(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(log_alpha), _ptr(beta), _ptr(gate), cu_h, N,
                                         _ptr(initial_state), _ptr(final_state), _ptr(out),
                                         int(segment_len), _ptr(workspace), workspace.numel(),
                                         _stream())
    _lib.check(st)
    return out, final_state


def prefill_backward(q, k, v, log_alpha, beta, gate, d_out, cu_seqlens=None,
                     initial_state=None, d_final_state=None, log_alpha_floor: float = -0.3,
                     scale: float = 1.0, cu_seqlens_host: Optional[Sequence[int]] = None,
                     workspace: Optional[torch.Tensor] = None,
                     max_workspace_bytes: Optional[int] = None):
    """Gradients of chunk_prefill (fp32).  Inputs as for chunk_prefill ([B, T, H, d] or
    packed [T_total, H, d] with cu_seqlens), d_out shaped like o, d_final_state fp32
    [N, H, dk, dv] or None.  Returns a dict with dq, dk, dv, dlog_alpha, dbeta, dgate
    (fp32, shaped like the inputs) and d_initial_state (fp32 [N, H, dk, dv]).

    workspace: a uint8 device tensor used as given (the library runs groups of sequences
    that fit it; it must hold the largest single sequence's need).  Without one, a workspace
    of the whole batch's need is allocated, or of max_workspace_bytes when that is smaller
    (but never below the largest single sequence's need)."""
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    shapes = {n: t.shape for n, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha),
                                      ("beta", beta), ("gate", gate))}
    if q.dim() == 4:
        B, T, H, dk = q.shape
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens is for packed [T_total, H, d] inputs")
        cu_host = [i * T for i in range(B + 1)]
        flat = lambda x: x.reshape(B * T, *x.shape[2:])
        q, k, v, log_alpha, beta, gate, d_out = (flat(x) for x in
                                                 (q, k, v, log_alpha, beta, gate, d_out))
    else:
        if cu_seqlens is None:
            raise ValueError("packed [T_total, H, d] inputs need cu_seqlens")
        if cu_seqlens_host is not None:
            cu_host = [int(x) for x in cu_seqlens_host]
        elif isinstance(cu_seqlens, torch.Tensor):
            cu_host = [int(x) for x in cu_seqlens.tolist()]
        else:
            cu_host = [int(x) for x in cu_seqlens]
    Ttot, H, dk = q.shape
    dv = v.shape[-1]
    N = len(cu_host) - 1
    for name, t, shp in (("q", q, (Ttot, H, dk)), ("k", k, (Ttot, H, dk)),
                         ("v", v, (Ttot, H, dv)), ("log_alpha", log_alpha, (Ttot, H, dk)),
                         ("beta", beta, (Ttot, H)), ("gate", gate, (Ttot, H, dv)),
                         ("d_out", d_out, (Ttot, H, dv))):
        _check_dev(name, t, dt)
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    dev = q.device
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None:
            _check_out(name, t, (N, H, dk, dv), torch.float32, dev)
    _check_cu_host(cu_host, Ttot)
    cu_dev = _device_cu(cu_seqlens, cu_host, dev)
    cu_h = (ctypes.c_int32 * len(cu_host))(*cu_host)
    p = _lib.params(_DT[dt], H, dk, dv, log_alpha_floor, scale)
    lib = _lib.load()
    need = lib.kda_prefill_backward_workspace(ctypes.byref(p), cu_h, N)
    if need < 0:
        raise _lib.KdaError(_lib.KDA_ERR_INVALID_ARGUMENT, lib.kda_last_error().decode())
    if workspace is None:
        size = need
        if max_workspace_bytes is not None and max_workspace_bytes < need:
            one = max(lib.kda_prefill_backward_workspace(
                ctypes.byref(p), (ctypes.c_int32 * 2)(0, cu_host[n + 1] - cu_host[n]), 1)
                for n in range(N))
            size = max(int(max_workspace_bytes), one)
        workspace = torch.empty(max(size, 256), dtype=torch.uint8, device=dev)
    else:
        _check_dev("workspace", workspace, torch.uint8)
        if workspace.device != dev:
            raise ValueError(f"workspace is on {workspace.device}, q on {dev}")
    f32 = lambda shp: torch.empty(shp, dtype=torch.float32, device=dev)
    g = dict(dq=f32((Ttot, H, dk)), dk=f32((Ttot, H, dk)), dv=f32((Ttot, H, dv)),
             dlog_alpha=f32((Ttot, H, dk)), dbeta=f32((Ttot, H)), dgate=f32((Ttot, H, dv)),
             d_initial_state=f32((N, H, dk, dv)))
    st = lib.kda_prefill_backward(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(gate),
        _ptr(cu_dev), cu_h, N, _ptr(initial_state), _ptr(d_out), _ptr(d_final_state),
        _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_alpha"]), _ptr(g["dbeta"]),
        _ptr(g["dgate"]), _ptr(g["d_initial_state"]), _ptr(workspace), workspace.numel(),
        _stream())
    _lib.check(st)
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_alpha", "dlog_alpha"),
                      ("beta", "dbeta"), ("gate", "dgate")):
        g[key] = g[key].reshape(shapes[name])
    return g
