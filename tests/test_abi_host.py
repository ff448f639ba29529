"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from linear_attention_sequence_chunked_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

A = 1 << 20  # a fake, 16-byte aligned "device" address; never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.kda_abi_version() == 1


def test_status_strings():
    lib = _lib.load()
    for s in range(4):
        assert lib.kda_status_string(s)
    assert lib.kda_status_string(99) == b"unknown status"


def cu(*vals):
    return (ctypes.c_int32 * len(vals))(*vals)


def prefill(p=None, q=A, k=A + 0x10000, v=A + 0x20000, la=A + 0x30000, beta=A + 0x40000,
            gate=A + 0x50000, cu_dev=A + 0x60000, cu_host=None, n=2, s0=None, sf=None,
            out=A + 0x70000):
    lib = _lib.load()
    if p is None:
        p = _lib.params(_lib.KDA_DTYPE_BF16, 2, 64, 64)
    if cu_host is None:
        cu_host = cu(0, 3, 5)
    pp = ctypes.byref(p) if p is not False else None
    st = lib.kda_chunk_prefill(pp, q, k, v, la, beta, gate, cu_dev, cu_host, n, s0, sf, out,
                               None)
    return st, lib.kda_last_error().decode()


def decode(p=None, q=A, k=A + 0x10000, v=A + 0x20000, la=A + 0x30000, beta=A + 0x40000,
           gate=A + 0x50000, n=2, state=A + 0x100000, out=A + 0x70000):
    lib = _lib.load()
    if p is None:
        p = _lib.params(_lib.KDA_DTYPE_BF16, 2, 64, 64)
    st = lib.kda_decode_step(ctypes.byref(p), q, k, v, la, beta, gate, n, state, out, None)
    return st, lib.kda_last_error().decode()


INV, UNS = _lib.KDA_ERR_INVALID_ARGUMENT, _lib.KDA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,status,msg", [
    (dict(p=False), INV, "params is NULL"),
    (dict(p=_lib.params(7, 2, 64, 64)), INV, "dtype"),
    (dict(p=_lib.params(0, 0, 64, 64)), INV, "num_heads"),
    (dict(p=_lib.params(0, 2, 64, 64, chunk=32)), UNS, "chunk"),
    (dict(p=_lib.params(0, 2, 96, 64)), UNS, "dk=96"),
    (dict(p=_lib.params(0, 2, 64, 256)), UNS, "dv=256"),
    (dict(p=_lib.params(0, 2, 64, 64, floor=0.5)), INV, "log_alpha_floor"),
    (dict(p=_lib.params(0, 2, 64, 64, floor=-6.0)), INV, "log_alpha_floor"),
    (dict(p=_lib.params(0, 2, 64, 64, floor=float("nan"))), INV, "log_alpha_floor"),
    (dict(p=_lib.params(0, 2, 64, 64, scale=float("inf"))), INV, "scale"),
    (dict(n=0), INV, "num_seqs"),
    (dict(cu_host=False), INV, "cu_seqlens_host is NULL"),
    (dict(cu_dev=None), INV, "cu_seqlens is NULL"),
    (dict(cu_host=cu(1, 3, 5)), INV, "must be 0"),
    (dict(cu_host=cu(0, 5, 3)), INV, "decreases"),
    (dict(q=None), INV, "q is NULL"),
    (dict(k=A + 8), INV, "k is not 16-byte aligned"),
    (dict(gate=None), INV, "gate is NULL"),
    (dict(beta=A + 1), INV, "beta is not 2-byte aligned"),
    (dict(out=None), INV, "out is NULL"),
    (dict(out=A + 0x10000), INV, "out overlaps k"),
    (dict(s0=A + 4), INV, "initial_state is not 16-byte aligned"),
    (dict(s0=A + 0x100000, sf=A + 0x100000 + 256), INV, "final_state overlaps initial_state"),
    (dict(sf=A + 0x70000), INV, "final_state overlaps out"),
    (dict(sf=A + 0x20000), INV, "final_state overlaps v"),
])
def test_prefill_rejects(kw, status, msg):
    if kw.get("cu_host") is False:
        kw["cu_host"] = None
        lib = _lib.load()
        p = _lib.params(_lib.KDA_DTYPE_BF16, 2, 64, 64)
        st = lib.kda_chunk_prefill(ctypes.byref(p), A, A, A, A, A, A, A, None, 2, None, None,
                                   A, None)
        assert st == status
        assert msg in lib.kda_last_error().decode()
        return
    st, err = prefill(**kw)
    assert st == status, err
    assert msg in err, err


@pytest.mark.parametrize("kw,status,msg", [
    (dict(p=_lib.params(0, 2, 64, 64, chunk=8)), UNS, "chunk"),
    (dict(n=-1), INV, "num_seqs"),
    (dict(state=None), INV, "state is NULL"),
    (dict(state=A + 0x100008), INV, "state is not 16-byte aligned"),
    (dict(out=A), INV, "out overlaps q"),
    (dict(out=A + 0x100000), INV, "out overlaps state"),
    (dict(state=A + 0x40000), INV, "state overlaps beta"),
    (dict(v=None), INV, "v is NULL"),
])
def test_decode_rejects(kw, status, msg):
    st, err = decode(**kw)
    assert st == status, err
    assert msg in err, err


def test_decode_zero_sequences_is_a_no_op():
    st, err = decode(n=0, q=None, state=None)
    assert st == _lib.KDA_OK and err == ""


def prefill_ckpt(m=16, ck=A + 0x200000, cu_host=None, sf=None, out=A + 0x70000):
    """Two sequences of 20 tokens (T_total = 40), H = 2, d = 64, bf16."""
    lib = _lib.load()
    p = _lib.params(_lib.KDA_DTYPE_BF16, 2, 64, 64)
    if cu_host is None:
        cu_host = cu(0, 20, 40)
    st = lib.kda_chunk_prefill_checkpointed(ctypes.byref(p), A, A + 0x10000, A + 0x20000,
                                            A + 0x30000, A + 0x40000, A + 0x50000, A + 0x60000,
                                            cu_host, 2, None, sf, out, m, ck, None)
    return st, lib.kda_last_error().decode()


@pytest.mark.parametrize("kw,msg", [
    (dict(m=0), "checkpoint_every 0"),
    (dict(m=-16), "checkpoint_every -16"),
    (dict(m=24), "checkpoint_every 24"),
    (dict(ck=None), "checkpoints is NULL"),
    (dict(ck=A + 0x200008), "checkpoints is not 16-byte aligned"),
    (dict(ck=A + 0x70000 + 64), "checkpoints overlaps out"),
    (dict(ck=A + 0x30000), "checkpoints overlaps log_alpha"),
    (dict(sf=A + 0x200000 + 0x8000), "checkpoints overlaps final_state"),
])
def test_prefill_checkpointed_rejects(kw, msg):
    st, err = prefill_ckpt(**kw)
    assert st == INV, err
    assert msg in err, err



def spec(verify=True, n=2, K=4, q=A, k=A + 0x10000, v=A + 0x20000, la=A + 0x30000,
         beta=A + 0x40000, gate=A + 0x50000, acc=A + 0x60000, state=A + 0x100000,
         out=A + 0x70000):
    lib = _lib.load()
    p = _lib.params(_lib.KDA_DTYPE_BF16, 2, 64, 64)
    if verify:
        st = lib.kda_spec_verify(ctypes.byref(p), q, k, v, la, beta, gate, n, K, state, out,
                                 None)
    else:
        st = lib.kda_spec_commit(ctypes.byref(p), k, v, la, beta, n, K, acc, state, None)
    return st, lib.kda_last_error().decode()


@pytest.mark.parametrize("verify", [True, False])
@pytest.mark.parametrize("kw,msg", [
    (dict(K=0), "num_draft 0"),
    (dict(K=17), "num_draft 17"),
    (dict(n=-1), "num_seqs"),
    (dict(k=None), "k is NULL"),
    (dict(v=A + 0x20004), "v is not 16-byte aligned"),
    (dict(beta=A + 0x40001), "beta is not 2-byte aligned"),
    (dict(state=None), "state is NULL"),
])
def test_spec_rejects(verify, kw, msg):
    st, err = spec(verify=verify, **kw)
    assert st == INV, err
    assert msg in err, err


@pytest.mark.parametrize("kw,msg", [
    (dict(q=None), "q is NULL"),
    (dict(gate=None), "gate is NULL"),
    (dict(out=None), "out is NULL"),
    (dict(out=A + 0x100000), "out overlaps state"),
    (dict(out=A + 0x20000), "out overlaps v"),
])
def test_spec_verify_rejects(kw, msg):
    st, err = spec(verify=True, **kw)
    assert st == INV, err
    assert msg in err, err


@pytest.mark.parametrize("kw,msg", [
    (dict(acc=None), "accepted is NULL"),
    (dict(acc=A + 0x60002), "accepted is not 4-byte aligned"),
    (dict(state=A + 0x30000), "state overlaps log_alpha"),
    (dict(state=A + 0x60000 - 16), "state overlaps"),
])
def test_spec_commit_rejects(kw, msg):
    st, err = spec(verify=False, **kw)
    assert st == INV, err
    assert msg in err, err


def test_spec_zero_sequences_is_a_no_op():
    for verify in (True, False):
        st, err = spec(verify=verify, n=0, q=None, state=None, acc=None)
        assert st == _lib.KDA_OK, err


def seg_ws(cu_host, L, p=None):
    lib = _lib.load()
    p = p or _lib.params(_lib.KDA_DTYPE_BF16, 2, 64, 64)
    n = len(cu_host) - 1
    return lib.kda_prefill_segmented_workspace(ctypes.byref(p), cu(*cu_host), n, L)


def test_segmented_workspace_size():
    """cu = (0, 40, 40, 100), L = 32: segments [0,32) [32,40) [40,72) [72,100) -> 4.
    Layout (256-byte aligned regions): segment table (5 int32), first-segment table
    (4 int32), transitions 4*H*dk*dk fp32, own states and incoming states 4*H*dk*dv fp32
    each."""
    M = 4 * 2 * 64 * 64 * 4
    assert seg_ws((0, 40, 40, 100), 32) == 512 + M + M + M
    # one segment per sequence when L covers it; empty sequences have none
    assert seg_ws((0, 16, 16), 512) == 256 + 256 + 3 * (1 * 2 * 64 * 64 * 4)


@pytest.mark.parametrize("L", [0, -16, 24])
def test_segmented_workspace_rejects_segment_len(L):
    assert seg_ws((0, 40), L) == -1
    assert "segment_len" in _lib.load().kda_last_error().decode()


def prefill_seg(L=32, ws=A + 0x400000, ws_bytes=1 << 22, cu_host=None, out=A + 0x70000):
    lib = _lib.load()
    p = _lib.params(_lib.KDA_DTYPE_BF16, 2, 64, 64)
    cu_host = cu_host or cu(0, 40, 100)
    st = lib.kda_chunk_prefill_segmented(ctypes.byref(p), A, A + 0x10000, A + 0x20000,
                                         A + 0x30000, A + 0x40000, A + 0x50000, cu_host, 2,
                                         None, None, out, L, ws, ws_bytes, None)
    return st, lib.kda_last_error().decode()


@pytest.mark.parametrize("kw,msg", [
    (dict(L=40), "segment_len 40"),
    (dict(ws=None), "workspace is NULL"),
    (dict(ws=A + 0x400010), "workspace is not 256-byte aligned"),
    (dict(ws_bytes=1024), "workspace_bytes 1024"),
    (dict(ws=A + 0x20000 - 0x100), "workspace overlaps"),
    (dict(out=A + 0x10000), "out overlaps k"),
    (dict(cu_host=cu(0, 50, 40)), "decreases"),
])
def test_segmented_rejects(kw, msg):
    st, err = prefill_seg(**kw)
    assert st == INV, err
    assert msg in err, err


def test_backward_workspace_size():
    """cu = (0, 40, 40, 100), H = 2, d = 64: the state entering each even chunk 2j at pair
    slot cu[n]/32 + n + j (at most 100 // 32 + 3 = 6 slots per head; the sequences of 3, 0
    and 4 chunks take slots {0, 1} and {3, 4}), then the gradient leaving each odd chunk (or
    the last) at the same slots, then three [16][dv] vectors per chunk slot cu[n]/16 + n + c
    (100 // 16 + 3 = 9) and head, then the chunk's A'^T and X^T ([16][16] each) per chunk
    slot and head."""
    lib = _lib.load()
    p = _lib.params(_lib.KDA_DTYPE_BF16, 2, 64, 64)
    ss = 64 * 64 * 4
    assert lib.kda_prefill_backward_workspace(ctypes.byref(p), cu(0, 40, 40, 100), 3) == \
        2 * 6 * 2 * ss + 3 * 9 * 2 * 16 * 64 * 4 + 9 * 2 * 2 * 16 * 16 * 4
    assert lib.kda_prefill_backward_workspace(ctypes.byref(p), cu(0, 40, 30), 2) == -1


def backward(dq=A + 0x100000, dk=A + 0x110000, dv=A + 0x120000, dla=A + 0x130000,
             dbeta=A + 0x140000, dgate=A + 0x150000, ds0=None, ws=A + 0x400000,
             ws_bytes=1 << 24, q=A, d_out=A + 0x80000):
    lib = _lib.load()
    p = _lib.params(_lib.KDA_DTYPE_BF16, 2, 64, 64)
    st = lib.kda_prefill_backward(ctypes.byref(p), q, A + 0x10000, A + 0x20000, A + 0x30000,
                                  A + 0x40000, A + 0x50000, A + 0x60000, cu(0, 3, 5), 2, None,
                                  d_out, None, dq, dk, dv, dla, dbeta, dgate, ds0, ws, ws_bytes,
                                  None)
    return st, lib.kda_last_error().decode()


@pytest.mark.parametrize("kw,msg", [
    (dict(dq=None), "dq is NULL"),
    (dict(dgate=A + 0x150008), "dgate is not 16-byte aligned"),
    (dict(d_out=None), "d_out is NULL"),
    (dict(ws=None), "workspace is NULL"),
    (dict(ws_bytes=100), "workspace_bytes 100"),
    (dict(dq=A + 0x10000), "dq overlaps k"),
    (dict(dk=A + 0x100000 + 64), "dk overlaps dq"),
    (dict(ws=A + 0x100000), "workspace overlaps dq"),
    (dict(ds0=A + 0x20000), "d_initial_state overlaps v"),
])
def test_backward_rejects(kw, msg):
    st, err = backward(**kw)
    assert st == INV, err
    assert msg in err, err


def test_noalloc_rejects_problems_beyond_its_fixed_buffer():
    """The no-alloc segmented prefill refuses, before any HIP call, a problem whose
    workspace would not fit the library's fixed buffer."""
    lib = _lib.load()
    assert lib.kda_noalloc_scratch_bytes() == 64 << 20
    p = _lib.params(_lib.KDA_DTYPE_BF16, 64, 128, 128)
    cu_h = cu(0, 1 << 20)
    need = lib.kda_prefill_segmented_workspace(ctypes.byref(p), cu_h, 1, 16384)
    assert need > lib.kda_noalloc_scratch_bytes()
    st = lib.kda_chunk_prefill_segmented_noalloc(ctypes.byref(p), A, A + 0x10000, A + 0x20000,
                                                 A + 0x30000, A + 0x40000, A + 0x50000, cu_h,
                                                 1, None, None, A + 0x70000, 16384, None)
    assert st == INV
    assert "fixed buffer" in lib.kda_last_error().decode()


def test_segment_plan_picks_segments_only_for_few_long_chains():
    """kda_prefill_segment_plan (host-only; 256 compute units assumed without a GPU): the
    long single sequence with 32 heads is cut into 8 segments of 16384 tokens; short
    sequences, many (sequence, head) chains and fp32 inputs keep the plain schedule."""
    lib = _lib.load()
    bf = lambda H: _lib.params(_lib.KDA_DTYPE_BF16, H, 128, 128)
    plan = lambda p, *c: lib.kda_prefill_segment_plan(ctypes.byref(p), cu(*c), len(c) - 1)
    assert plan(bf(32), 0, 131072) == 16384
    assert plan(bf(4), 0, 524288) == 8192
    assert plan(bf(16), 0, 4096, 8192, 12288, 16384) == 0          # 64 chains of 256 chunks
    assert plan(bf(32), *[4096 * i for i in range(65)]) == 0        # 2048 chains
    assert plan(_lib.params(_lib.KDA_DTYPE_F32, 32, 128, 128), 0, 131072) == 0
    assert plan(bf(32), 0, 100, 50) == -1                           # decreasing
