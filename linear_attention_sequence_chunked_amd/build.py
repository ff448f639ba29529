"""Build libkda.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m linear_attention_sequence_chunked_amd.build [-v]

Objects go to _build/ at the repository root; the library is written next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_plan.cpp", "kda_decode.hip", "kda_prefill.hip", "kda_prefill_bf16.hip",
           "kda_spec.hip", "kda_segment.hip", "kda_backward.hip", "kda_scratch.hip"]
HEADERS = ["kda_device.h", "kda_launch.h", "kda_mfma.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-munsafe-fp-atomics",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


# per-source extra flags: the compiler's ILP scheduling strategy measured faster with
# bit-identical results for these (backward 1-3%, decode 1.4%, verify/commit 1-1.5%,
# bf16 prefill 0.7%, each against the default strategy on one box)
_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
EXTRA_FLAGS = {"kda_backward.hip": _ILP, "kda_decode.hip": _ILP, "kda_spec.hip": _ILP,
               "kda_prefill_bf16.hip": _ILP}


def _obj(src: str) -> str:
    return os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")


def _stale(src: str) -> bool:
    o = _obj(src)
    if not os.path.exists(o):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in HEADERS] + [
        os.path.join(ROOT, "include", "kda.h"), os.path.abspath(__file__)]
    return any(os.path.getmtime(d) > os.path.getmtime(o) for d in deps)


def _compile(src: str, verbose: bool) -> None:
    cmd = [HIPCC] + FLAGS + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", _obj(src)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)


def build(verbose: bool = False, force: bool = True) -> str:
    """Compile every HIP source for gfx950 and link libkda.so.  force=False skips
    sources whose object is newer than the source and headers."""
    os.makedirs(OBJDIR, exist_ok=True)
    todo = [s for s in SOURCES if force or _stale(s)]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        list(ex.map(lambda s: _compile(s, verbose), todo))
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp"] + [
        _obj(s) for s in SOURCES]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, force="--incremental" not in sys.argv))
