"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one chunked-prefill launch over the whole workload.  The default (headline)
workload is the packed varlen batch: 64 sequences whose lengths follow the pages' mix
(8K / 32K / 128K / 256K), 3,768,320 tokens, H=32, dk=dv=128, bf16 inputs, fp32 per-sequence
states.  Inputs are generated once on the GPU and are resident in HBM before timing; a
1 GiB read flushes L2 and the MALL before every timed launch; each launch is timed with
HIP events on the stream the kernel runs on.  Prints one JSON line.

In the same run, each with its own timing: the fixed-length prefill B=4 H=16 T=4096 and
the long-context prefill B=1 H=32 T=131072 (keys under "other_prefill"), the decode step
(256 sequences x 32 heads, 128x128 fp32 states, 1000 consecutive steps), speculative
verify/commit, the backward of the B=4 prefill, the segmented prefill, and the CPU oracle
on a sample of the headline workload ("cpu_baseline").

    python bench.py --summarize {traffic,mfma,trace} ...

turns rocprofv3 CSV output of bench.py runs into the summaries under profiles/ (see
summarize()).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16 (256 CU x 4096 flop/clk x 2.4 GHz)
CSRC = os.path.join(ROOT, "linear_attention_sequence_chunked_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
BUILD_SCRIPT = os.path.join(ROOT, "linear_attention_sequence_chunked_amd", "build.py")
# sources whose change invalidates a stored counter summary of the prefill / decode kernels
PREFILL_SOURCES = ("kda_prefill_bf16.hip", "kda_mfma.h", "kda_prefill.hip", "kda_plan.cpp", "kda_device.h",
                   "kda_launch.h", "kda_api.cpp")
DECODE_SOURCES = ("kda_decode.hip", "kda_device.h", "kda_launch.h", "kda_api.cpp")
COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read + 1 GiB written
HEADLINE = "varlen_n64_h32"
OTHER_PREFILL = ("prefill_b4_h16_t4096", "prefill_b1_h32_t131072")


def _source_hash(names) -> str:
    """SHA-256 over the kernel sources and the build script (its flags shape the code)."""
    import hashlib
    h = hashlib.sha256()
    for path in [os.path.join(CSRC, n) for n in names] + [BUILD_SCRIPT]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def prefill_source_hash() -> str:
    return _source_hash(PREFILL_SOURCES)


def decode_source_hash() -> str:
    return _source_hash(DECODE_SOURCES)


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"{workload}_prefill_traffic.json")


def mfma_file(workload: str) -> str:
    return os.path.join(PROFILES, f"{workload}_prefill_mfma_counters.json")


DECODE_TRAFFIC_FILE = os.path.join(PROFILES, "decode_n256_h32_traffic.json")


def stored_summary(path: str, workload: str, source_hash: str):
    """A committed counter summary, or None when it is missing, is for another workload or
    predates the current kernel source."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("kernel_source_sha256") != source_hash:
        return None
    return t


def prefill_algorithmic(lengths, H, dk, dv, es, has_s0, chunk=16):
    """Bytes and flops a prefill launch must move/do at minimum.

    Per token-head: read q, k, log_alpha (dk each), v, gate (dv each), beta; write o (dv).
    Per (sequence, head): read S0 (if given) and write S_T, fp32 dk x dv each.
    Flops per token-head: 6 dk dv (W S, Qh S, Kb^T U) + 6 C dk (Gram pair, W) +
    4 C dv (T V, P U)."""
    tokens = sum(lengths)
    th = tokens * H
    bytes_ = th * (es * (3 * dk + 2 * dv) + es + es * dv)
    bytes_ += len(lengths) * H * 4 * dk * dv * (2 if has_s0 else 1)
    flops = th * (6 * dk * dv + 6 * chunk * dk + 4 * chunk * dv)
    return bytes_, flops


def cpu_model() -> str:
    """/proc/cpuinfo's model name (what lscpu prints as "Model name"), with the family, model
    and stepping numbers, which identify the part where a virtual machine shortens the name."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    k, v = line.split(":", 1)
                    fields.setdefault(k.strip(), v.strip())
    except OSError:
        pass
    name = fields.get("model name")
    if not name:
        import platform
        return platform.processor() or "unknown"
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


def varlen_sample(lengths, H, per_class: int):
    """per_class (sequence, head) pairs of every length class, spread over the class's
    sequences and the heads (the pairs the CPU baseline and the parity test use)."""
    out = []
    for c in sorted(set(lengths)):
        seqs = [n for n, L in enumerate(lengths) if L == c]
        out += [(seqs[j % len(seqs)], (5 * j + c // 8192) % H) for j in range(per_class)]
    return out


# ------------------------------------------------------------------------ measurement

def copy_calibration(steps: int) -> int:
    """Plain device copy of COPY_BYTES, the reference kernel for scaling the FETCH_SIZE /
    WRITE_SIZE counters (each launch must read and write exactly COPY_BYTES)."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "launches": steps}), flush=True)
    return 0


class Flush:
    """Evicts L2 and the MALL before a timed launch by reading 1 GiB (leaves only clean
    lines; a write would leave dirty lines whose write-back lands in the timed launch)."""

    def __init__(self, enabled: bool):
        import torch
        self.buf = torch.ones(256 << 20, dtype=torch.float32, device="cuda") if enabled else None
        self.out = torch.empty((), dtype=torch.float32, device="cuda")

    def __call__(self):
        import torch
        if self.buf is not None:
            torch.sum(self.buf, dim=0, out=self.out)


def time_launches(fn, steps: int, warmup: int, min_warmup_s: float, flush: Flush):
    """Warm up (at least `warmup` launches and `min_warmup_s` seconds, so the clocks have
    settled), then time `steps` launches, each after a cache flush, with HIP events on the
    current stream (the one the library launches on).  Returns (times in ms, wall s)."""
    import torch
    stream = torch.cuda.current_stream()
    n, t0 = 0, time.perf_counter()
    while n < warmup or time.perf_counter() - t0 < min_warmup_s:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    wall0 = time.perf_counter()
    for i in range(steps):
        flush()
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return [s.elapsed_time(e) for s, e in zip(starts, ends)], wall


def prefill_record(w, x, times_ms, wall, segment_len=0):
    """Throughput, roofline fractions and the stored counter summaries of one workload
    (segment_len > 0: the library's plan cut the sequences into segments of that many tokens,
    and a step is the segmented schedule's three launches)."""
    import numpy as np
    es = 2 if w.dtype == "bf16" else 4
    ms = float(np.mean(times_ms))
    tokens = sum(w.lengths)
    alg_bytes, alg_flops = prefill_algorithmic(w.lengths, w.H, w.dk, w.dv, es,
                                               x.initial_state is not None)
    gbps = alg_bytes / (ms * 1e-3) / 1e9
    tflops = alg_flops / (ms * 1e-3) / 1e12
    rec = {
        "workload": w.name, "tokens": tokens, "ms_per_step": ms,
        "ms_per_step_median": float(np.median(times_ms)), "tokens_per_s": tokens / (ms * 1e-3),
        "wall_s_timed_region_incl_cache_flush": wall,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "prefill_bf16_kernel" if w.dtype == "bf16" else "prefill_kernel",
                     "algorithmic_bytes_per_launch": alg_bytes},
        "schedule": ("plain" if segment_len <= 0 else
                     f"segmented, {segment_len}-token segments (the library's plan): a state and "
                     f"transition pass, the combine, and the output pass, timed together"),
        "mfma": {"achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "algorithmic_flops_per_launch": alg_flops},
    }
    src = prefill_source_hash()
    t = stored_summary(traffic_file(w.name), w.name, src)
    if t is not None:  # rocprofv3 FETCH_SIZE/WRITE_SIZE of the same kernel and workload
        rec["roofline"]["traffic"] = t["traffic_bytes_per_launch"]
        rec["roofline"]["traffic_over_algorithmic"] = t["traffic_bytes_per_launch"] / alg_bytes
        rec["roofline"]["traffic_source"] = os.path.relpath(traffic_file(w.name), ROOT)
    mc = stored_summary(mfma_file(w.name), w.name, src)
    if mc is not None:  # rocprofv3 MFMA counters of the same kernel, this launch's time
        ex = mc["executed_mfma_flops_per_launch"]
        rec["mfma"]["rocprof"] = {
            "executed_mfma_flops_per_launch": ex,
            "executed_bf16_flops_per_launch": mc["executed_bf16_flops_per_launch"],
            "executed_f16_flops_per_launch": mc["executed_f16_flops_per_launch"],
            "executed_TFLOPs": ex / (ms * 1e-3) / 1e12,
            "executed_frac": ex / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "mfma_busy_frac": mc["mfma_busy_frac"],
            "source": os.path.relpath(mfma_file(w.name), ROOT)}
    return rec


def run_prefill_workload(name, args, flush, seed=1):
    import torch
    import kda_inputs as ki
    import linear_attention_sequence_chunked_amd as kda
    w = ki.WORKLOADS[name]
    x = ki.make_workload_inputs(w, seed=seed, device="cuda")
    out = torch.empty((x.total_tokens, w.H, w.dv), dtype=x.q.dtype, device="cuda")
    Sf = torch.empty((len(w.lengths), w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")

    def step():
        kda.chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, cu_seqlens=x.cu_seqlens,
                          cu_seqlens_host=x.cu_seqlens_host, initial_state=x.initial_state,
                          out=out, final_state=Sf)

    import ctypes
    from linear_attention_sequence_chunked_amd import _lib as klib
    p = klib.params(klib.KDA_DTYPE_BF16 if w.dtype == "bf16" else klib.KDA_DTYPE_F32, w.H, w.dk, w.dv)
    cu_h = (ctypes.c_int32 * len(x.cu_seqlens_host))(*x.cu_seqlens_host)
    plan = kda.load_library().kda_prefill_segment_plan(ctypes.byref(p), cu_h, len(w.lengths))
    times, wall = time_launches(step, args.steps, args.warmup, args.min_warmup_s, flush)
    return w, x, prefill_record(w, x, times, wall, segment_len=plan)


def cpu_baseline(w, x, per_class: int, repeat_s: float):
    """The fp64 oracle (threads over (sequence, head) pairs) on a sample of the workload:
    per_class pairs of every length class, timed until repeat_s seconds have passed, scaled
    to the whole workload by its token-head count."""
    import oracle
    pairs = varlen_sample(w.lengths, w.H, per_class) if len(set(w.lengths)) > 1 else [
        (n, h) for n in range(len(w.lengths)) for h in range(w.H)]
    cu = x.cu_seqlens_host
    host = lambda t: t.detach().float().cpu().numpy()
    import numpy as np
    cat = lambda ts: np.concatenate(ts, axis=0)
    q, k, v, la, b, g, s0, cuh = [], [], [], [], [], [], [], [0]
    for n, h in pairs:
        a, e = cu[n], cu[n + 1]
        for lst, t in ((q, x.q), (k, x.k), (v, x.v), (la, x.log_alpha), (b, x.beta), (g, x.gate)):
            lst.append(host(t[a:e, h:h + 1]))
        if x.initial_state is not None:
            s0.append(host(x.initial_state[n, h:h + 1]))
        cuh.append(cuh[-1] + e - a)
    q, k, v, la, b, g = (cat(t) for t in (q, k, v, la, b, g))
    S0 = np.stack(s0) if s0 else None
    oracle.ensure_built()
    runs, t0 = 0, time.perf_counter()
    used = 0
    while runs == 0 or time.perf_counter() - t0 < repeat_s:
        _, _, used = oracle.run(q, k, v, la, b, g, cuh, S0, want_out=True)
        runs += 1
    dt = (time.perf_counter() - t0) / runs
    sample_th = cuh[-1]                     # token-heads in the sample
    rate = sample_th / dt                   # token-heads per second
    total_th = sum(w.lengths) * w.H
    return {"value": rate / w.H, "unit": "tokens/s", "cores": used, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{len(pairs)} (sequence, head) pairs of {w.name} ({per_class} per length "
                      f"class), {sample_th} token-heads = {sample_th / total_th:.4f} of the "
                      f"workload; fp64 token loop with outputs, {runs} run(s) of {dt:.2f} s; "
                      f"tokens/s = token-heads/s / H, i.e. the whole workload's rate"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--min-warmup-s", type=float, default=1.0,
                    help="warm up for at least this long (clocks settle); the B=4 T=4096 "
                         "prefill measured ~256 us per launch after 3 launches, ~235 us after "
                         "0.5-2 s of them")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--other-prefill", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the B=4 T=4096 and B=1 T=131072 prefills")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--spec-rounds", type=int, default=50)
    ap.add_argument("--spec-draft", type=int, default=4)
    ap.add_argument("--backward-steps", type=int, default=10)
    ap.add_argument("--segmented", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the segmented prefill on the few-head long workload")
    ap.add_argument("--segment-len", type=int, default=0,
                    help="segment length of the timed segmented prefill (0: the library's plan)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-pairs-per-class", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 1 GiB copy used to scale the HBM byte counters")
    ap.add_argument("--summarize", choices=("traffic", "mfma", "trace"))
    ap.add_argument("--pmc-dirs", nargs="*", default=[])
    ap.add_argument("--kernel", default="prefill_bf16_kernel")
    ap.add_argument("--per-step", action="store_true",
                    help="sum the matching dispatches between two cache flushes (one step)")
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--out")
    args = ap.parse_args()
    if args.summarize:
        return summarize(args)
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); "
              "the operator shards over (sequence, head) with no communication, so the "
              "N-GPU figure is N independent copies of this one.", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration(args.steps)

    import numpy as np
    import torch

    import kda_inputs as ki
    import linear_attention_sequence_chunked_amd as kda

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    flush = Flush(not args.no_flush)

    w, x, head = run_prefill_workload(args.workload, args, flush)
    result = {
        "metric": "KDA prefill tokens/s (%MFMA peak); decode state GB/s (%HBM peak), 1 MI355X",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_median": head["ms_per_step_median"],
        "wall_s_timed_region_incl_cache_flush": head["wall_s_timed_region_incl_cache_flush"],
        "cache_flush": None if args.no_flush else "1 GiB read before each launch",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1); v N(0,1); beta, gate "
                "sigmoid(N(0,1)); log_alpha max(-softplus(N(0,1)),-0.3); per-sequence S0 "
                "N(0,0.02^2) where the workload has one)",
        "config": {"workload": w.name, "sequences": len(w.lengths),
                   "length_classes": {str(L): w.lengths.count(L) for L in sorted(set(w.lengths))},
                   "longest": max(w.lengths), "tokens": x.total_tokens, "heads": w.H,
                   "dk": w.dk, "dv": w.dv, "chunk": 16, "state": "fp32",
                   "initial_state": x.initial_state is not None},
        "roofline": head["roofline"],
        "mfma": head["mfma"],
    }
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, x, args.cpu_pairs_per_class, args.cpu_seconds)
    del x
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- other prefill shapes
    if args.other_prefill:
        result["other_prefill"] = {}
        for name in OTHER_PREFILL:
            if name == args.workload:
                continue
            _, xo, rec = run_prefill_workload(name, args, flush)
            result["other_prefill"][name] = rec
            del xo
            torch.cuda.empty_cache()

    # ---------------------------------------------------------------- decode step
    if not args.no_decode and args.decode_steps > 0:
        d = ki.WORKLOADS["decode_n256_h32"]
        N = len(d.lengths)
        nsteps = args.decode_steps
        inp = ki.make_decode_inputs(nsteps, N, d.H, d.dk, d.dv, d.dtype, seed=3, device="cuda")
        state = ki.make_state(N, d.H, d.dk, d.dv, d.s0_std, seed=3, device="cuda")
        dout = torch.empty((N, d.H, d.dv), dtype=torch.bfloat16, device="cuda")

        def dstep(s):
            kda.decode_step(inp["q"][s], inp["k"][s], inp["v"][s], inp["log_alpha"][s],
                            inp["beta"][s], inp["gate"][s], state, out=dout)

        for s in range(min(5, nsteps)):
            dstep(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(nsteps):
            dstep(s)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / nsteps
        state_bytes = N * d.H * d.dk * d.dv * 4
        io_bytes = N * d.H * (2 * (3 * d.dk + 3 * d.dv) + 2)
        result["decode"] = {
            "workload": d.name, "steps": nsteps, "us_per_step": dms * 1e3,
            "state_GBps": 2 * state_bytes / (dms * 1e-3) / 1e9,
            "frac_hbm": 2 * state_bytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "total_GBps_incl_token_io": (2 * state_bytes + io_bytes) / (dms * 1e-3) / 1e9,
            "state_bytes": state_bytes,
        }
        dt = stored_summary(DECODE_TRAFFIC_FILE, d.name, decode_source_hash())
        if dt is not None:  # rocprofv3 HBM byte counters of the same kernel, this step's time
            result["decode"]["traffic_bytes_per_step"] = dt["traffic_bytes_per_step"]
            result["decode"]["traffic_GBps"] = dt["traffic_bytes_per_step"] / (dms * 1e-3) / 1e9
            result["decode"]["traffic_frac_hbm"] = result["decode"]["traffic_GBps"] / HBM_PEAK_GBPS
        del inp, state
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- speculative verify
    if not args.no_decode and args.spec_rounds > 0:
        d = ki.WORKLOADS["decode_n256_h32"]
        N, K = len(d.lengths), args.spec_draft
        sx = ki.make_prefill_inputs((K,) * N, d.H, d.dk, d.dv, d.dtype, d.s0_std, seed=6,
                                    device="cuda")
        state = sx.initial_state
        sout = torch.empty_like(sx.v)
        g = torch.Generator().manual_seed(6)
        accepted = torch.randint(0, K + 1, (args.spec_rounds, N), generator=g,
                                 dtype=torch.int32).cuda()
        sd = torch.cuda.Stream()
        with torch.cuda.stream(sd):
            for i in range(min(3, args.spec_rounds)):
                kda.spec_verify(sx.q, sx.k, sx.v, sx.log_alpha, sx.beta, sx.gate, state, out=sout)
                kda.spec_commit(sx.k, sx.v, sx.log_alpha, sx.beta, state, accepted[i])
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record(sd)
            for i in range(args.spec_rounds):
                kda.spec_verify(sx.q, sx.k, sx.v, sx.log_alpha, sx.beta, sx.gate, state,
                                out=sout)
            ev[1].record(sd)
            for i in range(args.spec_rounds):
                kda.spec_commit(sx.k, sx.v, sx.log_alpha, sx.beta, state, accepted[i])
            ev[2].record(sd)
        torch.cuda.synchronize()
        vus = ev[0].elapsed_time(ev[1]) / args.spec_rounds * 1e3
        cus = ev[1].elapsed_time(ev[2]) / args.spec_rounds * 1e3
        state_bytes = N * d.H * d.dk * d.dv * 4
        frac_committed = float((accepted > 0).float().mean())
        moved = state_bytes * (1 + 2 * frac_committed)  # verify reads; commit reads + writes
        result["spec_verify"] = {
            "workload": f"{d.name}, {K} bf16 drafts per sequence, accepted lengths uniform "
                        f"in 0..{K}",
            "rounds": args.spec_rounds, "verify_us": vus, "commit_us": cus,
            "state_GBps": moved / ((vus + cus) * 1e-6) / 1e9,
            "frac_hbm": moved / ((vus + cus) * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "draft_tokens_per_s": N * K / ((vus + cus) * 1e-6),
        }
        del sx, state, sout
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- backward
    if args.backward_steps > 0:
        import ctypes
        from linear_attention_sequence_chunked_amd import _lib as klib
        bw = ki.WORKLOADS["prefill_b4_h16_t4096"]
        bx = ki.make_workload_inputs(bw, seed=1, device="cuda")
        g = torch.Generator().manual_seed(1)
        dout = torch.randn(bx.v.shape, generator=g).to(bx.v.dtype).cuda()
        lib = kda.load_library()
        pp = klib.params(klib.KDA_DTYPE_BF16, bw.H, bw.dk, bw.dv)
        cu_h = (ctypes.c_int32 * len(bx.cu_seqlens_host))(*bx.cu_seqlens_host)
        need = lib.kda_prefill_backward_workspace(ctypes.byref(pp), cu_h, len(bw.lengths))
        bws = torch.empty(need, dtype=torch.uint8, device="cuda")
        fout = torch.empty_like(bx.v)

        def bstep():
            kda.prefill_backward(bx.q, bx.k, bx.v, bx.log_alpha, bx.beta, bx.gate, dout,
                                 cu_seqlens=bx.cu_seqlens, cu_seqlens_host=bx.cu_seqlens_host,
                                 initial_state=bx.initial_state, workspace=bws)

        def fstep():
            kda.chunk_prefill(bx.q, bx.k, bx.v, bx.log_alpha, bx.beta, bx.gate,
                              cu_seqlens=bx.cu_seqlens, cu_seqlens_host=bx.cu_seqlens_host,
                              initial_state=bx.initial_state, out=fout)

        bt, _ = time_launches(bstep, args.backward_steps, 3, 0.5, flush)
        ft, _ = time_launches(fstep, args.backward_steps, 3, 0.5, flush)
        bms, fms = float(np.median(bt)), float(np.median(ft))
        result["backward"] = {
            "workload": bw.name, "steps": args.backward_steps, "ms_per_step": bms,
            "tokens_per_s": bx.total_tokens / (bms * 1e-3), "forward_ms": fms,
            "vs_forward": bms / fms,
            "note": "chunk form, fp32 state and sums: forward and reverse chunk walks in one "
                    "launch storing every other state and gradient, then the pairs of chunks "
                    "on persistent workgroups (split-bf16 and fp32 MFMA); medians of launches "
                    "each after "
                    "the same cache flush as the forward's",
        }
        del bws, dout, bx, fout
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- segmented prefill
    if args.segmented:
        sw = ki.WORKLOADS["prefill_b1_h4_t524288"]
        sxx = ki.make_workload_inputs(sw, seed=2, device="cuda")
        import ctypes
        from linear_attention_sequence_chunked_amd import _lib as klib
        sp = klib.params(klib.KDA_DTYPE_BF16, sw.H, sw.dk, sw.dv)
        scu = (ctypes.c_int32 * len(sxx.cu_seqlens_host))(*sxx.cu_seqlens_host)
        plan = kda.load_library().kda_prefill_segment_plan(ctypes.byref(sp), scu, len(sw.lengths))
        L = args.segment_len if args.segment_len else plan
        sout = torch.empty_like(sxx.v)
        sSf = torch.empty((1, sw.H, sw.dk, sw.dv), dtype=torch.float32, device="cuda")
        ws = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")

        def plain_run():  # the plain schedule, forced
            kda.chunk_prefill(sxx.q, sxx.k, sxx.v, sxx.log_alpha, sxx.beta, sxx.gate,
                              cu_seqlens=sxx.cu_seqlens, cu_seqlens_host=sxx.cu_seqlens_host,
                              out=sout, final_state=sSf, segment_len=0)

        def seg_run():
            kda.chunk_prefill_segmented(sxx.q, sxx.k, sxx.v, sxx.log_alpha, sxx.beta, sxx.gate,
                                        sxx.cu_seqlens_host, L, out=sout, final_state=sSf,
                                        workspace=ws)

        pt, _ = time_launches(plain_run, 3, 1, 0.0, flush)
        st, _ = time_launches(seg_run, 5, 1, 0.0, flush)
        pms, sms = float(np.median(pt)), float(np.median(st))
        ttok = sum(sw.lengths)
        result["segmented"] = {
            "workload": sw.name, "segment_len": L, "planned_segment_len": plan,
            "plain_ms": pms, "segmented_ms": sms,
            "speedup": pms / sms, "segmented_tokens_per_s": ttok / (sms * 1e-3),
        }
        del sxx, sout, ws
        torch.cuda.empty_cache()

    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)
    return 0


# ------------------------------------------------------------------------ counter summaries

def _read_counters(dirs, kernel_substr):
    """{counter: [value per dispatch in dispatch order]} and the durations (us) of the
    dispatches whose kernel name contains kernel_substr, from rocprofv3 CSV directories."""
    vals, dur, names = {}, {}, {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if kernel_substr not in r["Kernel_Name"]:
                        continue
                    did = int(r["Dispatch_Id"])
                    vals.setdefault(r["Counter_Name"], {})[did] = float(r["Counter_Value"])
                    dur[did] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                    names[did] = r["Kernel_Name"]
    out = {c: [v[k] for k in sorted(v)] for c, v in vals.items()}
    order = sorted(dur)
    return out, [dur[k] for k in order], [names[k] for k in order]


def _read_steps(dirs, kernel_substr):
    """Like _read_counters, but per step: the dispatches whose kernel name contains
    kernel_substr, grouped into runs that other kernels (the cache flush before every timed
    launch) separate, each run summed -- one entry per step, however many kernels a step
    launches (the segmented schedule launches three)."""
    rows = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    did = int(r["Dispatch_Id"])
                    e = rows.setdefault(did, {"name": r["Kernel_Name"], "c": {},
                                              "dur": (int(r["End_Timestamp"]) -
                                                      int(r["Start_Timestamp"])) / 1e3})
                    e["c"][r["Counter_Name"]] = float(r["Counter_Value"])
    steps, cur = [], None
    for did in sorted(rows):
        e = rows[did]
        if kernel_substr not in e["name"]:
            cur = None
            continue
        if cur is None:
            cur = {"c": {}, "dur": 0.0, "names": []}
            steps.append(cur)
        for k, v in e["c"].items():
            cur["c"][k] = cur["c"].get(k, 0.0) + v
        cur["dur"] += e["dur"]
        cur["names"].append(e["name"])
    out = {}
    for st in steps:
        for k, v in st["c"].items():
            out.setdefault(k, []).append(v)
    return out, [st["dur"] for st in steps], [" + ".join(st["names"]) for st in steps]


def summarize(args) -> int:
    """traffic: --pmc-dirs FETCH WRITE COPYFETCH COPYWRITE (rocprofv3 --pmc FETCH_SIZE /
    WRITE_SIZE runs of `bench.py --steps S` and of `bench.py --copy-calibration`): HBM
    bytes per launch of the last S launches, each counter scaled by the factor that makes it
    read exactly 1 GiB for the plain 1 GiB copy.
    mfma: --pmc-dirs DIR (SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16
    SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE): executed bf16 and fp16 MFMA flops and the
    MFMA busy fraction.
    trace: --pmc-dirs DIR (--kernel-trace --stats): per-kernel call counts and durations."""
    import numpy as np
    import kda_inputs as ki
    w = ki.WORKLOADS.get(getattr(args, "workload", ""), None)
    steps = args.steps
    res = {"workload": args.workload, "commands": args.command}
    if args.summarize in ("traffic", "mfma"):
        res["kernel_source_sha256"] = (decode_source_hash() if "decode" in args.kernel
                                       else prefill_source_hash())
    if args.summarize == "traffic":
        rd = _read_steps if args.per_step else _read_counters
        fetch, fdur, names = rd([args.pmc_dirs[0]], args.kernel)
        write, _, _ = rd([args.pmc_dirs[1]], args.kernel)
        cf, _, _ = _read_counters([args.pmc_dirs[2]], "copyBuffer")
        cw, _, _ = _read_counters([args.pmc_dirs[3]], "copyBuffer")
        if not cf:  # torch's copy kernel, if the runtime did not use its blit
            cf, _, _ = _read_counters([args.pmc_dirs[2]], "copy")
            cw, _, _ = _read_counters([args.pmc_dirs[3]], "copy")
        f = fetch["FETCH_SIZE"][-steps:]
        wr = write["WRITE_SIZE"][-steps:]
        gib_kib = COPY_BYTES / 1024
        ff = gib_kib / float(np.mean(cf["FETCH_SIZE"]))
        wf = gib_kib / float(np.mean(cw["WRITE_SIZE"]))
        traffic = (float(np.mean(f)) * ff + float(np.mean(wr)) * wf) * 1024
        res.update({"kernel": names[-1], "fetch_kib_per_dispatch": float(np.mean(f)),
                    "write_kib_per_dispatch": float(np.mean(wr)), "fetch_dispatches": f,
                    "write_dispatches": wr,
                    "copy_calibration": {"bytes_read_and_written": COPY_BYTES,
                                         "fetch_kib": cf["FETCH_SIZE"],
                                         "write_kib": cw["WRITE_SIZE"], "fetch_factor": ff,
                                         "write_factor": wf},
                    "traffic_bytes_per_launch": traffic})
        key = "traffic_bytes_per_step" if "decode" in args.kernel else "traffic_bytes_per_launch"
        res[key] = traffic
        if w is not None and "decode" not in args.kernel:
            alg, _ = prefill_algorithmic(w.lengths, w.H, w.dk, w.dv, 2, w.s0_std > 0)
            res["algorithmic_bytes_per_launch"] = alg
            res["traffic_over_algorithmic"] = traffic / alg
        res["note"] = ("HBM bytes per launch = FETCH_SIZE*fetch_factor + WRITE_SIZE*write_factor "
                       "(KiB, mean over the last launches, each after the 1 GiB cache flush); the "
                       "factors make the counters read exactly 1 GiB for a plain 1 GiB copy.")
    elif args.summarize == "mfma":
        c, dur, names = (_read_steps if args.per_step else _read_counters)(args.pmc_dirs, args.kernel)
        mops = float(np.mean(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"][-steps:]))
        mops16 = float(np.mean(c["SQ_INSTS_VALU_MFMA_MOPS_F16"][-steps:]))
        busy = float(np.mean(c["SQ_VALU_MFMA_BUSY_CYCLES"][-steps:]))
        act = float(np.mean(c["GRBM_GUI_ACTIVE"][-steps:]))
        us = float(np.mean(dur[-steps:]))
        ex = (mops + mops16) * 512
        res.update({"kernel": names[-1], "dispatches": steps,
                    "SQ_INSTS_VALU_MFMA_MOPS_BF16_per_launch": mops,
                    "SQ_INSTS_VALU_MFMA_MOPS_F16_per_launch": mops16,
                    "SQ_VALU_MFMA_BUSY_CYCLES_per_launch": busy,
                    "GRBM_GUI_ACTIVE_per_launch": act,
                    "kernel_duration_us_under_counters": us,
                    "executed_bf16_flops_per_launch": mops * 512,
                    "executed_f16_flops_per_launch": mops16 * 512,
                    "executed_mfma_flops_per_launch": ex,
                    "mfma_busy_frac": busy / (act * 1024 / 8) if act else None})
        if w is not None:
            _, alg_f = prefill_algorithmic(w.lengths, w.H, w.dk, w.dv, 2, w.s0_std > 0)
            res["algorithmic_flops_per_launch"] = alg_f
            res["executed_over_algorithmic"] = ex / alg_f
        res["note"] = ("executed flops = (bf16 + fp16 MOPS) x 512 (the counters' unit); mfma_busy_frac = MFMA "
                       "busy cycles summed over the 1024 SIMDs / (GPU-active cycles per XCD x "
                       "1024), the MfmaUtil of rocprofv3 (GRBM_GUI_ACTIVE sums the 8 XCDs).")
    else:  # trace
        rows = []
        for path in glob.glob(os.path.join(args.pmc_dirs[0], "**", "*kernel_stats.csv"),
                              recursive=True):
            with open(path) as f:
                rows += list(csv.DictReader(f))
        lines = [f"rocprofv3 kernel trace of bench.py, one MI355X; workload {args.workload}",
                 "", "command:"] + [f"  {c}" for c in args.command] + ["",
                 f"{'kernel':70s} {'calls':>7s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} "
                 f"{'share%':>7s}"]
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:16]:
            lines.append(f"{r['Name'][:70]:70s} {int(r['Calls']):7d} "
                         f"{float(r['AverageNs']) / 1e3:10.1f} {float(r['MinNs']) / 1e3:10.1f} "
                         f"{float(r['MaxNs']) / 1e3:10.1f} {float(r['Percentage']):7.2f}")
        traces = glob.glob(os.path.join(args.pmc_dirs[0], "**", "*kernel_trace.csv"), recursive=True)
        durs = []
        for path in traces:
            with open(path) as f:
                for r in csv.DictReader(f):
                    if args.kernel in r["Kernel_Name"]:
                        durs.append((int(r["Start_Timestamp"]),
                                     (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
        durs = [d for _, d in sorted(durs)]
        if durs:
            tail = durs[-steps:]
            lines += ["", f"{args.kernel} dispatches: {len(durs)}; the timed ones (last {steps}): "
                          f"mean {np.mean(tail):.1f} us, median {np.median(tail):.1f} us"]
        with open(args.out, "w") as f:
            f.write("\n".join(lines) + "\n")
        return 0
    with open(args.out, "w") as f:
        json.dump(res, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
