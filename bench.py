"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one chunked-prefill launch over the whole workload (default: B=4, H=16,
T=4096, dk=dv=128, bf16 inputs, fp32 state).  Inputs are generated once on the GPU and are
resident in HBM before timing; the 256 MB last-level cache is flushed between timed steps
so no step reuses the previous step's inputs from cache.  Each step is timed with HIP
events on the stream the kernel runs on.  Prints one JSON line.

The decode step (256 sequences x 32 heads, 128x128 fp32 states, 1000 consecutive steps)
is measured in the same run and reported under "decode".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16 (256 CU x 4096 flop/clk x 2.4 GHz)
CSRC = os.path.join(ROOT, "linear_attention_sequence_chunked_amd", "csrc")
# sources whose change invalidates a stored traffic measurement of the prefill kernel
PREFILL_SOURCES = ("kda_prefill_bf16.hip", "kda_device.h", "kda_launch.h", "kda_api.cpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_bf16_b4_h16_t4096_traffic.json")
COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read + 1 GiB written


BUILD_SCRIPT = os.path.join(ROOT, "linear_attention_sequence_chunked_amd", "build.py")


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


def stored_traffic(workload: str):
    """HBM bytes per prefill launch from the committed counter summary, or None when the
    summary is missing, is for another workload or predates the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("kernel_source_sha256") != prefill_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


# the decode kernel's sources, and the committed counter summaries of MFMA use (prefill)
# and HBM bytes (decode)
DECODE_SOURCES = ("kda_decode.hip", "kda_device.h", "kda_launch.h", "kda_api.cpp")
MFMA_FILE = os.path.join(ROOT, "profiles", "prefill_bf16_b4_h16_t4096_mfma_counters.json")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_n256_h32_traffic.json")


def decode_source_hash() -> str:
    return _source_hash(DECODE_SOURCES)


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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # A few warmup launches leave the GPU below its steady clocks: the bench workload's
    # prefill measured ~256 us per launch after 3 warmup launches and ~235 us after 200
    # (0.5 s or 2 s of warmup: ~238 us).
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="prefill_b4_h16_t4096")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--spec-rounds", type=int, default=50)
    ap.add_argument("--spec-draft", type=int, default=4)
    ap.add_argument("--backward-steps", type=int, default=3)
    ap.add_argument("--segmented", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the segmented prefill on the few-head long workload")
    ap.add_argument("--segment-len", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--flush", choices=("read", "write"), default="read",
                    help="how the 1 GiB cache flush before each timed launch touches memory")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 1 GiB copy used to scale the HBM byte counters")
    args = ap.parse_args()
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
    w = ki.WORKLOADS[args.workload]
    x = ki.make_workload_inputs(w, seed=1, device="cuda")
    es = 2 if w.dtype == "bf16" else 4
    T_total = x.total_tokens
    out = torch.empty((T_total, w.H, w.dv), dtype=x.q.dtype, device="cuda")
    Sf = torch.empty((len(w.lengths), w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    # Cache flush before every timed launch: reading a 1 GiB buffer evicts the inputs from
    # L2 and the MALL and leaves only clean lines; writing it (--flush write) also leaves up
    # to the MALL's size of dirty lines, whose write-back then runs inside the timed launch.
    flush = None
    if not args.no_flush:
        flush = torch.ones(256 << 20, dtype=torch.float32, device="cuda")  # 1 GiB
        flush_out = torch.empty((), dtype=torch.float32, device="cuda")

    def do_flush():
        if args.flush == "write":
            flush.zero_()
        else:
            torch.sum(flush, dim=0, out=flush_out)

    def step():
        kda.chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, cu_seqlens=x.cu_seqlens,
                          cu_seqlens_host=x.cu_seqlens_host, initial_state=x.initial_state,
                          out=out, final_state=Sf)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            do_flush()
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    times_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms = float(np.mean(times_ms))
    tokens_per_s = T_total / (ms * 1e-3)
    alg_bytes, alg_flops = prefill_algorithmic(w.lengths, w.H, w.dk, w.dv, es,
                                               x.initial_state is not None)
    gbps = alg_bytes / (ms * 1e-3) / 1e9
    tflops = alg_flops / (ms * 1e-3) / 1e12

    result = {
        "metric": "KDA prefill tokens/s (%MFMA peak); decode state GB/s (%HBM peak), 1 MI355X",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": float(np.median(times_ms)),
        "wall_s_timed_region_incl_cache_flush": wall,
        "cache_flush": None if flush is None else f"1 GiB {args.flush} before each launch",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1); v N(0,1); beta, gate "
                "sigmoid(N(0,1)); log_alpha max(-softplus(N(0,1)),-0.3))",
        "config": {"workload": w.name, "batch": len(w.lengths), "seq_len": max(w.lengths),
                   "tokens": T_total, "heads": w.H, "dk": w.dk, "dv": w.dv, "chunk": 16,
                   "state": "fp32", "initial_state": x.initial_state is not None},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": stored_traffic(w.name) if w.dtype == "bf16" else None,
                     "kernel": "prefill_bf16_kernel" if w.dtype == "bf16" else "prefill_kernel",
                     "algorithmic_bytes_per_launch": alg_bytes},
        "mfma": {"achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                 "algorithmic_flops_per_launch": alg_flops},
    }
    mc = (stored_summary(MFMA_FILE, w.name, prefill_source_hash()) if w.dtype == "bf16" else None)
    if mc is not None:  # rocprofv3 counters of the same kernel, this launch's time
        ex = mc["executed_bf16_flops_per_launch"]
        result["mfma"]["rocprof"] = {
            "executed_bf16_flops_per_launch": ex,
            "executed_TFLOPs": ex / (ms * 1e-3) / 1e12,
            "executed_frac": ex / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "mfma_busy_frac": mc["mfma_busy_frac"],
            "source": os.path.basename(MFMA_FILE)}

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

        def spec_round(i):
            kda.spec_verify(sx.q, sx.k, sx.v, sx.log_alpha, sx.beta, sx.gate, state, out=sout)
            kda.spec_commit(sx.k, sx.v, sx.log_alpha, sx.beta, state, accepted[i])

        with torch.cuda.stream(sd):
            for i in range(min(3, args.spec_rounds)):
                spec_round(i)
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
        g = torch.Generator().manual_seed(1)
        dout = torch.randn(x.v.shape, generator=g).to(x.v.dtype).cuda()
        bws = None

        def bstep():
            kda.prefill_backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.gate, dout,
                                 cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_seqlens_host,
                                 initial_state=x.initial_state, workspace=bws)

        lib = kda.load_library()
        import ctypes
        from linear_attention_sequence_chunked_amd import _lib as klib
        pp = klib.params(klib.KDA_DTYPE_BF16 if w.dtype == "bf16" else klib.KDA_DTYPE_F32,
                         w.H, w.dk, w.dv)
        cu_h = (ctypes.c_int32 * len(x.cu_seqlens_host))(*x.cu_seqlens_host)
        need = lib.kda_prefill_backward_workspace(ctypes.byref(pp), cu_h, len(w.lengths))
        bws = torch.empty(need, dtype=torch.uint8, device="cuda")
        bstep()
        torch.cuda.synchronize()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(args.backward_steps):
            bstep()
        b1.record(stream)
        torch.cuda.synchronize()
        bms = b0.elapsed_time(b1) / args.backward_steps
        result["backward"] = {
            "workload": w.name, "steps": args.backward_steps, "ms_per_step": bms,
            "tokens_per_s": T_total / (bms * 1e-3), "vs_forward": bms / ms,
            "note": "chunk form, fp32 state and sums: forward and reverse chunk walks in one launch (split-bf16 products), then all chunks in parallel (fp32 MFMA)",
        }
        del bws, dout
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- segmented prefill
    if args.segmented:
        sw = ki.WORKLOADS["prefill_b1_h4_t524288"]
        sxx = ki.make_workload_inputs(sw, seed=2, device="cuda")
        L = args.segment_len
        sout = torch.empty_like(sxx.v)
        sSf = torch.empty((1, sw.H, sw.dk, sw.dv), dtype=torch.float32, device="cuda")
        ws = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")

        def plain_run():
            kda.chunk_prefill(sxx.q, sxx.k, sxx.v, sxx.log_alpha, sxx.beta, sxx.gate,
                              cu_seqlens=sxx.cu_seqlens, cu_seqlens_host=sxx.cu_seqlens_host,
                              out=sout, final_state=sSf)

        def seg_run():
            kda.chunk_prefill_segmented(sxx.q, sxx.k, sxx.v, sxx.log_alpha, sxx.beta, sxx.gate,
                                        sxx.cu_seqlens_host, L, out=sout, final_state=sSf,
                                        workspace=ws)

        def med_ms(fn, reps=5):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            return float(np.median(ts))

        pms, sms = med_ms(plain_run), med_ms(seg_run)
        ttok = sum(sw.lengths)
        result["segmented"] = {
            "workload": sw.name, "segment_len": L, "plain_ms": pms, "segmented_ms": sms,
            "speedup": pms / sms, "segmented_tokens_per_s": ttok / (sms * 1e-3),
        }
        del sxx, sout, ws
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- CPU oracle
    if not args.no_cpu_baseline:
        import oracle
        f = lambda t: None if t is None else t.detach().float().cpu().numpy()
        hq, hk, hv, hla, hb, hg, hs = (f(t) for t in (x.q, x.k, x.v, x.log_alpha, x.beta,
                                                      x.gate, x.initial_state))
        oracle.ensure_built()
        # the whole workload, repeated until about 10 s of CPU time have been spent
        runs, t0 = 0, time.perf_counter()
        while runs == 0 or (time.perf_counter() - t0 < 10.0 and runs < 50):
            _, _, used = oracle.run(hq, hk, hv, hla, hb, hg, x.cu_seqlens_host, hs,
                                    want_out=True)
            runs += 1
        dt = (time.perf_counter() - t0) / runs
        result["cpu_baseline"] = {
            "value": T_total / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"the whole workload: all {len(w.lengths) * w.H} (sequence, head) "
                      f"pairs, {T_total} tokens, fp64 token loop with outputs; mean of "
                      f"{runs} runs of {dt:.2f} s each"}

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
