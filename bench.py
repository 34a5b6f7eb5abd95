"""Benchmark of the ESA gated linear recurrence on one MI355X.

Headline: fwd + bwd scan tokens/s on the 64K-context workload (B=64, T=65536, H=8, Dh=64,
fp16 storage, controlled mode), with the dominant kernel's fraction of the HBM roofline,
plus decode steps/s on the generation workload (B=256, H=8, Dh=64, fp16; prefill at prompt
lengths 512 / 1K / 4K / 8K, then 1024 one-token steps).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = esa_scan_fwd (with checkpoint) + esa_scan_bwd over the whole batch, inputs
resident in HBM.  Timing uses HIP events on the stream the kernels run on, around every
launch, so the per-kernel averages come from the same timed region as the total.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
COUNTERS = os.path.join(ROOT, "profiles", "esa_scan_long64k_f16_hbm_counters.txt")


def kernel_source_hash() -> str:
    """sha256 over the kernel sources (name + bytes, sorted), to tell whether counters taken
    earlier still describe the kernels built now."""
    import glob
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_linear_recurrence_chunked_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.hpp"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's readings), or None when the summary is
    missing or was taken on different kernel sources."""
    try:
        text = open(COUNTERS).read()
    except OSError:
        return None
    vals = dict(line.strip().split(": ", 1) for line in text.splitlines()
                if line.strip().startswith(("kernel_source_sha256:", f"{kernel}_traffic_bytes:")))
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    v = vals.get(f"{kernel}_traffic_bytes")
    return int(float(v)) if v else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0, help="0 = min(16, cpu count)")
    ap.add_argument("--only", choices=["train", "decode", "variants", "all", "copy", "workloads",
                                       "lookback"],
                    default="all",
                    help="copy: a plain 4 GiB device copy, the reference for HBM counters; "
                         "variants: the fp8 and sequence-segment variants; "
                         "workloads: every synthetic workload's GPU time and oracle rate; "
                         "lookback: the look-back statistics of the 64K-context scans")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def bench_train(args, torch, binding, synth):
    wl = synth.WORKLOADS["long64k_f16"]
    B, T, H, Dh = wl.B, wl.T, wl.H, wl.Dh
    log(f"[bench] {wl.name}: generating inputs B={B} T={T} H={H} Dh={Dh} {wl.dtype}")
    g = synth.make_inputs(wl, device="cuda:0", with_dy=True)
    torch.cuda.synchronize()
    nelem = B * T * H * Dh
    sb = g["a"].element_size()
    ck_bytes = binding.ckpt_bytes(B, T, H, Dh)
    st_bytes = B * H * Dh * 4
    # algorithmic bytes per launch: what the method itself must read and write
    fwd_bytes = nelem * 4 * sb + ck_bytes + st_bytes  # a, v, q in; y out; ckpt + E_T out
    bwd_bytes = nelem * 7 * sb + ck_bytes  # a, v, q, dy in; da, dv, dq out; ckpt in

    y = torch.empty_like(g["a"])
    eT = torch.empty((B, H, Dh), dtype=torch.float32, device="cuda:0")

    def step():
        _, _, ck = binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode, return_ckpt=True,
                                    final_state=eT, y=y)
        return ck

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        ck = step()
        binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], ckpt=ck, mode=wl.mode)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record()
        ck = step()
        ev[k][1].record()
        binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], ckpt=ck, mode=wl.mode)
        ev[k][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in ev]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in ev]
    total_ms = ev[0][0].elapsed_time(ev[-1][2]) / args.steps
    out = {
        "B": B, "T": T, "H": H, "Dh": Dh, "nelem": nelem,
        "ms_per_step": total_ms, "wall_ms_per_step": wall * 1e3 / args.steps,
        "fwd_ms": sum(fwd_ms) / len(fwd_ms), "bwd_ms": sum(bwd_ms) / len(bwd_ms),
        "fwd_ms_median": sorted(fwd_ms)[len(fwd_ms) // 2],
        "bwd_ms_median": sorted(bwd_ms)[len(bwd_ms) // 2],
        "fwd_bytes": fwd_bytes, "bwd_bytes": bwd_bytes, "tokens": B * T,
    }
    out["tokens_per_s"] = B * T / (total_ms * 1e-3)
    out["fwd_gbs"] = fwd_bytes / (out["fwd_ms"] * 1e-3) / 1e9
    out["bwd_gbs"] = bwd_bytes / (out["bwd_ms"] * 1e-3) / 1e9
    out["fwd_tokens_per_s"] = B * T / (out["fwd_ms"] * 1e-3)
    # this box's streaming reference on the same 4 GiB tensors: what plain elementwise kernels
    # with the same read:write mixes reach (context for the roofline fraction; HBM speed
    # differs from box to box by several percent)
    def stream_gbs(fn, nbytes, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)

    out["stream_reference"] = {
        "copy_1r1w_GBs": stream_gbs(lambda: y.copy_(g["a"]), 2 * nelem * sb),
        "addcmul_3r1w_GBs": stream_gbs(lambda: torch.addcmul(g["a"], g["v"], g["q"], out=y),
                                       4 * nelem * sb),
    }
    if not args.no_cpu_baseline:  # the inputs of the oracle's timed sample (host copies)
        out["inputs"] = {k: g[k].cpu() for k in ("a", "v", "q", "dy")}
    del g, y, eT
    torch.cuda.empty_cache()
    return out


def bench_decode(args, torch, binding, synth):
    wl = synth.WORKLOADS["decode_f16"]
    B, H, Dh = wl.B, wl.H, wl.Dh
    res = {"B": B, "H": H, "Dh": Dh, "prefill": {}}
    n = args.decode_steps
    log(f"[bench] decode: {n} step inputs")
    steps = [synth.decode_step_inputs(wl, k, device="cuda:0") for k in range(n)]
    torch.cuda.synchronize()
    for T in wl.prompts:
        g = synth.make_inputs(wl, device="cuda:0", T=T)
        y, st = binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode)  # warm
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            y, st = binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode, y=y)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = B * T * H * Dh * 4 * 2 + B * H * Dh * 4
        # decode: 1024 eager steps chained from the prefill state, through a StepPlan (the
        # loop's fixed arguments validated once)
        ys = torch.empty((B, H, Dh), dtype=torch.float16, device="cuda:0")
        warm = binding.StepPlan(st.clone(), torch.float16, wl.mode)
        for s in steps[:8]:
            warm(s["a"], s["v"], s["q"], ys)
        plan = binding.StepPlan(st, torch.float16, wl.mode)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record()
        for s in steps:
            plan(s["a"], s["v"], s["q"], ys)
        d1.record()
        torch.cuda.synchronize()
        dms = d0.elapsed_time(d1)
        if T == wl.prompts[0]:  # the same loop through the general state_step call
            st2 = st.clone()
            torch.cuda.synchronize()
            d0.record()
            for s in steps:
                binding.state_step(s["a"], s["v"], s["q"], st2, mode=wl.mode, y=ys)
            d1.record()
            torch.cuda.synchronize()
            res["decode_state_step_call_us_per_step"] = d0.elapsed_time(d1) * 1e3 / n
        res["prefill"][str(T)] = {
            "ms": ms, "tokens_per_s": B * T / (ms * 1e-3), "gbs": nbytes / (ms * 1e-3) / 1e9,
            "decode_us_per_step": dms * 1e3 / n, "decode_steps_per_s": n / (dms * 1e-3),
        }
        del g, y
        torch.cuda.empty_cache()
    sps = [v["decode_steps_per_s"] for v in res["prefill"].values()]
    res["decode_steps_per_s"] = sum(sps) / len(sps)
    # the same chain of steps recorded once into a HIP graph (binding.DecodeGraph, which owns
    # the buffers it replays) and replayed from the last prefill's state: no host work per step
    dg = binding.DecodeGraph(B, H, Dh, n, dtype=torch.float16, mode=wl.mode, device="cuda:0")
    for k, s in enumerate(steps):
        dg.a[k].copy_(s["a"])
        dg.v[k].copy_(s["v"])
        dg.q[k].copy_(s["q"])
    dg.state.copy_(st)
    dg.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    g0.record()
    for _ in range(reps):
        dg.replay()
    g1.record()
    torch.cuda.synchronize()
    gms = g0.elapsed_time(g1) / reps
    res["decode_graph_us_per_step"] = gms * 1e3 / n
    res["decode_graph_steps_per_s"] = n / (gms * 1e-3)
    del dg
    res["decode_tokens_per_s"] = res["decode_steps_per_s"] * B
    res["decode_graph_tokens_per_s"] = res["decode_graph_steps_per_s"] * B
    res["decode_step_bytes"] = B * H * Dh * (4 * 2 + 2 * 4)
    # effective rate of a graph-replayed step (launch-bound: far below the HBM roofline)
    res["decode_graph_GB_s"] = res["decode_step_bytes"] / (res["decode_graph_us_per_step"] * 1e-6) / 1e9
    return res


def bench_variants(args, torch, binding, synth):
    """Two variants beside the headline, each timed with HIP events over 5 repetitions:
    fp8 (E4M3) storage on the 64K workload's shapes and draws, and one device's share of the
    64K workload cut into 8 sequence segments (T = 8192 per device), run through the
    two-pass segmented protocol against a plain scan of the same shape."""
    out = {}
    reps = 5

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    wl = synth.WORKLOADS["long64k_f8e4m3"]
    B, T, H, Dh = wl.B, wl.T, wl.H, wl.Dh
    log(f"[bench] variant {wl.name}")
    g = synth.make_inputs(wl, device="cuda:0", with_dy=True)
    nelem = B * T * H * Dh
    ckb = binding.ckpt_bytes(B, T, H, Dh)
    y = torch.empty_like(g["a"])
    eT = torch.empty((B, H, Dh), dtype=torch.float32, device="cuda:0")
    ck = {}

    def fwd():
        ck["c"] = binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode, return_ckpt=True,
                                   final_state=eT, y=y)[2]

    fwd_ms = timed(fwd)
    bwd_ms = timed(lambda: binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], ckpt=ck["c"],
                                            mode=wl.mode))
    fb = nelem * 4 + ckb + B * H * Dh * 4
    bb = nelem * 7 + ckb
    out[wl.name] = {"B": B, "T": T, "H": H, "Dh": Dh, "storage": "f8e4m3", "mode": wl.mode,
                    "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
                    "fwd_GB_s": round(fb / (fwd_ms * 1e-3) / 1e9, 1),
                    "bwd_GB_s": round(bb / (bwd_ms * 1e-3) / 1e9, 1),
                    "tokens_per_s": B * T / ((fwd_ms + bwd_ms) * 1e-3)}
    del g, y, eT, ck
    torch.cuda.empty_cache()

    nseg = 8
    wl = synth.WORKLOADS["long64k_f16"]
    B, T, H, Dh = wl.B, wl.T // nseg, wl.H, wl.Dh
    log(f"[bench] variant: one of {nseg} sequence segments of {wl.name} (T={T})")
    g = synth.make_inputs(wl, device="cuda:0", T=T, with_dy=True)
    st = {}

    def plain():
        _, _, c = binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode, return_ckpt=True)
        binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], ckpt=c, mode=wl.mode)

    def segmented():
        # this device's aggregate; the other devices' aggregates would arrive by an
        # all-gather, stood in for here by copies of this one (the composition's cost does
        # not depend on the values)
        e, pr = binding.segment_fwd(g["a"], g["v"], mode=wl.mode)
        carry, _ = binding.segment_compose(pr.expand(nseg, -1, -1, -1),
                                           e.expand(nseg, -1, -1, -1))
        k = nseg // 2
        _, _, c = binding.scan_fwd(g["a"], g["v"], g["q"], carry[k], mode=wl.mode,
                                   return_ckpt=True)
        lam = binding.segment_bwd(g["a"], g["v"], g["q"], g["dy"], carry[k], ckpt=c, mode=wl.mode)
        dcarry, _ = binding.segment_compose(pr.expand(nseg, -1, -1, -1),
                                            lam.expand(nseg, -1, -1, -1), reverse=True)
        binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], carry[k], dcarry[k], ckpt=c,
                         mode=wl.mode)

    plain_ms = timed(plain)
    seg_ms = timed(segmented)
    out[f"{wl.name}_segment_of_{nseg}"] = {
        "B": B, "T_per_device": T, "H": H, "Dh": Dh, "plain_fwd_bwd_ms": round(plain_ms, 4),
        "segmented_fwd_bwd_ms": round(seg_ms, 4), "overhead": round(seg_ms / plain_ms, 3),
        "note": "one device's kernels only; the all-gathers of the segment aggregates "
                "(2 x B*H*Dh fp32 per device each way) are not run"}
    del g
    torch.cuda.empty_cache()
    return out


def host_cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, train):
    """The oracle, as it stands, on the 64K workload's own inputs: whole batch rows (every row
    is an independent problem), one row per thread, fwd + bwd, in batches of `threads` rows
    until about 10 s of wall time or the whole batch has run."""
    import oracle

    threads = args.cpu_threads
    x = train["inputs"]
    B = x["a"].shape[0]
    log(f"[bench] cpu baseline: oracle fwd+bwd, T={x['a'].shape[1]}, {threads} threads, "
        f"batches of {threads} rows")
    rows = 0
    sec = 0.0
    while rows < B and sec < 10.0:
        r1 = min(B, rows + threads)
        a, v, q, dy = (oracle._f64(x[k][rows:r1]) for k in ("a", "v", "q", "dy"))
        t0 = time.perf_counter()
        oracle.scan_fwd(a, v, q, mode=1, threads=threads)
        oracle.scan_bwd(a, v, q, dy, mode=1, threads=threads)
        sec += time.perf_counter() - t0
        rows = r1
        del a, v, q, dy
    T = x["a"].shape[1]
    return {"value": rows * T / sec, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": sec, "host_cpus": os.cpu_count(), "cpu_model": host_cpu_model(),
            "sample": f"{rows} of the {B} batch rows x T={T} (H=8, Dh=64, fp64, controlled) "
                      f"fwd+bwd, one row per thread, {threads} threads"}


def bench_workloads(args, torch, binding, synth):
    """Every synthetic workload: the GPU path's time (HIP events, inputs resident) and the
    oracle's rate on a bounded sample of the same inputs, on 1 host thread and on N (one
    batch row per thread).  A token is one (batch, position) over all heads and channels."""
    import oracle

    def gpu_ms(fn, target_ms=20.0):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        reps = int(max(3, min(2000, target_ms / max(e0.elapsed_time(e1), 1e-3))))
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")

    def gpu_ms_cold(fn, reps=20):
        """Each launch after writing 1 GiB, more than the L2 caches and the 256 MB MALL hold,
        so the inputs come from HBM; the events bracket the scan launch only."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            flush.fill_(1)
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps

    def oracle_rate(g, mode, rows, T_s, threads, bwd):
        x = {k: oracle._f64(g[k][:rows, :T_s].cpu()) for k in g}
        t0 = time.perf_counter()
        oracle.scan_fwd(x["a"], x["v"], x["q"], mode=mode, threads=threads)
        if bwd:
            oracle.scan_bwd(x["a"], x["v"], x["q"], x["dy"], mode=mode, threads=threads)
        return rows * T_s / (time.perf_counter() - t0)

    if not args.no_cpu_baseline:
        oracle._load()  # load the library outside the timed samples
    specs = [("small_fwd_f32", None, False), ("layer_fwd_f16", None, False),
             ("long64k_f16", None, False), ("long64k_f16", None, True),
             ("train8k_bf16", None, True), ("long64k_f8e4m3", None, False),
             ("long64k_f8e4m3", None, True)]
    specs += [("decode_f16", T, False) for T in synth.WORKLOADS["decode_f16"].prompts]
    out = []
    for name, T_over, bwd in specs:
        wl = synth.WORKLOADS[name]
        T = T_over or wl.T
        B, H, Dh = wl.B, wl.H, wl.Dh
        log(f"[bench] workload {name} T={T} {'fwd+bwd' if bwd else 'fwd'}")
        g = synth.make_inputs(wl, device="cuda:0", T=T, with_dy=bwd)
        nelem = B * T * H * Dh
        sb = g["a"].element_size()
        y = torch.empty_like(g["a"])
        eT = torch.empty((B, H, Dh), dtype=torch.float32, device="cuda:0")
        if bwd:
            ck_b = binding.ckpt_bytes(B, T, H, Dh)
            nbytes = nelem * 4 * sb + ck_b + B * H * Dh * 4 + nelem * 7 * sb + ck_b

            def fn():
                _, _, ck = binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode,
                                            return_ckpt=True, final_state=eT, y=y)
                binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], ckpt=ck, mode=wl.mode)
        else:
            nbytes = nelem * 4 * sb + B * H * Dh * 4

            def fn():
                binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode, final_state=eT, y=y)
        ms = gpu_ms(fn)
        cold_ms = gpu_ms_cold(fn) if nbytes < (512 << 20) else None
        mode = 0 if wl.mode == "direct" else 1
        T_s = min(T, 8192)
        n_thr = min(B, args.cpu_threads)
        rec = {"workload": name, "B": B, "T": T, "H": H, "Dh": Dh, "dtype": wl.dtype,
               "mode": wl.mode, "path": "fwd+bwd" if bwd else "fwd", "gpu_ms": round(ms, 5),
               "gpu_tokens_per_s": B * T / (ms * 1e-3),
               "algorithmic_GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if cold_ms is not None:  # small enough to stay cache-resident between launches
            rec["gpu_ms_cache_flushed"] = round(cold_ms, 5)
        if not args.no_cpu_baseline:
            rec["oracle_sample"] = f"rows x T={T_s}: 1 row on 1 thread, {n_thr} rows on {n_thr}"
            rec["oracle_tokens_per_s_1thread"] = oracle_rate(g, mode, 1, T_s, 1, bwd)
            rec["oracle_tokens_per_s_nthreads"] = oracle_rate(g, mode, n_thr, T_s, n_thr, bwd)
            rec["oracle_threads"] = n_thr
        out.append(rec)
        del g, y, eT
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:  # the oracle's one-token update on the decode batch
        wl = synth.WORKLOADS["decode_f16"]
        s = {k: oracle._f64(t) for k, t in synth.decode_step_inputs(wl, 0).items()}
        st = oracle._f64(synth.random_state(wl.B, wl.H, wl.Dh, 1))
        n = 20
        t0 = time.perf_counter()
        for _ in range(n):
            _, st = oracle.state_step(s["a"], s["v"], s["q"], st, mode=1)
        out.append({"workload": "decode_f16", "path": "step", "B": wl.B,
                    "oracle_steps_per_s_1thread": n / (time.perf_counter() - t0)})
    return out


def bench_lookback(args, torch, binding, synth):
    """What the cross-tile look-back did in the 64K-context scans (fp16 and fp8 E4M3), from
    the statistics instance of the kernels (ESA_LOOKBACK_STATS): per launch, the lanes that
    found their neighbouring tile's inclusive value published, the lanes that walked back, the
    tiles those walks folded, the longest walk and the unproductive polls.  Each launch is
    also timed (HIP events) beside a launch of the default instance."""
    out = {}
    for name in ("long64k_f16", "long64k_f8e4m3"):
        wl = synth.WORKLOADS[name]
        B, T, H, Dh = wl.B, wl.T, wl.H, wl.Dh
        log(f"[bench] look-back statistics {name}")
        g = synth.make_inputs(wl, device="cuda:0", with_dy=True)
        ws = torch.zeros(binding.workspace_bytes(B, T, H, Dh, g["a"].dtype), dtype=torch.uint8,
                         device="cuda:0")
        y = torch.empty_like(g["a"])
        m = binding.MODES[wl.mode]
        rec = {}
        ck = binding.scan_fwd(g["a"], g["v"], g["q"], mode=m, return_ckpt=True, y=y,
                              workspace=ws)[2]
        for kind in ("fwd", "bwd"):
            runs = []
            for r in range(args.steps if args.steps <= 5 else 5):
                for mode, label in ((m | binding.LOOKBACK_STATS, "stats"), (m, "default")):
                    ws.zero_()
                    e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
                    e0.record()
                    if kind == "fwd":
                        binding.scan_fwd(g["a"], g["v"], g["q"], mode=mode, return_ckpt=True,
                                         y=y, workspace=ws)
                    else:
                        binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], ckpt=ck, mode=mode,
                                         workspace=ws)
                    e1.record()
                    torch.cuda.synchronize()
                    st = binding.workspace_status(ws)
                    st["ms"] = round(e0.elapsed_time(e1), 4)
                    if label == "stats":
                        runs.append(st)
                    else:
                        runs[-1]["default_ms"] = st["ms"]
            rec[kind] = runs
        out[name] = rec
        del g, y, ws, ck
        torch.cuda.empty_cache()
    return out


def bench_copy(args, torch):
    """A plain device-to-device copy of 4 GiB: reads and writes exactly 4 GiB each, the
    reference that scales the HBM traffic counters (FETCH_SIZE, WRITE_SIZE)."""
    n = 1 << 32
    x = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(args.warmup + args.steps):
        y.copy_(x)
    torch.cuda.synchronize()
    return {"copy_bytes": n, "launches": args.warmup + args.steps}


def main():
    args = parse()
    args.cpu_threads = args.cpu_threads or min(16, os.cpu_count() or 1)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: every lane is "
                                   "independent, so several GPUs would each run the one-GPU "
                                   "kernels on their share of the batch or heads",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from gated_linear_recurrence_chunked_amd import binding, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.load_library()
    result = {"metric": "scan fwd+bwd tokens/s and % of HBM peak at 64K ctx; decode steps/s",
              "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
              # dtype: the type the path computes in (fp32 arithmetic and states); the
              # storage type of the sequences (fp16) is config["storage"]
              "scaling": "weak", "vs_baseline": None, "dtype": "f32",
              "data": "synthetic (seeded N(mu, sigma) draws shaped like the pages' workloads)"}
    train = None
    if args.only == "copy":
        result["copy"] = bench_copy(args, torch)
        print(json.dumps(result), flush=True)
        return
    if args.only == "workloads":
        result["workloads"] = bench_workloads(args, torch, binding, synth)
        print(json.dumps(result), flush=True)
        return
    if args.only == "lookback":
        result["lookback"] = bench_lookback(args, torch, binding, synth)
        print(json.dumps(result), flush=True)
        return
    if args.only in ("train", "all"):
        train = bench_train(args, torch, binding, synth)
        result["value"] = train["tokens_per_s"]
        result["ms_per_step"] = train["ms_per_step"]
        result["config"] = {"workload": "long64k_f16: 64K-context fwd+bwd scan", "B": train["B"],
                            "T": train["T"], "H": train["H"], "Dh": train["Dh"],
                            "mode": "controlled", "storage": "f16", "accumulate": "f32",
                            "global_batch": train["B"], "seq_len": train["T"],
                            "parallelism": "single GPU"}
        dom = "bwd" if train["bwd_ms"] >= train["fwd_ms"] else "fwd"
        ach = train[f"{dom}_gbs"]
        result["roofline"] = {"kernel": f"esa {dom}_kernel (f16, controlled, Dh=64)",
                              "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                              "traffic": measured_traffic(dom),
                              "algorithmic_bytes_per_launch": train[f"{dom}_bytes"],
                              "avg_launch_ms": round(train[f"{dom}_ms"], 4)}
        result["stream_reference"] = train["stream_reference"]
        result["kernels"] = {
            "fwd": {"ms": round(train["fwd_ms"], 4), "ms_median": round(train["fwd_ms_median"], 4),
                    "GB_s": round(train["fwd_gbs"], 1),
                    "frac_hbm": round(train["fwd_gbs"] / HBM_PEAK_GBS, 4),
                    "tokens_per_s": train["fwd_tokens_per_s"],
                    "algorithmic_bytes": train["fwd_bytes"]},
            "bwd": {"ms": round(train["bwd_ms"], 4), "ms_median": round(train["bwd_ms_median"], 4),
                    "GB_s": round(train["bwd_gbs"], 1),
                    "frac_hbm": round(train["bwd_gbs"] / HBM_PEAK_GBS, 4),
                    "algorithmic_bytes": train["bwd_bytes"]},
        }
    if args.only in ("decode", "all"):
        dec = bench_decode(args, torch, binding, synth)
        result["decode"] = dec
    if args.only in ("variants", "all"):
        result["variants"] = bench_variants(args, torch, binding, synth)
    if train is not None and not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, train)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
