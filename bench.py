#!/usr/bin/env python3
"""Benchmark: LUT-GEMV over decoupled row-column binary bases on one MI355X.

Workload: the 7B-shaped attention projection — N = K = 4096, 2 binary bases, 5% salient
columns (205) with 2 refinement bases, fp16 activations, batch 1, group width 8. One step is
the whole per-token hot path for that matrix in one launch: the main table-lookup GEMV
(LUT-BSF tables built in LDS, pattern lookups, alpha_r) and the VCM salient refinement into the
same output.

Cold weights: the packed bases, scales, indices, activations and outputs are replicated into
enough distinct copies (>= 512 MiB, twice the 256 MB Infinity Cache) and the steps rotate
through them, so every step streams its weights from HBM rather than from a cache.

Prints one JSON line (see the keys below). The oracle is timed on the host cores for the
cpu_baseline entry; the GPU path never touches it.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LUT-GEMV HBM GB/s (% of peak) + µs/call, 4096×4096 batch-1, 2 bases"
PEAK_GBS = 8000.0          # MI355X HBM3E peak, 8 TB/s
COLD_BYTES = 512 << 20     # rotate through at least this much distinct input data


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="bound on the oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the headline line: time every GEMV and layer of the 7B MLP and the "
                         "70B layer at their batches, the group-scale variant, the offline fit and the saliency search")
    ap.add_argument("--profile-shape", type=str, default=None, metavar="N,K,NB,B",
                    help="instead of the headline line: run `--steps` cold ubw_lut_gemv calls of an N x K GEMV with "
                         "NB bases at batch B (no refinement), for counter collection under rocprofv3")
    ap.add_argument("--profile-run", action="store_true",
                    help="for hardware-counter runs: a 64 MiB device copy (known bytes, to scale the counters) "
                         "then --steps cold steps; prints one line, no timing")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gemv8_proj4096_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "ultra_bit_weight_uint32_amd", "csrc", "kernels.hip")


def measured_traffic():
    """HBM bytes per step-kernel launch from the committed counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    import hashlib
    try:
        fields = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line)
    except OSError:
        return None
    digest = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256", "").strip() != digest:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (the per-GPU share of a "
              "sharded matrix is the same kernel at a smaller N). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import ultra_bit_weight_uint32_amd as ubw
    from workloads import algorithmic_bytes, attn_proj_7b

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_shape:
        profile_shape(torch, ubw, dev, args.profile_shape, args.steps)
        return
    if args.configs:
        small_sweep(torch, ubw, dev)
        load_time_sweep(torch, ubw, dev)
        config_sweep(torch, ubw, dev)
        gs_sweep(torch, ubw, dev)
        fit_sweep(torch, ubw, dev)
        saliency_sweep(torch, ubw, dev)
        return
    wl = attn_proj_7b(seed=0)
    g = wl.gemvs[0]
    n, k, nb, s, ns, batch = g.n, g.k, g.nb, g.s, g.ns, g.batch

    def t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint32:
            a = a.view(np.int32)
        return torch.from_numpy(a).to(dev)

    # load time: pack once on the device, then replicate (not timed)
    packed0 = ubw.pack_bases(t(g.bits), nb, n, k)
    packed_s0 = ubw.pack_bases(t(g.bits_s), ns, n, s)
    base = dict(packed=packed0, ar=t(g.alpha_r), ac=t(g.alpha_c), packed_s=packed_s0, ar_s=t(g.alpha_r_s),
                ac_s=t(g.alpha_c_s), idx=t(g.idx), x=t(g.x))
    per_copy = sum(v.numel() * v.element_size() for v in base.values()) + batch * n * 4
    ncopy = max(2, -(-COLD_BYTES // per_copy))
    copies = []
    for _ in range(ncopy):
        c = {key: v.clone() for key, v in base.items()}
        c["y"] = torch.empty((batch, n), dtype=torch.float32, device=dev)
        copies.append(c)
    del base
    torch.cuda.synchronize()

    ws = ubw.workspace(n, dev)

    def step(c):
        """The whole per-token hot path for this matrix: one launch (main bases + VCM refinement,
        y = result via the workspace's row-group counters)."""
        ubw.lut_gemv_refined(c["packed"], c["ar"], c["ac"], c["idx"], c["packed_s"], c["ar_s"], c["ac_s"], c["x"],
                             n, k, y=c["y"], workspace=ws)

    def main_only(c):
        ubw.lut_gemv(c["packed"], c["ar"], c["ac"], c["x"], n, k, y=c["y"], workspace=ws)

    def step_g4(c):
        """The same step at group width 4 (whole rows per workgroup, 16-entry tables of the full
        row in LDS, one plain store per output; no workspace needed)."""
        ubw.lut_gemv_refined(c["packed"], c["ar"], c["ac"], c["idx"], c["packed_s"], c["ar_s"], c["ac_s"], c["x"],
                             n, k, g=4, y=c["y"])

    wbytes = packed0.numel() * 4
    outw = torch.empty(-(-wbytes // 8192), dtype=torch.int32, device=dev)

    def read_only(c):
        ubw.bench_stream_read(c["packed"], wbytes, outw)

    def tiny(c):  # one 16-byte read by one workgroup: the floor of any launch
        ubw.bench_stream_read(c["packed"], 16, outw)

    # warmup: W untimed steps (and touch every copy once)
    for i in range(max(args.warmup, ncopy)):
        step(copies[i % ncopy])
    torch.cuda.synchronize()

    # Every timed launch reads a copy that no launch has touched for at least COLD_BYTES of other
    # data: one position runs on through the copies across all legs, and a COLD_BYTES write
    # evicts the caches before each leg.
    evict = torch.empty(COLD_BYTES // 4, dtype=torch.float32, device=dev)
    pos = [0]

    def leg(fn):
        evict.zero_()
        start = pos[0]

        def launch(i):
            fn(copies[(start + i) % ncopy])
        return launch

    def timed(fn, count, isolated=False):
        """Per-launch us: K queued launches (pipelined) or the median of single launches."""
        launch = leg(fn)
        us = (run_isolated(torch, launch, count) if isolated else run_queued(torch, launch, count) * 1e3 / count)
        pos[0] += count
        return us

    if args.profile_run:
        src = torch.ones(16 << 20, dtype=torch.float32, device=dev)   # 64 MiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        for i in range(args.steps):
            step(copies[i % ncopy])
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": True, "steps": args.steps, "copy_bytes": src.numel() * 4}), flush=True)
        return

    # A. the timed region: exactly K steps, synchronized on both sides, queued behind a GPU
    # sleep so the GPU runs them back to back (host launch overhead would otherwise dominate).
    # A step is one launch of the step kernel, so the time per step is also that kernel's
    # average launch duration, dispatch gap between back-to-back launches included.
    ms_per_step = timed(step, args.steps) * 1e-3
    # B. main bases only (ubw_lut_gemv, one launch per call), same protocol
    main_us = timed(main_only, args.steps)
    # C. size-matched streaming read of the same weight bytes (ceiling of one read that size), and
    # the launch floor (a one-workgroup kernel that reads 16 bytes)
    read_us = timed(read_only, args.steps)
    floor_us = timed(tiny, args.steps)
    # C'. the step at group width 4
    g4_us = timed(step_g4, args.steps)
    # D. the same three, one launch at a time: each launch alone on the GPU between two events
    # (median), i.e. dispatch, the kernel and its end, with nothing of a neighbour overlapping
    iso = min(args.steps, 100)
    iso_step, iso_main, iso_read = (timed(f, iso, isolated=True) for f in (step, main_only, read_only))
    st, word = ubw.workspace_check(ws)
    if st != ubw.UBW_OK:
        raise RuntimeError(f"workspace reports {ubw.status_str(st)} (word {word:#x})")
    # E. a dependent chain: call i + 1 reads call i's output as its activations (fp32 x, which
    # the kernel reads directly), so no call can start before the previous one has finished and
    # its output is written: the per-token latency of a chain of such layers. The chain's copies
    # get alpha_c / 8 so that values stay finite along it (same work, same bytes).
    for c in copies:
        c["ac"].mul_(0.125)
        c["ac_s"].mul_(0.125)
    ys = [torch.empty((batch, n), dtype=torch.float32, device=dev) for _ in range(2)]
    ys[1].copy_(copies[0]["x"].float())

    def chained(i):
        c = copies[(chain_start + i) % ncopy]
        ubw.lut_gemv_refined(c["packed"], c["ar"], c["ac"], c["idx"], c["packed_s"], c["ar_s"], c["ac_s"],
                             ys[(i + 1) % 2], n, k, y=ys[i % 2], workspace=ws)

    evict.zero_()
    chain_start = pos[0]
    chain_us = run_queued(torch, chained, args.steps) * 1e3 / args.steps
    pos[0] += args.steps
    st, word = ubw.workspace_check(ws)
    if st != ubw.UBW_OK or not torch.isfinite(ys[(args.steps - 1) % 2]).all():
        raise RuntimeError(f"dependent chain: {ubw.status_str(st)} (word {word:#x}) or non-finite output")

    # sanity: the last outputs are finite (parity itself is the test suite's job)
    if not torch.isfinite(copies[(args.steps - 1) % ncopy]["y"]).all():
        raise RuntimeError("non-finite output")

    step_bytes = algorithmic_bytes(n, k, nb, batch, 2, s, ns)
    main_bytes = algorithmic_bytes(n, k, nb, batch, 2)
    chain_bytes = algorithmic_bytes(n, k, nb, batch, 4, s, ns)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    step_mean = ms_per_step * 1e3
    achieved = step_bytes / (step_mean * 1e-6) / 1e9
    main_mean = main_us

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(g, step_bytes, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "7B attention projection: N=K=4096, 2 binary bases, 5% salient columns (s=205) with "
                        "2 refinement bases, fp16 x, batch 1, g=8; step = one ubw_lut_gemv_refined launch (main + VCM)",
            "N": n, "K": k, "nb": nb, "s": s, "ns": ns, "batch": batch, "x_dtype": "fp16", "g": 8,
            "cold_copies": ncopy, "bytes_per_copy": per_copy,
        },
        "pct_of_peak": round(100 * value / PEAK_GBS, 2),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "step_algorithmic_bytes": step_bytes,
        "roofline": {
            "kernel": "k_gemv8 (the step's single launch: main bases + VCM refinement)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "bytes_per_launch": step_bytes,
            "us_per_launch": round(step_mean, 3),
            "timing": "K back-to-back launches between two events on the launch stream, divided by K",
        },
        "main_only": {
            "what": "ubw_lut_gemv alone (2 bases, no salient columns), one launch per call",
            "bytes_per_launch": main_bytes,
            "us_per_launch": round(main_mean, 3),
            "GBps": round(main_bytes / (main_mean * 1e-6) / 1e9, 2),
            "pct_of_peak": round(100 * main_bytes / (main_mean * 1e-6) / 1e9 / PEAK_GBS, 2),
        },
        "read_ceiling": {
            "what": "one streaming read of the same weight bytes, same access shape, cold",
            "bytes": wbytes,
            "us_per_launch": round(read_us, 3),
            "GBps": round(wbytes / (read_us * 1e-6) / 1e9, 2),
            "us_isolated": round(iso_read, 3),
            "GBps_isolated": round(wbytes / (iso_read * 1e-6) / 1e9, 2),
        },
        "launch_floor": {
            "what": "a one-workgroup kernel reading 16 bytes, same protocol: the per-launch cost of any kernel",
            "us_per_launch": round(floor_us, 3),
        },
        "g4_step": {
            "what": "the same step at group width 4 (ubw_lut_gemv_refined, g=4: whole rows per workgroup, "
                    "no workspace)",
            "us_per_launch": round(g4_us, 3),
            "GBps": round(step_bytes / (g4_us * 1e-6) / 1e9, 2),
            "pct_of_peak": round(100 * step_bytes / (g4_us * 1e-6) / 1e9 / PEAK_GBS, 2),
        },
        "isolated": {
            "what": "median of single launches, each alone on the GPU between two events (dispatch, kernel "
                    "and its end; no neighbouring launch overlapping), cold",
            "launches": iso,
            "step_us": round(iso_step, 3),
            "step_GBps": round(step_bytes / (iso_step * 1e-6) / 1e9, 2),
            "main_only_us": round(iso_main, 3),
            "read_us": round(iso_read, 3),
        },
        "dependent_chain": {
            "what": "K steps where step i + 1 reads step i's fp32 output as x (each waits for the previous "
                    "one's result), weights cold",
            "us_per_step": round(chain_us, 3),
            "bytes_per_step": chain_bytes,
            "GBps": round(chain_bytes / (chain_us * 1e-6) / 1e9, 2),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def run_isolated(torch, launch, count):
    """Median time of `count` single launches in us: each is queued behind a short GPU sleep
    (so the host's launch overhead is not counted) between two events on the launch stream and
    synchronized before the next."""
    times = []
    for i in range(count):
        torch.cuda._sleep(2_000_000)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch(i)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    return float(np.median(times))


def run_queued(torch, launch, count):
    """Queue `count` launches behind a GPU sleep so the host is far ahead when the GPU starts,
    then time them with two events on the launch stream (synchronized on both sides). Returns
    the total in ms. Retries with a longer sleep if the host could not queue everything before
    the sleep ended."""
    cycles = 100_000_000
    for _ in range(5):
        torch.cuda.synchronize()
        torch.cuda._sleep(cycles)
        gate = torch.cuda.Event()
        gate.record()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(count):
            launch(i)
        end.record()
        queued_in_time = not gate.query()
        torch.cuda.synchronize()
        if queued_in_time:
            return start.elapsed_time(end)
        cycles *= 4
    raise RuntimeError("could not queue the timed launches ahead of the GPU")


def config_sweep(torch, ubw, dev):
    """Per-GEMV and per-layer times of configs 4 and 5 (cold: each timed loop rotates through at least
    COLD_BYTES of distinct copies), printed as one JSON line per measurement."""
    from workloads import algorithmic_bytes, mlp_7b, decoder_layer_70b

    def t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int32) if a.dtype == np.uint32 else a).to(dev)

    for label, wl in (("7B MLP", mlp_7b(seed=0)), ("70B decoder layer", decoder_layer_70b(seed=0))):
        base = []
        for g in wl.gemvs:
            base.append(dict(packed=ubw.pack_bases(t(g.bits), g.nb, g.n, g.k), ar=t(g.alpha_r), ac=t(g.alpha_c),
                             x=t(g.x), packed_s=ubw.pack_bases(t(g.bits_s), g.ns, g.n, g.s), ar_s=t(g.alpha_r_s),
                             ac_s=t(g.alpha_c_s), idx=t(g.idx), ws=ubw.workspace(g.n, dev)))
        size = [sum(v.numel() * v.element_size() for v in d.values()) for d in base]

        def copies_of(gis):
            n = max(2, -(-COLD_BYTES // sum(size[i] for i in gis)))
            return [[{k: v.clone() for k, v in base[i].items()} for i in gis] for _ in range(n)]

        def call(d, g, b, y):
            ubw.lut_gemv_refined(d["packed"], d["ar"], d["ac"], d["idx"], d["packed_s"], d["ar_s"], d["ac_s"],
                                 d["x"][:b], g.n, g.k, y=y, workspace=d["ws"])

        def call_group(ds, gs, b, ys):
            # GEMVs that read the same x in one launch (the first one's x serves all)
            ubw.lut_gemv_multi([dict(packed=d["packed"], alpha_r=d["ar"], alpha_c=d["ac"], n=g.n, y=y, idx=d["idx"],
                                     packed_s=d["packed_s"], alpha_r_s=d["ar_s"], alpha_c_s=d["ac_s"],
                                     workspace=d["ws"]) for d, g, y in zip(ds, gs, ys)], ds[0]["x"][:b], gs[0].k)

        names = [g.name for g in wl.gemvs]
        runs = [(list(range(len(wl.gemvs))), "layer", None)]
        # groups of GEMVs on one input: q/k/v and gate/up
        groups = [[names.index(m) for m in grp] for grp in (("q", "k", "v"), ("gate", "up")) if set(grp) <= set(names)]
        if groups:
            parts = groups + [[i] for i in range(len(names)) if not any(i in grp for grp in groups)]
            runs.append((list(range(len(wl.gemvs))), "layer_grouped", parts))
            runs += [(grp, "+".join(names[i] for i in grp) + "_grouped", [list(grp)]) for grp in groups]
        runs += [([i], g.name, None) for i, g in enumerate(wl.gemvs)]
        for gis, name, parts in runs:
            C = copies_of(gis)
            for b in wl.batches:
                ys = [torch.zeros((b, wl.gemvs[i].n), device=dev) for i in gis]
                pos = {i: j for j, i in enumerate(gis)}

                def launch(k):
                    c = C[k % len(C)]
                    if parts is None:
                        for j, i in enumerate(gis):
                            call(c[j], wl.gemvs[i], b, ys[j])
                        return
                    for grp in parts:
                        if len(grp) == 1:
                            call(c[pos[grp[0]]], wl.gemvs[grp[0]], b, ys[pos[grp[0]]])
                        else:
                            call_group([c[pos[i]] for i in grp], [wl.gemvs[i] for i in grp], b,
                                       [ys[pos[i]] for i in grp])

                for k in range(len(C)):
                    launch(k)
                reps = 100 if sum(size[i] for i in gis) < (64 << 20) else 20
                us = run_queued(torch, launch, reps) * 1e3 / reps
                by = sum(algorithmic_bytes(wl.gemvs[i].n, wl.gemvs[i].k, wl.gemvs[i].nb, b, 2, wl.gemvs[i].s,
                                           wl.gemvs[i].ns) for i in gis)
                print(json.dumps({"sweep": label, "gemv": name, "batch": b, "us": round(us, 2),
                                  "GBps": round(by / us / 1e3, 1), "pct_of_peak": round(by / us / 1e3 / PEAK_GBS * 100, 2),
                                  "algorithmic_bytes": by, "cold_copies": len(C)}), flush=True)
            del C
            torch.cuda.empty_cache()
        del base
        torch.cuda.empty_cache()


def profile_shape(torch, ubw, dev, spec, steps):
    """Cold calls of one GEMV shape (for rocprofv3 --pmc / --kernel-trace runs)."""
    from workloads import make_gemv
    n, k, nb, b = (int(v) for v in spec.split(","))
    g = make_gemv(np.random.default_rng(1), "profile", n, k, nb, batch=b)

    def t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int32) if a.dtype == np.uint32 else a).to(dev)

    base = dict(packed=ubw.pack_bases(t(g.bits), nb, n, k), ar=t(g.alpha_r), ac=t(g.alpha_c), x=t(g.x))
    per = sum(v.numel() * v.element_size() for v in base.values())
    copies = [{kk: v.clone() for kk, v in base.items()} for _ in range(max(2, -(-COLD_BYTES // per)))]
    for c in copies:
        c["ws"] = ubw.workspace(n, dev)
    y = torch.zeros((b, n), device=dev)
    for i in range(steps):
        c = copies[i % len(copies)]
        ubw.lut_gemv(c["packed"], c["ar"], c["ac"], c["x"], n, k, y=y, workspace=c["ws"])
    torch.cuda.synchronize()
    print(json.dumps({"profile_shape": [n, k, nb, b], "steps": steps, "cold_copies": len(copies)}), flush=True)


def small_sweep(torch, ubw, dev):
    """The two cache-resident workloads, reported as time per call (launch-latency bound):
    the single 256 x 512 GEMV (1 base, fp32 x) and the ternary stack (4 x 256 -> 768 -> 256, two
    half-scale bases per layer), 64 tokens one after another, each through 8 chained launches.
    The timed chain feeds each layer's fp32 output straight to the next layer as fp32 x (the
    kernel reads fp32 activations); the parity test rounds to fp16 between layers instead."""
    from workloads import single_gemv_256x512, ternary_stack_256x768

    def t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int32) if a.dtype == np.uint32 else a).to(dev)

    g = single_gemv_256x512(seed=0).gemvs[0]
    packed = ubw.pack_bases(t(g.bits), g.nb, g.n, g.k)
    ar, ac, x = t(g.alpha_r), t(g.alpha_c), t(g.x)
    ws = ubw.workspace(g.n, dev)
    y = torch.empty((1, g.n), dtype=torch.float32, device=dev)
    ubw.lut_gemv(packed, ar, ac, x, g.n, g.k, y=y, workspace=ws)
    us = run_queued(torch, lambda i: ubw.lut_gemv(packed, ar, ac, x, g.n, g.k, y=y, workspace=ws), 400) * 1e3 / 400
    print(json.dumps({"sweep": "single GEMV 256 x 512, 1 base, fp32 x", "batch": 1, "us": round(us, 2),
                      "note": "cache-resident: launch-latency bound"}), flush=True)

    wl = ternary_stack_256x768(seed=0)
    enc = [ubw.ternary_encode(t(L.w), t(L.scale)) for L in wl.ternary]
    shapes = [L.w.shape for L in wl.ternary]
    wss = [ubw.workspace(n, dev) for n, _ in shapes]
    outs = [torch.empty((1, n), dtype=torch.float32, device=dev) for n, _ in shapes]
    toks = t(wl.tokens.astype(np.float32))

    def token(i):
        a = toks[i % toks.shape[0]:i % toks.shape[0] + 1]
        for (packed, ar, ac), (n, k), w, o in zip(enc, shapes, wss, outs):
            a = ubw.lut_gemv(packed, ar, ac, a, n, k, y=o, workspace=w)

    token(0)
    ntok = toks.shape[0]
    ms = run_queued(torch, token, ntok)
    print(json.dumps({"sweep": "ternary stack 4 x (256 -> 768 -> 256), 8 chained GEMVs per token",
                      "tokens": ntok, "us_per_token": round(ms * 1e3 / ntok, 2),
                      "us_per_gemv": round(ms * 1e3 / ntok / len(enc), 2),
                      "tokens_per_s": round(ntok / ms * 1e3, 1)}), flush=True)


def load_time_sweep(torch, ubw, dev):
    """The load-time kernels at the 70B gate shape (28672 x 8192, 3 bases): packing canonical
    words into tiles, packing from int8 signs, the ternary two-base encoding (one 28672 x 8192
    int8 matrix), and the tables written to memory (batch 16, 3 bases, K = 8192). HBM-bound:
    bytes = what each must read and write."""
    n, k, nb = 28672, 8192, 3
    kw = (k + 31) // 32
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    words = torch.randint(-2**31, 2**31 - 1, (nb, n, kw), dtype=torch.int32, device=dev, generator=gen)
    signs = torch.randint(-1, 2, (nb, n, k), dtype=torch.int8, device=dev, generator=gen)
    out = torch.empty(ubw.packed_words(nb, n, k), dtype=torch.int32, device=dev)
    tern = signs[0].contiguous()
    scale = torch.rand(n, device=dev, generator=gen)
    x = torch.randn((16, k), device=dev, generator=gen).half()
    ac = torch.rand((nb, k), device=dev, generator=gen)
    packed_bytes = out.numel() * 4
    cases = [
        ("pack canonical words -> tiles", lambda i: ubw.pack_bases(words, nb, n, k, out=out), words.numel() * 4 + packed_bytes),
        ("pack int8 signs -> tiles", lambda i: ubw.pack_bases(signs, nb, n, k, out=out), signs.numel() + packed_bytes),
        ("ternary encode (one int8 matrix -> 2 bases)", lambda i: ubw.ternary_encode(tern, scale),
         tern.numel() + ubw.packed_words(2, n, k) * 4 + 4 * (3 * n + 2 * k)),
        ("tables into memory (b 16, 3 bases, K 8192)", lambda i: ubw.build_lut(x, ac),
         16 * nb * (k // 8) * 256 * 4 + x.numel() * 2 + ac.numel() * 4),
    ]
    for name, fn, by in cases:
        fn(0)
        reps = 20
        ms = run_queued(torch, fn, reps) / reps
        print(json.dumps({"sweep": "load-time kernels", "kernel": name, "ms": round(ms, 4),
                          "GBps": round(by / ms / 1e6, 1), "pct_of_peak": round(by / ms / 1e6 / PEAK_GBS * 100, 2),
                          "bytes": by}), flush=True)
    del words, signs, out
    torch.cuda.empty_cache()


def gs_sweep(torch, ubw, dev):
    """The group-scale variant (one fp16 row scale per 128 columns) on the 7B attention
    projection (with its refinement) and the 7B MLP up projection, batch 1, cold, one JSON line
    each, next to the per-row call on the same data."""
    from workloads import algorithmic_bytes, attn_proj_7b, mlp_7b

    def t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int32) if a.dtype == np.uint32 else a).to(dev)

    rng = np.random.default_rng(5)
    for label, g in (("7B attention projection", attn_proj_7b(seed=0).gemvs[0]),
                     ("7B MLP up", mlp_7b(seed=0).gemvs[0].with_batch(1))):
        cols = ubw.group_scale_cols(g.k)
        arg = rng.uniform(0.05, 0.5, size=(g.nb, g.n, cols)).astype(np.float16)
        base = dict(packed=ubw.pack_bases(t(g.bits), g.nb, g.n, g.k), arg=t(ubw.arrange_group_scales(arg)),
                    ar=t(g.alpha_r), ac=t(g.alpha_c),
                    x=t(g.x), packed_s=ubw.pack_bases(t(g.bits_s), g.ns, g.n, g.s), ar_s=t(g.alpha_r_s),
                    ac_s=t(g.alpha_c_s), idx=t(g.idx), ws=ubw.workspace(g.n, dev))
        size = sum(v.numel() * v.element_size() for v in base.values())
        C = [{k: v.clone() for k, v in base.items()} for _ in range(max(2, -(-COLD_BYTES // size)))]
        y = torch.zeros((1, g.n), device=dev)
        per_row = algorithmic_bytes(g.n, g.k, g.nb, 1, 2, g.s, g.ns)
        grouped = per_row - g.nb * g.n * 4 + g.nb * g.n * cols * 2   # fp16 block scales instead of fp32 per row

        def launch_gs(k):
            c = C[k % len(C)]
            ubw.lut_gemv_gs(c["packed"], c["arg"], c["ac"], c["x"], g.n, g.k, idx=c["idx"], packed_s=c["packed_s"],
                            alpha_r_s=c["ar_s"], alpha_c_s=c["ac_s"], y=y, workspace=c["ws"])

        def launch_row(k):
            c = C[k % len(C)]
            ubw.lut_gemv_refined(c["packed"], c["ar"], c["ac"], c["idx"], c["packed_s"], c["ar_s"], c["ac_s"], c["x"],
                                 g.n, g.k, y=y, workspace=c["ws"])

        for name, fn, by in (("group scales (g128, fp16)", launch_gs, grouped), ("per-row scales", launch_row, per_row)):
            for k in range(len(C)):
                fn(k)
            us = run_queued(torch, fn, 200) * 1e3 / 200
            print(json.dumps({"sweep": label, "gemv": name, "batch": 1, "us": round(us, 2),
                              "GBps": round(by / us / 1e3, 1), "pct_of_peak": round(by / us / 1e3 / PEAK_GBS * 100, 2),
                              "algorithmic_bytes": by, "cold_copies": len(C)}), flush=True)
        del C
        torch.cuda.empty_cache()


def fit_bytes(n, k, nb, iters, w_bytes=4):
    """HBM bytes the fit's passes must move: W read and the residual written once, then per
    base after the first a residual update (read + write), the sign words, 2 reads of the
    residual per ALS round, and the final update."""
    nk = n * k
    return (w_bytes + 4) * nk + (nb - 1) * 8 * nk + nb * nk // 8 + nb * iters * 8 * nk + 8 * nk


def fit_sweep(torch, ubw, dev):
    """The offline fit (residual binarization + alternating least squares) at the 7B projection
    and the 70B q/o shapes: one JSON line each, GPU time next to the oracle's on the host."""
    import oracle
    rng = np.random.default_rng(6)
    for n, k, nb, iters in ((4096, 4096, 2, 5), (8192, 8192, 3, 5)):
        w = (rng.standard_normal((n, k)) * rng.uniform(0.2, 3, (n, 1))).astype(np.float32)
        wt = torch.from_numpy(w).to(dev)
        res = torch.empty((n, k), dtype=torch.float32, device=dev)
        ws = torch.empty(ubw.fit_workspace_bytes(n, k) // 4, dtype=torch.float32, device=dev)
        for _ in range(2):
            ubw.fit_bases(wt, nb, iters, residual=res, workspace=ws)
        reps = 5
        ms = run_queued(torch, lambda i: ubw.fit_bases(wt, nb, iters, residual=res, workspace=ws), reps) / reps
        by = fit_bytes(n, k, nb, iters)
        t0 = time.perf_counter()
        oracle.fit(w, nb, iters)
        cpu = time.perf_counter() - t0
        print(json.dumps({"sweep": "offline fit", "shape": [n, k], "nb": nb, "iters": iters, "ms": round(ms, 3),
                          "GBps": round(by / ms / 1e6, 1), "pct_of_peak": round(by / ms / 1e6 / PEAK_GBS * 100, 2),
                          "algorithmic_bytes": by, "oracle_s": round(cpu, 3), "oracle_cores": oracle.max_threads()}),
              flush=True)
        del wt, res, ws
        torch.cuda.empty_cache()


def saliency_sweep(torch, ubw, dev):
    """Hessian-guided salient-column search at the 7B projection (K = 4096) and the 70B q/o
    (K = 8192) shapes, 2048 calibration rows: the Gram matrix on the matrix cores (TFLOP/s
    against the fp16 dense peak) and the whole search (damped Cholesky, inverse diagonal,
    scores, selection); the oracle (numpy fp64) is timed beside the first."""
    import oracle
    rng = np.random.default_rng(7)
    for k, n, s in ((4096, 4096, 205), (8192, 8192, 410)):
        t = 2048
        x = torch.from_numpy((rng.standard_normal((t, k)) * rng.uniform(0.2, 2, (1, k))).astype(np.float16)).to(dev)
        w = torch.from_numpy(rng.standard_normal((n, k)).astype(np.float32)).to(dev)
        h = torch.empty((k, k), dtype=torch.float32, device=dev)
        ws = torch.empty(ubw.saliency_workspace_bytes(n, k) // 4, dtype=torch.float32, device=dev)
        ubw.gram(x, out=h)
        reps = 10
        gms = run_queued(torch, lambda i: ubw.gram(x, out=h), reps) / reps
        flops = 2.0 * t * k * k
        ubw.hessian_saliency(h, w, s, workspace=ws)
        ms = run_queued(torch, lambda i: (ubw.gram(x, out=h), ubw.hessian_saliency(h, w, s, workspace=ws)), 3) / 3
        line = {"sweep": "hessian saliency", "K": k, "T": t, "N": n, "s": s, "gram_ms": round(gms, 3),
                "gram_TFLOPs": round(flops / gms / 1e9, 1), "gram_pct_of_fp16_peak": round(flops / gms / 1e9 / 2500 * 100, 2),
                "search_ms": round(ms, 3)}
        if k == 4096:
            xh = x.cpu().numpy()
            wh = w.cpu().numpy()
            t0 = time.perf_counter()
            oracle.saliency(oracle.hessian(xh), wh, s)
            line["oracle_s"] = round(time.perf_counter() - t0, 3)
        print(json.dumps(line), flush=True)
        del x, w, h, ws
        torch.cuda.empty_cache()


def host_cpu_model():
    """The host CPU's model name with its family and model numbers (/proc/cpuinfo: a virtualized
    host may report only the brand), or the platform's processor string."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (t.strip() for t in line.split(":", 1))
                if k in ("model name", "cpu family", "model") and k not in fields:
                    fields[k] = v
            if not line.strip() and fields:
                break
    except OSError:
        pass
    if "model name" in fields:
        extra = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model") if k in fields)
        return fields["model name"] + (f" ({extra})" if extra else "")
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(g, step_bytes, seconds):
    """The oracle as it stands (fp64 dequantize + naive matvec, OpenMP over rows) on the host
    cores, on whole calls of the step until about `seconds` have passed."""
    import oracle
    cores = oracle.max_threads()
    kw = g.refine_kwargs()
    t0 = time.perf_counter()
    oracle.gemv(g.bits, g.alpha_r, g.alpha_c, g.x, **kw)
    first = time.perf_counter() - t0
    reps = max(1, int(seconds / max(first, 1e-3)) - 1)
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.gemv(g.bits, g.alpha_r, g.alpha_c, g.x, **kw)
    dt = (time.perf_counter() - t0) / reps
    return {
        "value": round(step_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "cpu_model": host_cpu_model(),
        "host_logical_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{reps} full calls of the same step (4096x4096, 2 bases + 205 salient columns, batch 1), "
                  f"{dt * 1e3:.1f} ms per call",
    }


if __name__ == "__main__":
    main()
