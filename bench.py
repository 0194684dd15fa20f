#!/usr/bin/env python3
"""Benchmark of the submanifold 3x3x3 convolution on one MI355X.

One step = the whole path on one synthetic batch: build the neighbour map of
the coordinate set (pack, radix sort, resolve, status read-back), then run the
forward pass on it (4 forward passes reusing the map for the 4-grid workload).
Inputs are resident in device memory before the timed region starts.

Prints ONE JSON line.  `value` is forward active voxels per second (N divided
by the mean forward kernel time from HIP events on the launch stream);
`ms_per_step` is the GPU time of a whole step (map build + forward, HIP events;
the map build's span includes its host-side status read-back); `host_ms_per_step`
is the host wall time of a step, which also holds a short spin kernel that keeps
the GPU busy while the forward is enqueued.

    python bench.py [--steps K] [--warmup W] [--config 3] [--dtype f32|bf16]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SubMConv3d fwd active-voxels/s + TFLOP/s at 128^3/128ch; map-build ms"
PEAK_HBM_GBPS = 8000.0
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}
CSRC = os.path.join(ROOT, "submanifold_sparse_convolution_submconv3d_amd", "csrc")
CONV_SRCS = [os.path.join(CSRC, f) for f in ("conv.hip", "conv_win.hip", "conv_big.hip")]
MAP_SRCS = [os.path.join(CSRC, f) for f in ("mapbuild.hip", "sort_scan.hip", "conv_win.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
BOUND = {1: "hbm", 2: "mfma", 3: "mfma", 4: "mfma", 5: "hbm"}


def src_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, dtype: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = data.get("%s/%s/%s" % (workload, dtype, kernel))
    if not entry:
        return None
    srcs = CONV_SRCS if kernel == "forward" else MAP_SRCS
    if entry.get("source_hash") != src_hash(srcs):
        return None
    return entry.get("bytes_per_launch")


def algorithmic(n, p, cin, cout, dtype):
    s = 4 if dtype == "f32" else 2
    flops = 2.0 * cin * cout * p
    bytes_ = n * (cin * s + cout * s + 27 * 4) + 27 * cin * cout * s + 4 * cout
    return flops, float(bytes_)


def cpu_baseline(coords, feats, weight, bias, res, batch, budget_s):
    """The oracle (C, dense volume, fp64) on a bounded sample of the same workload."""
    import numpy as np
    import oracle

    oracle.build_oracle(force=False)
    t0 = time.perf_counter()
    nbr = oracle.dense.neighbor_table(coords, res, batch)
    t_map = time.perf_counter() - t0
    n = len(coords)
    f64, w64 = feats.astype(np.float64), weight.astype(np.float64)
    probe = min(n, 256)
    t0 = time.perf_counter()
    oracle.dense.forward(f64, w64, bias, nbr, rows=(0, probe))
    per_row = max((time.perf_counter() - t0) / probe, 1e-9)
    rows = int(min(n, max(probe, (budget_s - t_map) / per_row)))
    t0 = time.perf_counter()
    oracle.dense.forward(f64, w64, bias, nbr, rows=(0, rows))
    t_fwd = time.perf_counter() - t0
    return {
        "value": rows / t_fwd, "unit": "voxels/s", "cores": oracle.dense.num_threads(), "kind": "oracle",
        "sample": "C dense-volume oracle, fp64: neighbour table of all %d voxels (%.2f s), forward of the "
                  "first %d rows (%.2f s)" % (n, t_map, rows, t_fwd),
        "map_build_s": t_map,
    }


def bench_helpers(args):
    """The coordinate-set helpers on the 256^3 noisy-sphere parent shell (32 channels
    bf16) and its 512^3 subdivision: each op's mean event time over the reps, its
    algorithmic HBM bytes (inputs read once, outputs written once) against 8 TB/s,
    and the oracle on a bounded sample of the same input."""
    import numpy as np
    import torch

    import synth
    import submanifold_sparse_convolution_submconv3d_amd as sc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sc.load_library()
    w, parent = synth.workload(5)
    c, s_el = w.cin, 2
    pc = torch.from_numpy(parent).to(dev)
    np_ = len(parent)
    pf_h, _, _ = synth.make_values(np_, c, 1, 31)
    pf = torch.from_numpy(synth.bf16_bits(pf_h).view(np.int16)).view(torch.bfloat16).to(dev)
    mask_h = (np.random.default_rng(31).random((np_, 8)) < 0.4).astype(np.uint8)
    mask = torch.from_numpy(mask_h).to(dev)
    kids, kf = sc.submconv_subdivide(pc, pf)
    nk = kids.shape[0]
    res = w.res
    reps, warm = max(3, args.steps), max(1, args.warmup)

    def timed(fn):
        for _ in range(warm):
            out = fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            out = fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.mean(ts)), out

    def rec(ms, nbytes, n_in, n_out, host_s=None, host_n=None):
        r = {"ms": ms, "voxels_in": n_in, "voxels_out": n_out, "algorithmic_bytes": nbytes,
             "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBPS,
                          "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}}
        if host_s is not None:
            r["oracle"] = {"voxels_per_s": host_n / host_s, "sample_voxels": host_n, "cores": 1,
                           "kind": "oracle (Python reference)"}
        return r

    def host_time(fn, *a):
        t0 = time.perf_counter()
        fn(*a)
        return time.perf_counter() - t0

    from oracle import reference as ref
    sample = 20000
    ops = {}
    ms, _ = timed(lambda: sc.submconv_subdivide(pc, pf))
    ops["subdivide"] = rec(ms, np_ * (16 + c * s_el) + nk * (16 + c * s_el), np_, nk,
                           host_time(ref.subdivide, parent[:sample], pf_h[:sample]), sample)
    ms, (uc, _) = timed(lambda: sc.submconv_upsample_masked(pc, pf, mask))
    nu = uc.shape[0]
    ops["upsample_masked"] = rec(ms, np_ * (16 + 8 + c * s_el) + nu * (16 + c * s_el), np_, nu,
                                 host_time(ref.upsample_masked, parent[:sample], pf_h[:sample], mask_h[:sample]),
                                 sample)
    kids_h, kf_h = kids.cpu().numpy(), pf_h.repeat(8, axis=0)
    for mode in ("max", "mean"):
        ms, (dc, _) = timed(lambda: sc.submconv_downsample(kids, kf, res, 1, mode))
        nd = dc.shape[0]
        ops["downsample_" + mode] = rec(ms, nk * (16 + c * s_el) + nd * (16 + c * s_el), nk, nd,
                                        host_time(ref.downsample, kids_h[:8 * sample], kf_h[:8 * sample], mode),
                                        8 * sample)
    ms, (cc, cf, cm) = timed(lambda: sc.submconv_space_to_depth(kids, kf, res, 1))
    ncs = cc.shape[0]
    ops["space_to_depth"] = rec(ms, nk * (16 + c * s_el) + ncs * (16 + 8 * c * s_el + 8), nk, ncs)
    ms, (bc, _) = timed(lambda: sc.submconv_depth_to_space(cc, cf, cm))
    ops["depth_to_space_masked"] = rec(ms, ncs * (16 + 8 * c * s_el + 8) + bc.shape[0] * (16 + c * s_el), ncs,
                                       bc.shape[0])
    total = sum(o["ms"] for o in ops.values())
    out = {
        "metric": "sparse helper ops on the 512^3 subdivided shell: total ms (each op's ms and HBM fraction inside)",
        "value": total, "unit": "ms", "n_gpus": 1, "steps": reps, "warmup": warm, "ms_per_step": total,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "subdiv512_c32_bf16 helpers", "parent_voxels": np_, "voxels": nk, "channels": c,
                   "upsample_mask": "seeded Bernoulli(0.4) per child slot"},
        "ops": ops,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_chain(args):
    """A decoder-like chain on one GPU: per level, build the map of the level's set, run
    its SubMConv3d layers on that one map, then subdivide (features replicated) into the
    next level; 64^3 -> 512^3, 18 layers, bf16.  Reports the whole chain's time, the
    share of it spent building maps, and the layers' throughput (voxel-layers/s and
    algorithmic TFLOP/s over present taps)."""
    import numpy as np
    import torch

    import synth
    import submanifold_sparse_convolution_submconv3d_amd as sc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sc.load_library()
    levels = synth.CHAIN_LEVELS
    c0 = synth.chain_start(levels[0][0])
    feats, layers = synth.chain_values(levels, len(c0))

    def bf(a):
        return torch.from_numpy(synth.bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x0, coords0 = bf(feats), torch.from_numpy(c0).to(dev)
    dw = [(li, bf(w), torch.from_numpy(b).to(dev)) for li, w, b in layers]
    stream = torch.cuda.current_stream()

    def chain(record):
        coords, x = coords0, x0
        ev = []
        info = []
        for li, (res, ch, convs) in enumerate(levels):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record(stream)
            rb = sc.submconv_build_map(coords, res, 1)
            e[1].record(stream)
            for lj, w, b in dw:
                if lj == li:
                    x = sc.submconv_forward(x, w, b, rb)
            e[2].record(stream)
            n, p = rb.n, rb.taps_present
            rb.free()
            if li + 1 < len(levels):
                coords, x = sc.submconv_subdivide(coords, x)
            e[3].record(stream)
            ev.append(e)
            info.append((n, p))
        torch.cuda.synchronize()
        if record:
            return [(e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])) for e in ev], info
        return None, info

    steps, warm = max(2, args.steps), max(1, args.warmup)
    for _ in range(warm):
        chain(False)
    per = []
    wall = 0.0
    for _ in range(steps):
        t0 = time.perf_counter()
        t, info = chain(True)
        wall += time.perf_counter() - t0
        per.append(t)
    per = np.array(per)  # steps x levels x (map, convs, subdivide)
    mean = per.mean(axis=0)
    total = float(mean.sum())
    vl, flops, lv = 0.0, 0.0, []
    cin = levels[0][1]
    for li, (res, ch, convs) in enumerate(levels):
        n, p = info[li]
        fl = 0.0
        for j in range(convs):
            fl += 2.0 * cin * ch * p
            cin = ch
        vl += n * convs
        flops += fl
        lv.append({"grid": "%d^3" % res, "voxels": n, "taps_present": p, "channels": ch, "convs": convs,
                   "map_build_ms": float(mean[li, 0]), "convs_ms": float(mean[li, 1]),
                   "subdivide_ms": float(mean[li, 2]), "conv_tflops": fl / (mean[li, 1] * 1e-3) / 1e12})
    conv_ms = float(mean[:, 1].sum())
    out = {
        "metric": "decoder-like chain 64^3 -> 512^3 (18 SubMConv3d, bf16): voxel-layers/s over the whole chain",
        "value": vl / (total * 1e-3), "unit": "voxel-layers/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": total, "host_ms_per_step": wall * 1e3 / steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "chain64to512_bf16", "levels": [list(l) for l in levels], "start_voxels": len(c0),
                   "weights": "LeCun-normal, seeded"},
        "chain_ms": total, "convs_ms": conv_ms, "map_build_ms": float(mean[:, 0].sum()),
        "subdivide_ms": float(mean[:, 2].sum()), "map_build_share": float(mean[:, 0].sum()) / total,
        "conv_tflops": flops / (conv_ms * 1e-3) / 1e12, "chain_tflops": flops / (total * 1e-3) / 1e12,
        "levels": lv,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_peaks(args):
    """What the box reaches on plain work, beside the vendor peaks the roofline fractions use: a device
    copy (torch's copy kernel, 1 GiB each way) and dense GEMMs (torch.matmul, 8192^3, bf16 and fp32 with
    TF32 off; the vendor's library GEMMs, not this package's code)."""
    import torch
    dev = torch.device("cuda:0")
    torch.backends.cuda.matmul.allow_tf32 = False
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    copy_ms = timed(lambda: b.copy_(a), max(args.steps, 10))
    copy_tbps = 2.0 * a.numel() * 4 / (copy_ms * 1e-3) / 1e12
    del a, b
    out = {"metric": "measured device copy and dense GEMM rates (context for the roofline peaks)",
           "copy_TBps": copy_tbps, "copy_frac_of_8TBps": copy_tbps / 8.0}
    m = 8192
    for name, dt, peak in (("bf16", torch.bfloat16, 2500.0), ("f32", torch.float32, 157.3)):
        x = torch.randn(m, m, device=dev).to(dt)
        y = torch.randn(m, m, device=dev).to(dt)
        ms = timed(lambda: torch.matmul(x, y), 5 if dt == torch.float32 else 10)
        tf = 2.0 * m ** 3 / (ms * 1e-3) / 1e12
        out["gemm_%s_TFLOPs" % name] = tf
        out["gemm_%s_frac_of_peak" % name] = tf / peak
        del x, y
    out["n_gpus"] = 1
    print(json.dumps(out), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--dtype", default=None, choices=[None, "f32", "bf16"])
    ap.add_argument("--variant", default="auto", choices=["auto", "generic", "lowc", "mfma", "window", "persistent"])
    ap.add_argument("--shuffled", action="store_true", help="seeded random row order")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the second dtype and the cold-cache pass")
    ap.add_argument("--chain", action="store_true",
                    help="time the decoder-like chain 64^3 -> 512^3 (18 convolutions) instead (own JSON line)")
    ap.add_argument("--peaks", action="store_true",
                    help="measure a device copy and dense library GEMMs instead (context; own JSON line)")
    ap.add_argument("--helpers", action="store_true",
                    help="time the coordinate-set helpers on the 512^3 subdivided shell instead (own JSON line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        return 2
    if args.peaks:
        return bench_peaks(args)
    if args.helpers:
        return bench_helpers(args)
    if args.chain:
        return bench_chain(args)

    import numpy as np
    import torch

    import synth
    import submanifold_sparse_convolution_submconv3d_amd as sc

    variant = {"auto": sc.KERNEL_AUTO, "generic": sc.KERNEL_GENERIC, "lowc": sc.KERNEL_LOWC,
               "mfma": sc.KERNEL_MFMA, "window": sc.KERNEL_WINDOW,
               "persistent": sc.KERNEL_PERSISTENT}[args.variant]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sc.load_library()
    w, coords = synth.workload(args.config)
    dtype = args.dtype or w.dtypes[0]
    subdivide_ms = None
    if w.subdivide_parent:                       # the set is the device subdivision of the parent shell
        parent = torch.from_numpy(coords).to(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kids, _ = sc.submconv_subdivide(parent)
        e1.record()
        torch.cuda.synchronize()
        subdivide_ms = e0.elapsed_time(e1)
        tc = kids
        coords = kids.cpu().numpy()
    else:
        tc = torch.from_numpy(coords).to(dev)
    n = len(coords)
    feats, weight, bias = synth.make_values(n, w.cin, w.cout, w.value_seed, w.weight_std, w.bias)
    if args.shuffled:
        p = synth.shuffle_rows(n, 1000 + args.config)
        coords, feats = np.ascontiguousarray(coords[p]), np.ascontiguousarray(feats[p])
        tc = torch.from_numpy(coords).to(dev)

    def dev_values(dt):
        if dt == "f32":
            return torch.from_numpy(feats).to(dev), torch.from_numpy(weight).to(dev)
        fb, wb = synth.bf16_bits(feats), synth.bf16_bits(weight)
        return (torch.from_numpy(fb.view(np.int16)).view(torch.bfloat16).to(dev),
                torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).to(dev).reshape(weight.shape))

    tb = torch.from_numpy(bias).to(dev)
    reps = 4 if args.config == 4 else 1
    stream = torch.cuda.current_stream()

    def gpu_busy():
        try:
            torch.cuda._sleep(200000)
        except (AttributeError, RuntimeError):
            pass

    def run(dt, steps, warmup, flush=None):
        tf, tw = dev_values(dt)
        out = torch.empty((n, w.cout), dtype=tf.dtype, device=dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3 + reps)] for _ in range(steps)]
        taps = None
        for _ in range(warmup):
            rb = sc.submconv_build_map(tc, w.res, w.batch)
            for _ in range(reps):
                sc.submconv_forward(tf, tw, tb, rb, out=out, variant=variant)
            taps = rb.taps_present
            rb.free()
        torch.cuda.synchronize()
        wall = 0.0
        for s in range(steps):
            if flush is not None:
                flush.fill_(s)                 # evict caches (outside the timed events and wall time)
                torch.cuda.synchronize()
            t0 = time.perf_counter()
            e = ev[s]
            e[0].record(stream)
            rb = sc.submconv_build_map(tc, w.res, w.batch)
            e[1].record(stream)
            # The map build ends with a host sync, so the GPU would sit idle while the host
            # enqueues the forward; a short spin kernel first keeps it busy, so the forward
            # events time the kernels rather than the launch latency.
            gpu_busy()
            e[2].record(stream)
            for r in range(reps):
                sc.submconv_forward(tf, tw, tb, rb, out=out, variant=variant)
                e[3 + r].record(stream)
            taps = rb.taps_present
            rb.free()
            torch.cuda.synchronize()
            wall += time.perf_counter() - t0
        t_map = [e[0].elapsed_time(e[1]) for e in ev]
        t_fwd = [e[2 + r].elapsed_time(e[3 + r]) for e in ev for r in range(reps)]
        step_ms = [t_map[i] + sum(t_fwd[i * reps:(i + 1) * reps]) for i in range(steps)]
        return dict(t_map=t_map, t_fwd=t_fwd, step_ms=float(np.mean(step_ms)), wall_ms=wall * 1e3 / steps, taps=taps,
                    out=out)

    torch.cuda.synchronize()
    res = run(dtype, args.steps, args.warmup)
    p = res["taps"]
    fwd_ms = float(np.mean(res["t_fwd"]))
    map_ms = float(np.mean(res["t_map"]))
    flops, abytes = algorithmic(n, p, w.cin, w.cout, dtype)
    bound = BOUND[args.config]
    if bound == "mfma":
        achieved, peak, unit = flops / (fwd_ms * 1e-3) / 1e12, PEAK_TFLOPS[dtype], "TFLOP/s"
    else:
        achieved, peak, unit = abytes / (fwd_ms * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"
    kname = "forward"
    traffic = load_traffic(w.name + ("_shuffled" if args.shuffled else ""), dtype, kname)
    rec = {
        "metric": METRIC,
        "value": n / (fwd_ms * 1e-3),
        "unit": "voxels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["step_ms"],
        "host_ms_per_step": res["wall_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "grid": "%d^3" % w.res, "batch": w.batch, "n_voxels": n, "taps_present": p,
            "cin": w.cin, "cout": w.cout, "geometry": w.note,
            "row_order": "seeded shuffle" if args.shuffled else ("parent-major subdivide" if w.subdivide_parent
                                                                   else "C order"),
            "forward_calls_per_step": reps, "kernel": args.variant,
        },
        "fwd_ms": fwd_ms,
        "fwd_ms_min": float(np.min(res["t_fwd"])),
        "fwd_tflops": flops / (fwd_ms * 1e-3) / 1e12,
        "fwd_tflops_dense27": 2.0 * w.cin * w.cout * 27 * n / (fwd_ms * 1e-3) / 1e12,
        "fwd_algorithmic_GBps": abytes / (fwd_ms * 1e-3) / 1e9,
        "map_build_ms": map_ms,
        "map_build_ms_min": float(np.min(res["t_map"])),
        "map_algorithmic_GBps": n * 124.0 / (map_ms * 1e-3) / 1e9,
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
                     "traffic": traffic, "kernel": "forward (%s)" % args.variant,
                     "per_launch": {"flops": flops, "algorithmic_bytes": abytes}},
    }
    if subdivide_ms is not None:
        rec["subdivide_ms"] = subdivide_ms
    if not args.no_extra:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB > 4x the 256 MB MALL
        cold = run(dtype, max(3, args.steps // 4), 1, flush)
        cf = float(np.mean(cold["t_fwd"]))
        rec["cold"] = {"fwd_ms": cf, "map_build_ms": float(np.mean(cold["t_map"])),
                       "voxels_per_s": n / (cf * 1e-3), "fwd_tflops": flops / (cf * 1e-3) / 1e12,
                       "fwd_algorithmic_GBps": abytes / (cf * 1e-3) / 1e9}
        del flush
        for other in w.dtypes:
            if other == dtype:
                continue
            o = run(other, args.steps, args.warmup)
            of = float(np.mean(o["t_fwd"]))
            ofl, oby = algorithmic(n, p, w.cin, w.cout, other)
            rec[other] = {"fwd_ms": of, "voxels_per_s": n / (of * 1e-3), "fwd_tflops": ofl / (of * 1e-3) / 1e12,
                          "map_build_ms": float(np.mean(o["t_map"])),
                          "roofline": {"bound": "mfma", "achieved": ofl / (of * 1e-3) / 1e12,
                                       "peak": PEAK_TFLOPS[other], "unit": "TFLOP/s",
                                       "frac": ofl / (of * 1e-3) / 1e12 / PEAK_TFLOPS[other],
                                       "hbm_frac": oby / (of * 1e-3) / 1e9 / PEAK_HBM_GBPS}}
    if args.no_cpu_baseline:
        rec["cpu_baseline"] = None
    else:
        rec["cpu_baseline"] = cpu_baseline(coords, feats, weight, bias, w.res, w.batch, args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
