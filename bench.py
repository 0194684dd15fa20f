#!/usr/bin/env python3
"""Benchmark of the submanifold 3x3x3 convolution on one MI355X.

One step = the whole path on one synthetic batch: build the neighbour map of
the coordinate set (pack, sort, resolve, the wait for its status), then run the
forward pass on it (4 forward passes reusing the map for the 4-grid workload).
Inputs are resident in device memory before the timed region starts.

Prints ONE JSON line.  The headline workload (default: the 128^3 shell at 128
channels, fp32) is timed with cold caches: 1 GiB is written between steps,
outside the timed spans, so no input is left in the 256 MB last-level cache.
`value` is forward active voxels per second (N divided by the mean forward
kernel time from HIP events on the launch stream); `ms_per_step` is the GPU
time of a whole step (map build + forward, HIP events; the map build's span
includes the host's wait for its status); `host_ms_per_step` is the host wall
time of a step, which also holds a short spin kernel that keeps the GPU busy
while the forward is enqueued.  `roofline` is taken from the same cold reps.

Unless --no-extra: warm reps of the headline, a `configs` record with every
workload (cold reps for the roofline figures, warm beside them) and the CPU
oracle legs (`cpu_baseline`).

    python bench.py [--steps K] [--warmup W] [--config 3] [--dtype f32|bf16] [--no-extra]
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
COMMON_SRCS = [os.path.join(CSRC, f) for f in ("common.h", "winplan.h")]


def kernel_sources(kernel: str):
    """The sources a forward kernel's code depends on (counter figures are valid while
    their hash is unchanged)."""
    f = "conv_win.hip" if "win32" in kernel else ("conv_big.hip" if "conv_big" in kernel else "conv.hip")
    return [os.path.join(CSRC, f)] + COMMON_SRCS
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
BOUND = {1: "hbm", 2: "mfma", 3: "mfma", 4: "mfma", 5: "hbm"}


def src_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, dtype: str, kernel: str, algorithmic_bytes: float, runs: str = ""):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    kernel that runs now (`runs`: its name without namespace or template arguments), on
    that kernel's current source and on the same input (same algorithmic bytes); else None."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = data.get("%s/%s/%s" % (workload, dtype, kernel))
    if not entry:
        return None
    recorded = entry.get("kernel", "")
    if runs and recorded.replace("sc::", "").split("<")[0] != runs.split("<")[0]:
        return None
    if (entry.get("source_hash") != src_hash(kernel_sources(recorded))
            or entry.get("algorithmic_bytes") != float(algorithmic_bytes)):
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


KERNEL_OF_VARIANT = {"auto": 0, "generic": 1, "lowc": 2, "mfma": 3, "window": 4, "persistent": 5}


def _forward_kernel(cin, cout, dtype, n):
    """Name of the kernel the automatic choice runs (for the record; the library decides)."""
    if dtype == "bf16" and cin == cout == 32 and n * 64 <= 2 ** 31 - 1:
        return "k_conv_win32"
    if dtype == "bf16" and cin == cout == 64 and n >= 2 ** 19:
        return "k_conv_mfma_rows"
    if dtype == "bf16" and cin == cout and cin in (64, 128) and n * cin * 2 <= 2 ** 31 - 1:
        return "k_conv_big<%d,%d,8>" % (cin, cout)
    if dtype == "f32" and cin == cout == 128:
        return "k_conv_mfma<float,128,128>"
    if cin in (32, 64, 128) and cout in (32, 64, 128):
        return "k_conv_mfma_rows"
    if cin == cout == 16 and n * 16 * (4 if dtype == "f32" else 2) <= 2 ** 31 - 1:
        return "k_conv_mfma16<%s>" % ("float" if dtype == "f32" else "unsigned short")
    return "k_conv_lowc" if cin <= 32 and cout <= 32 else "k_conv_generic"


class Workbench:
    """Inputs of one workload resident on the device, and the timed step (map build,
    then the forward pass(es) on it) in a warm or a cold-cache protocol."""

    def __init__(self, idx, shuffled=False):
        import numpy as np
        import torch

        import synth
        import submanifold_sparse_convolution_submconv3d_amd as sc

        self.np, self.torch, self.sc = np, torch, sc
        self.dev = torch.device("cuda:0")
        w, coords = synth.workload(idx)
        self.w, self.idx = w, idx
        self.subdivide_ms = None
        if w.subdivide_parent:                   # the set is the device subdivision of the parent shell
            parent = torch.from_numpy(coords).to(self.dev)
            ts = []
            for _ in range(4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                kids, _ = sc.submconv_subdivide(parent)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            self.subdivide_ms = float(np.mean(ts[1:]))
            coords = kids.cpu().numpy()
        n = len(coords)
        feats, weight, bias = synth.make_values(n, w.cin, w.cout, w.value_seed, w.weight_std, w.bias)
        if shuffled:
            p = synth.shuffle_rows(n, 1000 + idx)
            coords, feats = np.ascontiguousarray(coords[p]), np.ascontiguousarray(feats[p])
        self.coords, self.feats, self.weight, self.bias = coords, feats, weight, bias
        self.n = n
        self.tc = torch.from_numpy(coords).to(self.dev)
        self.tb = torch.from_numpy(bias).to(self.dev)
        self.calls = 4 if idx == 4 else 1
        self.taps = None
        self._flush = None

    def values(self, dt):
        np, torch = self.np, self.torch
        import synth
        if dt == "f32":
            return torch.from_numpy(self.feats).to(self.dev), torch.from_numpy(self.weight).to(self.dev)
        fb, wb = synth.bf16_bits(self.feats), synth.bf16_bits(self.weight)
        return (torch.from_numpy(fb.view(np.int16)).view(torch.bfloat16).to(self.dev),
                torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).to(self.dev).reshape(self.weight.shape))

    def flush(self, s):
        """Evict the caches: a 1 GiB write (4x the 256 MB MALL), outside the timed spans."""
        if self._flush is None:
            self._flush = self.torch.empty(1 << 28, dtype=self.torch.float32, device=self.dev)
        self._flush.fill_(float(s))
        self.torch.cuda.synchronize()

    def run(self, dt, steps, warmup, cold, variant=0):
        """Timed steps; returns per-step map-build ms, per-call forward ms, step ms, host ms."""
        np, torch, sc, w = self.np, self.torch, self.sc, self.w
        tf, tw = self.values(dt)
        out = torch.empty((self.n, w.cout), dtype=tf.dtype, device=self.dev)
        stream = torch.cuda.current_stream()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3 + self.calls)] for _ in range(steps)]

        def gpu_busy():
            # The map build ends with a host sync, so the GPU would sit idle while the host
            # enqueues the forward; a short spin kernel keeps it busy, so the forward's
            # events time the kernel rather than the launch latency.
            try:
                torch.cuda._sleep(200000)
            except (AttributeError, RuntimeError):
                pass

        for s in range(warmup):
            if cold:
                self.flush(s)
            rb = sc.submconv_build_map(self.tc, w.res, w.batch)
            for _ in range(self.calls):
                sc.submconv_forward(tf, tw, self.tb, rb, out=out, variant=variant)
            self.taps = rb.taps_present
            rb.free()
        torch.cuda.synchronize()
        wall = 0.0
        for s in range(steps):
            if cold:
                self.flush(s)
            t0 = time.perf_counter()
            e = ev[s]
            e[0].record(stream)
            rb = sc.submconv_build_map(self.tc, w.res, w.batch)
            e[1].record(stream)
            gpu_busy()
            e[2].record(stream)
            for r in range(self.calls):
                sc.submconv_forward(tf, tw, self.tb, rb, out=out, variant=variant)
                e[3 + r].record(stream)
            self.taps = rb.taps_present
            rb.free()
            torch.cuda.synchronize()
            wall += time.perf_counter() - t0
        t_map = [e[0].elapsed_time(e[1]) for e in ev]
        t_fwd = [e[2 + r].elapsed_time(e[3 + r]) for e in ev for r in range(self.calls)]
        step_ms = [t_map[i] + sum(t_fwd[i * self.calls:(i + 1) * self.calls]) for i in range(steps)]
        return dict(t_map=t_map, t_fwd=t_fwd, step_ms=float(np.mean(step_ms)), wall_ms=wall * 1e3 / steps)


def _fwd_roofline(wb, dt, fwd_ms, bound):
    """Roofline figures of one forward launch of mean duration fwd_ms."""
    w = wb.w
    flops, abytes = algorithmic(wb.n, wb.taps, w.cin, w.cout, dt)
    if bound == "mfma":
        ach, peak, unit = flops / (fwd_ms * 1e-3) / 1e12, PEAK_TFLOPS[dt], "TFLOP/s"
    else:
        ach, peak, unit = abytes / (fwd_ms * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"
    return ach, peak, unit, flops, abytes


def config_record(wb, dt, warm, cold):
    """One workload's figures: cold-cache reps are the roofline numbers, warm beside them."""
    np, w = wb.np, wb.w
    bound = BOUND[wb.idx]
    fc, fw = float(np.mean(cold["t_fwd"])), float(np.mean(warm["t_fwd"]))
    mc, mw = float(np.mean(cold["t_map"])), float(np.mean(warm["t_map"]))
    ach, peak, unit, flops, abytes = _fwd_roofline(wb, dt, fc, bound)
    ach_w = _fwd_roofline(wb, dt, fw, bound)[0]
    rec = {
        "workload": w.name, "dtype": dt, "n_voxels": wb.n, "taps_present": wb.taps, "cin": w.cin, "cout": w.cout,
        "kernel": _forward_kernel(w.cin, w.cout, dt, wb.n), "forward_calls_per_step": wb.calls,
        "fwd_ms": fc, "fwd_ms_warm": fw, "fwd_ms_min": float(np.min(cold["t_fwd"])),
        "voxels_per_s": wb.n / (fc * 1e-3), "voxels_per_s_warm": wb.n / (fw * 1e-3),
        "fwd_tflops": flops / (fc * 1e-3) / 1e12, "fwd_tflops_warm": flops / (fw * 1e-3) / 1e12,
        "fwd_algorithmic_GBps": abytes / (fc * 1e-3) / 1e9,
        "map_build_ms": mc, "map_build_ms_warm": mw, "map_build_ms_min": float(np.min(cold["t_map"] + warm["t_map"])),
        "map_build_hbm_frac": wb.n * 124.0 / (mc * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "map_build_hbm_frac_warm": wb.n * 124.0 / (mw * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "step_ms": cold["step_ms"], "step_ms_warm": warm["step_ms"],
        "roofline": {"bound": bound, "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
                     "frac_warm": ach_w / peak,
                     "traffic": load_traffic(w.name, dt, "forward", abytes, _forward_kernel(w.cin, w.cout, dt, wb.n)),
                     "per_launch": {"flops": flops, "algorithmic_bytes": abytes}},
    }
    if bound == "mfma":
        rec["roofline"]["hbm_frac"] = abytes / (fc * 1e-3) / 1e9 / PEAK_HBM_GBPS
    if wb.idx == 1:
        rec["roofline"]["note"] = "134 KB per launch: launch-latency bound, the HBM fraction is not meaningful"
    if wb.idx == 4:
        rec["fwd_ms_per_call"] = fc
        rec["map_plus_4_calls_ms"] = mc + 4 * fc
    if wb.subdivide_ms is not None:
        rec["subdivide_ms"] = wb.subdivide_ms
    return rec


def cpu_legs(budget_s):
    """The oracle as it stands on configs 1-3: O2 (C) single-threaded and O1 (Python
    dict + numpy), each on a bounded sample of the workload's rows."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from oracle import reference as ref
    import synth

    legs = []
    per = budget_s / 6.0
    for idx in (1, 2, 3):
        w, coords = synth.workload(idx)
        n = len(coords)
        feats, weight, bias = synth.make_values(n, w.cin, w.cout, w.value_seed, w.weight_std, w.bias)
        f64, w64 = feats.astype(np.float64), weight.astype(np.float64)
        # O2, one thread
        threads = oracle.dense.num_threads()
        oracle.dense.set_threads(1)
        try:
            t0 = time.perf_counter()
            nbr = oracle.dense.neighbor_table(coords, w.res, w.batch)
            t_map = time.perf_counter() - t0
            probe = min(n, 64)
            t0 = time.perf_counter()
            oracle.dense.forward(f64, w64, bias, nbr, rows=(0, probe))
            per_row = max((time.perf_counter() - t0) / probe, 1e-9)
            rows = int(min(n, max(probe, per / per_row)))
            t0 = time.perf_counter()
            oracle.dense.forward(f64, w64, bias, nbr, rows=(0, rows))
            t_fwd = time.perf_counter() - t0
        finally:
            oracle.dense.set_threads(threads)
        legs.append({"kind": "oracle O2 (C dense volume, fp64), 1 thread", "workload": w.name, "cores": 1,
                     "voxels_per_s": rows / t_fwd, "table_s": t_map, "sample_rows": rows, "n_voxels": n})
        # O1, Python dict + numpy per tap, numpy's BLAS held to one thread
        blas_one = threadpool_limits(limits=1)
        t0 = time.perf_counter()
        nbr1 = ref.neighbor_table(coords, w.res, w.batch)
        t_map1 = time.perf_counter() - t0
        rows1 = min(n, 256)
        t0 = time.perf_counter()
        ref.forward(f64, w64, bias, nbr1[:rows1])
        per_row1 = max((time.perf_counter() - t0) / rows1, 1e-9)
        rows1 = int(min(n, max(rows1, per / per_row1)))
        t0 = time.perf_counter()
        ref.forward(f64, w64, bias, nbr1[:rows1])
        t_fwd1 = time.perf_counter() - t0
        blas_one.restore_original_limits()
        legs.append({"kind": "oracle O1 (Python dict, numpy fp64 per tap), 1 thread", "workload": w.name,
                     "cores": 1, "voxels_per_s": rows1 / t_fwd1, "table_s": t_map1,
                     "table_lookups_per_s": 27.0 * n / t_map1, "sample_rows": rows1, "n_voxels": n})
    return legs


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--dtype", default=None, choices=[None, "f32", "bf16"])
    ap.add_argument("--variant", default="auto", choices=list(KERNEL_OF_VARIANT))
    ap.add_argument("--shuffled", action="store_true", help="seeded random row order")
    ap.add_argument("--warm", action="store_true",
                    help="time the headline without the cache flush between steps (default: cold)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="headline only: no per-workload sweep, no warm reps, no CPU legs")
    ap.add_argument("--chain", action="store_true",
                    help="time the decoder-like chain 64^3 -> 512^3 (18 convolutions) instead (own JSON line)")
    ap.add_argument("--peaks", action="store_true",
                    help="measure a device copy and dense library GEMMs instead (context; own JSON line)")
    ap.add_argument("--helpers", action="store_true",
                    help="time the coordinate-set helpers on the 512^3 subdivided shell instead (own JSON line)")
    ap.add_argument("--ingest-traffic", metavar="DIR",
                    help="host only: read rocprofv3 FETCH_SIZE / WRITE_SIZE runs under DIR into profiles/traffic.json")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        return 2
    if args.ingest_traffic:
        return ingest_traffic(args.ingest_traffic)
    if args.peaks:
        return bench_peaks(args)
    if args.helpers:
        return bench_helpers(args)
    if args.chain:
        return bench_chain(args)

    import numpy as np
    import torch

    import submanifold_sparse_convolution_submconv3d_amd as sc

    variant = KERNEL_OF_VARIANT[args.variant]
    torch.cuda.set_device(torch.device("cuda:0"))
    sc.load_library()
    wb = Workbench(args.config, args.shuffled)
    w, n = wb.w, wb.n
    dtype = args.dtype or w.dtypes[0]
    cold = not args.warm
    torch.cuda.synchronize()
    res = wb.run(dtype, args.steps, args.warmup, cold, variant)
    p = wb.taps
    fwd_ms = float(np.mean(res["t_fwd"]))
    map_ms = float(np.mean(res["t_map"]))
    bound = BOUND[args.config]
    achieved, peak, unit, flops, abytes = _fwd_roofline(wb, dtype, fwd_ms, bound)
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
            "forward_calls_per_step": wb.calls, "kernel": args.variant,
            "cache": "cold: 1 GiB written between steps, outside the timed spans" if cold else "warm",
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
                     "traffic": load_traffic(w.name + ("_shuffled" if args.shuffled else ""), dtype, "forward", abytes,
                                             _forward_kernel(w.cin, w.cout, dtype, n) if variant == 0 else "(forced)"),
                     "kernel": _forward_kernel(w.cin, w.cout, dtype, n) if variant == 0 else args.variant,
                     "kernel_ms": fwd_ms, "reps": "cold" if cold else "warm",
                     "per_launch": {"flops": flops, "algorithmic_bytes": abytes}},
    }
    if wb.subdivide_ms is not None:
        rec["subdivide_ms"] = wb.subdivide_ms
    if not args.no_extra:
        warm = wb.run(dtype, args.steps, args.warmup, not cold, variant)
        rec["warm" if cold else "cold"] = {"fwd_ms": float(np.mean(warm["t_fwd"])),
                                           "map_build_ms": float(np.mean(warm["t_map"]))}
        # every workload of the metric, cold reps for the roofline and warm beside them
        hw, hc = (warm, res) if cold else (res, warm)
        configs = {"%d_%s" % (args.config, dtype): config_record(wb, dtype, hw, hc)} if variant == 0 else {}
        steps_c, warm_c = max(5, args.steps // 2), max(1, args.warmup)
        for idx in (1, 2, 3, 4, 5):
            ob = wb if idx == args.config and not args.shuffled else Workbench(idx)
            for dt in ob.w.dtypes:
                key = "%d_%s" % (idx, dt)
                if key in configs:
                    continue
                wr = ob.run(dt, steps_c, warm_c, False)
                cr = ob.run(dt, max(3, steps_c // 2), 1, True)
                configs[key] = config_record(ob, dt, wr, cr)
            if ob is not wb:
                del ob
                torch.cuda.empty_cache()
        rec["configs"] = configs
    if args.no_cpu_baseline or args.no_extra:
        rec["cpu_baseline"] = None
    else:
        rec["cpu_baseline"] = cpu_baseline(wb.coords, wb.feats, wb.weight, wb.bias, w.res, w.batch,
                                           args.cpu_seconds)
        rec["cpu_baseline"]["legs"] = cpu_legs(args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


def ingest_traffic(root):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE of the forward kernels from rocprofv3 csv runs
    named pmc_<workload>_<dtype>_<COUNTER> (and pmc_copy_<COUNTER> for the 1 GiB copy that
    calibrates them) into profiles/traffic.json, keyed to the current kernel sources."""
    import csv
    import glob

    def per_dispatch(d, kernel_filter):
        sums = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                name = row.get("Kernel_Name", "")
                if not kernel_filter(name):
                    continue
                key = (name, row.get("Dispatch_Id"))
                sums[key] = sums.get(key, 0.0) + float(row["Counter_Value"])
        by_kernel = {}
        for (name, _), v in sums.items():
            by_kernel.setdefault(name, []).append(v)
        return {k: sum(v) / len(v) for k, v in by_kernel.items()}

    cal = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        got = per_dispatch(os.path.join(root, "pmc_copy_" + ctr), lambda k: "copyBuffer" in k)
        cal[ctr] = max(got.values())
    copy_kib = float(1 << 30) / 1024.0
    fscale, wscale = copy_kib / cal["FETCH_SIZE"], copy_kib / cal["WRITE_SIZE"]
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        data = {}
    data["_note"] = ("HBM bytes per forward launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each "
                     "scaled by what the same counter reads for a 1 GiB device copy; keyed workload/dtype/kernel; "
                     "valid while source_hash matches the kernel's source file with common.h and winplan.h, and "
                     "the workload's algorithmic bytes are unchanged.")
    data["calibration"] = {"copy_bytes": 1 << 30, "fetch_kib": cal["FETCH_SIZE"], "write_kib": cal["WRITE_SIZE"],
                           "fetch_scale": fscale, "write_scale": wscale}
    import synth
    for d in sorted(glob.glob(os.path.join(root, "pmc_*_FETCH_SIZE"))):
        tag = os.path.basename(d)[len("pmc_"):-len("_FETCH_SIZE")]
        if tag == "copy":
            continue
        wname, dt = tag.rsplit("_", 1)
        fetch = per_dispatch(d, lambda k: "sc::k_conv" in k)
        write = per_dispatch(os.path.join(root, "pmc_%s_WRITE_SIZE" % tag), lambda k: "sc::k_conv" in k)
        if not fetch:
            continue
        kfull = max(fetch, key=lambda k: fetch[k])           # the forward kernel of the run
        kname = kfull.split("(")[0].replace("void ", "")
        idx = [i for i, w in synth.WORKLOADS.items() if wname.startswith(w.name)][0]
        w, coords = synth.workload(idx)
        n = len(coords) * (8 if w.subdivide_parent else 1)
        rb, wbytes = fetch[kfull] * 1024 * fscale, write.get(kfull, 0.0) * 1024 * wscale
        s_el = 4 if dt == "f32" else 2
        data["%s/%s/forward" % (wname, dt)] = {
            "kernel": kname, "fetch_kib_raw": fetch[kfull], "write_kib_raw": write.get(kfull, 0.0),
            "read_bytes": rb, "write_bytes": wbytes, "bytes_per_launch": rb + wbytes,
            "algorithmic_bytes": float(n * (w.cin * s_el + w.cout * s_el + 108) + 27 * w.cin * w.cout * s_el
                                       + 4 * w.cout),
            "source_hash": src_hash(kernel_sources(kname))}
    json.dump(data, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps({k: (v.get("bytes_per_launch"), v.get("algorithmic_bytes")) for k, v in data.items()
                      if isinstance(v, dict) and "bytes_per_launch" in v}))
    return 0


if __name__ == "__main__":
    sys.exit(main())
