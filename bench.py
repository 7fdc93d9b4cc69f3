#!/usr/bin/env python3
"""Benchmark of radial block-sparse attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one forward pass of radial attention over the whole workload
(every batch and head in a single launch) with inputs already resident in
device memory; the static layout is compiled once, outside the timed region
(its host build time is reported separately).  Default workload: the
HunyuanVideo-shaped 5 s 720p forward (B=1, H=24, 33 frames x 3600 tokens,
N = 118,800, D = 128, 128 x 128 tiles, sink on), synthetic N(0,1) bf16
inputs.

Prints one JSON line on stdout.  `value` is the effective throughput over
the kept (nonzero) tiles: 4 * D flops per kept token pair, per batch and
head, divided by the measured step time.  Extra objects:
  roofline     -- the forward kernel against the MI355X dense bf16 MFMA peak
                  (2.5 PFLOP/s), timed per launch with HIP events on the
                  launch stream; `traffic` is HBM bytes per launch from
                  rocprofv3 counters committed under profiles/ (null if the
                  kernel source changed since they were taken);
  cpu_baseline -- the CPU oracle (float64 numpy) on a bounded sample of the
                  same workload, scaled to the same unit;
  dense        -- the same kernel on an all-tiles layout (dense attention);
  bwd          -- the backward pass (dQ, dK, dV) on the same workload;
  token_exact  -- forward and backward with token-exact masking inside the
                  partly covered tiles (same kept tiles, same flop count);
  variants     -- the mask variants of the ablations (central band d, width
                  scale c, harmonic-series decay) on the same workload:
                  their tiles, density and forward/backward times.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "radial attn fwd latency (ms) + effective TFLOP/s on nonzero tiles vs bf16 peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
FWD_SOURCES = ["attn_fwd.hip", "device_common.h", "kernels.h"]
# mask variants of the ablations (central band d, width scale c, decay)
VARIANTS = [("d=0", dict(central_band=0)), ("d=2", dict(central_band=2)),
            ("c=1.5", dict(width_scale=(3, 2))), ("c=3", dict(width_scale=(3, 1))),
            ("c=4", dict(width_scale=(4, 1))), ("harmonic", dict(decay="harmonic"))]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "static_block_sparse_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic(workload: str):
    """HBM bytes per forward launch from the committed counter summary, or
    None when it is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"radial_fwd_kernel_{workload}_hbm.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_hash(FWD_SOURCES):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_launches(fn, steps: int, warmup: int):
    """Run fn warmup + steps times on the current stream.  Returns the total
    time of the timed steps (ms) and the per-launch event durations (ms)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1), [a.elapsed_time(b) for a, b in evs]


def cpu_baseline(w, layout_kept, budget_s: float = 15.0):
    """The oracle (float64 numpy) on a bounded sample: query tiles of head 0,
    spread evenly over the sequence, until about budget_s seconds."""
    import numpy as np
    import torch

    import workloads
    from oracle import attention as oa
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    q, k, v = workloads.workload_inputs(w, with_dout=False, heads=[0])
    qh, kh, vh = (t[0, 0].to(torch.float64).numpy() for t in (q, k, v))
    nb = layout_kept.shape[0]
    sizes = np.full(nb, w.T)
    sizes[-1] = w.N - (nb - 1) * w.T
    t_start = time.perf_counter()
    order = list(range(0, nb, max(1, nb // 512)))
    done, pairs = 0, 0
    for u in order:
        oa.fwd_tile(qh, kh, vh, layout_kept, w.T, w.scale, u)
        pairs += int(sizes[u] * (layout_kept[u] * sizes).sum())
        done += 1
        if time.perf_counter() - t_start > budget_s:
            break
    secs = time.perf_counter() - t_start
    flops = 4 * w.D * pairs
    per_head_pairs = int(sizes @ layout_kept.astype(np.int64) @ sizes)
    full_est = secs * (per_head_pairs * w.B * w.H) / pairs
    return {
        "value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": f"float64 numpy oracle forward, head 0 of {w.H}, {done} of {nb} query tiles "
                  f"(evenly spaced), {secs:.1f} s measured; full workload extrapolated "
                  f"{full_est:.0f} s on {threads} threads",
        "seconds_measured": round(secs, 2), "full_workload_seconds_extrapolated": round(full_est, 1),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="hunyuan_5s_720p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the dense and backward legs")
    ap.add_argument("--only", choices=["fwd", "bwd", "dense", "exact", "variants", "copy"],
                    help="run only one leg (for profiler runs); prints no JSON")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(heads would shard across GPUs with no exchange between them)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import static_block_sparse_amd as sba
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = workloads.WORKLOADS[args.workload]
    BH = w.B * w.H

    if args.only == "copy":
        # calibration: a plain device copy of known size (1 GiB read + 1 GiB written)
        a = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).normal_()
        b = torch.empty_like(a)
        for _ in range(args.warmup + args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy: 1 GiB x", args.warmup + args.steps)
        return

    t = time.perf_counter()
    L = sba.Layout(w.frames, w.tokens_per_frame, w.T, sink=True)
    build_ms = (time.perf_counter() - t) * 1e3
    L.upload(dev)
    log(f"workload {w.name}: N={w.N} H={w.H} D={w.D} tiles/head={L.nnz_tiles} "
        f"density={L.nnz_tiles / L.n_blocks ** 2:.4f} (layout built in {build_ms:.1f} ms)")
    q, k, v = workloads.workload_inputs(w, with_dout=False, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    fwd_flops = 4 * w.D * L.nnz_pairs * BH

    def fwd():
        sba.attn_fwd(q, k, v, L, w.scale, out=o, lse=lse)

    result = None
    if args.only in (None, "fwd"):
        total_ms, per = time_launches(fwd, args.steps, args.warmup)
        ms = total_ms / args.steps
        launch_ms = float(np.mean(per))
        log(f"fwd: {ms:.3f} ms/step, {fwd_flops / ms / 1e9:.1f} TFLOP/s "
            f"(launch avg {launch_ms:.3f} ms, min {min(per):.3f})")
        achieved = fwd_flops / (launch_ms / 1e3) / 1e12
        traffic = read_traffic(w.name)
        result = {
            "metric": METRIC,
            "value": round(fwd_flops / (ms / 1e3) / 1e12, 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": w.desc, "name": w.name, "B": w.B, "H": w.H, "frames": w.frames,
                       "tokens_per_frame": w.tokens_per_frame, "N": w.N, "D": w.D, "tile": w.T,
                       "sink": True, "nnz_tiles_per_head": L.nnz_tiles,
                       "tile_density": round(L.nnz_tiles / L.n_blocks ** 2, 5),
                       "kept_pairs_per_head": L.nnz_pairs},
            "fwd_latency_ms": round(ms, 4),
            "fwd_latency_min_ms": round(min(per), 4),
            "fwd_latency_median_ms": round(float(np.median(per)), 4),
            "roofline": {"bound": "mfma", "kernel": "radial_fwd_kernel<128,128>",
                         "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic, "traffic_unit": "bytes per launch (HBM side)",
                         "alg_flops_per_launch": fwd_flops, "avg_launch_ms": round(launch_ms, 4)},
            "mask_build_ms": round(build_ms, 2),
        }

    if args.only in (None, "dense") and not args.no_extras:
        Ld = sba.Layout(w.frames, w.tokens_per_frame, w.T, dense=True)
        Ld.upload(dev)
        dflops = 4 * w.D * Ld.nnz_pairs * BH

        def dfwd():
            sba.attn_fwd(q, k, v, Ld, w.scale, out=o, lse=lse)

        st = 2 if args.only is None else args.steps
        total_ms, per = time_launches(dfwd, st, 1)
        dms = total_ms / st
        log(f"dense fwd: {dms:.2f} ms, {dflops / dms / 1e9:.1f} TFLOP/s")
        if result is not None:
            result["dense"] = {"ms": round(dms, 3), "tflops": round(dflops / dms / 1e9, 2),
                               "speedup_radial_vs_dense": round(dms / result["ms_per_step"], 3),
                               "frac": round(dflops / dms / 1e9 / PEAK_BF16_TFLOPS, 4)}
        del Ld

    bflops = 10 * w.D * L.nnz_pairs * BH
    do = ws = None
    if args.only in (None, "bwd", "exact", "variants") and not args.no_extras:
        g = torch.Generator(dev).manual_seed(w.seed + 1000)
        do = torch.randn(q.shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        ws = torch.empty(sba.lib().radial_attn_bwd_workspace_bytes(L.handle, w.B, w.H, w.N, w.D),
                         dtype=torch.uint8, device=dev)

    if args.only in (None, "bwd") and not args.no_extras:
        fwd()

        def bwd():
            sba.attn_bwd(q, k, v, o, lse, do, L, w.scale, workspace=ws)

        st = 3 if args.only is None else args.steps
        total_ms, per = time_launches(bwd, st, 1)
        bms = total_ms / st
        log(f"bwd: {bms:.2f} ms, {bflops / bms / 1e9:.1f} TFLOP/s")
        if result is not None:
            result["bwd"] = {"ms": round(bms, 3), "tflops": round(bflops / bms / 1e9, 2),
                             "frac": round(bflops / bms / 1e9 / PEAK_BF16_TFLOPS, 4),
                             "fwd_plus_bwd_ms": round(bms + result["ms_per_step"], 3),
                             "alg_flops": bflops}

    if args.only in (None, "exact") and not args.no_extras:
        Lx = sba.Layout(w.frames, w.tokens_per_frame, w.T, sink=True, token_exact=True)
        Lx.upload(dev)
        n_full = int(Lx.tile_flags()[0].sum())

        def xfwd():
            sba.attn_fwd(q, k, v, Lx, w.scale, out=o, lse=lse)

        def xbwd():
            sba.attn_bwd(q, k, v, o, lse, do, Lx, w.scale, workspace=ws)

        st = 2 if args.only is None else args.steps
        total_ms, _ = time_launches(xfwd, st, 1)
        xf = total_ms / st
        xfwd()
        total_ms, _ = time_launches(xbwd, st, 1)
        xb = total_ms / st
        log(f"token-exact: fwd {xf:.2f} ms, bwd {xb:.2f} ms "
            f"({n_full} of {Lx.nnz_tiles} kept tiles full)")
        if result is not None:
            result["token_exact"] = {
                "fwd_ms": round(xf, 3), "bwd_ms": round(xb, 3),
                "fwd_tflops": round(fwd_flops / xf / 1e9, 2),
                "bwd_tflops": round(bflops / xb / 1e9, 2),
                "fwd_overhead_vs_tile_mode": round(xf / result["ms_per_step"] - 1, 4),
                "full_tile_fraction": round(n_full / Lx.nnz_tiles, 4)}
            if "bwd" in result:
                result["token_exact"]["bwd_overhead_vs_tile_mode"] = round(
                    xb / result["bwd"]["ms"] - 1, 4)
        del Lx

    if args.only in (None, "variants") and not args.no_extras:
        rows = []
        st = 2 if args.only is None else args.steps
        for name, kw in VARIANTS:
            Lv = sba.Layout(w.frames, w.tokens_per_frame, w.T, sink=True, **kw)
            Lv.upload(dev)
            vf = 4 * w.D * Lv.nnz_pairs * BH
            vb = 10 * w.D * Lv.nnz_pairs * BH

            def vfwd():
                sba.attn_fwd(q, k, v, Lv, w.scale, out=o, lse=lse)

            def vbwd():
                sba.attn_bwd(q, k, v, o, lse, do, Lv, w.scale, workspace=ws)

            total_ms, _ = time_launches(vfwd, st, 1)
            f_ms = total_ms / st
            vfwd()
            total_ms, _ = time_launches(vbwd, st, 1)
            b_ms = total_ms / st
            dens = Lv.nnz_tiles / Lv.n_blocks ** 2
            log(f"variant {name}: tiles {Lv.nnz_tiles} (density {dens:.4f}), fwd {f_ms:.2f} ms "
                f"({vf / f_ms / 1e9:.0f} TFLOP/s), bwd {b_ms:.2f} ms ({vb / b_ms / 1e9:.0f} TFLOP/s)")
            rows.append({"variant": name, "nnz_tiles_per_head": Lv.nnz_tiles,
                         "tile_density": round(dens, 5), "fwd_ms": round(f_ms, 3),
                         "fwd_tflops": round(vf / f_ms / 1e9, 2), "bwd_ms": round(b_ms, 3),
                         "bwd_tflops": round(vb / b_ms / 1e9, 2)})
            del Lv
        if result is not None:
            result["variants"] = rows

    if result is None:
        return
    if not args.no_cpu_baseline:
        from oracle import mask as om
        log("cpu baseline (oracle) ...")
        t = time.perf_counter()
        kept = om.kept_tiles(w.frames, w.tokens_per_frame, w.T, True)
        oracle_mask_s = time.perf_counter() - t
        result["cpu_baseline"] = cpu_baseline(w, kept)
        result["cpu_baseline"]["oracle_mask_build_s"] = round(oracle_mask_s, 3)
        log("cpu baseline:", result["cpu_baseline"]["sample"])
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
