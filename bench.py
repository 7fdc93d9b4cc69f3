#!/usr/bin/env python3
"""Benchmark of radial block-sparse attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one forward pass of radial attention over the whole workload
(every batch and head in a single launch) with inputs already resident in
device memory; the static layout is compiled once, outside the timed region
(its host build time is reported separately).  Default workload: the
largest one that fits one GPU, the 4x longer HunyuanVideo-shaped forward
(B=1, H=24, 129 frames x 3600 tokens, N = 464,400, D = 128, 128 x 128
tiles, sink on), synthetic N(0,1) bf16 inputs.

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
  dense        -- the same kernel on an all-tiles layout (dense attention)
                  on the same workload;
  train        -- the training step (66 frames x 3600 tokens, H=24): forward,
                  backward (dQ, dK, dV from a random dO) and their total,
                  10 * D flops per kept pair for the backward (bwd_hw_frac:
                  the 14 * D per pair of matrix work its kernels issue);
  others       -- the HunyuanVideo 5 s 720p and Wan2.1 720p forwards (and
                  the 720p backward);
  token_exact  -- 720p forward and backward with token-exact masking inside
                  the partly covered tiles (same kept tiles, same flops);
  variants     -- 720p mask variants of the ablations (central band d,
                  width scale c, harmonic-series decay): their tiles,
                  density and forward/backward times.
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
# what the forward's HBM traffic depends on: the kernel and the mask
# compiler's query-tile grouping
FWD_SOURCES = ["attn_fwd.hip", "device_common.h", "kernels.h", "mask.cpp", "layout.h"]
HEADLINE = "hunyuan_4x_long"
TRAIN = "train_f66"
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


def cpu_baseline(w, layout_kept, head0, budget_s: float = 15.0):
    """The oracle (float64 numpy) on a bounded sample: query tiles of head 0
    (the same values the GPU ran, as float64 arrays [N, D]), spread evenly
    over the sequence, until about budget_s seconds."""
    import numpy as np

    from oracle import attention as oa
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    qh, kh, vh = head0
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


def leg_fwd(sba, w, L, q, k, v, o, lse, steps, warmup):
    """Forward over the whole workload: total ms per step and per-launch
    HIP-event durations (launch stream = torch's current stream, which the
    binding passes to the library)."""
    def fwd():
        sba.attn_fwd(q, k, v, L, w.scale, out=o, lse=lse)
    total_ms, per = time_launches(fwd, steps, warmup)
    return total_ms / steps, per


def leg_bwd(sba, w, L, q, k, v, o, lse, do, ws, steps, warmup):
    sba.attn_fwd(q, k, v, L, w.scale, out=o, lse=lse)

    def bwd():
        sba.attn_bwd(q, k, v, o, lse, do, L, w.scale, workspace=ws)
    total_ms, per = time_launches(bwd, steps, warmup)
    return total_ms / steps, per


def fwd_entry(w, L, ms, per):
    import numpy as np
    flops = 4 * w.D * L.nnz_pairs * w.B * w.H
    return {"ms": round(ms, 4), "median_ms": round(float(np.median(per)), 4),
            "min_ms": round(min(per), 4), "tflops": round(flops / ms / 1e9, 2),
            "frac": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4), "alg_flops": flops,
            "nnz_tiles_per_head": L.nnz_tiles,
            "tile_density": round(L.nnz_tiles / L.n_blocks ** 2, 5)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline forward only (no dense, training, 720p legs)")
    ap.add_argument("--only", choices=["fwd", "bwd", "dense", "exact", "variants", "copy"],
                    help="run only one leg on --workload (for profiler runs); prints no JSON")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
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

    if args.only == "copy":
        # calibration: a plain device copy of known size (1 GiB read + 1 GiB written)
        a = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).normal_()
        b = torch.empty_like(a)
        for _ in range(args.warmup + args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy: 1 GiB x", args.warmup + args.steps)
        return

    def setup(name, dout=False):
        w = workloads.WORKLOADS[name]
        t = time.perf_counter()
        L = sba.Layout(w.frames, w.tokens_per_frame, w.T, sink=True)
        build_ms = (time.perf_counter() - t) * 1e3
        L.upload(dev)
        log(f"workload {w.name}: N={w.N} H={w.H} D={w.D} tiles/head={L.nnz_tiles} "
            f"density={L.nnz_tiles / L.n_blocks ** 2:.4f} (layout built in {build_ms:.1f} ms)")
        ins = workloads.workload_inputs(w, with_dout=False, device=dev)
        q, k, v = ins
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        do = ws = None
        if dout:
            g = torch.Generator(dev).manual_seed(w.seed + 1000)
            do = torch.randn(q.shape, generator=g, device=dev,
                             dtype=torch.float32).to(torch.bfloat16)
            ws = torch.empty(sba.lib().radial_attn_bwd_workspace_bytes(L.handle, w.B, w.H, w.N,
                                                                         w.D),
                             dtype=torch.uint8, device=dev)
        return w, L, build_ms, q, k, v, o, lse, do, ws

    # ---- profiler legs: one leg on one workload, no JSON ------------------------
    if args.only is not None:
        need_do = args.only in ("bwd", "exact", "variants")
        w, L, _, q, k, v, o, lse, do, ws = setup(args.workload, dout=need_do)
        if args.only == "fwd":
            ms, per = leg_fwd(sba, w, L, q, k, v, o, lse, args.steps, args.warmup)
            log(f"fwd: {ms:.3f} ms/step, {fwd_entry(w, L, ms, per)['tflops']} TFLOP/s")
        elif args.only == "bwd":
            ms, _ = leg_bwd(sba, w, L, q, k, v, o, lse, do, ws, args.steps, args.warmup)
            log(f"bwd: {ms:.3f} ms/step, {10 * w.D * L.nnz_pairs * w.B * w.H / ms / 1e9:.1f} TFLOP/s")
        elif args.only == "dense":
            Ld = sba.Layout(w.frames, w.tokens_per_frame, w.T, dense=True).upload(dev)
            ms, per = leg_fwd(sba, w, Ld, q, k, v, o, lse, args.steps, args.warmup)
            log(f"dense fwd: {ms:.2f} ms")
        elif args.only == "exact":
            Lx = sba.Layout(w.frames, w.tokens_per_frame, w.T, token_exact=True).upload(dev)
            ms, _ = leg_fwd(sba, w, Lx, q, k, v, o, lse, args.steps, args.warmup)
            bms, _ = leg_bwd(sba, w, Lx, q, k, v, o, lse, do, ws, args.steps, args.warmup)
            log(f"token-exact: fwd {ms:.2f} ms, bwd {bms:.2f} ms")
        elif args.only == "variants":
            for name, kw in VARIANTS:
                Lv = sba.Layout(w.frames, w.tokens_per_frame, w.T, **kw).upload(dev)
                ms, _ = leg_fwd(sba, w, Lv, q, k, v, o, lse, args.steps, args.warmup)
                bms, _ = leg_bwd(sba, w, Lv, q, k, v, o, lse, do, ws, args.steps, args.warmup)
                log(f"variant {name}: fwd {ms:.2f} ms, bwd {bms:.2f} ms")
        return

    # ---- headline: the forward at the workload ----------------------------------
    w, L, build_ms, q, k, v, o, lse, _, _ = setup(args.workload)
    BH = w.B * w.H
    fwd_flops = 4 * w.D * L.nnz_pairs * BH
    ms, per = leg_fwd(sba, w, L, q, k, v, o, lse, args.steps, args.warmup)
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

    # head 0 of the inputs, for the CPU baseline at the end
    head0 = None if args.no_cpu_baseline else tuple(
        t[0, 0].to("cpu", torch.float64).numpy() for t in (q, k, v))
    if not args.no_extras:
        # the in-repo dense kernel on the same inputs
        Ld = sba.Layout(w.frames, w.tokens_per_frame, w.T, dense=True).upload(dev)
        dms, dper = leg_fwd(sba, w, Ld, q, k, v, o, lse, 2, 1)
        dflops = 4 * w.D * Ld.nnz_pairs * BH
        log(f"dense fwd: {dms:.2f} ms, {dflops / dms / 1e9:.1f} TFLOP/s")
        result["dense"] = {"ms": round(dms, 3), "tflops": round(dflops / dms / 1e9, 2),
                           "speedup_radial_vs_dense": round(dms / ms, 3),
                           "frac": round(dflops / dms / 1e9 / PEAK_BF16_TFLOPS, 4)}
        del Ld
    del q, k, v, o, lse
    torch.cuda.empty_cache()

    if not args.no_extras and args.workload != TRAIN:
        # the training step: forward + backward
        tw, tL, _, q, k, v, o, lse, do, ws = setup(TRAIN, dout=True)
        fms, fper = leg_fwd(sba, tw, tL, q, k, v, o, lse, 5, 1)
        bms, bper = leg_bwd(sba, tw, tL, q, k, v, o, lse, do, ws, 3, 1)
        tpairs = tL.nnz_pairs * tw.B * tw.H
        ff, bf = 4 * tw.D * tpairs, 10 * tw.D * tpairs
        log(f"train {tw.name}: fwd {fms:.2f} ms, bwd {bms:.2f} ms, total {fms + bms:.2f} ms "
            f"({(ff + bf) / (fms + bms) / 1e9:.0f} TFLOP/s)")
        result["train"] = {
            "workload": tw.desc, "name": tw.name, "N": tw.N, "H": tw.H,
            "nnz_tiles_per_head": tL.nnz_tiles,
            "fwd_ms": round(fms, 3), "bwd_ms": round(bms, 3), "fwd_plus_bwd_ms": round(fms + bms, 3),
            "fwd_tflops": round(ff / fms / 1e9, 2), "bwd_tflops": round(bf / bms / 1e9, 2),
            "total_tflops": round((ff + bf) / (fms + bms) / 1e9, 2),
            "fwd_frac": round(ff / fms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "bwd_frac": round(bf / bms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "total_frac": round((ff + bf) / (fms + bms) / 1e9 / PEAK_BF16_TFLOPS, 4),
            "fwd_alg_flops": ff, "bwd_alg_flops": bf,
            "bwd_flop_convention": "10 * D per kept token pair (4 * D forward)",
            # the matrix work the backward kernels issue: S and dP are computed
            # in both the dK/dV and the dQ kernel (8 D + 6 D per kept pair)
            "bwd_hw_frac": round(14 * tw.D * tpairs / bms / 1e9 / PEAK_BF16_TFLOPS, 4)}
        del q, k, v, o, lse, do, ws
        torch.cuda.empty_cache()

    if not args.no_extras:
        others = {}
        for name in ("hunyuan_5s_720p", "wan21_720p"):
            if name == args.workload:
                continue
            ow, oL, _, q, k, v, o, lse, do, ws = setup(name, dout=name == "hunyuan_5s_720p")
            oms, oper = leg_fwd(sba, ow, oL, q, k, v, o, lse, 5, 1)
            others[name] = fwd_entry(ow, oL, oms, oper)
            log(f"{name} fwd: {oms:.2f} ms, {others[name]['tflops']} TFLOP/s")
            if name != "hunyuan_5s_720p":
                continue
            # the 720p backward, token-exact masking and the mask variants
            bflops = 10 * ow.D * oL.nnz_pairs * ow.B * ow.H
            bms, _ = leg_bwd(sba, ow, oL, q, k, v, o, lse, do, ws, 3, 1)
            others[name]["bwd_ms"] = round(bms, 3)
            others[name]["bwd_tflops"] = round(bflops / bms / 1e9, 2)
            log(f"{name} bwd: {bms:.2f} ms")
            Lx = sba.Layout(ow.frames, ow.tokens_per_frame, ow.T, token_exact=True).upload(dev)
            n_full = int(Lx.tile_flags()[0].sum())
            xf, _ = leg_fwd(sba, ow, Lx, q, k, v, o, lse, 2, 1)
            xb, _ = leg_bwd(sba, ow, Lx, q, k, v, o, lse, do, ws, 2, 1)
            log(f"token-exact {name}: fwd {xf:.2f} ms, bwd {xb:.2f} ms "
                f"({n_full} of {Lx.nnz_tiles} kept tiles full)")
            result["token_exact"] = {
                "workload": name, "fwd_ms": round(xf, 3), "bwd_ms": round(xb, 3),
                "fwd_overhead_vs_tile_mode": round(xf / oms - 1, 4),
                "bwd_overhead_vs_tile_mode": round(xb / bms - 1, 4),
                "full_tile_fraction": round(n_full / Lx.nnz_tiles, 4)}
            del Lx
            rows = []
            for vname, kw in VARIANTS:
                Lv = sba.Layout(ow.frames, ow.tokens_per_frame, ow.T, sink=True, **kw).upload(dev)
                vf = 4 * ow.D * Lv.nnz_pairs * ow.B * ow.H
                vb = 10 * ow.D * Lv.nnz_pairs * ow.B * ow.H
                f_ms, _ = leg_fwd(sba, ow, Lv, q, k, v, o, lse, 2, 1)
                b_ms, _ = leg_bwd(sba, ow, Lv, q, k, v, o, lse, do, ws, 2, 1)
                dens = Lv.nnz_tiles / Lv.n_blocks ** 2
                log(f"variant {vname}: tiles {Lv.nnz_tiles} (density {dens:.4f}), fwd {f_ms:.2f} "
                    f"ms ({vf / f_ms / 1e9:.0f} TFLOP/s), bwd {b_ms:.2f} ms "
                    f"({vb / b_ms / 1e9:.0f} TFLOP/s)")
                rows.append({"variant": vname, "nnz_tiles_per_head": Lv.nnz_tiles,
                             "tile_density": round(dens, 5), "fwd_ms": round(f_ms, 3),
                             "fwd_tflops": round(vf / f_ms / 1e9, 2), "bwd_ms": round(b_ms, 3),
                             "bwd_tflops": round(vb / b_ms / 1e9, 2)})
                del Lv
            result["variants"] = {"workload": name, "rows": rows}
            del q, k, v, o, lse, do, ws
            torch.cuda.empty_cache()
        result["others"] = others

    if not args.no_cpu_baseline:
        from oracle import mask as om
        log("cpu baseline (oracle) ...")
        t = time.perf_counter()
        kept = om.kept_tiles(w.frames, w.tokens_per_frame, w.T, True)
        oracle_mask_s = time.perf_counter() - t
        result["cpu_baseline"] = cpu_baseline(w, kept, head0)
        result["cpu_baseline"]["oracle_mask_build_s"] = round(oracle_mask_s, 3)
        log("cpu baseline:", result["cpu_baseline"]["sample"])
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
