#!/usr/bin/env python3
"""Benchmark of one GDN tree-speculation layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
    gdn_tree_desc_build -> conv_ancestry_gather -> gdn_tree_verify -> gdn_tree_commit
on the 27-node-tree workload (B = 128 requests, 32 value heads over 16 qk heads,
d_k = d_v = 128, causal conv kernel 4 over 8192 channels, bf16 operands, fp32
state).  Inputs are resident in HBM before the timed region; two independent
layers' inputs (about 0.9 GB each) alternate step by step so that no step
reads data the previous step left in the 256 MB last-level cache.

Prints ONE JSON line (rank 0): metric, value = tree nodes verified per second,
per-kernel roofline of the dominant kernel (HIP events on the launch stream),
and the fp64 CPU oracle timed on the host on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree nodes verified/sec (GDN layer, 1 GPU) + achieved HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0
# file stem of the committed profile summaries for each workload
WORKLOAD_TAG = {"tree27_b128_h32_conv4": "tree27_b128_conv4"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, case):
    """Bytes each kernel must move through its interface, read once / written
    once ("Byte model")."""
    B, N, D, Hv, Hqk = case["B"], cfg.N, cfg.D, cfg.Hv, cfg.Hqk
    L = case["path_len"].astype(np.int64)
    W = max(cfg.conv_W, 1)
    C = cfg.conv_C
    out = {}
    out["desc"] = B * N * (4 + 4) + B * N * (4 + 8 + 4 * (W - 1)) + B * 4
    if cfg.conv_W > 0:
        out["conv"] = B * N * C * 2 + B * (W - 1) * C * 2 + C * W * 2 + B * N * C * 2
    else:
        out["conv"] = 0
    out["verify"] = (B * Hv * D * D * 4 + B * N * (2 * Hqk * D + Hv * D) * 2 + B * N * Hv * 8
                     + B * N * Hv * D * 4)
    active = int((L > 0).sum())
    hist_bytes = 0
    if cfg.conv_W > 1:
        hist_bytes = active * 2 * (W - 1) * C * 2 + int(np.minimum(L, W - 1).sum()) * C * 2
    out["commit"] = (active * Hv * D * D * 4 * 2 + int(L.sum()) * (Hqk * D + Hv * D) * 2
                     + int(L.sum()) * Hv * 8 + hist_bytes)
    return out


KERNEL_PREFIX = {"conv": "gdn::conv_gather_kernel", "verify": "gdn::verify_",
                 "commit": "gdn::commit_kernel", "desc": "gdn::desc_build_kernel"}


def library_source_hash():
    """sha256[:16] over the library's kernel sources and the ABI header, in
    the order the profile summaries under profiles/ record it."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "tree_speculative_verification_gdn_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    with open(os.path.join(ROOT, "include", "gdn_tree.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, stage):
    """HBM bytes per launch of ``stage``'s kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE passes, scaled by a known-size copy),
    or None when there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256_16") != library_source_hash():
        return None
    for name, k in rec["kernels"].items():
        if name.startswith(KERNEL_PREFIX[stage]):
            return int(round(k["traffic_bytes"]))
    return None


def cpu_baseline(cfg, seed, budget_s):
    """The fp64 oracle (as it stands) on the host cores, on the same workload
    (all B requests of one layer), repeated until ``budget_s`` of wall time."""
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from harness import run_oracle
    import gdn_inputs as gi
    case = gi.make_case(cfg, seed=seed, layer=0, packing="bfs")
    run_oracle(subset_first(case, 1))  # build / load outside the timing
    reps, t0 = 0, time.perf_counter()
    while True:
        run_oracle(case)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    nodes = reps * case["B"] * cfg.N
    return dict(value=nodes / el, unit="tree nodes/s", cores=oracle.threads(), kind="oracle",
                sample=f"full layer of {cfg.name} (B={case['B']}, N={cfg.N}): desc+conv+verify+commit "
                       f"in fp64, {reps} repetition(s), {el:.1f} s wall, inputs converted per call")


def subset_first(case, n):
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from harness import subset
    return subset(case, np.arange(n))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--seed", type=int, default=2026)
    ap.add_argument("--sets", type=int, default=2, help="independent layer input sets rotated per step")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain fp32 copy kernel (out = in * 1) over MIB MiB, three "
                         "times, as the known-size reference for HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build runs the path on a single MI355X; "
              "see DESIGN.md for how it would shard. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gdn_inputs as gi
    import tree_speculative_verification_gdn_amd as g

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    g.load_library()
    cfg = gi.CONFIGS[args.config]
    dev = "cuda"

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x {args.copy_calibration} MiB read + written")
        del src, dst

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    t0 = time.perf_counter()
    sets = []
    for layer in range(args.sets):
        case = gi.make_case(cfg, seed=args.seed, layer=layer, packing="bfs")
        s = dict(case=case)
        W = max(cfg.conv_W, 1)
        s["desc"] = g.TreeDesc(to_dev(case["parent"]), to_dev(case["node_row"]), cfg.R, W)
        for key in ("alpha", "beta", "pool", "state_idx", "path", "path_len"):
            s[key] = to_dev(case[key])
        B, R, D, Hv, Hqk = case["B"], cfg.R, cfg.D, cfg.Hv, cfg.Hqk
        if cfg.conv_W > 0:
            C = cfg.conv_C
            s["x"], s["hist"], s["w"] = to_dev(case["x"]), to_dev(case["hist"]), to_dev(case["w"])
            s["y"] = torch.zeros((B, R, C), dtype=torch.bfloat16, device=dev)
            s["q"] = s["y"][:, :, :Hqk * D].unflatten(-1, (Hqk, D))
            s["k"] = s["y"][:, :, Hqk * D:2 * Hqk * D].unflatten(-1, (Hqk, D))
            s["v"] = s["y"][:, :, 2 * Hqk * D:].unflatten(-1, (Hv, D))
        else:
            s["x"] = s["hist"] = None
            s["q"], s["k"], s["v"] = to_dev(case["q"]), to_dev(case["k"]), to_dev(case["v"])
        s["out"] = torch.zeros((B, R, Hv, D), dtype=torch.float32, device=dev)
        s["bytes"] = algorithmic_bytes(cfg, case)
        sets.append(s)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    flags = g.GDN_F_NORM_QK if cfg.norm_qk else 0
    torch.cuda.synchronize()
    log(f"[bench] inputs for {cfg.name} x{args.sets} ready in {time.perf_counter() - t0:.1f} s")

    names = ("desc", "conv", "verify", "commit")

    def step(s, ev=None):
        if ev is not None:
            ev[0].record()
        g.gdn_tree_desc_build(s["desc"], err)
        if ev is not None:
            ev[1].record()
        if cfg.conv_W > 0:
            g.conv_ancestry_gather(s["desc"], s["x"], s["hist"], s["state_idx"], s["w"], None,
                                   s["y"], cfg.act, err)
        if ev is not None:
            ev[2].record()
        g.gdn_tree_verify(s["desc"], s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["pool"],
                          s["state_idx"], s["out"], err, flags=flags)
        if ev is not None:
            ev[3].record()
        g.gdn_tree_commit(s["desc"], s["path"], s["path_len"], s["k"], s["v"], s["alpha"],
                          s["beta"], s["pool"], s["state_idx"], err, Hqk=cfg.Hqk,
                          flags=flags & g.GDN_F_NORM_QK, x=s["x"], hist=s["hist"])
        if ev is not None:
            ev[4].record()

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    if int(err.item()) != 0:
        log(f"[bench] device error word {int(err.item())}")
        sys.exit(3)

    per = {n: [] for n in names}
    for ev in evs:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]))
    total_ms = evs[0][0].elapsed_time(evs[-1][4])
    ms_per_step = total_ms / args.steps
    avg = {n: float(np.mean(per[n])) for n in names}
    bytes_avg = {n: float(np.mean([s["bytes"][n] for s in sets])) for n in names}
    B, N = cfg.B, cfg.N
    nodes_per_s = B * N / (ms_per_step / 1e3)
    step_bytes = sum(bytes_avg.values())
    for n in names:
        gbs = bytes_avg[n] / (avg[n] / 1e3) / 1e9 if avg[n] > 0 else 0.0
        log(f"[bench] {n:7s} {avg[n] * 1e3:9.1f} us  {bytes_avg[n] / 1e6:8.1f} MB  "
            f"{gbs:8.1f} GB/s  {gbs / PEAK_HBM_GBS * 100:5.1f}% of 8 TB/s")
    log(f"[bench] step {ms_per_step * 1e3:.1f} us (events), wall {wall / args.steps * 1e6:.1f} us, "
        f"{step_bytes / 1e6:.1f} MB -> {step_bytes / (ms_per_step / 1e3) / 1e9:.1f} GB/s")

    dom = max(("conv", "verify", "commit"), key=lambda n: avg[n])
    achieved = bytes_avg[dom] / (avg[dom] / 1e3) / 1e9
    roofline = dict(bound="hbm", kernel=dom, achieved=round(achieved, 1), peak=PEAK_HBM_GBS,
                    unit="GB/s", frac=round(achieved / PEAK_HBM_GBS, 4),
                    traffic=measured_traffic(WORKLOAD_TAG.get(cfg.name, cfg.name), dom),
                    avg_us=round(avg[dom] * 1e3, 2), algorithmic_bytes=int(bytes_avg[dom]))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.seed, args.cpu_budget)
        cpu["value"] = round(cpu["value"], 1)

    line = {
        "metric": METRIC,
        "value": round(nodes_per_s, 1),
        "unit": "tree nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {N}-node draft trees (branching<={cfg.bmax}, depth<={cfg.depth_max}), "
                        f"B={B}, Hv={cfg.Hv} over Hqk={cfg.Hqk}, d={cfg.D}, bf16 operands, fp32 state"
                        + (f", causal conv W={cfg.conv_W} C={cfg.conv_C} SiLU, q/k normalised in-kernel"
                           if cfg.conv_W else ""),
            "step": "desc_build + conv_ancestry_gather + gdn_tree_verify + gdn_tree_commit (one layer)",
            "global_batch": B,
            "nodes_per_request": N,
            "parallelism": "single GPU",
            "step_hbm_gbs": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
            "step_frac_of_peak": round(step_bytes / (ms_per_step / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "kernel_us": {n: round(avg[n] * 1e3, 2) for n in names},
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
