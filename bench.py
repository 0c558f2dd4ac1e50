#!/usr/bin/env python3
"""Benchmark of one GDN tree-speculation layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input on
the 27-node-tree workload (B = 128 requests, 32 value heads over 16 qk heads,
d_k = d_v = 128, causal conv kernel 4 over 8192 channels, bf16 operands, fp32
state): the descriptor build, the ancestry-gathered conv, the tree verify, the
commit of an accepted path into the state and the conv-history publication.

Three step shapes (``--mode``):
  layer     (default) the steady-state decode step in one launch per layer:
              gdn_step_prepare -> gdn_layer_step
            (the first once per step for all layers: the new tree's
            descriptor and the previous path's rows); the layer step
            commits the previous step's accepted path, publishes its conv
            history into the other of two history buffers, and convolves and
            verifies the new tree: the state is read once and written once,
            the conv output never goes to memory.
  fused     the same step in two launches per layer:
              gdn_step_prepare -> conv_ancestry_gather_publish ->
              gdn_tree_commit_verify
            (the conv output goes to memory and is read back).
  separate  gdn_tree_desc_build -> conv_ancestry_gather -> gdn_tree_verify
            -> gdn_tree_commit (this step's own path), the state read twice.
  factored  the stored-U form: gdn_step_prepare -> conv_ancestry_gather_publish
            -> gdn_tree_verify_store_u -> gdn_tree_commit_factored (this
            step's own path, from the corrections the verify stored; its conv
            history published by the next step's conv).
All four commit one path and verify one tree per step.

Before the W warm-up steps the step runs back to back for --settle-ms
(300 ms by default) so that the GPU's clocks are at their steady state, as
in a decode loop that runs continuously.  Inputs are resident in HBM before
the timed region.  Two independent layer
instances (pool, history, weights, about 0.5 GB each with their step data)
alternate step by step, so no step reads data the previous step left in the
256 MB last-level cache; in fused mode each instance alternates between two
step slots, the previous step's slot supplying the path and its recorded
operands.

Prints ONE JSON line: metric, value = tree nodes verified per second, the
roofline of the dominant kernel (HIP events on the launch stream) and the
fp64 CPU oracle timed on the host on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
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
KERNEL_PREFIX = {"conv": "gdn::conv_gather_kernel", "verify": "gdn::verify_",
                 "commit": "gdn::commit_kernel", "desc": "gdn::desc_build_kernel",
                 "commit_verify": "gdn::verify_", "prepare": "gdn::step_prepare_kernel",
                 "layer": "gdn::verify_", "verify_u": "gdn::verify_",
                 "commit_factored": "gdn::commit_factored_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# byte model: what the method must move (read once, written once), per the
# survey's measurement section: the state read once per step (by verify, or
# by the fused kernels that verify from it) and written for requests with an
# accepted path; q/k/v counted once as the conv input x when the conv feeds
# them (the conv output y is never credited, whichever kernel reads or writes
# it); outputs, gates, the accepted path's k/v rows and gates, the conv
# history read and written, the weights and the accepted rows' conv inputs
# that enter the history.  Re-reads, padding rows and cache effects are
# never credited.
# --------------------------------------------------------------------------

def _common(cfg, case):
    return case["B"], cfg.N, cfg.D, cfg.Hv, cfg.Hqk, max(cfg.conv_W, 1), cfg.conv_C


def bytes_desc(cfg, case):
    B, N, D, Hv, Hqk, W, C = _common(cfg, case)
    return B * N * (4 + 4) + B * N * (4 + 8 + 4 * (W - 1)) + B * 4


def bytes_resolve(cfg, prev):
    """Path validation: path ids and length in, parents and rows of the path
    nodes, the slots for the duplicate check; rows and counts out."""
    B, Lmax = prev["path"].shape
    return B * Lmax * (4 + 4 + 4 + 4) + B * (4 + 4 + 4 + 4)


def bytes_conv(cfg, case, path_case):
    """x rows of the tree, the history read and written, the weights, and the
    conv inputs of the accepted path's rows that enter the history."""
    B, N, D, Hv, Hqk, W, C = _common(cfg, case)
    if cfg.conv_W == 0:
        return 0
    L = path_case["path_len"].astype(np.int64)
    return (B * N * C * 2 + B * (W - 1) * C * 2 * 2 + C * W * 2
            + int(np.minimum(L, W - 1).sum()) * C * 2)


def bytes_verify_io(cfg, case):
    """Verify's bytes besides the state: q/k/v (unless the conv produced
    them), gates and outputs."""
    B, N, D, Hv, Hqk, W, C = _common(cfg, case)
    qkv = 0 if cfg.conv_W > 0 else B * N * (2 * Hqk * D + Hv * D) * 2
    return qkv + B * N * Hv * 8 + B * N * Hv * D * 4


def bytes_commit_parts(cfg, case):
    """(state bytes of one pass over the committed requests' states, the
    accepted path's k/v rows and gates)."""
    B, N, D, Hv, Hqk, W, C = _common(cfg, case)
    L = case["path_len"].astype(np.int64)
    active = int((L > 0).sum())
    return active * Hv * D * D * 4, int(L.sum()) * ((Hqk * D + Hv * D) * 2 + Hv * 8)


def byte_model(cfg, cur, prev, mode):
    """Algorithmic bytes per launch of each kernel of one step."""
    B, N, D, Hv, Hqk, W, C = _common(cfg, cur)
    state = B * Hv * D * D * 4
    if mode in ("fused", "layer"):
        # the step commits prev's path and verifies cur's tree from that state
        sw, path = bytes_commit_parts(cfg, prev)
        commit_verify = state + sw + bytes_verify_io(cfg, cur) + path
        conv = bytes_conv(cfg, cur, prev)
        prep = bytes_desc(cfg, cur) + bytes_resolve(cfg, prev)
        if mode == "layer":
            return {"prepare": prep, "layer": commit_verify + conv}
        out = {"prepare": prep}
        if cfg.conv_W > 0:
            out["conv"] = conv
        out["commit_verify"] = commit_verify
        return out
    if mode == "factored":
        # verify also writes every node's correction u (fp32, node rows); the
        # commit reads the state, the path's k rows, u rows and decays, and
        # writes the state
        sw, _ = bytes_commit_parts(cfg, cur)
        L = int(cur["path_len"].astype(np.int64).sum())
        out = {"prepare": bytes_desc(cfg, cur) + bytes_resolve(cfg, prev)}
        if cfg.conv_W > 0:
            out["conv"] = bytes_conv(cfg, cur, prev)
        out["verify_u"] = state + bytes_verify_io(cfg, cur) + B * N * Hv * D * 4
        out["commit_factored"] = 2 * sw + L * (Hqk * D * 2 + Hv * D * 4 + Hv * 4)
        return out
    # separate calls: this step's own path; verify and commit each pass over the state
    sw, path = bytes_commit_parts(cfg, cur)
    out = {"desc": bytes_desc(cfg, cur)}
    if cfg.conv_W > 0:
        out["conv"] = bytes_conv(cfg, cur, cur)
    out["verify"] = state + bytes_verify_io(cfg, cur)
    out["commit"] = 2 * sw + path
    return out


# --------------------------------------------------------------------------
# measured traffic from the committed counter summaries
# --------------------------------------------------------------------------

ATTN_SOURCES = ("tree_attention.hip", "gdn_internal.h")


def library_source_hash(scope="gdn"):
    """sha256[:16] over the kernel sources a workload's kernels are built
    from, the value its counter summary under profiles/ records: the tree
    attention's file and the shared header for scope "attention", every
    other csrc/*.hip and csrc/*.h for scope "gdn" (documentation of the ABI
    header does not invalidate either)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "tree_speculative_verification_gdn_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if not f.endswith((".hip", ".h")):
            continue
        if scope == "attention" and f not in ATTN_SOURCES:
            continue
        if scope == "gdn" and f == "tree_attention.hip":
            continue
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _scope(workload):
    return "attention" if "attention" in workload or "ctx" in workload else "gdn"


def measured_traffic_sum(workload, mode, prefix):
    """HBM bytes of one call of every kernel whose name starts with ``prefix``
    (summed), from the committed counter summary, or None (as below)."""
    path = os.path.join(ROOT, "profiles", f"{workload}_{mode}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256_16") != library_source_hash(_scope(workload)):
        return None
    tot = [k["traffic_bytes"] for name, k in rec["kernels"].items() if name.startswith(prefix)]
    return int(round(sum(tot))) if tot else None


def measured_traffic(workload, mode, stage):
    """HBM bytes per launch of ``stage``'s kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE passes, scaled by a known-size copy),
    or None when there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_{mode}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256_16") != library_source_hash(_scope(workload)):
        return None
    for name, k in rec["kernels"].items():
        if name.startswith(KERNEL_PREFIX[stage]):
            return int(round(k["traffic_bytes"]))
    return None


# --------------------------------------------------------------------------
# CPU baseline: the oracle as it stands
# --------------------------------------------------------------------------

def cpu_baseline(cfg, seed, budget_s, B=None):
    """The fp64 oracle on the host cores, on the same workload (all B
    requests of one layer, or the first ``B`` of them: desc, conv, verify,
    commit), repeated until ``budget_s`` of wall time."""
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from harness import run_oracle, subset
    import gdn_inputs as gi
    case = gi.make_case(cfg, seed=seed, layer=0, packing="bfs", B=B)
    run_oracle(subset(case, np.arange(1)))  # build / load outside the timing
    reps, t0 = 0, time.perf_counter()
    while True:
        run_oracle(case)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    nodes = reps * case["B"] * cfg.N
    cores = oracle.threads()
    out = dict(value=nodes / el, unit="tree nodes/s", cores=cores, kind="oracle",
               sample=f"{'full layer' if case['B'] == cfg.B else 'one layer, first %d requests,' % case['B']} "
                      f"of {cfg.name} (B={case['B']}, N={cfg.N}): "
                      f"{'desc+conv+verify+commit' if cfg.conv_W else 'desc+verify+commit'} "
                      f"in fp64, {reps} repetition(s), {el:.1f} s wall, inputs converted per call",
               cpu_model=cpu_model())
    # the same oracle on one thread, over the first requests of the layer
    # (a bounded sample: about a sixteenth of the layer, repeated up to half
    # the budget)
    nb = max(1, case["B"] // 16)
    sub = subset(case, np.arange(nb))
    oracle.set_threads(1)
    try:
        reps1, t1 = 0, time.perf_counter()
        while True:
            run_oracle(sub)
            reps1 += 1
            el1 = time.perf_counter() - t1
            if el1 >= budget_s / 2 or reps1 >= 50:
                break
    finally:
        oracle.set_threads(cores)
    out["single_thread"] = dict(
        value=round(reps1 * nb * cfg.N / el1, 1), unit="tree nodes/s", cores=1,
        sample=f"first {nb} request(s) of the same layer, {reps1} repetition(s), {el1:.1f} s wall")
    return out


def cpu_model():
    """The host CPU's model name (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def settle(step_fn, ms, torch):
    """Run the step back to back for ``ms`` of wall time before the warm-up
    steps and return how many ran.  After idle this GPU runs the first
    100-200 steps of the conv-fed workload 6-19% slower than in steady state
    (its clocks and power settle over tens of ms under load); a decode loop
    runs continuously, so the timed steps are taken at the steady state."""
    if ms <= 0:
        return 0
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(16):
            step_fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def stream_ceiling(torch, dev, mib=1024, reps=20):
    """A measured streaming ceiling for read-modify-write traffic: an
    in-place fp32 scale (x *= 0.5, then x *= 2, exact) over ``mib`` MiB, far
    larger than the 256 MB last-level cache, timed with HIP events on the
    current stream after 5 untimed passes.  Returns GB/s counting each pass's
    read and write of the buffer."""
    x = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    for i in range(5):
        x.mul_(0.5 if i % 2 == 0 else 2.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        x.mul_(0.5 if i % 2 == 0 else 2.0)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x
    return 2.0 * mib * (1 << 20) / (ms / 1e3) / 1e9


def spread(xs):
    """[p10, median, p90] of a list of durations in ms, as us."""
    return [round(float(v) * 1e3, 2) for v in np.percentile(np.asarray(xs), [10, 50, 90])]


# --------------------------------------------------------------------------
# device inputs
# --------------------------------------------------------------------------

class Slot:
    """One step's data of one layer instance: tree, rows, operands, path."""

    def __init__(self, g, cfg, case, to_dev, dev, torch):
        W = max(cfg.conv_W, 1)
        self.case = case
        self.desc = g.TreeDesc(to_dev(case["parent"]), to_dev(case["node_row"]), cfg.R, W)
        for key in ("alpha", "beta", "path", "path_len"):
            setattr(self, key, to_dev(case[key]))
        B, R, D, Hv, Hqk = case["B"], cfg.R, cfg.D, cfg.Hv, cfg.Hqk
        if cfg.conv_W > 0:
            C = cfg.conv_C
            self.x = to_dev(case["x"])
            self.y = torch.zeros((B, R, C), dtype=torch.bfloat16, device=dev)
            self.q = self.y[:, :, :Hqk * D].unflatten(-1, (Hqk, D))
            self.k = self.y[:, :, Hqk * D:2 * Hqk * D].unflatten(-1, (Hqk, D))
            self.v = self.y[:, :, 2 * Hqk * D:].unflatten(-1, (Hv, D))
        else:
            self.x = None
            self.q, self.k, self.v = to_dev(case["q"]), to_dev(case["k"]), to_dev(case["v"])
        self.out = torch.zeros((B, R, Hv, D), dtype=torch.float32, device=dev)
        self.u = None  # stored corrections (factored mode)


class Instance:
    """One layer instance: its pool, history (two buffers in layer mode, used
    in turn as the step's input and output), weights and step slots."""

    def __init__(self, g, cfg, seed, layer, to_dev, dev, torch, slots):
        import gdn_inputs as gi
        cases = [gi.make_case(cfg, seed=seed + 7919 * j, layer=layer, packing="bfs") for j in range(slots)]
        base = cases[0]
        for c in cases[1:]:
            for key in ("pool", "state_idx", "P", "hist", "w"):
                if key in base:
                    c[key] = base[key]
        self.pool = to_dev(base["pool"])
        self.state_idx = to_dev(base["state_idx"])
        self.hist = to_dev(base["hist"]) if cfg.conv_W > 0 else None
        self.hist2 = self.hist.clone() if cfg.conv_W > 0 else None
        self.w = to_dev(base["w"]) if cfg.conv_W > 0 else None
        self.slots = [Slot(g, cfg, c, to_dev, dev, torch) for c in cases]
        B, Lmax = base["path"].shape
        self.path_rows = torch.zeros((B, Lmax), dtype=torch.int32, device=dev)
        self.path_n = torch.zeros((B,), dtype=torch.int32, device=dev)
        self.P = int(base["P"])
        self.turn = 0


class LayerStack:
    """L layers back to back on the same requests: one tree and accepted path
    per request for every layer (host-drawn, two step slots), and per layer
    its own operands and state pool, drawn on the device with the workload's
    distributions (q, k unit rows in bf16, v ~N(0,1) bf16, a = exp(-softplus(n)),
    b = sigmoid(n), state ~N(0, s_std^2)) from a seeded generator per layer and
    slot.  Outputs share one buffer per slot (no layer reads them)."""

    def __init__(self, g, cfg, seed, layers, to_dev, dev, torch):
        import gdn_inputs as gi
        cases = [gi.make_case(cfg, seed=seed + 7919 * j, layer=0, packing="bfs", with_pool=False)
                 for j in range(2)]
        B, R, D, Hv, Hqk, N = cfg.B, cfg.R, cfg.D, cfg.Hv, cfg.Hqk, cfg.N
        self.cases = cases
        self.desc = [g.TreeDesc(to_dev(c["parent"]), to_dev(c["node_row"]), R, 1) for c in cases]
        self.path = [to_dev(c["path"]) for c in cases]
        self.path_len = [to_dev(c["path_len"]) for c in cases]
        self.state_idx = to_dev(cases[0]["state_idx"])
        self.P = int(cases[0]["P"])
        self.out = [torch.empty((B, R, Hv, D), dtype=torch.float32, device=dev) for _ in range(2)]
        self.path_rows = torch.zeros(cases[0]["path"].shape, dtype=torch.int32, device=dev)
        self.path_n = torch.zeros((B,), dtype=torch.int32, device=dev)
        used = torch.zeros((2, B, R), dtype=torch.bool, device=dev)
        for j, c in enumerate(cases):
            for b in range(B):
                used[j, b, torch.as_tensor(c["node_row"][b], device=dev).long()] = True
        # stacked per kind ([L, ...] with layer l at index l) so that one
        # launch can commit every layer; layer l's tensors are views
        L = layers
        self.pool_all = torch.empty((L, self.P, Hv, D, D), dtype=torch.float32, device=dev)
        self.slot_all = [{"q": torch.empty((L, B, R, Hqk, D), dtype=torch.bfloat16, device=dev),
                          "k": torch.empty((L, B, R, Hqk, D), dtype=torch.bfloat16, device=dev),
                          "v": torch.empty((L, B, R, Hv, D), dtype=torch.bfloat16, device=dev),
                          "alpha": torch.empty((L, B, R, Hv), dtype=torch.float32, device=dev),
                          "beta": torch.empty((L, B, R, Hv), dtype=torch.float32, device=dev)}
                         for _ in range(2)]
        self.layers = []
        for l in range(L):
            gen = torch.Generator(device=dev)
            gen.manual_seed(seed * 1000003 + l)

            def unit_rows(shape):
                x = torch.randn(shape, generator=gen, device=dev)
                return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

            self.pool_all[l].copy_(torch.randn((self.P, Hv, D, D), generator=gen, device=dev) * cfg.s_std)
            lay = {"pool": self.pool_all[l], "slots": []}
            for j in range(2):
                sl = {key: t[l] for key, t in self.slot_all[j].items()}
                sl["q"].copy_(unit_rows((B, R, Hqk, D)))
                sl["k"].copy_(unit_rows((B, R, Hqk, D)))
                sl["v"].copy_(torch.randn((B, R, Hv, D), generator=gen, device=dev).to(torch.bfloat16))
                sl["alpha"].copy_(torch.exp(-torch.nn.functional.softplus(
                    torch.randn((B, R, Hv), generator=gen, device=dev))))
                sl["beta"].copy_(torch.sigmoid(torch.randn((B, R, Hv), generator=gen, device=dev)))
                pad = ~used[j]
                for key in ("alpha", "beta"):
                    sl[key][pad] = float("nan")
                lay["slots"].append(sl)
            self.layers.append(lay)
        self.turn = 0


def run_layers(args, cfg, g, torch, dev, to_dev):
    """The step of an L-layer model: the step's shared prepare (descriptor,
    path rows), then every layer's commit + verify (fused: one launch per
    layer; separate: every layer's verify, then one launch that commits this
    step's path into all layers)."""
    L = args.layers
    fused = args.mode == "fused"
    t0 = time.perf_counter()
    st = LayerStack(g, cfg, args.seed, L, to_dev, dev, torch)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] {args.mode} mode: {L} layers of {cfg.name} ready in {time.perf_counter() - t0:.1f} s")

    def step(ev=None):
        cur, prev = st.turn % 2, (st.turn - 1) % 2
        st.turn += 1
        marks = iter(ev) if ev is not None else None

        def mark():
            if marks is not None:
                next(marks).record()

        mark()
        if fused:
            g.gdn_step_prepare(st.desc[cur], st.desc[prev], st.path[prev], st.path_len[prev],
                               st.state_idx, st.P, st.path_rows, st.path_n, err)
        else:
            g.gdn_tree_desc_build(st.desc[cur], err)
        mark()
        for lay in st.layers:
            c, p = lay["slots"][cur], lay["slots"][prev]
            if fused:
                g.gdn_tree_commit_verify(st.desc[cur], c["q"], c["k"], c["v"], c["alpha"], c["beta"],
                                         lay["pool"], st.state_idx, st.out[cur], st.desc[prev],
                                         st.path_rows, st.path_n, p["k"], p["v"], p["alpha"],
                                         p["beta"], err)
            else:
                g.gdn_tree_verify(st.desc[cur], c["q"], c["k"], c["v"], c["alpha"], c["beta"],
                                  lay["pool"], st.state_idx, st.out[cur], err)
            mark()
        if not fused:
            # after acceptance: this step's path into every layer's state, one launch
            sa = st.slot_all[cur]
            g.gdn_tree_commit_layers(st.desc[cur], st.path[cur], st.path_len[cur], sa["k"], sa["v"],
                                     sa["alpha"], sa["beta"], st.pool_all, st.state_idx, err,
                                     Hqk=cfg.Hqk)
            mark()
        return cur, prev

    settle_steps = settle(lambda i: step(), args.settle_ms, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    steps_bytes = []
    for _ in range(args.steps):
        cur, prev = step()
        ccase, pcase = st.cases[cur], st.cases[prev]
        steps_bytes.append(byte_model(cfg, ccase, pcase, args.mode))
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    # per-layer launch durations, in a second pass with an event between launches
    nsteps_b = min(args.steps, 10)
    nev = L + 2 if fused else L + 3
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(nsteps_b)]
    for i in range(nsteps_b):
        step(evs[i])
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        log(f"[bench] device error word {int(err.item())}")
        sys.exit(3)
    prep_ms = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in evs]))
    layer_ms = float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in evs for j in range(1, L + 1)]))
    if not fused:
        commit_ms = float(np.mean([ev[L + 1].elapsed_time(ev[L + 2]) for ev in evs]))
        log(f"[bench] verify {layer_ms * 1e3:.1f} us per layer; commit of {L} layers in one launch "
            f"{commit_ms * 1e3:.1f} us ({commit_ms * 1e3 / L:.1f} us per layer)")
        layer_ms += commit_ms / L
    kname = "commit_verify" if fused else "verify+commit"
    per_layer_bytes = float(np.mean([sum(v for k, v in b.items() if k not in ("desc", "prepare"))
                                     for b in steps_bytes]))
    step_bytes = L * per_layer_bytes + float(np.mean([b.get("prepare", b.get("desc", 0)) for b in steps_bytes]))
    B, N = cfg.B, cfg.N
    value = B * N * L / (ms_per_step / 1e3)
    achieved = per_layer_bytes / (layer_ms / 1e3) / 1e9
    # measured HBM bytes per layer from the committed counter summaries (taken
    # at this workload's full layer count), while the kernels are unchanged
    traffic = None
    if L == cfg.layers and cfg.name == "tree64_b256_h32_l48":
        if fused:
            traffic = measured_traffic("tree64_b256_l48", "fused", "commit_verify")
        else:
            tv = measured_traffic("tree64_b256_l48", "separate", "verify")
            tc = measured_traffic("tree64_b256_l48", "separate", "commit")
            traffic = tv + tc // L if tv is not None and tc is not None else None
    log(f"[bench] prepare {prep_ms * 1e3:.1f} us; per layer {layer_ms * 1e3:.1f} us "
        f"{per_layer_bytes / 1e6:.1f} MB -> {achieved:.1f} GB/s ({achieved / PEAK_HBM_GBS * 100:.1f}% of 8 TB/s)")
    log(f"[bench] step of {L} layers {ms_per_step * 1e3:.1f} us (wall {wall / args.steps * 1e6:.1f} us): "
        f"{ms_per_step * 1e3 / L:.1f} us per layer, {step_bytes / (ms_per_step / 1e3) / 1e9:.1f} GB/s")
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tree nodes/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {N}-node draft trees (branching<={cfg.bmax}, depth<={cfg.depth_max}), "
                        f"B={B}, Hv={cfg.Hv} over Hqk={cfg.Hqk}, d={cfg.D}, bf16 operands, fp32 state, "
                        f"{L} GDN layers back to back (own operands and state pool per layer; one tree "
                        f"and accepted path per request shared by the layers)",
            "mode": args.mode,
            "step": ("gdn_step_prepare + gdn_tree_commit_verify per layer" if fused else
                     "gdn_tree_desc_build + gdn_tree_verify per layer + one gdn_tree_commit_layers"),
            "settle_ms": args.settle_ms, "settle_steps": settle_steps,
            "value_is": "tree nodes verified per second per GDN layer: B*N*layers / step time",
            "global_batch": B, "nodes_per_request": N, "layers": L, "parallelism": "single GPU",
            "step_bytes": int(step_bytes), "us_per_layer": round(ms_per_step * 1e3 / L, 2),
            "step_hbm_gbs": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
            "node_heads_per_s": round(value * cfg.Hv, 1),
            # spread over the launches of the pass with an event between launches
            "layer_us_p10_p50_p90": spread([ev[j].elapsed_time(ev[j + 1]) for ev in evs
                                            for j in range(1, L + 1)]),
            "prepare_us_p10_p50_p90": spread([ev[0].elapsed_time(ev[1]) for ev in evs]),
        },
        "roofline": dict(bound="hbm", kernel=kname, achieved=round(achieved, 1), peak=PEAK_HBM_GBS,
                         unit="GB/s", frac=round(achieved / PEAK_HBM_GBS, 4), traffic=traffic,
                         traffic_over_algorithmic=(round(traffic / per_layer_bytes, 3) if traffic else None),
                         avg_us=round(layer_ms * 1e3, 2), algorithmic_bytes=int(per_layer_bytes)),
        "cpu_baseline": None,
    }
    if not args.no_ceiling:
        ceil = stream_ceiling(torch, dev)
        log(f"[bench] streaming ceiling (in-place fp32 scale over 1 GiB, read + write): {ceil:.1f} GB/s")
        line["roofline"]["stream_rmw_ceiling"] = dict(
            kind="in-place fp32 x *= c over 1 GiB (torch elementwise kernel), read + write counted",
            gbs=round(ceil, 1), frac_of_ceiling=round(achieved / ceil, 4))
    if not args.no_cpu_baseline:
        # one layer's oracle on a bounded sample of the requests (a full
        # layer of this workload is minutes of fp64 work); per layer, so the
        # 48-layer step is this rate divided by the layer count
        cpu = cpu_baseline(cfg, args.seed, args.cpu_budget, B=min(cfg.B, 16))
        cpu["value"] = round(cpu["value"], 1)
        cpu["per_step_of_layers"] = round(cpu["value"] / L, 2)
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


ATTN = dict(N=27, R=32, Hq=16, Hkv=2, D=256, bmax=3, depth_max=6)


def attention_cpu_baseline(args, budget_s):
    """The fp64 oracle's tree attention on the host, on one request of the
    same workload (all its nodes and heads), repeated until ``budget_s``."""
    import oracle  # noqa: F401  (the package; the attention oracle is NumPy)
    from oracle.attention import tree_attention
    import gdn_inputs as gi
    a = ATTN
    c = gi.make_attention_case(args.seed, 1, a["N"], a["R"], a["Hq"], a["Hkv"], a["D"], [args.ctx],
                               args.ctx + a["R"], bmax=a["bmax"], depth_max=a["depth_max"], packing="bfs")
    st = np.zeros(1, np.int32)
    reps, t0 = 0, time.perf_counter()
    while True:
        tree_attention(c["parent"], c["node_row"], st, c["q"], c["k"], c["v"], c["ctx"], a["R"], a["Hq"],
                       a["Hkv"], 1.0 / np.sqrt(a["D"]))
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 20:
            break
    return dict(value=reps * a["N"] / el, unit="tree nodes/s", cores=1, kind="oracle",
                sample=f"one request of the workload (N={a['N']}, {args.ctx} prefix positions, all "
                       f"{a['Hq']} heads) in fp64 NumPy, {reps} repetition(s), {el:.1f} s wall")


def run_attention(args, g, torch, dev):
    """Tree attention of one softmax-attention layer: B requests, each a
    27-node tree (branching <= 3, depth <= 6, breadth-first rows) over a
    committed prefix of ``--ctx`` positions; 16 query heads over 2 kv heads,
    d = 256, bf16 cache.  Inputs drawn on the device; three instances in turn
    so a step's 134 MB per request of keys and values do not stay in the
    256 MB last-level cache."""
    import gdn_inputs as gi
    a = ATTN
    B, N, R, Hq, Hkv, D = args.batch, a["N"], a["R"], a["Hq"], a["Hkv"], a["D"]
    S = args.ctx + R
    splits = args.splits
    t0 = time.perf_counter()
    insts = []
    for j in range(3):
        parents = np.stack([gi.random_tree(gi.rng(args.seed + j, gi.ATTN_CFG, b, 0), N, a["bmax"], a["depth_max"])
                            for b in range(B)]).astype(np.int32)
        rows = np.stack([gi.bfs_rows(p) for p in parents]).astype(np.int32)
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed * 7 + j)
        inst = dict(desc=g.TreeDesc(torch.from_numpy(parents).to(dev), torch.from_numpy(rows).to(dev), R, 1, B=B),
                    q=torch.randn((B, N, Hq, D), generator=gen, device=dev).to(torch.bfloat16),
                    k=torch.randn((B, S, Hkv, D), generator=gen, device=dev).to(torch.bfloat16),
                    v=torch.randn((B, S, Hkv, D), generator=gen, device=dev).to(torch.bfloat16),
                    ctx=torch.full((B,), args.ctx, dtype=torch.int32, device=dev),
                    out=torch.empty((B, N, Hq, D), dtype=torch.float32, device=dev))
        insts.append(inst)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for inst in insts:
        g.gdn_tree_desc_build(inst["desc"], err)
    nbytes = g.gdn_tree_attention_workspace_bytes(B, N, Hq, D, splits)
    ws = torch.empty((nbytes // 4 + 4,), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] attention mode: {B} x {N}-node trees over {args.ctx} prefix positions, Hq={Hq} "
        f"Hkv={Hkv} d={D}, {splits} partitions; inputs ready in {time.perf_counter() - t0:.1f} s")

    def step(i):
        inst = insts[i % 3]
        g.gdn_tree_attention(inst["desc"], inst["q"], inst["k"], inst["v"], inst["ctx"], inst["out"], ws, err,
                             splits=splits)

    settle_steps = settle(step, args.settle_ms, torch)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        log(f"[bench] device error word {int(err.item())}")
        sys.exit(3)
    ms = e0.elapsed_time(e1) / args.steps
    # algorithmic bytes: the prefix keys and values once, the candidates',
    # the queries and the outputs; flops of Q K^T and P V
    kv = B * args.ctx * Hkv * D * 2 * 2
    byts = kv + B * R * Hkv * D * 2 * 2 + B * N * Hq * D * 2 + B * N * Hq * D * 4
    flops = 2 * 2 * B * N * Hq * (args.ctx + 7) * D
    achieved = byts / (ms / 1e3) / 1e9
    log(f"[bench] tree attention {ms * 1e3:.1f} us per layer: {byts / 1e6:.1f} MB -> {achieved:.1f} GB/s "
        f"({achieved / PEAK_HBM_GBS * 100:.1f}% of 8 TB/s); {flops / 1e9:.1f} GFLOP -> "
        f"{flops / (ms / 1e3) / 1e12:.1f} TFLOP/s")
    cpu = None if args.no_cpu_baseline else attention_cpu_baseline(args, args.cpu_budget)
    line = {
        "metric": METRIC, "value": round(B * N / (ms / 1e3), 1), "unit": "tree nodes/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"tree attention: {B} request(s), {N}-node trees (branching<=3, depth<=6), "
                               f"{args.ctx} prefix positions, Hq={Hq} over Hkv={Hkv}, d={D}, bf16 KV cache, "
                               f"{splits} prefix partitions",
                   "mode": "attention", "step": "gdn_tree_attention (partitions + merge), one layer",
                   "settle_ms": args.settle_ms, "settle_steps": settle_steps,
                   "value_is": "tree nodes attended per second per attention layer",
                   "global_batch": B, "nodes_per_request": N, "parallelism": "single GPU",
                   "step_bytes": int(byts), "step_gflop": round(flops / 1e9, 2)},
        "roofline": dict(bound="hbm", kernel="tree_attention (partitions + merge launches)",
                         achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                         frac=round(achieved / PEAK_HBM_GBS, 4),
                         traffic=(measured_traffic_sum("tree27_ctx64k", "attention", "gdn::tree_attn")
                                  if (B, args.ctx, splits) == (1, 65536, 63) else None),
                         avg_us=round(ms * 1e3, 2), algorithmic_bytes=int(byts)),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # after idle the GPU runs the first 100-200 steps of this workload about
    # 6% slower than in steady state (clocks and power ramping up over tens of
    # ms); 200 untimed steps (about 40 ms) reach the steady state
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--mode", choices=("fused", "layer", "separate", "factored", "attention"),
                    default="layer")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="run the step for this long before the warm-up steps: after idle the GPU's "
                         "clocks take tens of ms of load to reach their steady state")
    ap.add_argument("--ctx", type=int, default=65536, help="attention mode: committed prefix per request")
    ap.add_argument("--splits", type=int, default=63,
                    help="attention mode: prefix partitions (63: with the candidate partition, "
                         "2 kv heads x 2 head groups x 64 = 256 workgroups, one per CU)")
    ap.add_argument("--batch", type=int, default=1, help="attention mode: requests")
    ap.add_argument("--seed", type=int, default=2026)
    ap.add_argument("--sets", type=int, default=2, help="independent layer instances rotated per step")
    ap.add_argument("--layers", type=int, default=0,
                    help="layers per step for the multi-layer workload (default: the workload's)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming read-modify-write ceiling measured after the timed run")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain fp32 copy kernel (out = in * 1) over MIB MiB, three "
                         "times, as the known-size reference for HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the path runs on a single MI355X, one process "
              "and one device. Use --gpus 1.", file=sys.stderr)
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
    fused = args.mode == "fused"
    layer = args.mode == "layer"
    factored = args.mode == "factored"
    if layer and cfg.conv_W == 0:
        print("--mode layer needs a conv workload (the layer step starts from the conv input)",
              file=sys.stderr)
        sys.exit(2)

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

    if args.mode == "attention":
        run_attention(args, g, torch, dev)
        return
    if args.layers == 0:
        args.layers = cfg.layers
    if args.layers > 1:
        if cfg.conv_W > 0 or layer or factored:
            print("--layers > 1 covers the workloads without conv (fused or separate mode)",
                  file=sys.stderr)
            sys.exit(2)
        run_layers(args, cfg, g, torch, dev, to_dev)
        return

    t0 = time.perf_counter()
    insts = [Instance(g, cfg, args.seed, li, to_dev, dev, torch, 2 if (fused or layer or factored) else 1)
             for li in range(args.sets)]
    if factored:
        for inst in insts:
            for sl in inst.slots:
                sl.u = torch.zeros_like(sl.out)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    flags = g.GDN_F_NORM_QK if cfg.norm_qk else 0
    torch.cuda.synchronize()
    log(f"[bench] {args.mode} mode: inputs for {cfg.name} x{args.sets} ready in "
        f"{time.perf_counter() - t0:.1f} s")

    has_conv = cfg.conv_W > 0
    names = (("prepare", "layer") if layer else
             ("prepare",) + (("conv",) if has_conv else ()) + ("commit_verify",) if fused else
             ("prepare",) + (("conv",) if has_conv else ()) + ("verify_u", "commit_factored") if factored else
             ("desc",) + (("conv",) if has_conv else ()) + ("verify", "commit"))

    def step(inst, ev=None):
        cur = inst.slots[inst.turn % len(inst.slots)]
        prev = inst.slots[(inst.turn - 1) % len(inst.slots)]
        inst.turn += 1
        marks = iter(ev) if ev is not None else None

        def mark():
            if marks is not None:
                next(marks).record()

        mark()
        if layer:
            # once per step for every layer: the new tree's descriptor and the
            # previous path's rows
            g.gdn_step_prepare(cur.desc, prev.desc, prev.path, prev.path_len, inst.state_idx, inst.P,
                               inst.path_rows, inst.path_n, err)
            mark()
            hist_in, hist_out = (inst.hist, inst.hist2) if inst.turn % 2 else (inst.hist2, inst.hist)
            g.gdn_layer_step(cur.desc, cur.x, inst.w, None, cfg.act, hist_in, hist_out, cur.alpha,
                             cur.beta, inst.pool, inst.state_idx, cur.out, prev.desc, prev.x,
                             prev.alpha, prev.beta, inst.path_rows, inst.path_n, err, cfg.Hqk,
                             flags=flags)
            mark()
            return cur, prev
        if factored:
            g.gdn_step_prepare(cur.desc, prev.desc, prev.path, prev.path_len, inst.state_idx, inst.P,
                               inst.path_rows, inst.path_n, err)
            mark()
            if has_conv:
                g.conv_ancestry_gather_publish(cur.desc, cur.x, inst.hist, inst.state_idx, inst.w,
                                               None, cur.y, cfg.act, prev.desc, inst.path_rows,
                                               inst.path_n, prev.x, err)
                mark()
            g.gdn_tree_verify_store_u(cur.desc, cur.q, cur.k, cur.v, cur.alpha, cur.beta, inst.pool,
                                      inst.state_idx, cur.out, cur.u, err, flags=flags)
            mark()
            g.gdn_tree_commit_factored(cur.desc, cur.path, cur.path_len, cur.k, cur.u, cur.alpha,
                                       inst.pool, inst.state_idx, err, flags=flags & g.GDN_F_NORM_QK)
            mark()
            return cur, prev
        if fused:
            g.gdn_step_prepare(cur.desc, prev.desc, prev.path, prev.path_len, inst.state_idx, inst.P,
                               inst.path_rows, inst.path_n, err)
            mark()
            if has_conv:
                g.conv_ancestry_gather_publish(cur.desc, cur.x, inst.hist, inst.state_idx, inst.w,
                                               None, cur.y, cfg.act, prev.desc, inst.path_rows,
                                               inst.path_n, prev.x, err)
                mark()
            g.gdn_tree_commit_verify(cur.desc, cur.q, cur.k, cur.v, cur.alpha, cur.beta,
                                     inst.pool, inst.state_idx, cur.out, prev.desc, inst.path_rows,
                                     inst.path_n, prev.k, prev.v, prev.alpha, prev.beta, err,
                                     flags=flags)
        else:
            g.gdn_tree_desc_build(cur.desc, err)
            mark()
            if has_conv:
                g.conv_ancestry_gather(cur.desc, cur.x, inst.hist, inst.state_idx, inst.w, None,
                                       cur.y, cfg.act, err)
                mark()
            g.gdn_tree_verify(cur.desc, cur.q, cur.k, cur.v, cur.alpha, cur.beta, inst.pool,
                              inst.state_idx, cur.out, err, flags=flags)
            mark()
            g.gdn_tree_commit(cur.desc, cur.path, cur.path_len, cur.k, cur.v, cur.alpha,
                              cur.beta, inst.pool, inst.state_idx, err, Hqk=cfg.Hqk,
                              flags=flags & g.GDN_F_NORM_QK, x=cur.x, hist=inst.hist)
        mark()
        return cur, prev

    # clock settle, then the warm-up steps (the first step of each instance
    # also fills its slots' conv outputs)
    settle_steps = settle(lambda i: step(insts[i % len(insts)]), args.settle_ms, torch)
    for i in range(args.warmup + (2 * args.sets if (fused or factored) else 0)):
        step(insts[i % len(insts)])
    torch.cuda.synchronize()

    # the timed steps: events only around the whole run (an event recorded
    # between two launches adds a few µs of its own to the timeline)
    bytes_steps = []
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        cur, prev = step(insts[i % len(insts)])
        bytes_steps.append(byte_model(cfg, cur.case, prev.case, args.mode))
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = e0.elapsed_time(e1)
    # then the same number of steps again with an event between launches, for
    # the per-kernel durations
    nmarks = len(names) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nmarks)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(insts[i % len(insts)], evs[i])
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        log(f"[bench] device error word {int(err.item())}")
        sys.exit(3)

    per = {n: [ev[j].elapsed_time(ev[j + 1]) for ev in evs] for j, n in enumerate(names)}
    ms_per_step = total_ms / args.steps
    avg = {n: float(np.mean(per[n])) for n in names}
    bytes_avg = {n: float(np.mean([b[n] for b in bytes_steps])) for n in names}
    B, N = cfg.B, cfg.N
    nodes_per_s = B * N / (ms_per_step / 1e3)
    step_bytes = sum(bytes_avg.values())
    for n in names:
        gbs = bytes_avg[n] / (avg[n] / 1e3) / 1e9 if avg[n] > 0 else 0.0
        log(f"[bench] {n:13s} {avg[n] * 1e3:9.1f} us  {bytes_avg[n] / 1e6:8.1f} MB  "
            f"{gbs:8.1f} GB/s  {gbs / PEAK_HBM_GBS * 100:5.1f}% of 8 TB/s")
    log(f"[bench] step {ms_per_step * 1e3:.1f} us (events around the run), wall "
        f"{wall / args.steps * 1e6:.1f} us; with an event between launches "
        f"{evs[0][0].elapsed_time(evs[-1][-1]) / args.steps * 1e3:.1f} us; "
        f"{step_bytes / 1e6:.1f} MB -> {step_bytes / (ms_per_step / 1e3) / 1e9:.1f} GB/s")

    dom = max((n for n in names if n not in ("desc", "prepare")), key=lambda n: avg[n])
    achieved = bytes_avg[dom] / (avg[dom] / 1e3) / 1e9
    tag = WORKLOAD_TAG.get(cfg.name, cfg.name)
    traffic = measured_traffic(tag, args.mode, dom)
    roofline = dict(bound="hbm", kernel=dom, achieved=round(achieved, 1), peak=PEAK_HBM_GBS,
                    unit="GB/s", frac=round(achieved / PEAK_HBM_GBS, 4), traffic=traffic,
                    traffic_over_algorithmic=(round(traffic / bytes_avg[dom], 3) if traffic else None),
                    avg_us=round(avg[dom] * 1e3, 2), algorithmic_bytes=int(bytes_avg[dom]))
    if not args.no_ceiling:
        ceil = stream_ceiling(torch, dev)
        log(f"[bench] streaming ceiling (in-place fp32 scale over 1 GiB, read + write): {ceil:.1f} GB/s; "
            f"{dom} at {achieved / ceil * 100:.1f}% of it")
        roofline["stream_rmw_ceiling"] = dict(
            kind="in-place fp32 x *= c over 1 GiB (torch elementwise kernel), read + write counted",
            gbs=round(ceil, 1), frac_of_ceiling=round(achieved / ceil, 4))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.seed, args.cpu_budget)
        cpu["value"] = round(cpu["value"], 1)

    steps_desc = ("gdn_step_prepare + gdn_layer_step (steady state: the previous "
                  "step's accepted path committed and its conv history published inside the "
                  "layer step, the conv output kept on chip)" if layer else
                  "gdn_step_prepare + conv_ancestry_gather_publish + gdn_tree_commit_verify (steady "
                  "state: the previous step's accepted path committed and its conv history "
                  "published inside this step)" if fused else
                  "gdn_step_prepare + conv_ancestry_gather_publish + gdn_tree_verify_store_u + "
                  "gdn_tree_commit_factored (the stored-U form: this step's path committed from the "
                  "verify's corrections, its conv history published by the next step)" if factored else
                  "desc_build + conv_ancestry_gather + gdn_tree_verify + gdn_tree_commit")
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
            "mode": args.mode,
            "step": steps_desc + " (one layer)",
            "global_batch": B,
            "nodes_per_request": N,
            "parallelism": "single GPU",
            "step_bytes": int(step_bytes),
            "step_hbm_gbs": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
            "step_frac_of_peak": round(step_bytes / (ms_per_step / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "settle_ms": args.settle_ms, "settle_steps": settle_steps,
            "kernel_us": {n: round(avg[n] * 1e3, 2) for n in names},
            # per-launch spread from the pass with an event between launches
            "kernel_us_p10_p50_p90": {n: spread(per[n]) for n in names},
            "step_us_p10_p50_p90": spread([ev[0].elapsed_time(ev[-1]) for ev in evs]),
            "node_heads_per_s": round(nodes_per_s * cfg.Hv, 1),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
