"""Shared helpers for the parity tests: upload a seeded case, run the HIP path
through the binding, run the oracle on the same host inputs, compare.

The oracle never sees a value the GPU produced: for conv configurations it
computes its own conv output and rounds it to bf16 itself.
"""
from __future__ import annotations

import numpy as np

import gdn_inputs as gi
import oracle
from oracle.gates import gates_from_raw as oracle_gate_eval

NAN_BF16 = 0x7FC0


# --------------------------------------------------------------------------
# metrics
# --------------------------------------------------------------------------

def max_rel_rows(gpu, ref, axis_rows):
    """Max over rows of max|gpu - ref| / max(max|ref|, 1e-30): the error of a
    row (an output vector, or a state matrix) relative to that row's largest
    magnitude.  ``axis_rows`` = number of leading axes that index rows.
    NaN anywhere in gpu where ref is finite counts as infinite error."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    lead = g.shape[:axis_rows]
    g = g.reshape(int(np.prod(lead)) if lead else 1, -1)
    r = r.reshape(g.shape)
    if np.isnan(g).any() or np.isinf(g).any():
        return float("inf")
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((np.abs(g - r).max(axis=1) / den).max())


def bf16_ulp_diff(a_bits, b_bits):
    """Distance in bf16 units in the last place (ordered integer view)."""
    def ordered(u):
        u = np.asarray(u, np.uint16).astype(np.int32)
        mag = u & 0x7FFF
        return np.where(u & 0x8000, -mag, mag)
    return np.abs(ordered(a_bits) - ordered(b_bits))


# --------------------------------------------------------------------------
# device plumbing
# --------------------------------------------------------------------------

def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def bits(t):
    """bf16 tensor -> uint16 numpy bit patterns."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def subset(case, bs):
    """The same problem restricted to requests ``bs`` (their own pool slots,
    re-indexed 0..len(bs)-1).  Requests are independent, so the oracle's
    answer for request b in the subset is its answer in the full batch."""
    bs = np.asarray(bs)
    out = dict(case)
    out["B"] = len(bs)
    for key in ("parent", "node_row", "path", "path_len", "alpha", "beta", "q", "k", "v", "x"):
        if key in case:
            out[key] = case[key][bs]
    slots = case["state_idx"][bs]
    out["state_idx"] = np.arange(len(bs), dtype=np.int32)
    out["pool"] = case["pool"][slots]
    if "hist" in case:
        out["hist"] = case["hist"][slots]
    out["P"] = len(bs)
    return out


def run_gpu(case, flags=0, commit=True, shared=False, out_bf16=False, raise_on_error=True,
            y_override=None):
    """desc_build -> [conv] -> verify -> [commit] on the device for one case.
    Returns host copies of everything produced.  With ``y_override`` (bf16
    bits [B][R][C]) the conv output the device produced is kept in res["y"]
    but verify and commit read ``y_override`` instead (stage-wise parity:
    downstream stages compared on identical inputs)."""
    import torch
    import tree_speculative_verification_gdn_amd as g

    cfg = case["cfg"]
    B, N, R, D, Hv, Hqk = case["B"], cfg.N, cfg.R, cfg.D, cfg.Hv, cfg.Hqk
    W = cfg.conv_W if cfg.conv_W > 0 else 1
    parent = case["parent"][:1] if shared else case["parent"]
    rows = case["node_row"][:1] if shared else case["node_row"]
    desc = g.TreeDesc(to_dev(parent), to_dev(rows), R, W, B=B, shared=shared)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = {}
    res["rc_desc"] = g.gdn_tree_desc_build(desc, err, raise_on_error=raise_on_error)
    pool = to_dev(case["pool"])
    sidx = to_dev(case["state_idx"])
    alpha, beta = to_dev(case["alpha"]), to_dev(case["beta"])
    if cfg.conv_W > 0:
        C = cfg.conv_C
        x = to_dev(case["x"])
        hist = to_dev(case["hist"])
        w = to_dev(case["w"])
        y = torch.full((B, R, C), float("nan"), dtype=torch.bfloat16, device="cuda")
        res["rc_conv"] = g.conv_ancestry_gather(desc, x, hist, sidx, w, dev_bias(case), y, cfg.act, err,
                                                raise_on_error=raise_on_error)
        if y_override is not None:
            res["y_own"] = bits(y)
            y.copy_(to_dev(np.where(y_override == NAN_BF16, res["y_own"], y_override).astype(np.uint16)))
        q = y[:, :, :Hqk * D].unflatten(-1, (Hqk, D))
        k = y[:, :, Hqk * D:2 * Hqk * D].unflatten(-1, (Hqk, D))
        v = y[:, :, 2 * Hqk * D:].unflatten(-1, (Hv, D))
        flags |= g.GDN_F_NORM_QK if cfg.norm_qk else 0
    else:
        x = hist = None
        q, k, v = to_dev(case["q"]), to_dev(case["k"]), to_dev(case["v"])
    odt = torch.bfloat16 if out_bf16 else torch.float32
    out = torch.full((B, R, Hv, D), float("nan"), dtype=odt, device="cuda")
    vflags = flags | (g.GDN_F_OUT_BF16 if out_bf16 else 0)
    gp = dev_gate_params(case)
    res["rc_verify"] = g.gdn_tree_verify(desc, q, k, v, alpha, beta, pool, sidx, out, err,
                                         flags=vflags, raise_on_error=raise_on_error,
                                         gate_params=gp)
    if commit:
        res["rc_commit"] = g.gdn_tree_commit(desc, to_dev(case["path"]), to_dev(case["path_len"]),
                                             k, v, alpha, beta, pool, sidx, err, Hqk=Hqk,
                                             flags=flags & g.GDN_F_NORM_QK, x=x, hist=hist,
                                             raise_on_error=raise_on_error, gate_params=gp)
    torch.cuda.synchronize()
    res.update(err=int(err.item()), depth=desc.depth.cpu().numpy(),
               anc=desc.anc.cpu().numpy().view(np.uint64), conv_src=desc.conv_src.cpu().numpy()[:, :, :W - 1],
               status=desc.status.cpu().numpy(), pool=pool.cpu().numpy())
    res["out"] = (bits(out) if out_bf16 else out.cpu().numpy())
    if cfg.conv_W > 0:
        res["y"] = res.get("y_own", bits(y))
        res["hist"] = bits(hist)
    return res


def run_oracle(case, commit=True, shared=False):
    """The oracle on the same host inputs (conv output rounded to bf16 by the
    oracle itself when the config has a conv)."""
    cfg = case["cfg"]
    R, Hv, Hqk, D = cfg.R, cfg.Hv, cfg.Hqk, cfg.D
    W = cfg.conv_W if cfg.conv_W > 0 else 1
    parent = case["parent"][:1] if shared else case["parent"]
    rows = case["node_row"][:1] if shared else case["node_row"]
    d = oracle.desc_build(parent, rows, R, W)
    res = dict(err=d["err"], depth=d["depth"], anc=d["anc"], conv_src=d["conv_src"], status=d["status"])
    if cfg.conv_W > 0:
        y, e = oracle.conv(rows, d["conv_src"], d["status"], case["x"], case["hist"], case["state_idx"],
                           case["w"], case.get("bias"), cfg.act, R, cfg.conv_C, W, shared=shared)
        res["err"] |= e
        ybits = oracle.round_f64_to_bf16_bits(y)
        ybits = np.where(np.isnan(y), NAN_BF16, ybits).astype(np.uint16)
        res["y"] = ybits
        B = case["B"]
        q = ybits[:, :, :Hqk * D].reshape(B, R, Hqk, D)
        k = ybits[:, :, Hqk * D:2 * Hqk * D].reshape(B, R, Hqk, D)
        v = ybits[:, :, 2 * Hqk * D:].reshape(B, R, Hv, D)
        norm = cfg.norm_qk
    else:
        q, k, v = case["q"], case["k"], case["v"]
        norm = False
    alpha, beta = oracle_gates(case)
    out, e = oracle.verify(parent, rows, d["status"], q, k, v, alpha, beta,
                           case["pool"], case["state_idx"], Hqk, Hv, norm, shared=shared)
    res["err"] |= e
    res["out"] = out
    if commit:
        pool, hist, e = oracle.commit(parent, rows, d["status"], case["path"], case["path_len"], k, v,
                                      alpha, beta, case["pool"], case["state_idx"],
                                      Hqk, Hv, norm, x=case.get("x"), hist=case.get("hist"), W=W,
                                      shared=shared)
        res["err"] |= e
        res["pool"] = pool
        if hist is not None:
            res["hist"] = hist
    return res


def oracle_gates(case):
    """The gates the oracle uses: the case's own, or, for raw gate inputs,
    the oracle's fp64 evaluation of them."""
    if "gate_params" in case:
        return oracle_gate_eval(case["alpha"], case["beta"], case["gate_params"])
    return case["alpha"], case["beta"]


def dev_bias(case):
    return to_dev(case["bias"]) if "bias" in case else None


def dev_gate_params(case):
    return to_dev(case["gate_params"]) if "gate_params" in case else None


def hist_to_bits(h64):
    """The oracle's published history holds copies of bf16 values: back to bits."""
    return oracle.round_f64_to_bf16_bits(h64)


def node_rows_mask(case):
    B, R = case["B"], case["cfg"].R
    m = np.zeros((B, R), bool)
    for b in range(B):
        m[b, case["node_row"][b]] = True
    return m


def straddle_rows(case, y_gpu, y_ref):
    """Output rows [B][R][Hv] and committed states [B][Hv] downstream of a conv
    element where the device's bf16 rounding differs from the oracle's (a value
    straddling a rounding boundary): the node's own row and its descendants'
    rows, for the value heads that read the differing channel."""
    cfg = case["cfg"]
    B, N, R, D, Hv, Hqk = case["B"], cfg.N, cfg.R, cfg.D, cfg.Hv, cfg.Hqk
    out_mask = np.zeros((B, R, Hv), bool)
    state_mask = np.zeros((B, Hv), bool)
    diff = (y_gpu != y_ref)
    from oracle.closed_form import ancestors
    for b in range(B):
        rows = case["node_row"][b]
        anc = ancestors(case["parent"][b])
        path = set(case["path"][b, :case["path_len"][b]].tolist())
        for i in range(N):
            cs = np.nonzero(diff[b, rows[i]])[0]
            if cs.size == 0:
                continue
            heads = set()
            for c in cs:
                if c < 2 * Hqk * D:
                    gq = (c % (Hqk * D)) // D
                    heads |= {h for h in range(Hv) if h * Hqk // Hv == gq}
                else:
                    heads.add((c - 2 * Hqk * D) // D)
            hs = sorted(heads)
            for i2 in range(N):
                if i2 == i or i in anc[i2]:
                    out_mask[b, rows[i2], hs] = True
            if i in path:
                state_mask[b, hs] = True
    return out_mask, state_mask


# --------------------------------------------------------------------------
# the fused steady-state step: commit of step 1's accepted path, then the
# conv and verify of step 2's tree (same requests, pool and history)
# --------------------------------------------------------------------------

def two_step_case(cfg, seed, B=None, extra_slots=0, packing="perm", conv_values="normal"):
    """Two consecutive steps of one layer: step 2 has its own trees, rows,
    operands and paths, and the requests' pool slots, history and conv
    weights of step 1."""
    c1 = gi.make_case(cfg, seed=seed, B=B, extra_slots=extra_slots, packing=packing,
                      conv_values=conv_values)
    c2 = gi.make_case(cfg, seed=seed + 7919, B=B, extra_slots=extra_slots, packing=packing,
                      conv_values=conv_values)
    # the pool, the history and the conv weights belong to the layer: the
    # same at both steps
    for key in ("pool", "state_idx", "P", "hist", "w", "bias"):
        if key in c1:
            c2[key] = c1[key]
    return c1, c2


def _qkv_of(cfg, B, ybits):
    R, D, Hv, Hqk = cfg.R, cfg.D, cfg.Hv, cfg.Hqk
    q = ybits[:, :, :Hqk * D].reshape(B, R, Hqk, D)
    k = ybits[:, :, Hqk * D:2 * Hqk * D].reshape(B, R, Hqk, D)
    v = ybits[:, :, 2 * Hqk * D:].reshape(B, R, Hv, D)
    return q, k, v


def run_oracle_two_steps(c1, c2):
    """The oracle: commit step 1's path (with the history publication), then
    step 2's conv and verify from the committed state and history."""
    cfg = c1["cfg"]
    R, Hv, Hqk = cfg.R, cfg.Hv, cfg.Hqk
    W = cfg.conv_W if cfg.conv_W > 0 else 1
    B = c1["B"]
    d1 = oracle.desc_build(c1["parent"], c1["node_row"], R, W)
    d2 = oracle.desc_build(c2["parent"], c2["node_row"], R, W)
    res = dict(err=d1["err"] | d2["err"], status1=d1["status"], status2=d2["status"])
    norm = cfg.norm_qk if cfg.conv_W > 0 else False
    if cfg.conv_W > 0:
        y1, e = oracle.conv(c1["node_row"], d1["conv_src"], d1["status"], c1["x"], c1["hist"],
                            c1["state_idx"], c1["w"], c1.get("bias"), cfg.act, R, cfg.conv_C, W)
        res["err"] |= e
        y1b = np.where(np.isnan(y1), NAN_BF16, oracle.round_f64_to_bf16_bits(y1)).astype(np.uint16)
        q1, k1, v1 = _qkv_of(cfg, B, y1b)
        res["y1"] = y1b
    else:
        k1, v1 = c1["k"], c1["v"]
    a1, b1 = oracle_gates(c1)
    pool, hist, e = oracle.commit(c1["parent"], c1["node_row"], d1["status"], c1["path"],
                                  c1["path_len"], k1, v1, a1, b1, c1["pool"],
                                  c1["state_idx"], Hqk, Hv, norm, x=c1.get("x"), hist=c1.get("hist"),
                                  W=W)
    res["err"] |= e
    res["pool"] = pool
    if cfg.conv_W > 0:
        res["hist"] = hist
        hbits = oracle.round_f64_to_bf16_bits(hist)
        y2, e = oracle.conv(c2["node_row"], d2["conv_src"], d2["status"], c2["x"], hbits,
                            c2["state_idx"], c2["w"], c2.get("bias"), cfg.act, R, cfg.conv_C, W)
        res["err"] |= e
        y2b = np.where(np.isnan(y2), NAN_BF16, oracle.round_f64_to_bf16_bits(y2)).astype(np.uint16)
        q2, k2, v2 = _qkv_of(cfg, B, y2b)
        res["y2"] = y2b
    else:
        q2, k2, v2 = c2["q"], c2["k"], c2["v"]
    a2, b2 = oracle_gates(c2)
    out, e = oracle.verify(c2["parent"], c2["node_row"], d2["status"], q2, k2, v2, a2, b2, pool,
                           c2["state_idx"], Hqk, Hv, norm)
    res["err"] |= e
    res["out"] = out
    return res


def run_gpu_two_steps(c1, c2, fused=True, y1_override=None, y2_override=None, flags=0):
    """Step 1's recorded operands (its conv output for conv configs), then
    step 2 through the fused calls (conv_ancestry_gather_publish and
    gdn_tree_commit_verify), or through the separate calls (commit with the
    history, conv, verify) when fused is False.  With y*_override the
    device's own conv outputs are kept in res but the GDN stages read the
    given ones (stage-wise parity)."""
    import torch
    import tree_speculative_verification_gdn_amd as g

    cfg = c1["cfg"]
    B, R, D, Hv, Hqk = c1["B"], cfg.R, cfg.D, cfg.Hv, cfg.Hqk
    W = cfg.conv_W if cfg.conv_W > 0 else 1
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    d1 = g.TreeDesc(to_dev(c1["parent"]), to_dev(c1["node_row"]), R, W)
    d2 = g.TreeDesc(to_dev(c2["parent"]), to_dev(c2["node_row"]), R, W)
    g.gdn_tree_desc_build(d1, err)
    pool = to_dev(c1["pool"])
    sidx = to_dev(c1["state_idx"])
    a1, b1 = to_dev(c1["alpha"]), to_dev(c1["beta"])
    a2, b2 = to_dev(c2["alpha"]), to_dev(c2["beta"])
    gp = dev_gate_params(c1)  # the layer's gate parameters (both steps)
    p1, l1 = to_dev(c1["path"]), to_dev(c1["path_len"])
    if fused:  # the fused calls take the path resolved; step 2's descriptor in the same launch
        prow = torch.full(p1.shape, -7, dtype=torch.int32, device="cuda")
        pn = torch.full((B,), -9, dtype=torch.int32, device="cuda")
        g.gdn_step_prepare(d2, d1, p1, l1, sidx, int(pool.shape[0]), prow, pn, err)
    else:
        g.gdn_tree_desc_build(d2, err)
    res = {}
    if cfg.conv_W > 0:
        C = cfg.conv_C
        flags |= g.GDN_F_NORM_QK if cfg.norm_qk else 0
        hist = to_dev(c1["hist"])
        w1, w2 = to_dev(c1["w"]), to_dev(c2["w"])
        x1, x2 = to_dev(c1["x"]), to_dev(c2["x"])
        y1 = torch.full((B, R, C), float("nan"), dtype=torch.bfloat16, device="cuda")
        bias = dev_bias(c1)  # the layer's (both steps)
        g.conv_ancestry_gather(d1, x1, hist, sidx, w1, bias, y1, cfg.act, err)
        res["y1"] = bits(y1)
        if y1_override is not None:
            y1.copy_(to_dev(np.where(y1_override == NAN_BF16, res["y1"], y1_override).astype(np.uint16)))
        q1 = y1[:, :, :Hqk * D].unflatten(-1, (Hqk, D))
        k1 = y1[:, :, Hqk * D:2 * Hqk * D].unflatten(-1, (Hqk, D))
        v1 = y1[:, :, 2 * Hqk * D:].unflatten(-1, (Hv, D))
        y2 = torch.full((B, R, C), float("nan"), dtype=torch.bfloat16, device="cuda")
        if fused:
            g.conv_ancestry_gather_publish(d2, x2, hist, sidx, w2, bias, y2, cfg.act, d1, prow, pn,
                                           x1, err)
        else:
            g.gdn_tree_commit(d1, p1, l1, k1, v1, a1, b1, pool, sidx, err, Hqk=Hqk,
                              flags=flags & g.GDN_F_NORM_QK, x=x1, hist=hist, gate_params=gp)
            g.conv_ancestry_gather(d2, x2, hist, sidx, w2, bias, y2, cfg.act, err)
        res["y2"] = bits(y2)
        if y2_override is not None:
            y2.copy_(to_dev(np.where(y2_override == NAN_BF16, res["y2"], y2_override).astype(np.uint16)))
        q2 = y2[:, :, :Hqk * D].unflatten(-1, (Hqk, D))
        k2 = y2[:, :, Hqk * D:2 * Hqk * D].unflatten(-1, (Hqk, D))
        v2 = y2[:, :, 2 * Hqk * D:].unflatten(-1, (Hv, D))
    else:
        hist = None
        k1, v1 = to_dev(c1["k"]), to_dev(c1["v"])
        q2, k2, v2 = to_dev(c2["q"]), to_dev(c2["k"]), to_dev(c2["v"])
    out = torch.full((B, R, Hv, D), float("nan"), dtype=torch.float32, device="cuda")
    if fused:
        g.gdn_tree_commit_verify(d2, q2, k2, v2, a2, b2, pool, sidx, out, d1, prow, pn, k1, v1, a1,
                                 b1, err, flags=flags, gate_params=gp)
    else:
        if cfg.conv_W == 0:
            g.gdn_tree_commit(d1, p1, l1, k1, v1, a1, b1, pool, sidx, err, Hqk=Hqk,
                              flags=flags & g.GDN_F_NORM_QK, gate_params=gp)
        g.gdn_tree_verify(d2, q2, k2, v2, a2, b2, pool, sidx, out, err, flags=flags, gate_params=gp)
    torch.cuda.synchronize()
    res.update(err=int(err.item()), out=out.cpu().numpy(), pool=pool.cpu().numpy(),
               status1=d1.status.cpu().numpy(), status2=d2.status.cpu().numpy())
    if hist is not None:
        res["hist"] = bits(hist)
    return res


def run_gpu_layer(c1, c2, flags=0, with_y=True, prepare=False):
    """Step 2 of a conv configuration through the one-launch layer step:
    step 2's descriptor and the resolution of step 1's path (two calls, or
    gdn_step_prepare with prepare=True), then gdn_layer_step with step 1's
    conv input, gates and history (hist_in) and a separate hist_out."""
    import torch
    import tree_speculative_verification_gdn_amd as g

    cfg = c1["cfg"]
    B, R, D, Hv, Hqk, C, W = c1["B"], cfg.R, cfg.D, cfg.Hv, cfg.Hqk, cfg.conv_C, cfg.conv_W
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    d1 = g.TreeDesc(to_dev(c1["parent"]), to_dev(c1["node_row"]), R, W)
    d2 = g.TreeDesc(to_dev(c2["parent"]), to_dev(c2["node_row"]), R, W)
    g.gdn_tree_desc_build(d1, err)
    pool = to_dev(c1["pool"])
    sidx = to_dev(c1["state_idx"])
    P = int(pool.shape[0])
    path = to_dev(c1["path"])
    Lmax = int(path.shape[1])
    path_rows = torch.full((B, Lmax), -7, dtype=torch.int32, device="cuda")
    path_n = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    if prepare:
        g.gdn_step_prepare(d2, d1, path, to_dev(c1["path_len"]), sidx, P, path_rows, path_n, err)
    else:
        g.gdn_tree_desc_build(d2, err)
        g.gdn_path_resolve(d1, path, to_dev(c1["path_len"]), sidx, P, path_rows, path_n, err)
    hist_in = to_dev(c1["hist"])
    hist_out = torch.full_like(hist_in, float("nan"))
    out = torch.full((B, R, Hv, D), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((B, R, C), float("nan"), dtype=torch.bfloat16, device="cuda") if with_y else None
    flags |= g.GDN_F_NORM_QK if cfg.norm_qk else 0
    g.gdn_layer_step(d2, to_dev(c2["x"]), to_dev(c2["w"]), dev_bias(c1), cfg.act, hist_in, hist_out,
                     to_dev(c2["alpha"]), to_dev(c2["beta"]), pool, sidx, out, d1, to_dev(c1["x"]),
                     to_dev(c1["alpha"]), to_dev(c1["beta"]), path_rows, path_n, err, Hqk,
                     flags=flags, y=y, gate_params=dev_gate_params(c1))
    torch.cuda.synchronize()
    res = dict(err=int(err.item()), out=out.cpu().numpy(), pool=pool.cpu().numpy(),
               hist_out=bits(hist_out), hist_in=bits(hist_in), path_n=path_n.cpu().numpy(),
               path_rows=path_rows.cpu().numpy(), status2=d2.status.cpu().numpy(),
               desc2=[t.cpu().numpy() for t in (d2.depth, d2.anc, d2.conv_src, d2.status)])
    if with_y:
        res["y2"] = bits(y)
    return res
