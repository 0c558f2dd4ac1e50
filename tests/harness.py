"""Shared helpers for the parity tests: upload a seeded case, run the HIP path
through the binding, run the oracle on the same host inputs, compare.

The oracle never sees a value the GPU produced: for conv configurations it
computes its own conv output and rounds it to bf16 itself.
"""
from __future__ import annotations

import numpy as np

import gdn_inputs as gi
import oracle

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
        res["rc_conv"] = g.conv_ancestry_gather(desc, x, hist, sidx, w, None, y, cfg.act, err,
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
    res["rc_verify"] = g.gdn_tree_verify(desc, q, k, v, alpha, beta, pool, sidx, out, err,
                                         flags=vflags, raise_on_error=raise_on_error)
    if commit:
        res["rc_commit"] = g.gdn_tree_commit(desc, to_dev(case["path"]), to_dev(case["path_len"]),
                                             k, v, alpha, beta, pool, sidx, err, Hqk=Hqk,
                                             flags=flags & g.GDN_F_NORM_QK, x=x, hist=hist,
                                             raise_on_error=raise_on_error)
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
                           case["w"], None, cfg.act, R, cfg.conv_C, W, shared=shared)
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
    out, e = oracle.verify(parent, rows, d["status"], q, k, v, case["alpha"], case["beta"],
                           case["pool"], case["state_idx"], Hqk, Hv, norm, shared=shared)
    res["err"] |= e
    res["out"] = out
    if commit:
        pool, hist, e = oracle.commit(parent, rows, d["status"], case["path"], case["path_len"], k, v,
                                      case["alpha"], case["beta"], case["pool"], case["state_idx"],
                                      Hqk, Hv, norm, x=case.get("x"), hist=case.get("hist"), W=W,
                                      shared=shared)
        res["err"] |= e
        res["pool"] = pool
        if hist is not None:
            res["hist"] = hist
    return res


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
