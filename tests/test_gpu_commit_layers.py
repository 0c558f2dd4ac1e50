"""GPU parity of gdn_tree_commit_layers: one launch that replays the accepted
path into every layer's state pool (same trees, paths and slots for all
layers; per-layer k, v, gates and pools at fixed strides).

Bars: every layer's pool bit-identical to gdn_tree_commit called on that
layer alone (the same kernel arithmetic); committed states within 2e-3 of the
oracle's commit (max relative per state row); skipped requests and unused
slots bit-unchanged; error bits equal to the oracle's.
"""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from harness import max_rel_rows, subset, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _g():
    import tree_speculative_verification_gdn_amd as g
    return g


def layers_case(cfg, seed, L, B=None, extra_slots=0):
    """L layers over one set of trees, paths and slots (layer 0's); each layer
    draws its own k, v, gates and pool.  Pool slots no request uses hold NaN."""
    c0 = gi.make_case(cfg, seed=seed, layer=0, B=B, extra_slots=extra_slots)
    per = [gi.make_case(cfg, seed=seed, layer=l, B=B, extra_slots=extra_slots, poison=False)
           for l in range(L)]
    unused = np.ones(c0["P"], bool)
    unused[c0["state_idx"]] = False
    pools = []
    for c in per:
        p = c["pool"].copy()
        p[unused] = np.nan
        pools.append(p)
    rows_used = np.zeros((c0["B"], cfg.R), bool)
    for b in range(c0["B"]):
        rows_used[b, c0["node_row"][b]] = True
    out = dict(c0)
    for key in ("k", "v", "alpha", "beta"):
        arrs = []
        for c in per:
            a = c[key].copy()
            a[~rows_used] = np.nan if a.dtype != np.uint16 else 0x7FC0
            arrs.append(a)
        out[key] = np.stack(arrs)
    out["pool"] = np.stack(pools)
    out["L"] = L
    return out


def layer_slice(lc, l):
    c = dict(lc)
    for key in ("k", "v", "alpha", "beta", "pool"):
        c[key] = lc[key][l]
    return c


def oracle_commit(c, norm):
    cfg = c["cfg"]
    d = oracle.desc_build(c["parent"], c["node_row"], cfg.R, 1)
    pool, _, e = oracle.commit(c["parent"], c["node_row"], d["status"], c["path"], c["path_len"],
                               c["k"], c["v"], c["alpha"], c["beta"], c["pool"], c["state_idx"],
                               cfg.Hqk, cfg.Hv, norm)
    return pool, d["err"] | e


def run_layers(lc, flags=0, pad_slots=0, pad_rows=0):
    """gdn_tree_commit_layers on the device; with pad_slots / pad_rows the
    layers sit at larger strides than their extent (the extra slots / rows
    are NaN and must stay so).  Returns (pools [L][P]..., err)."""
    import torch
    g = _g()
    cfg = lc["cfg"]
    L, B, R = lc["L"], lc["B"], cfg.R
    desc = g.TreeDesc(to_dev(lc["parent"]), to_dev(lc["node_row"]), R, 1, B=B)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.gdn_tree_desc_build(desc, err)

    def padded(a, extra):
        t = to_dev(a)
        if extra == 0:
            return t
        shape = list(t.shape)
        shape[1] += extra
        big = torch.full(shape, float("nan"), dtype=t.dtype, device="cuda")
        big[:, :a.shape[1]] = t
        return big[:, :a.shape[1]]

    # rows of k / v: pad along the batch axis keeps each layer's [B, R, H, D] dense
    k, v = padded(lc["k"], pad_rows), padded(lc["v"], pad_rows)
    alpha, beta = padded(lc["alpha"], pad_rows), padded(lc["beta"], pad_rows)
    pool_full = padded(lc["pool"], pad_slots)
    g.gdn_tree_commit_layers(desc, to_dev(lc["path"]), to_dev(lc["path_len"]), k, v, alpha, beta,
                             pool_full, to_dev(lc["state_idx"]), err, flags=flags)
    torch.cuda.synchronize()
    base = pool_full._base if pool_full._base is not None else pool_full
    if pad_slots:
        assert torch.isnan(base[:, lc["P"]:]).all()
    return pool_full.cpu().numpy(), int(err.item())


def run_per_layer(lc, flags=0):
    import torch
    g = _g()
    cfg = lc["cfg"]
    B, R = lc["B"], cfg.R
    desc = g.TreeDesc(to_dev(lc["parent"]), to_dev(lc["node_row"]), R, 1, B=B)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.gdn_tree_desc_build(desc, err)
    path, plen, sidx = to_dev(lc["path"]), to_dev(lc["path_len"]), to_dev(lc["state_idx"])
    pools = []
    for l in range(lc["L"]):
        pool = to_dev(lc["pool"][l])
        g.gdn_tree_commit(desc, path, plen, to_dev(lc["k"][l]), to_dev(lc["v"][l]),
                          to_dev(lc["alpha"][l]), to_dev(lc["beta"][l]), pool, sidx, err,
                          Hqk=cfg.Hqk, flags=flags)
        pools.append(pool)
    torch.cuda.synchronize()
    return np.stack([p.cpu().numpy() for p in pools]), int(err.item())


def _check(lc, gp, gerr, norm, skipped=()):
    sidx = lc["state_idx"]
    unused = np.setdiff1d(np.arange(lc["P"]), sidx)
    for l in range(lc["L"]):
        c = layer_slice(lc, l)
        op, oerr = oracle_commit(c, norm)
        assert gerr == oerr, (gerr, oerr)
        rel = max_rel_rows(gp[l][sidx], op[sidx], 2)
        assert rel <= TOL, f"layer {l}: state max rel {rel:.3e}"
        assert np.array_equal(gp[l][unused], lc["pool"][l][unused], equal_nan=True)
        for b in skipped:
            assert np.array_equal(gp[l][sidx[b]], lc["pool"][l][sidx[b]])


@pytest.mark.parametrize("norm", [False, True])
def test_three_layers_tree27_against_oracle_and_per_layer(norm):
    g = _g()
    cfg = gi.CONFIGS[3]
    lc = layers_case(cfg, seed=31, L=3, B=6, extra_slots=2)
    flags = g.GDN_F_NORM_QK if norm else 0
    gp, gerr = run_layers(lc, flags=flags)
    sp, serr = run_per_layer(lc, flags=flags)
    assert gerr == serr == 0
    assert np.array_equal(gp, sp, equal_nan=True)
    _check(lc, gp, gerr, norm)


def test_layer_strides_larger_than_the_layers():
    # each layer's operands and pool followed by unused rows / slots
    cfg = gi.CONFIGS[2]
    lc = layers_case(cfg, seed=5, L=4, B=5, extra_slots=1)
    gp, gerr = run_layers(lc, pad_slots=3, pad_rows=2)
    sp, _ = run_per_layer(lc)
    assert np.array_equal(gp, sp, equal_nan=True)
    _check(lc, gp, gerr, False)


def test_f32_small_tree_many_layers():
    cfg = gi.CONFIGS[1]
    lc = layers_case(cfg, seed=9, L=7, B=3, extra_slots=1)
    gp, gerr = run_layers(lc)
    sp, _ = run_per_layer(lc)
    assert np.array_equal(gp, sp, equal_nan=True)
    _check(lc, gp, gerr, False)


def test_malformed_requests_skipped_in_every_layer():
    g = _g()
    cfg = gi.CONFIGS[3].replace(B=8)
    lc = layers_case(cfg, seed=21, L=3, extra_slots=2)
    lc["parent"][1, 4] = 20                      # malformed tree
    lc["path"][3, 0] = lc["path"][3, 1] if lc["path_len"][3] > 1 else 5
    lc["path_len"][3] = max(int(lc["path_len"][3]), 1)   # path not a parent chain
    lc["path_len"][4] = cfg.Lmax + 1             # longer than Lmax
    lc["path_len"][0] = 0                        # nothing accepted
    lc["state_idx"][5] = lc["state_idx"][6]      # shared slot
    gp, gerr = run_layers(lc)
    sp, serr = run_per_layer(lc)
    assert gerr == serr == (g.GDN_EV_PARENT | g.GDN_EV_PATH | g.GDN_EV_STATE)
    assert np.array_equal(gp, sp, equal_nan=True)
    _check(lc, gp, gerr, False, skipped=(0, 1, 3, 4, 5, 6))


def test_tree64_b256_four_of_48_layers_sampled():
    # the 64-node workload at full batch: bitwise against per-layer commits,
    # the oracle on a sample of requests (including the longest paths)
    cfg = gi.CONFIGS[5]
    lc = layers_case(cfg, seed=2026, L=4)
    gp, gerr = run_layers(lc)
    assert gerr == 0
    sp, _ = run_per_layer(lc)
    assert np.array_equal(gp, sp, equal_nan=True)
    order = np.argsort(-lc["path_len"], kind="stable")
    bs = np.unique(np.concatenate([order[:2], [0, 100, 255]]))
    assert lc["path_len"][bs].max() > 8
    for l in (0, 3):
        sub = subset(layer_slice(lc, l), bs)
        op, oerr = oracle_commit(sub, False)
        assert oerr == 0
        rel = max_rel_rows(gp[l][lc["state_idx"][bs]], op, 2)
        assert rel <= TOL, f"layer {l}: state max rel {rel:.3e}"
