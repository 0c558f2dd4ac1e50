"""Pins of the oracle's tree attention and KV publication (oracle/attention.py)
against what fixes them independently of the oracle's own code:
- every root-to-leaf path equals ordinary causal attention over (prefix ++
  the path's tokens in order), computed by torch's scaled_dot_product_attention
  in float64 on the CPU (a library routine) -- this covers chains, the GQA
  head mapping, the scale, and the physical slot map;
- a node never sees a sibling branch (changing another branch's keys and
  values leaves its output bit-identical), nor padding rows;
- a single visible key returns its value; equal keys average the values;
- publication is a gather through the slot map with every source read first
  (checked against a copy made before the move)."""
import numpy as np
import pytest
import torch

from oracle.attention import EV_CTX, kv_publish, root_path, tree_attention

import gdn_inputs as gi


def _case(seed, B=2, N=11, R=14, Hq=4, Hkv=2, D=16, ctx=(5, 9), S=32, bmax=3, depth=4):
    g = np.random.default_rng(seed)
    cfg = gi.CONFIGS[3].replace(N=N, R=R, bmax=bmax, depth_max=depth)
    parent = np.stack([gi.random_tree(np.random.default_rng(seed * 7 + b), N, bmax, depth)
                       for b in range(B)]).astype(np.int32)
    node_row = np.stack([g.permutation(R)[:N] for _ in range(B)]).astype(np.int32)
    q = g.standard_normal((B, N, Hq, D))
    k = g.standard_normal((B, S, Hkv, D))
    v = g.standard_normal((B, S, Hkv, D))
    return dict(cfg=cfg, parent=parent, node_row=node_row, q=q, k=k, v=v,
                ctx=np.array(ctx[:B], np.int32), R=R, Hq=Hq, Hkv=Hkv, D=D)


def _run(c, scale=None):
    scale = 1.0 / np.sqrt(c["D"]) if scale is None else scale
    status = np.zeros(c["parent"].shape[0], np.int32)
    return tree_attention(c["parent"], c["node_row"], status, c["q"], c["k"], c["v"], c["ctx"],
                          c["R"], c["Hq"], c["Hkv"], scale)


def _sdpa_causal(q, k, v, scale):
    """torch causal attention for one sequence: q [T][Hq][D], k, v [T][Hkv][D]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1)).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_every_root_path_is_causal_attention(seed):
    c = _case(seed)
    scale = 0.37
    out, err = _run(c, scale)
    assert err == 0
    B, N = c["parent"].shape
    for b in range(B):
        L = int(c["ctx"][b])
        for i in range(N):
            path = root_path(c["parent"][b], i)
            # the sequence: prefix tokens, then the path's candidates in order
            # (queries of prefix positions are irrelevant: take node i's query
            # at the last position)
            slots = list(range(L)) + [L + int(c["node_row"][b, a]) for a in path]
            T = len(slots)
            qs = np.zeros((T, c["Hq"], c["D"]))
            qs[-1] = c["q"][b, i]
            o = _sdpa_causal(qs, c["k"][b, slots], c["v"][b, slots], scale)
            np.testing.assert_allclose(out[b, i], o[-1], rtol=1e-12, atol=1e-12)


def test_chain_tree_is_causal_decoding():
    c = _case(4, B=1, N=8, R=8, ctx=(6,))
    c["parent"][0] = np.arange(-1, 7)
    c["node_row"][0] = np.arange(8)
    out, _ = _run(c)
    L = 6
    qs = np.concatenate([np.zeros((L, c["Hq"], c["D"])), c["q"][0]])
    o = _sdpa_causal(qs, c["k"][0, :L + 8], c["v"][0, :L + 8], 1.0 / np.sqrt(c["D"]))
    np.testing.assert_allclose(out[0], o[L:], rtol=1e-12, atol=1e-12)


def test_siblings_and_padding_are_invisible():
    c = _case(5, B=1, N=11, R=16)
    out, _ = _run(c)
    par, rows = c["parent"][0], c["node_row"][0]
    i = 10
    on_path = set(root_path(par, i))
    c2 = dict(c)
    c2["k"], c2["v"] = c["k"].copy(), c["v"].copy()
    L = int(c["ctx"][0])
    for a in range(11):
        if a not in on_path:
            c2["k"][0, L + rows[a]] = 1e3
            c2["v"][0, L + rows[a]] = np.nan
    unused = sorted(set(range(16)) - set(int(r) for r in rows))
    for r in unused:
        c2["k"][0, L + r] = np.nan
        c2["v"][0, L + r] = np.nan
    c2["k"][0, L + 16:] = np.nan  # past the tree's rows
    out2, _ = _run(c2)
    assert np.array_equal(out[0, i], out2[0, i])


def test_single_key_and_equal_keys():
    c = _case(6, B=1, N=1, R=1, ctx=(0,))
    c["parent"][0, 0] = -1
    c["node_row"][0, 0] = 0
    out, _ = _run(c)
    np.testing.assert_allclose(out[0, 0], np.repeat(c["v"][0, 0], 2, axis=0), rtol=0, atol=0)
    c = _case(7, B=1, ctx=(9,))
    c["k"][:] = 0.25
    out, _ = _run(c)
    L = 9
    for i in range(c["parent"].shape[1]):
        slots = list(range(L)) + [L + int(c["node_row"][0, a]) for a in root_path(c["parent"][0], i)]
        mean = c["v"][0, slots].mean(axis=0)
        np.testing.assert_allclose(out[0, i], np.repeat(mean, 2, axis=0), rtol=1e-13, atol=1e-14)


def test_context_out_of_range_is_reported_and_skipped():
    c = _case(8, ctx=(5, 19), S=32, R=14)  # 19 + 14 > 32
    out, err = _run(c)
    assert err == EV_CTX
    assert np.isnan(out[1]).all() and not np.isnan(out[0]).any()


def test_publication_gathers_through_the_slot_map():
    g = np.random.default_rng(9)
    B, S, Hkv, D, R, Lmax = 3, 24, 2, 8, 10, 6
    k = g.standard_normal((B, S, Hkv, D))
    v = g.standard_normal((B, S, Hkv, D))
    ctx = np.array([3, 7, 0], np.int32)
    path_rows = np.array([[4, 0, 9, 1, 0, 0], [0, 1, 2, 3, 0, 0], [5, 4, 3, 2, 1, 0]], np.int32)
    path_n = np.array([4, 4, 6], np.int32)
    k2, v2, err = kv_publish(path_rows, path_n, k, v, ctx, R)
    assert err == 0
    for b in range(B):
        L, n = int(ctx[b]), int(path_n[b])
        for j in range(n):
            assert np.array_equal(k2[b, L + j], k[b, L + path_rows[b, j]])
            assert np.array_equal(v2[b, L + j], v[b, L + path_rows[b, j]])
        rest = [p for p in range(S) if not (L <= p < L + n)]
        assert np.array_equal(k2[b, rest], k[b, rest])
    # rows already in place: nothing moves
    assert np.array_equal(k2[1], k[1])
    # nothing accepted, or a context past the end: untouched (the latter reported)
    k3, _, err = kv_publish(path_rows, np.array([0, -1, 2], np.int32), k, v, np.array([3, 7, 20]), R)
    assert err == EV_CTX and np.array_equal(k3, k)
