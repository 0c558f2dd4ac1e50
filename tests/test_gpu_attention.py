"""GPU parity of the tree attention and the accepted path's KV publication
against the fp64 oracle (oracle/attention.py) on the same seeded inputs.

Bars: outputs within 2e-3 of the oracle in the max-relative-per-row metric
(each (request, node, head) row normalised by its largest magnitude); rows of
skipped requests untouched (NaN); error bits equal; the publication
bit-exact (a data movement).  The cache holds NaN past each request's
candidates and in candidate rows no node occupies: nothing may read them."""
import numpy as np
import pytest

import gdn_inputs as gi
from harness import max_rel_rows, to_dev
from oracle.attention import kv_publish as oracle_kv_publish
from oracle.attention import tree_attention as oracle_tree_attention

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _g():
    import tree_speculative_verification_gdn_amd as g
    return g


def run_attention(c, splits, out_bf16=False, shared=False, scale=None, ctx=None):
    import torch
    g = _g()
    B, N, Hq, D = c["B"], c["N"], c["Hq"], c["D"]
    parent = c["parent"][:1] if shared else c["parent"]
    rows = c["node_row"][:1] if shared else c["node_row"]
    desc = g.TreeDesc(to_dev(parent), to_dev(rows), c["R"], 1, B=B, shared=shared)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.gdn_tree_desc_build(desc, err)
    nbytes = g.gdn_tree_attention_workspace_bytes(B, N, Hq, D, splits)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    odt = torch.bfloat16 if out_bf16 else torch.float32
    out = torch.full((B, N, Hq, D), float("nan"), dtype=odt, device="cuda")
    ctx = c["ctx"] if ctx is None else ctx
    g.gdn_tree_attention(desc, to_dev(c["q"]), to_dev(c["k"]), to_dev(c["v"]), to_dev(ctx), out, ws, err,
                         splits=splits, scale=scale, flags=g.GDN_F_OUT_BF16 if out_bf16 else 0)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    return o, int(err.item()), desc.status.cpu().numpy()


def oracle(c, status, shared=False, scale=None, nodes=None, ctx=None):
    scale = 1.0 / np.sqrt(c["D"]) if scale is None else scale
    parent = c["parent"][:1] if shared else c["parent"]
    rows = c["node_row"][:1] if shared else c["node_row"]
    return oracle_tree_attention(parent, rows, status, c["q"], c["k"], c["v"],
                                 c["ctx"] if ctx is None else ctx, c["R"], c["Hq"], c["Hkv"],
                                 scale, shared=shared, nodes=nodes)


def _cmp(go, oo, tol=TOL):
    m = ~np.isnan(oo[..., 0])
    assert np.isnan(go[~m]).all()
    rel = max_rel_rows(go[m], oo[m], 1)
    assert rel <= tol, f"attention max rel {rel:.3e}"
    return rel


@pytest.mark.parametrize("D", [128, 256])
def test_small_trees_several_partitions(D):
    c = gi.make_attention_case(11, B=3, N=11, R=14, Hq=8, Hkv=2, D=D, ctx=[0, 37, 100], S=128)
    go, err, st = run_attention(c, splits=3)
    oo, oerr = oracle(c, st)
    assert err == oerr == 0
    _cmp(go, oo)


def test_tree27_long_prefix_bf16_output():
    c = gi.make_attention_case(12, B=2, N=27, R=32, Hq=16, Hkv=2, D=256, ctx=[1000, 2047], S=2100,
                               packing="bfs")
    go, err, st = run_attention(c, splits=8, out_bf16=True)
    oo, _ = oracle(c, st)
    assert err == 0
    # the fp32 bar plus the output's own rounding to bf16 (half an ulp, 2^-9
    # relative), as the GDN outputs' bf16 test
    _cmp(go, oo, tol=TOL + 2.0 ** -9)
    go32, _, _ = run_attention(c, splits=8)
    _cmp(go32, oo)


@pytest.mark.parametrize("splits", [1, 2, 7, 64])
def test_partition_counts_agree(splits):
    # more partitions than prefix tiles leaves some empty
    c = gi.make_attention_case(13, B=2, N=20, R=24, Hq=4, Hkv=1, D=128, ctx=[300, 5], S=340)
    go, err, st = run_attention(c, splits=splits)
    oo, _ = oracle(c, st)
    _cmp(go, oo)


def test_wide_tree_two_heads_per_workgroup():
    # N > 32: the N rows of two query heads per workgroup
    c = gi.make_attention_case(14, B=2, N=40, R=48, Hq=4, Hkv=4, D=128, ctx=[64, 250], S=320,
                               bmax=4, depth_max=8)
    go, err, st = run_attention(c, splits=4)
    oo, _ = oracle(c, st)
    _cmp(go, oo)


def test_odd_group_size_and_scale():
    # three query heads per kv head: pairs of 2 and 1
    c = gi.make_attention_case(15, B=2, N=9, R=12, Hq=6, Hkv=2, D=128, ctx=[17, 64], S=96)
    go, err, st = run_attention(c, splits=2, scale=0.05)
    oo, _ = oracle(c, st, scale=0.05)
    _cmp(go, oo)


@pytest.mark.parametrize("scale", [1e-4, 2.0])
def test_extreme_scales(scale):
    # a large scale makes each row's softmax nearly one-hot, so the rows'
    # reference maxima move on many tiles (the cross-lane maximum and the
    # rescale run often); a tiny one makes the weights nearly uniform and the
    # references never move after the first tile
    c = gi.make_attention_case(31, B=2, N=11, R=16, Hq=4, Hkv=2, D=256, ctx=[700, 300], S=720)
    go, err, st = run_attention(c, splits=3, scale=scale)
    assert err == 0
    oo, _ = oracle(c, st, scale=scale)
    _cmp(go, oo)


# seeded random shapes: tree size, candidate rows, head grouping, head
# dimension, context lengths (0 and lengths that end inside a tile among
# them), partition count and softmax scale
_SWEEP = [
    # seed, B, N, R, Hq, Hkv, D, ctx, S, splits, scale
    (101, 2, 1, 1, 2, 1, 128, [0, 33], 40, 1, 0.09),
    (102, 3, 7, 8, 8, 2, 256, [31, 32, 95], 110, 5, 0.0625),
    (103, 1, 40, 48, 4, 4, 128, [257], 320, 8, 0.3),
    (104, 2, 64, 64, 2, 2, 256, [1, 200], 270, 3, 0.02),
    (105, 2, 23, 30, 12, 4, 128, [63, 64], 100, 2, 0.125),
    (106, 4, 5, 16, 6, 3, 256, [0, 17, 48, 160], 180, 7, 1.0),
]


@pytest.mark.parametrize("case", _SWEEP, ids=[str(c[0]) for c in _SWEEP])
def test_random_shape_sweep(case):
    seed, B, N, R, Hq, Hkv, D, ctx, S, splits, scale = case
    c = gi.make_attention_case(seed, B=B, N=N, R=R, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, S=S)
    go, err, st = run_attention(c, splits=splits, scale=scale)
    assert err == 0
    oo, _ = oracle(c, st, scale=scale)
    _cmp(go, oo)


def test_shared_topology():
    c = gi.make_attention_case(16, B=3, N=13, R=16, Hq=4, Hkv=2, D=128, ctx=[5, 40, 77], S=100,
                               shared=True)
    go, err, st = run_attention(c, splits=2, shared=True)
    oo, _ = oracle(c, st, shared=True)
    _cmp(go, oo)


def test_bad_context_and_malformed_tree_are_skipped():
    g = _g()
    c = gi.make_attention_case(17, B=4, N=10, R=12, Hq=4, Hkv=2, D=128, ctx=[10, 20, 30, 40], S=64)
    c["parent"][1, 5] = 7          # malformed tree: no output, error from the descriptor build
    ctx = np.array([10, 60, 30, -1], np.int32)  # 60 + 12 > 64 and -1: EV_CTX
    go, err, st = run_attention(c, splits=2, ctx=ctx)
    oo, oerr = oracle(c, st, ctx=ctx)
    assert err == g.GDN_EV_PARENT | g.GDN_EV_CTX
    assert oerr == g.GDN_EV_CTX
    assert np.isnan(go[3]).all() and np.isnan(go[1]).all()
    _cmp(go, oo)


def test_tree27_64k_prefix_sampled():
    # the benchmarked shape: one request, 64 Ki prefix positions, 16 query
    # heads over 2 kv heads, d = 256; the oracle on a sample of nodes
    c = gi.make_attention_case(2026, B=1, N=27, R=32, Hq=16, Hkv=2, D=256, ctx=[65536], S=65536 + 32,
                               packing="bfs")
    go, err, st = run_attention(c, splits=64)
    assert err == 0
    nodes = {(0, 0), (0, 5), (0, 13), (0, 26)}
    oo, _ = oracle(c, st, nodes=nodes)
    m = ~np.isnan(oo[..., 0])
    rel = max_rel_rows(go[m], oo[m], 1)
    assert rel <= TOL, f"attention max rel {rel:.3e}"
    assert not np.isnan(go).any()


@pytest.mark.parametrize("D", [128, 256])
def test_kv_publish_through_the_slot_map(D):
    import torch
    g = _g()
    c = gi.make_attention_case(18, B=5, N=14, R=16, Hq=4, Hkv=2, D=D, ctx=[0, 9, 33, 50, 4], S=72,
                               poison=False)
    # the accepted paths, resolved on the device from a previous-step tree
    rg = np.random.default_rng(18)
    Lmax = 7
    path = np.full((c["B"], Lmax), -1, np.int32)
    plen = np.zeros(c["B"], np.int32)
    for b in range(c["B"]):
        leaf = int(rg.integers(c["N"]))
        chain = []
        while leaf >= 0:
            chain.append(leaf)
            leaf = int(c["parent"][b, leaf])
        chain = chain[::-1][:Lmax]
        path[b, :len(chain)] = chain
        plen[b] = len(chain)
    plen[2] = 0                                   # nothing accepted
    ctx = c["ctx"].copy()
    ctx[4] = 60                                   # 60 + 16 > 72: EV_CTX
    desc = g.TreeDesc(to_dev(c["parent"]), to_dev(c["node_row"]), c["R"], 1, B=c["B"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.gdn_tree_desc_build(desc, err)
    sidx = torch.arange(c["B"], dtype=torch.int32, device="cuda")
    prow = torch.zeros((c["B"], Lmax), dtype=torch.int32, device="cuda")
    pn = torch.zeros(c["B"], dtype=torch.int32, device="cuda")
    g.gdn_path_resolve(desc, to_dev(path), to_dev(plen), sidx, c["B"], prow, pn, err)
    k, v = to_dev(c["k"]), to_dev(c["v"])
    g.gdn_tree_kv_publish(desc, prow, pn, k, v, to_dev(ctx), err)
    torch.cuda.synchronize()
    from harness import bits
    rows = prow.cpu().numpy()
    n = pn.cpu().numpy()
    assert (n == plen).all()
    ko, vo, oerr = oracle_kv_publish(rows, n, c["k"], c["v"], ctx, c["R"])
    assert int(err.item()) == oerr == g.GDN_EV_CTX
    assert np.array_equal(bits(k), ko)
    assert np.array_equal(bits(v), vo)


def test_repeat_runs_are_bit_identical():
    # a multi-tile partition (online-softmax rescaling across tiles) run
    # several times: every run gives the same bits and meets the bar
    c = gi.make_attention_case(19, B=1, N=20, R=20, Hq=2, Hkv=1, D=128, ctx=[64], S=90)
    first, _, st = run_attention(c, splits=1)
    oo, _ = oracle(c, st)
    _cmp(first, oo)
    for splits in (1, 2, 1, 2):
        again, _, _ = run_attention(c, splits=splits)
        if splits == 1:
            assert np.array_equal(again, first)
        _cmp(again, oo)


@pytest.mark.parametrize("profile", ["rising", "falling", "spike"])
def test_score_range_across_tiles(profile):
    # keys scaled along the prefix so that a partition's running maximum
    # climbs far past the 2^8 slack the kernel allows before it rescales the
    # output rows (rising), is set by the first tiles with later weights
    # many orders of magnitude smaller (falling), or jumps at one late key
    # (spike); about 14 tiles per partition
    c = gi.make_attention_case(30, B=2, N=11, R=14, Hq=4, Hkv=2, D=128, ctx=[900, 640], S=1000)
    k = (c["k"].astype(np.uint32) << 16).view(np.float32).copy()
    for b in range(c["B"]):
        L = int(c["ctx"][b])
        pos = np.arange(L, dtype=np.float32) / max(L - 1, 1)
        if profile == "rising":
            f = 0.25 + 5.0 * pos
        elif profile == "falling":
            f = 5.25 - 5.0 * pos
        else:
            f = np.full(L, 0.5, np.float32)
            f[(2 * L) // 3] = 12.0
        k[b, :L] *= f[:, None, None]
    c["k"] = gi.f32_to_bf16_bits(k)
    go, err, st = run_attention(c, splits=2)
    oo, oerr = oracle(c, st)
    assert err == oerr == 0
    _cmp(go, oo)


@pytest.mark.parametrize("N,R,ctx", [(1, 1, [0, 3]), (64, 64, [37, 0]), (32, 64, [100, 1])])
def test_node_count_edges(N, R, ctx):
    # a single node (its own key, or the prefix and itself), the largest tree
    # (64 nodes in 64 rows, two heads filling a workgroup's 128 query rows)
    # and 32 nodes spread over 64 rows
    c = gi.make_attention_case(20 + N, B=2, N=N, R=R, Hq=4, Hkv=2, D=128, ctx=ctx, S=max(ctx) + R + 5,
                               bmax=4, depth_max=12)
    go, err, st = run_attention(c, splits=3)
    oo, oerr = oracle(c, st)
    assert err == oerr == 0
    _cmp(go, oo)
