"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Bars: descriptor indices, status, error bits, conv history and untouched
padding / pool slots bit-exact; conv output within 1 bf16 ulp; outputs and
committed states within 2e-3 of the oracle in the max-relative-per-row metric
(each output row (b, node, h) and each committed state (b, h) is normalised by
its own largest magnitude).
"""
import os

import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from harness import (bf16_ulp_diff, hist_to_bits, max_rel_rows, node_rows_mask, run_gpu,
                     run_oracle, straddle_rows, subset)

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _g():
    import tree_speculative_verification_gdn_amd as g
    return g


def _cmp_desc(gr, orr):
    assert np.array_equal(gr["status"], orr["status"])
    assert np.array_equal(gr["depth"], orr["depth"])
    assert np.array_equal(gr["anc"], orr["anc"])
    assert np.array_equal(gr["conv_src"], orr["conv_src"])


def _cmp_out(case, gr, orr, tol=TOL):
    m = node_rows_mask(case)
    rel = max_rel_rows(gr["out"][m], orr["out"][m], 2)
    assert rel <= tol, f"output max rel {rel:.3e}"
    # padding rows never written (NaN poison survives)
    assert np.isnan(gr["out"][~m]).all()
    return rel


def _cmp_pool(case, gr, orr, tol=TOL):
    used = case["state_idx"]
    rel = max_rel_rows(gr["pool"][used], orr["pool"][used], 2)
    assert rel <= tol, f"state max rel {rel:.3e}"
    unused = np.setdiff1d(np.arange(gr["pool"].shape[0]), used)
    assert np.array_equal(gr["pool"][unused], case["pool"][unused], equal_nan=True)
    # len 0 requests: bit-unchanged
    z = used[case["path_len"] == 0]
    assert np.array_equal(gr["pool"][z], case["pool"][z])
    return rel


# ---------------------------------------------------------------------------
# descriptor
# ---------------------------------------------------------------------------

def test_desc_build_bit_exact_with_invalid_trees():
    rng = np.random.default_rng(5)
    cfg = gi.CONFIGS[5]
    case = gi.make_case(cfg, seed=11, B=40, with_pool=False, extra_slots=0)
    parent = case["parent"].copy()
    rows = case["node_row"].copy()
    parent[3, 10] = 12          # parent not before child
    parent[4, 5] = -2
    rows[5, 7] = rows[5, 8]     # shared row
    rows[6, 0] = cfg.R          # out of range
    parent[7] = np.arange(-1, cfg.N - 1)  # a 64-deep chain
    parent[8, 1:] = -1          # forest of 64 root-level nodes
    for W in (1, 2, 4):
        import torch
        g = _g()
        from harness import to_dev
        desc = g.TreeDesc(to_dev(parent), to_dev(rows), cfg.R, W)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        g.gdn_tree_desc_build(desc, err)
        torch.cuda.synchronize()
        d = oracle.desc_build(parent, rows, cfg.R, W)
        assert int(err.item()) == d["err"] == (oracle.EV_PARENT | oracle.EV_ROW)
        assert np.array_equal(desc.status.cpu().numpy(), d["status"])
        assert np.array_equal(desc.depth.cpu().numpy(), d["depth"])
        assert np.array_equal(desc.anc.cpu().numpy().view(np.uint64), d["anc"])
        if W > 1:
            assert np.array_equal(desc.conv_src.cpu().numpy(), d["conv_src"])


# ---------------------------------------------------------------------------
# verify + commit, no conv
# ---------------------------------------------------------------------------

def test_binary7_d32_f32_full():
    case = gi.make_case(gi.CONFIGS[1], seed=2026, extra_slots=1)
    gr, orr = run_gpu(case), run_oracle(case)
    _cmp_desc(gr, orr)
    assert gr["err"] == orr["err"] == 0
    _cmp_out(case, gr, orr)
    _cmp_pool(case, gr, orr)


@pytest.mark.parametrize("valu", [False, True])
def test_chain8_equals_sequential_decode_full(valu):
    g = _g()
    case = gi.make_case(gi.CONFIGS[2], seed=2026, extra_slots=3)
    gr = run_gpu(case, flags=g.GDN_F_VALU if valu else 0)
    orr = run_oracle(case)
    assert gr["err"] == orr["err"] == 0
    _cmp_out(case, gr, orr)
    _cmp_pool(case, gr, orr)


@pytest.mark.parametrize("valu", [False, True])
def test_tree27_b32_full(valu):
    g = _g()
    case = gi.make_case(gi.CONFIGS[3], seed=2026, extra_slots=2)
    gr = run_gpu(case, flags=g.GDN_F_VALU if valu else 0)
    orr = run_oracle(case)
    _cmp_desc(gr, orr)
    assert gr["err"] == orr["err"] == 0
    _cmp_out(case, gr, orr)
    _cmp_pool(case, gr, orr)


def test_tree27_bfs_packing_and_shared_topology():
    cfg = gi.CONFIGS[3]
    case = gi.make_case(cfg, seed=77, B=8, packing="bfs")
    # one topology for all requests; accepted paths redrawn on that tree
    case["parent"][:] = case["parent"][0]
    case["node_row"][:] = case["node_row"][0]
    rng = np.random.default_rng(1)
    case["path"][:] = -1
    for b in range(case["B"]):
        p = gi.draw_path(rng, case["parent"][0], "uniform_len")
        case["path"][b, :len(p)] = p
        case["path_len"][b] = len(p)
    gr = run_gpu(case, shared=True)
    orr = run_oracle(case, shared=True)
    assert gr["err"] == orr["err"] == 0
    _cmp_out(case, gr, orr)
    _cmp_pool(case, gr, orr)


@pytest.mark.parametrize("N,bmax,depth", [(1, 1, 0), (16, 2, 5), (17, 4, 3), (32, 3, 6),
                                          (33, 64, 1), (37, 3, 8), (48, 2, 12), (50, 2, 9),
                                          (64, 1, 63), (64, 64, 1)])
def test_node_count_edges(N, bmax, depth):
    # MB = 1..4 kernel variants, deepest chain, widest star; two blocks with
    # a node count off the multiples of four and paths of length 9 (solved in
    # the 8-lane pass) with and without longer ones
    tree = "chain" if bmax == 1 else "random"
    cfg = gi.CONFIGS[3].replace(N=N, R=N + 3, bmax=bmax, depth_max=depth, tree=tree, B=6)
    case = gi.make_case(cfg, seed=N * 7 + bmax, extra_slots=1)
    gr, orr = run_gpu(case), run_oracle(case)
    _cmp_desc(gr, orr)
    assert gr["err"] == orr["err"] == 0
    _cmp_out(case, gr, orr)
    _cmp_pool(case, gr, orr)


@pytest.mark.parametrize("dtype,valu,tree", [("f32", False, "chain"), ("f32", False, "random"),
                                             ("bf16", True, "chain"), ("bf16", True, "random")])
def test_n64_d128_vector_alu_paths(dtype, valu, tree):
    # 64 nodes at d = 128 on the vector-ALU kernel (fp32 operands, or bf16 with
    # GDN_F_VALU): its layout keeps the ancestor Gram entries as lower
    # triangles, so this size fits the 160 KiB of LDS
    cfg = gi.CONFIGS[3].replace(N=64, R=67, dtype=dtype, tree=tree, bmax=4 if tree == "random" else 1,
                                depth_max=8 if tree == "random" else 63, B=4, Hv=4, Hqk=2)
    case = gi.make_case(cfg, seed=640 + (dtype == "f32") + 2 * (tree == "chain"), extra_slots=1)
    gr = run_gpu(case, flags=_g().GDN_F_VALU if valu else 0)
    orr = run_oracle(case)
    assert gr["err"] == orr["err"] == 0
    _cmp_out(case, gr, orr)
    _cmp_pool(case, gr, orr)


def test_wide_tree_every_depth_class():
    # 64 nodes: a 24-node spine with 40 leaves hung at depths 7 .. 24, so the
    # M solve meets nodes of path length <= 8, more than 16 of length 9 .. 16
    # (two rounds of 16-lane groups) and longer ones (one thread per node);
    # each request commits the root chain of one of its leaves
    cfg = gi.CONFIGS[3].replace(N=64, R=67, bmax=64, depth_max=30, B=4)
    case = gi.make_case(cfg, seed=64, extra_slots=1)
    rng = np.random.default_rng(64)
    for b in range(cfg.B):
        par = np.arange(-1, 63, dtype=np.int32)
        par[24:] = rng.integers(6, 24, 40)
        case["parent"][b] = par
        chain, i = [], int(rng.integers(24, 64))
        while i >= 0:
            chain.append(i)
            i = int(par[i])
        case["path"][b] = -1
        case["path"][b, :len(chain)] = chain[::-1]
        case["path_len"][b] = len(chain)
    gr, orr = run_gpu(case), run_oracle(case)
    d = orr["depth"]
    assert (((d > 8) & (d <= 16)).sum(axis=1) > 16).all() and (d > 16).any(axis=1).all()
    _cmp_desc(gr, orr)
    assert gr["err"] == orr["err"] == 0
    _cmp_out(case, gr, orr)
    _cmp_pool(case, gr, orr)


def test_forest_and_len0_paths():
    cfg = gi.CONFIGS[3].replace(B=6)
    case = gi.make_case(cfg, seed=3, extra_slots=1)
    # request 0: a forest (several children of the committed state)
    case["parent"][0, [5, 9, 14]] = -1
    case["path"][0] = -1
    case["path"][0, 0] = 9
    case["path_len"][0] = 1
    case["path_len"][[1, 3]] = 0
    gr, orr = run_gpu(case), run_oracle(case)
    assert gr["err"] == orr["err"] == 0
    _cmp_out(case, gr, orr)
    _cmp_pool(case, gr, orr)


def test_out_bf16_flag():
    case = gi.make_case(gi.CONFIGS[3], seed=9, B=4)
    gr = run_gpu(case, out_bf16=True, commit=False)
    orr = run_oracle(case, commit=False)
    m = node_rows_mask(case)
    got = gi.bf16_bits_to_f32(gr["out"][m])
    # the fp32 bar plus bf16's own rounding (half an ulp, 2^-9 relative)
    assert max_rel_rows(got, orr["out"][m], 2) <= TOL + 2.0 ** -9
    ref = oracle.round_f64_to_bf16_bits(orr["out"])
    d = bf16_ulp_diff(gr["out"][m], ref[m])
    assert (d <= 1).mean() > 0.99


def test_tree64_out_bf16_and_shared_topology():
    # the wide-tree kernel with one topology for every request and bf16 outputs
    cfg = gi.CONFIGS[5]
    case = gi.make_case(cfg, seed=78, B=4, packing="bfs")
    case["parent"][:] = case["parent"][0]
    case["node_row"][:] = case["node_row"][0]
    gr = run_gpu(case, shared=True, out_bf16=True, commit=False)
    orr = run_oracle(case, shared=True, commit=False)
    assert gr["err"] == orr["err"] == 0
    m = node_rows_mask(case)
    got = gi.bf16_bits_to_f32(gr["out"][m])
    assert max_rel_rows(got, orr["out"][m], 2) <= TOL + 2.0 ** -9


def test_malformed_inputs_skip_requests():
    g = _g()
    cfg = gi.CONFIGS[3].replace(B=8)
    case = gi.make_case(cfg, seed=21, extra_slots=2)
    case["parent"][1, 4] = 20             # tree error -> desc status, skipped everywhere
    case["node_row"][2, 3] = case["node_row"][2, 4]
    case["path"][3, 0] = case["path"][3, 1] if case["path_len"][3] > 1 else 5
    if case["path_len"][3] < 2:
        case["path_len"][3] = 1
    case["path_len"][4] = cfg.Lmax + 1     # longer than Lmax
    case["state_idx"][5] = case["state_idx"][6]   # shared slot: both skipped by commit
    gr = run_gpu(case)
    orr = run_oracle(case)
    assert gr["err"] == orr["err"]
    assert gr["err"] == (g.GDN_EV_PARENT | g.GDN_EV_ROW | g.GDN_EV_PATH | g.GDN_EV_STATE)
    assert np.array_equal(gr["status"], orr["status"])
    m = node_rows_mask(case)
    for b in (1, 2):
        assert np.isnan(gr["out"][b]).all()
    ok = [b for b in range(cfg.B) if b not in (1, 2)]
    mo = m[ok]
    assert max_rel_rows(gr["out"][ok][mo], orr["out"][ok][mo], 2) <= TOL
    for b in (1, 2, 3, 4, 5, 6):
        s = case["state_idx"][b]
        assert np.array_equal(gr["pool"][s], case["pool"][s])
    for b in (0, 7):
        s = case["state_idx"][b]
        assert max_rel_rows(gr["pool"][s], orr["pool"][s], 1) <= TOL


def test_bad_state_index_in_verify():
    g = _g()
    case = gi.make_case(gi.CONFIGS[3], seed=4, B=4)
    case["state_idx"][2] = 99
    gr = run_gpu(case, commit=False)
    orr = run_oracle(case, commit=False)
    assert gr["err"] == orr["err"] == g.GDN_EV_STATE
    assert np.isnan(gr["out"][2]).all()


def test_deterministic_repeat():
    case = gi.make_case(gi.CONFIGS[3], seed=12, B=8)
    a = run_gpu(case)
    b = run_gpu(case)
    assert np.array_equal(a["out"], b["out"], equal_nan=True)
    assert np.array_equal(a["pool"], b["pool"], equal_nan=True)


def test_bitwise_identical_across_processes():
    """Two runs here and one in a fresh process give the same bits: outputs,
    committed states, conv outputs and published histories of the fused
    step, the layer step and the separate calls (no atomics or
    order-dependent reductions on the path)."""
    import json
    import subprocess
    import sys

    from repeat_digest import digests

    first = digests()
    assert digests() == first
    script = os.path.join(os.path.dirname(os.path.abspath(__file__)), "repeat_digest.py")
    proc = subprocess.run([sys.executable, script], capture_output=True, text=True, timeout=300)
    assert proc.returncode == 0, proc.stderr[-2000:]
    other = json.loads(proc.stdout.strip().splitlines()[-1])
    assert other == first


# ---------------------------------------------------------------------------
# conv-fed configuration (27-node, conv kernel 4, 8192 channels)
# ---------------------------------------------------------------------------

def _cmp_conv(case, gr, orr):
    m = node_rows_mask(case)
    yg, yo = gr["y"][m], orr["y"][m]
    d = bf16_ulp_diff(yg, yo)
    tiny = (np.abs(gi.bf16_bits_to_f32(yo)) < 2.0 ** -126) & (np.abs(gi.bf16_bits_to_f32(yg)) < 2.0 ** -126)
    assert (d[~tiny] <= 1).all(), f"conv ulp diff {d.max()}"
    assert (gr["y"][~m] == 0x7FC0).all()  # padding rows untouched
    return int((d != 0).sum())


def _cmp_end_to_end(case, gr, orr):
    """Own conv output downstream: rows that no straddled conv element reaches
    meet the strict bar; the rest must be finite (their gap is the oracle's own
    sensitivity to a one-ulp input change, covered stage-wise)."""
    m = node_rows_mask(case)
    om, sm = straddle_rows(case, gr["y"], orr["y"])
    clean = m[:, :, None] & ~om
    assert max_rel_rows(gr["out"][clean], orr["out"][clean], 1) <= TOL
    assert np.isfinite(gr["out"][m]).all()
    used = case["state_idx"]
    for b in range(case["B"]):
        for h in range(case["cfg"].Hv):
            if not sm[b, h]:
                assert max_rel_rows(gr["pool"][used[b], h], orr["pool"][used[b], h], 0) <= TOL


def test_conv4_tree27_b8_end_to_end():
    case = gi.make_case(gi.CONFIGS[4], seed=2026, B=8, extra_slots=1)
    orr = run_oracle(case)
    # stage-wise: verify/commit read the oracle's own bf16 conv output
    gs = run_gpu(case, y_override=orr["y"])
    _cmp_desc(gs, orr)
    assert gs["err"] == orr["err"] == 0
    n_straddle = _cmp_conv(case, gs, orr)
    _cmp_out(case, gs, orr)
    _cmp_pool(case, gs, orr)
    assert np.array_equal(gs["hist"], hist_to_bits(orr["hist"]))
    # end to end on the device's own conv output
    gr = run_gpu(case)
    assert np.array_equal(gr["y"], gs["y"])
    _cmp_end_to_end(case, gr, orr)
    print(f"conv elements differing by one bf16 ulp: {n_straddle}")


def test_conv4_variants():
    for W, act in ((1, 0), (2, 1), (3, 0)):
        cfg = gi.CONFIGS[4].replace(conv_W=W, act=act, conv_C=2048 + 8 * W, Hv=4, Hqk=2, B=3)
        cfg = cfg.replace(conv_C=2 * cfg.Hqk * cfg.D + cfg.Hv * cfg.D)
        case = gi.make_case(cfg, seed=W, extra_slots=1)
        orr = run_oracle(case)
        gr = run_gpu(case, y_override=orr["y"])
        assert gr["err"] == orr["err"] == 0
        _cmp_conv(case, gr, orr)
        _cmp_out(case, gr, orr)
        _cmp_pool(case, gr, orr)
        assert np.array_equal(gr["hist"], hist_to_bits(orr["hist"]))


def test_conv4_tree27_b128_full_size_sampled():
    # the full workload on the GPU; the oracle on a sample of requests
    case = gi.make_case(gi.CONFIGS[4], seed=2026)
    bs = np.array([0, 17, 63, 64, 101, 127])
    sub = subset(case, bs)
    orr = run_oracle(sub)
    # sampled requests read the oracle's conv output downstream (stage-wise)
    yo = np.full((case["B"],) + orr["y"].shape[1:], 0x7FC0, np.uint16)
    yo[bs] = orr["y"]
    gr = run_gpu(case, y_override=yo)
    assert gr["err"] == 0
    gsub = dict(gr)
    gsub["out"] = gr["out"][bs]
    gsub["y"] = gr["y"][bs]
    gsub["pool"] = gr["pool"][case["state_idx"][bs]]
    gsub["hist"] = gr["hist"][case["state_idx"][bs]]
    _cmp_conv(sub, gsub, orr)
    _cmp_out(sub, gsub, orr)
    m = sub["state_idx"]
    assert max_rel_rows(gsub["pool"], orr["pool"][m], 2) <= TOL
    assert np.array_equal(gsub["hist"], hist_to_bits(orr["hist"]))
    # every request: untouched padding, finite outputs on node rows
    mm = node_rows_mask(case)
    assert np.isfinite(gr["out"][mm]).all() and np.isnan(gr["out"][~mm]).all()


# ---------------------------------------------------------------------------
# wide 64-node tree, B = 256, two of the 48 layers back to back
# ---------------------------------------------------------------------------

def test_tree64_b256_two_layers_sampled():
    cfg = gi.CONFIGS[5]
    bs = np.array([0, 5, 77, 128, 200, 255])
    for layer in (0, 1):
        case = gi.make_case(cfg, seed=2026, layer=layer)
        gr = run_gpu(case)
        assert gr["err"] == 0
        sub = subset(case, bs)
        orr = run_oracle(sub)
        m = node_rows_mask(sub)
        assert max_rel_rows(gr["out"][bs][m], orr["out"][m], 2) <= TOL
        assert max_rel_rows(gr["pool"][case["state_idx"][bs]], orr["pool"], 2) <= TOL


@pytest.mark.parametrize("N,R,C,act,with_bias", [(27, 32, 1024, 0, False), (27, 40, 1024, 0, True),
                                                 (27, 32, 1028, 0, True), (40, 48, 1024, 0, False),
                                                 (40, 70, 1024, 1, True), (64, 64, 512, 1, False)])
def test_conv_row_layouts(N, R, C, act, with_bias):
    # row counts and padding of one and two passes of rows, 8- and 4-channel
    # accesses (C = 1028), with and without the activation and the bias
    import torch
    g = _g()
    from harness import bits, to_dev
    import oracle
    cfg = gi.CONFIGS[4].replace(N=N, R=R, conv_C=C, act=act, B=5, bmax=4, depth_max=8)
    case = gi.make_case(cfg, seed=N + R + C, extra_slots=1, conv_values="dyadic" if act == 0 else "normal")
    W = cfg.conv_W
    desc = g.TreeDesc(to_dev(case["parent"]), to_dev(case["node_row"]), R, W)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.gdn_tree_desc_build(desc, err)
    y = torch.full((case["B"], R, C), float("nan"), dtype=torch.bfloat16, device="cuda")
    hist = to_dev(case["hist"])
    bias = gi.conv_bias(cfg, seed=N, dyadic=act == 0) if with_bias else None
    g.conv_ancestry_gather(desc, to_dev(case["x"]), hist, to_dev(case["state_idx"]), to_dev(case["w"]),
                           None if bias is None else to_dev(bias), y, act, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    d = oracle.desc_build(case["parent"], case["node_row"], R, W)
    yo, e = oracle.conv(case["node_row"], d["conv_src"], d["status"], case["x"], case["hist"],
                        case["state_idx"], case["w"], bias, act, R, C, W)
    assert e == 0
    yb = bits(y)
    m = node_rows_mask(case)
    ob = oracle.round_f64_to_bf16_bits(yo)
    if act == 0:
        assert np.array_equal(yb[m], ob[m])
    else:
        assert (bf16_ulp_diff(yb[m], ob[m]) <= 1).all()
    assert (yb[~m] == 0x7FC0).all()
