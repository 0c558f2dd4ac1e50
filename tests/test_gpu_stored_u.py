"""GPU parity of the stored-U mode: gdn_tree_verify_store_u writes every
node's delta correction u_i = b_i (v_i - a_i S_parent(i) k^_i) beside the
outputs, and gdn_tree_commit_factored publishes the accepted frontier's state
from them, S_new = P_a S_pre + sum_j (P_a / P_j) u_j k^_j^T (Bole review,
Sec. 5.2 and Eq. (10); TreeWY, Sec. 3).

Bars: u within 2e-3 of the oracle's u (max relative per row, as the
outputs); the factored commit within 2e-3 of the oracle's replay commit,
both from the device's u and from the oracle's own u (the latter checks the
commit kernel on its own); the verify's outputs bitwise those of
gdn_tree_verify on the same inputs; error bits and every slot or row the
mode must not write bit-exact."""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from harness import dev_gate_params, max_rel_rows, node_rows_mask, oracle_gates, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _g():
    import tree_speculative_verification_gdn_amd as g
    return g


def _gpu(case, flags=0, u_from=None, commit=True, also_plain=False):
    """desc_build -> verify_store_u -> [commit_factored] on the device.  With
    ``u_from`` (host [B][R][Hv][D]) the commit reads those corrections
    instead of the ones the verify wrote."""
    import torch
    g = _g()
    cfg = case["cfg"]
    B, R, D, Hv, Hqk = case["B"], cfg.R, cfg.D, cfg.Hv, cfg.Hqk
    desc = g.TreeDesc(to_dev(case["parent"]), to_dev(case["node_row"]), R, 1, B=B)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.gdn_tree_desc_build(desc, err, raise_on_error=False)
    q, k, v = to_dev(case["q"]), to_dev(case["k"]), to_dev(case["v"])
    alpha, beta = to_dev(case["alpha"]), to_dev(case["beta"])
    pool, sidx = to_dev(case["pool"]), to_dev(case["state_idx"])
    gp = dev_gate_params(case)
    out = torch.full((B, R, Hv, D), float("nan"), dtype=torch.float32, device="cuda")
    u = torch.full((B, R, Hv, D), float("nan"), dtype=torch.float32, device="cuda")
    res = {}
    if also_plain:
        out2 = torch.full_like(out, float("nan"))
        e2 = torch.zeros_like(err)
        g.gdn_tree_verify(desc, q, k, v, alpha, beta, pool, sidx, out2, e2, flags=flags, gate_params=gp,
                          raise_on_error=False)
        torch.cuda.synchronize()
        res["out_plain"] = out2.cpu().numpy()
    g.gdn_tree_verify_store_u(desc, q, k, v, alpha, beta, pool, sidx, out, u, err, flags=flags,
                              gate_params=gp, raise_on_error=False)
    torch.cuda.synchronize()
    res["out"] = out.cpu().numpy()
    res["u"] = u.cpu().numpy()
    if commit:
        uc = u if u_from is None else to_dev(np.asarray(u_from, np.float32))
        g.gdn_tree_commit_factored(desc, to_dev(case["path"]), to_dev(case["path_len"]), k, uc, alpha, pool,
                                   sidx, err, flags=flags & (g.GDN_F_NORM_QK | g.GDN_F_RAW_GATES),
                                   gate_params=gp, raise_on_error=False)
    torch.cuda.synchronize()
    res["pool"] = pool.cpu().numpy()
    res["err"] = int(err.item())
    return res


def _oracle(case, norm=False):
    cfg = case["cfg"]
    d = oracle.desc_build(case["parent"], case["node_row"], cfg.R, 1)
    alpha, beta = oracle_gates(case)
    out, e, u = oracle.verify(case["parent"], case["node_row"], d["status"], case["q"], case["k"], case["v"],
                              alpha, beta, case["pool"], case["state_idx"], cfg.Hqk, cfg.Hv, norm, want_u=True)
    pool, _, e2 = oracle.commit(case["parent"], case["node_row"], d["status"], case["path"], case["path_len"],
                                case["k"], case["v"], alpha, beta, case["pool"], case["state_idx"],
                                cfg.Hqk, cfg.Hv, norm)
    return dict(out=out, u=u, pool=pool, err=d["err"] | e | e2)


def _cmp(case, gr, orr, tol=TOL):
    assert gr["err"] == orr["err"]
    m = node_rows_mask(case)
    assert np.isnan(gr["u"][~m]).all(), "u written on a row no node uses"
    assert np.isnan(gr["out"][~m]).all()
    rel = max_rel_rows(gr["u"][m], orr["u"][m], 2)
    assert rel <= tol, f"u max rel {rel:.3e}"
    rel = max_rel_rows(gr["out"][m], orr["out"][m], 2)
    assert rel <= tol, f"output max rel {rel:.3e}"
    used = case["state_idx"]
    rel = max_rel_rows(gr["pool"][used], orr["pool"][used], 2)
    assert rel <= tol, f"state max rel {rel:.3e}"
    untouched = np.setdiff1d(np.arange(case["P"]), used[case["path_len"] > 0])
    assert np.array_equal(gr["pool"][untouched], case["pool"][untouched], equal_nan=True)


@pytest.mark.parametrize("valu", [False, True])
def test_tree27_u_and_factored_commit(valu):
    # N = 27: the matrix-core kernel (or the vector-ALU one with GDN_F_VALU)
    g = _g()
    case = gi.make_case(gi.CONFIGS[3], seed=271 + valu, B=6, extra_slots=1)
    case["path_len"][2] = 0
    gr = _gpu(case, flags=g.GDN_F_VALU if valu else 0, also_plain=True)
    orr = _oracle(case)
    _cmp(case, gr, orr)
    # the stored-U verify's outputs are the plain verify's, bit for bit
    assert np.array_equal(gr["out"], gr["out_plain"], equal_nan=True)


def test_chain8_and_full_paths():
    # the speculative-decoding chain: every path is the whole chain
    case = gi.make_case(gi.CONFIGS[2], seed=82, B=8)
    _cmp(case, _gpu(case), _oracle(case))


@pytest.mark.parametrize("tree", ["random", "chain"])
def test_n64_vector_alu_u(tree):
    # 64 nodes: the stored-U mode runs on the vector-ALU kernel; the chain
    # commits paths of up to 64 nodes (eight matrix-core segments)
    cfg = gi.CONFIGS[5].replace(B=3, Hv=4, Hqk=2, tree=tree, bmax=4 if tree == "random" else 1,
                                depth_max=8 if tree == "random" else 63,
                                path="uniform_len" if tree == "random" else "full")
    case = gi.make_case(cfg, seed=641 + (tree == "chain"), extra_slots=1)
    gr, orr = _gpu(case), _oracle(case)
    _cmp(case, gr, orr)
    if tree == "chain":
        assert (case["path_len"] == 64).all()


def test_factored_commit_from_oracle_u():
    # the commit kernel alone: the oracle's own u (rounded to fp32) in, the
    # oracle's replay commit out
    case = gi.make_case(gi.CONFIGS[3], seed=277, B=8, extra_slots=2)
    orr = _oracle(case)
    gr = _gpu(case, u_from=orr["u"])
    used = case["state_idx"]
    assert gr["err"] == orr["err"] == 0
    rel = max_rel_rows(gr["pool"][used], orr["pool"][used], 2)
    assert rel <= TOL, f"state max rel {rel:.3e}"


def test_norm_qk_and_raw_gates():
    g = _g()
    case = gi.with_raw_gates(gi.make_case(gi.CONFIGS[3], seed=279, B=6))
    gr = _gpu(case, flags=g.GDN_F_NORM_QK)
    orr = _oracle(case, norm=True)
    _cmp(case, gr, orr)


def test_malformed_paths_and_shared_slots():
    g = _g()
    cfg = gi.CONFIGS[3].replace(B=8)
    case = gi.make_case(cfg, seed=283, extra_slots=2)
    case["parent"][1, 4] = 20                       # tree error: nothing of request 1 is touched
    case["path"][3, 0] = case["path"][3, 1] if case["path_len"][3] > 1 else 5
    if case["path_len"][3] < 2:
        case["path_len"][3] = 1
    case["path_len"][4] = cfg.Lmax + 1              # longer than Lmax
    case["state_idx"][5] = case["state_idx"][6]     # shared slot: both skipped by the commit
    gr, orr = _gpu(case), _oracle(case)
    assert gr["err"] == orr["err"] == (g.GDN_EV_PARENT | g.GDN_EV_PATH | g.GDN_EV_STATE)
    assert np.isnan(gr["u"][1]).all() and np.isnan(gr["out"][1]).all()
    for b in (1, 3, 4, 5, 6):
        s = case["state_idx"][b]
        assert np.array_equal(gr["pool"][s], case["pool"][s])
    for b in (0, 2, 7):
        s = case["state_idx"][b]
        assert max_rel_rows(gr["pool"][s], orr["pool"][s], 1) <= TOL
    ok = [b for b in range(cfg.B) if b != 1]
    m = node_rows_mask(case)[ok]
    assert max_rel_rows(gr["u"][ok][m], orr["u"][ok][m], 2) <= TOL


def test_f32_small_u():
    # fp32 operands at d = 32 (vector-ALU kernel): u only; the factored
    # commit is for bf16 k at d = 128
    case = gi.make_case(gi.CONFIGS[1], seed=11)
    gr, orr = _gpu(case, commit=False), _oracle(case)
    m = node_rows_mask(case)
    assert gr["err"] == orr["err"] == 0
    assert max_rel_rows(gr["u"][m], orr["u"][m], 2) <= TOL


def test_state_dump_and_commit_consistency():
    """GDN_F_DUMP_STATES: every node's state S_i next to the oracle's, the
    outputs against S_i q_i, and the frontier's dumped state against both
    commits of the accepted path (LumoTree, Sec. IV-B: the native replay and
    the verifier may differ numerically).  The factored commit rebuilds the
    frontier with the dump's own arithmetic, so it matches bit for bit; the
    replay commit is held to the 2e-3 bar, and how many of its elements are
    bitwise equal to the dump is reported."""
    import torch
    g = _g()
    cfg = gi.CONFIGS[3].replace(Hv=8, Hqk=4)
    case = gi.make_case(cfg, seed=291, B=5, extra_slots=1)
    case["path_len"][1] = 0
    B, N, R, D, Hv = case["B"], cfg.N, cfg.R, cfg.D, cfg.Hv
    desc = g.TreeDesc(to_dev(case["parent"]), to_dev(case["node_row"]), R, 1, B=B)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.gdn_tree_desc_build(desc, err)
    q, k, v = to_dev(case["q"]), to_dev(case["k"]), to_dev(case["v"])
    alpha, beta = to_dev(case["alpha"]), to_dev(case["beta"])
    pool0, sidx = to_dev(case["pool"]), to_dev(case["state_idx"])
    out = torch.full((B, R, Hv, D), float("nan"), dtype=torch.float32, device="cuda")
    u = torch.full_like(out, float("nan"))
    dump = torch.full((B, N, Hv, D, D), float("nan"), dtype=torch.float32, device="cuda")
    g.gdn_tree_verify_store_u(desc, q, k, v, alpha, beta, pool0, sidx, out, u, err, dump=dump)
    path, plen = to_dev(case["path"]), to_dev(case["path_len"])
    pool_f, pool_r = pool0.clone(), pool0.clone()
    g.gdn_tree_commit_factored(desc, path, plen, k, u, alpha, pool_f, sidx, err)
    g.gdn_tree_commit(desc, path, plen, k, v, alpha, beta, pool_r, sidx, err, Hqk=cfg.Hqk)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    dump_h, out_h = dump.cpu().numpy(), out.cpu().numpy()
    pf, pr = pool_f.cpu().numpy(), pool_r.cpu().numpy()
    assert np.array_equal(pool0.cpu().numpy(), case["pool"], equal_nan=True)  # the dump only reads the pool

    # every node's state against the oracle's S_i
    d = oracle.desc_build(case["parent"], case["node_row"], R, 1)
    _, e, states = oracle.verify(case["parent"], case["node_row"], d["status"], case["q"], case["k"], case["v"],
                                 case["alpha"], case["beta"], case["pool"], case["state_idx"], cfg.Hqk, Hv,
                                 False, want_states=True)
    rel = max_rel_rows(dump_h, states, 3)
    assert rel <= TOL, f"dumped states max rel {rel:.3e}"
    # each output against its own node's dumped state: o_i = S_i q_i
    qf = gi.bf16_bits_to_f32(case["q"]).astype(np.float64)
    g_of_h = np.arange(Hv) * cfg.Hqk // Hv
    worst = 0.0
    for b in range(B):
        for i in range(N):
            r = case["node_row"][b, i]
            o_ref = np.einsum("hvk,hk->hv", dump_h[b, i].astype(np.float64), qf[b, r, g_of_h])
            worst = max(worst, max_rel_rows(out_h[b, r], o_ref, 1))
    assert worst <= TOL, f"outputs vs S_i q_i max rel {worst:.3e}"

    # the frontier's dumped state against both commits
    n_eq = n_all = 0
    rel_r = 0.0
    for b in range(B):
        s = case["state_idx"][b]
        L = case["path_len"][b]
        if L == 0:
            assert np.array_equal(pf[s], case["pool"][s]) and np.array_equal(pr[s], case["pool"][s])
            continue
        f = case["path"][b, L - 1]
        assert np.array_equal(pf[s], dump_h[b, f]), f"factored commit of request {b} differs from its dump"
        rel_r = max(rel_r, max_rel_rows(pr[s], dump_h[b, f], 1))
        n_eq += int((pr[s] == dump_h[b, f]).sum())
        n_all += pr[s].size
    print(f"\n[consistency] replay commit vs dumped frontier: max rel {rel_r:.3e}, "
          f"{n_eq}/{n_all} elements bitwise equal ({100.0 * n_eq / n_all:.1f}%); "
          f"factored commit: bitwise equal on every committed slot")
    assert rel_r <= TOL
