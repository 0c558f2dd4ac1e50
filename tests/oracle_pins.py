"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` function runs the oracle (through ``lib``, so planted-mistake
variants can be checked too) and raises AssertionError if the pin does not
hold.  None of them re-types the oracle's own formula:

* pin_chain_textbook     chain tree == sequential decode written in the matrix
                         form a S (I - b k k^T) + b v k^T (TreeWY, Sec. 1)
* pin_paths_are_chains   every root-to-node path == an independent chain run
                         (Bole review, Lemma 1: a node depends only on its path)
* pin_sibling_isolation  NaN in one node touches only its subtree (LumoTree,
                         Sec. VII-D negative controls; packed-row trap)
* pin_commit_is_replay   commit(path) == the path's sequential run and == the
                         frontier node's verify state (LumoTree, Sec. IV-B)
* pin_closed_form        outputs == Theorem 1 by dense solve (Bole review, Eq. (2))
* pin_treewy_states      node states == TreeWY pseudo-value reconstruction
* pin_nilpotent          G^{d+1} == 0 exactly, G^d != 0, Neumann == solve (Eq. (6))
* pin_factorized_commit  commit == Eq. (10) of the Bole review
* pin_pure_decay         beta == 0: o_i = P_i S_pre q_i, S_i = P_i S_pre
* pin_delta_write        alpha = beta = 1, |k| = 1: S_i k_i == v_i
* pin_conv_chain         chain conv == numpy.convolve over history ++ inputs
* pin_conv_tree_paths    a tree node's conv == numpy.convolve over its own path
* pin_conv_w1            W = 1 conv == pointwise scale
* pin_desc_enumeration   depth / ancestors / conv sources == explicit path walk
* pin_norm_flag          normalise flag == pre-normalised operands
* pin_norm_invariance    normalised outputs do not change when a q/k row is
                         scaled by a positive factor; unit rows are (nearly)
                         left alone; a row of tiny norm becomes the first D
                         coordinates of the unit vector of (x, sqrt(1e-6))
* pin_u_closed_form      the oracle's per-node delta corrections u_i == the
                         rows of U from the dense solve of (I + G) U = R
                         (Bole review, Lemma 2), and Eq. (10) from them ==
                         the oracle's commit
* pin_conv_publish       the history a commit publishes continues the causal
                         conv: the next tree's conv == numpy.convolve over
                         old history ++ accepted inputs ++ new inputs
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle import closed_form as cf


# --------------------------------------------------------------------------
# small problem builder (test-local; operands drawn here, nothing from the GPU)
# --------------------------------------------------------------------------

def small_problem(seed, parents, R=None, Hv=2, Hqk=1, D=8, P_extra=1, unit_k=True,
                  alpha_range=(0.5, 1.0), s_std=0.3):
    g = np.random.default_rng(seed)
    parents = [np.asarray(p, np.int32) for p in parents]
    B = len(parents)
    N = len(parents[0])
    R = R or N + 2
    rows = np.stack([g.permutation(R)[:N] for _ in range(B)]).astype(np.int32)
    q = g.standard_normal((B, R, Hqk, D))
    k = g.standard_normal((B, R, Hqk, D))
    if unit_k:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((B, R, Hv, D))
    alpha = g.uniform(*alpha_range, (B, R, Hv))
    beta = g.uniform(0.0, 1.0, (B, R, Hv))
    P = B + P_extra
    pool = g.standard_normal((P, Hv, D, D)) * s_std
    state_idx = g.permutation(P)[:B].astype(np.int32)
    return dict(parent=np.stack(parents), node_row=rows, q=q, k=k, v=v, alpha=alpha,
                beta=beta, pool=pool, state_idx=state_idx, Hv=Hv, Hqk=Hqk, D=D, R=R,
                B=B, N=N)


def random_parent(g, N, bmax=3):
    par = [-1]
    ch = [0]
    for i in range(1, N):
        cand = [j for j in range(i) if ch[j] < bmax]
        p = int(cand[g.integers(len(cand))])
        par.append(p)
        ch[p] += 1
        ch.append(0)
    return np.array(par, np.int32)


def run_verify(pb, lib, norm=False, want_states=True):
    d = oracle.desc_build(pb["parent"], pb["node_row"], pb["R"], 1, lib=lib)
    return oracle.verify(pb["parent"], pb["node_row"], d["status"], pb["q"], pb["k"], pb["v"],
                         pb["alpha"], pb["beta"], pb["pool"], pb["state_idx"], pb["Hqk"],
                         pb["Hv"], norm, want_states=want_states, lib=lib)


def operands(pb, b, h, node):
    """(q, k, v, a, beta) of one node of request b, value head h."""
    row = pb["node_row"][b][node]
    gq = h * pb["Hqk"] // pb["Hv"]
    return (pb["q"][b, row, gq], pb["k"][b, row, gq], pb["v"][b, row, h],
            pb["alpha"][b, row, h], pb["beta"][b, row, h])


def chain_textbook(S0, steps):
    """Sequential gated delta rule in TreeWY's matrix form:
    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t."""
    S = S0.copy()
    outs = []
    D = S.shape[1]
    for (q, k, v, a, b) in steps:
        S = a * S @ (np.eye(D) - b * np.outer(k, k)) + b * np.outer(v, k)
        outs.append(S @ q)
    return S, outs


def relerr(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_chain_textbook(lib):
    N = 9
    pb = small_problem(11, [np.arange(-1, N - 1)] * 2, D=12, Hv=2, Hqk=1)
    out, err, states = run_verify(pb, lib)
    assert err == 0
    for b in range(pb["B"]):
        for h in range(pb["Hv"]):
            S0 = pb["pool"][pb["state_idx"][b], h]
            steps = [operands(pb, b, h, i) for i in range(N)]
            S_end, outs = chain_textbook(S0, steps)
            for i in range(N):
                row = pb["node_row"][b][i]
                assert relerr(out[b, row, h], outs[i]) < 1e-12, "chain output differs from textbook decode"
            assert relerr(states[b, N - 1, h], S_end) < 1e-12
    # commit of the whole chain == textbook final state
    path = np.tile(np.arange(N, dtype=np.int32), (pb["B"], 1))
    plen = np.full(pb["B"], N, np.int32)
    d = oracle.desc_build(pb["parent"], pb["node_row"], pb["R"], 1, lib=lib)
    pool_new, _, err = oracle.commit(pb["parent"], pb["node_row"], d["status"], path, plen,
                                     pb["k"], pb["v"], pb["alpha"], pb["beta"], pb["pool"],
                                     pb["state_idx"], pb["Hqk"], pb["Hv"], False, lib=lib)
    assert err == 0
    for b in range(pb["B"]):
        for h in range(pb["Hv"]):
            S_end, _ = chain_textbook(pb["pool"][pb["state_idx"][b], h],
                                      [operands(pb, b, h, i) for i in range(N)])
            assert relerr(pool_new[pb["state_idx"][b], h], S_end) < 1e-12


def pin_paths_are_chains(lib):
    g = np.random.default_rng(5)
    par = random_parent(g, 14)
    pb = small_problem(12, [par], D=8, Hv=2, Hqk=1)
    out, err, _ = run_verify(pb, lib)
    assert err == 0
    anc = cf.ancestors(par)
    for node in range(len(par)):
        nodes = anc[node] + [node]
        L = len(nodes)
        # the same operands, re-indexed as a chain over this path only
        chain = dict(pb)
        chain["parent"] = np.arange(-1, L - 1, dtype=np.int32)[None, :]
        chain["node_row"] = pb["node_row"][:, nodes]
        cout, cerr, _ = run_verify(chain, lib)
        assert cerr == 0
        for h in range(pb["Hv"]):
            row = pb["node_row"][0][node]
            assert np.array_equal(cout[0, row, h], out[0, row, h]), "path output differs from its chain run"


def pin_sibling_isolation(lib):
    g = np.random.default_rng(6)
    par = random_parent(g, 13, bmax=2)
    pb = small_problem(13, [par], D=8)
    base, _, _ = run_verify(pb, lib)
    anc = cf.ancestors(par)
    for j in range(len(par)):
        bad = {k: v.copy() if isinstance(v, np.ndarray) else v for k, v in pb.items()}
        row = pb["node_row"][0][j]
        bad["k"][0, row] = np.nan
        bad["v"][0, row] = np.nan
        out, _, _ = run_verify(bad, lib)
        for i in range(len(par)):
            ri = pb["node_row"][0][i]
            in_subtree = (i == j) or (j in anc[i])
            if in_subtree:
                assert np.isnan(out[0, ri]).all(), "poison did not reach a descendant"
            else:
                assert np.array_equal(out[0, ri], base[0, ri]), "a non-descendant was touched"


def pin_commit_is_replay(lib):
    g = np.random.default_rng(7)
    pars = [random_parent(g, 12) for _ in range(3)]
    pb = small_problem(14, pars, D=10, Hv=2, Hqk=1)
    out, err, states = run_verify(pb, lib)
    assert err == 0
    B = pb["B"]
    Lmax = 12
    path = np.full((B, Lmax), -1, np.int32)
    plen = np.zeros(B, np.int32)
    fronts = []
    for b in range(B):
        fr = int(g.integers(len(pars[b])))
        p = cf.ancestors(pars[b])[fr] + [fr]
        path[b, :len(p)] = p
        plen[b] = len(p)
        fronts.append(fr)
    d = oracle.desc_build(pb["parent"], pb["node_row"], pb["R"], 1, lib=lib)
    pool_new, _, err = oracle.commit(pb["parent"], pb["node_row"], d["status"], path, plen,
                                     pb["k"], pb["v"], pb["alpha"], pb["beta"], pb["pool"],
                                     pb["state_idx"], pb["Hqk"], pb["Hv"], False, lib=lib)
    assert err == 0
    for b in range(B):
        for h in range(pb["Hv"]):
            got = pool_new[pb["state_idx"][b], h]
            assert np.array_equal(got, states[b, fronts[b], h]), "commit != frontier verify state"
            seq, _ = chain_textbook(pb["pool"][pb["state_idx"][b], h],
                                    [operands(pb, b, h, n) for n in path[b, :plen[b]]])
            assert relerr(got, seq) < 1e-12
    # the unused pool slot is untouched
    unused = sorted(set(range(pb["pool"].shape[0])) - set(pb["state_idx"].tolist()))
    for s in unused:
        assert np.array_equal(pool_new[s], pb["pool"][s])


def pin_closed_form(lib):
    g = np.random.default_rng(8)
    pars = [random_parent(g, 16, bmax=3), random_parent(g, 16, bmax=1), random_parent(g, 16, bmax=6)]
    pb = small_problem(15, pars, D=12, Hv=2, Hqk=1)
    out, err, _ = run_verify(pb, lib)
    assert err == 0
    for b in range(pb["B"]):
        for h in range(pb["Hv"]):
            ops = [operands(pb, b, h, i) for i in range(pb["N"])]
            Q = np.stack([o[0] for o in ops])
            K = np.stack([o[1] for o in ops])
            V = np.stack([o[2] for o in ops])
            al = np.array([o[3] for o in ops])
            be = np.array([o[4] for o in ops])
            O, _ = cf.solve_tree(pars[b], al, be, Q, K, V, pb["pool"][pb["state_idx"][b], h])
            rows = pb["node_row"][b]
            assert relerr(out[b, rows, h], O) < 1e-11, "closed form disagrees"


def pin_treewy_states(lib):
    g = np.random.default_rng(9)
    par = random_parent(g, 11)
    pb = small_problem(16, [par], D=8, Hv=1, Hqk=1)
    _, _, states = run_verify(pb, lib)
    ops = [operands(pb, 0, 0, i) for i in range(pb["N"])]
    K = np.stack([o[1] for o in ops])
    V = np.stack([o[2] for o in ops])
    al = np.array([o[3] for o in ops])
    be = np.array([o[4] for o in ops])
    St = cf.treewy_states(par, al, be, K, V, pb["pool"][pb["state_idx"][0], 0])
    assert relerr(states[0, :, 0], St) < 1e-11


def pin_nilpotent(lib):
    g = np.random.default_rng(10)
    for trial in range(6):
        par = random_parent(g, 15, bmax=1 + trial % 3)
        pb = small_problem(20 + trial, [par], D=6, Hv=1)
        ops = [operands(pb, 0, 0, i) for i in range(pb["N"])]
        Q = np.stack([o[0] for o in ops])
        K = np.stack([o[1] for o in ops])
        V = np.stack([o[2] for o in ops])
        al = np.array([o[3] for o in ops])
        be = np.array([o[4] for o in ops])
        G = cf.g_matrix(par, al, be, K)
        d = max(len(a) for a in cf.ancestors(par))
        assert np.all(np.linalg.matrix_power(G, d + 1) == 0.0)
        if d > 0:
            assert np.any(np.linalg.matrix_power(G, d) != 0.0)
        S0 = pb["pool"][pb["state_idx"][0], 0]
        O1, U1 = cf.solve_tree(par, al, be, Q, K, V, S0)
        O2, U2 = cf.solve_tree(par, al, be, Q, K, V, S0, use_neumann=True)
        assert relerr(O2, O1) < 1e-12 and relerr(U2, U1) < 1e-12
        out, _, _ = run_verify(pb, lib)
        assert relerr(out[0, pb["node_row"][0], 0], O2) < 1e-11


def pin_factorized_commit(lib):
    g = np.random.default_rng(11)
    par = random_parent(g, 14)
    pb = small_problem(17, [par], D=8, Hv=2, Hqk=1)
    d = oracle.desc_build(pb["parent"], pb["node_row"], pb["R"], 1, lib=lib)
    for fr in range(len(par)):
        p = cf.ancestors(par)[fr] + [fr]
        path = np.full((1, 14), -1, np.int32)
        path[0, :len(p)] = p
        pool_new, _, err = oracle.commit(pb["parent"], pb["node_row"], d["status"], path,
                                         np.array([len(p)], np.int32), pb["k"], pb["v"],
                                         pb["alpha"], pb["beta"], pb["pool"], pb["state_idx"],
                                         pb["Hqk"], pb["Hv"], False, lib=lib)
        assert err == 0
        for h in range(pb["Hv"]):
            ops = [operands(pb, 0, h, i) for i in range(pb["N"])]
            Q = np.stack([o[0] for o in ops])
            K = np.stack([o[1] for o in ops])
            V = np.stack([o[2] for o in ops])
            al = np.array([o[3] for o in ops])
            be = np.array([o[4] for o in ops])
            S0 = pb["pool"][pb["state_idx"][0], h]
            _, U = cf.solve_tree(par, al, be, Q, K, V, S0)
            Snew = cf.commit_factorized(par, al, p, K, U, S0)
            assert relerr(pool_new[pb["state_idx"][0], h], Snew) < 1e-11


def pin_pure_decay(lib):
    g = np.random.default_rng(12)
    par = random_parent(g, 12)
    pb = small_problem(18, [par], D=8, Hv=2)
    pb["beta"][:] = 0.0
    out, _, states = run_verify(pb, lib)
    for h in range(pb["Hv"]):
        ops = [operands(pb, 0, h, i) for i in range(pb["N"])]
        al = np.array([o[3] for o in ops])
        P = cf.path_decay(par, al)
        S0 = pb["pool"][pb["state_idx"][0], h]
        for i in range(pb["N"]):
            assert relerr(states[0, i, h], P[i] * S0) < 1e-14
            assert relerr(out[0, pb["node_row"][0][i], h], P[i] * (S0 @ ops[i][0])) < 1e-13


def pin_delta_write(lib):
    g = np.random.default_rng(13)
    par = random_parent(g, 10)
    pb = small_problem(19, [par], D=8, Hv=2, unit_k=True)
    pb["alpha"][:] = 1.0
    pb["beta"][:] = 1.0
    _, _, states = run_verify(pb, lib)
    for h in range(pb["Hv"]):
        for i in range(pb["N"]):
            _, k, v, _, _ = operands(pb, 0, h, i)
            assert np.max(np.abs(states[0, i, h] @ k - v)) < 1e-12 * max(1.0, np.max(np.abs(v)))


def _conv_problem(seed, pars, W, C=5, R=None):
    g = np.random.default_rng(seed)
    B = len(pars)
    N = len(pars[0])
    R = R or N + 3
    rows = np.stack([g.permutation(R)[:N] for _ in range(B)]).astype(np.int32)
    x = g.standard_normal((B, R, C))
    P = B + 1
    hist = g.standard_normal((P, W - 1, C))
    w = g.standard_normal((C, W))
    sidx = g.permutation(P)[:B].astype(np.int32)
    return dict(parent=np.stack(pars).astype(np.int32), node_row=rows, x=x, hist=hist, w=w,
                state_idx=sidx, R=R, C=C, W=W, B=B, N=N)


def _conv_run(cp, lib, act=0, bias=None):
    d = oracle.desc_build(cp["parent"], cp["node_row"], cp["R"], cp["W"], lib=lib)
    y, err = oracle.conv(cp["node_row"], d["conv_src"], d["status"], cp["x"], cp["hist"],
                         cp["state_idx"], cp["w"], bias, act, cp["R"], cp["C"], cp["W"], lib=lib)
    return y, err


def _np_causal(seq, wc):
    """Causal conv1d by numpy.convolve: output at position t uses seq[t-W+1..t]
    with weight w[W-1] on the newest element."""
    full = np.convolve(seq, wc[::-1], mode="full")
    return full[len(wc) - 1:len(seq)]


def pin_conv_chain(lib):
    for W in (2, 3, 4):
        N = 7
        cp = _conv_problem(30 + W, [np.arange(-1, N - 1)] * 2, W)
        y, err = _conv_run(cp, lib)
        assert err == 0
        for b in range(cp["B"]):
            for c in range(cp["C"]):
                seq = np.concatenate([cp["hist"][cp["state_idx"][b], :, c],
                                      cp["x"][b, cp["node_row"][b], c]])
                ref = _np_causal(seq, cp["w"][c])
                got = y[b, cp["node_row"][b], c]
                assert np.max(np.abs(got - ref)) < 1e-12


def pin_conv_tree_paths(lib):
    g = np.random.default_rng(31)
    for W in (3, 4):
        par = random_parent(g, 12, bmax=3)
        cp = _conv_problem(40 + W, [par], W)
        y, err = _conv_run(cp, lib, act=1)
        assert err == 0
        for i, anc in enumerate(cf.ancestors(par)):
            nodes = anc + [i]
            for c in range(cp["C"]):
                seq = np.concatenate([cp["hist"][cp["state_idx"][0], :, c],
                                      cp["x"][0, cp["node_row"][0][nodes], c]])
                z = _np_causal(seq, cp["w"][c])[-1]
                ref = z / (1.0 + np.exp(-z))
                assert abs(y[0, cp["node_row"][0][i], c] - ref) < 1e-12


def pin_conv_w1(lib):
    g = np.random.default_rng(32)
    par = random_parent(g, 9)
    cp = _conv_problem(50, [par], 1)
    y, err = _conv_run(cp, lib)
    assert err == 0
    rows = cp["node_row"][0]
    assert np.array_equal(y[0, rows], cp["x"][0, rows] * cp["w"][:, 0][None, :])


def pin_desc_enumeration(lib):
    g = np.random.default_rng(33)
    for trial in range(20):
        N = int(g.integers(1, 20))
        par = random_parent(g, N, bmax=1 + trial % 4)
        R = N + int(g.integers(0, 4))
        rows = g.permutation(R)[:N].astype(np.int32)
        for W in (1, 2, 4):
            d = oracle.desc_build(par[None], rows[None], R, W, lib=lib)
            assert d["err"] == 0
            for i, anc in enumerate(cf.ancestors(par)):
                assert d["depth"][0, i] == len(anc) + 1
                assert int(d["anc"][0, i]) == sum(1 << j for j in anc)
                H = W - 1
                if H == 0:
                    continue
                # explicit: the H entries before node i in the sequence
                # (history slots 0..H-1) ++ (rows of the root-to-parent path)
                seq = [-(s + 1) for s in range(H)] + [int(rows[j]) for j in anc]
                assert list(d["conv_src"][0, i]) == seq[-H:]


def pin_norm_flag(lib):
    g = np.random.default_rng(34)
    par = random_parent(g, 10)
    pb = small_problem(60, [par], D=8, unit_k=False)
    pb["q"] *= 3.0
    pb["k"] *= 0.5
    out_flag, _, _ = run_verify(pb, lib, norm=True)
    pre = dict(pb)
    pre["q"] = pb["q"] / np.sqrt((pb["q"] ** 2).sum(-1, keepdims=True) + 1e-6)
    pre["k"] = pb["k"] / np.sqrt((pb["k"] ** 2).sum(-1, keepdims=True) + 1e-6)
    out_pre, _, _ = run_verify(pre, lib, norm=False)
    rows = pb["node_row"][0]
    assert relerr(out_flag[0, rows], out_pre[0, rows]) < 1e-13


def pin_norm_invariance(lib):
    """q/k normalisation is a property of direction, not length (LumoTree,
    Sec. IV-B: the verifier normalises q and k itself).  Three facts that do
    not restate the normalisation formula:
      (1) large rows (|x| ~ 1e3, so the 1e-6 floor moves nothing by more than
          ~1e-12): scaling each q/k row by its own positive factor leaves every
          output unchanged, and the result equals the outputs on rows divided
          by numpy.linalg.norm;
      (2) rows already of unit length change the outputs by at most ~1e-6;
      (3) rows of tiny norm (|x|^2 ~ 1e-6): the normalised row is the first D
          coordinates of the unit vector of x with one more coordinate
          sqrt(1e-6) appended (the floor inside the square root, read R4)."""
    g = np.random.default_rng(35)
    par = random_parent(g, 11)
    D = 8
    pb = small_problem(61, [par], D=D, unit_k=False)
    rows = pb["node_row"][0]
    big = dict(pb)
    big["q"] = pb["q"] * 1e3
    big["k"] = pb["k"] * 1e3
    out_big, err = run_verify(big, lib, norm=True, want_states=False)
    assert err == 0
    scaled = dict(big)
    scaled["q"] = big["q"] * g.uniform(0.25, 4.0, big["q"].shape[:-1] + (1,))
    scaled["k"] = big["k"] * g.uniform(0.25, 4.0, big["k"].shape[:-1] + (1,))
    out_scaled, _ = run_verify(scaled, lib, norm=True, want_states=False)
    assert relerr(out_scaled[0, rows], out_big[0, rows]) < 1e-10
    unit = dict(pb)
    unit["q"] = pb["q"] / np.linalg.norm(pb["q"], axis=-1, keepdims=True)
    unit["k"] = pb["k"] / np.linalg.norm(pb["k"], axis=-1, keepdims=True)
    out_unit_raw, _ = run_verify(unit, lib, norm=False, want_states=False)
    assert relerr(out_big[0, rows], out_unit_raw[0, rows]) < 1e-10
    out_unit_norm, _ = run_verify(unit, lib, norm=True, want_states=False)
    d_unit = relerr(out_unit_norm[0, rows], out_unit_raw[0, rows])
    assert d_unit < 2e-6
    tiny = dict(pb)
    tiny["q"] = pb["q"] / np.linalg.norm(pb["q"], axis=-1, keepdims=True) * 1e-3
    tiny["k"] = pb["k"] / np.linalg.norm(pb["k"], axis=-1, keepdims=True) * 2e-3
    out_tiny, _ = run_verify(tiny, lib, norm=True, want_states=False)

    def aug_unit(x):
        ext = np.concatenate([x, np.full(x.shape[:-1] + (1,), np.sqrt(1e-6))], axis=-1)
        return (ext / np.linalg.norm(ext, axis=-1, keepdims=True))[..., :-1]

    ref = dict(pb)
    ref["q"], ref["k"] = aug_unit(tiny["q"]), aug_unit(tiny["k"])
    out_ref, _ = run_verify(ref, lib, norm=False, want_states=False)
    assert relerr(out_tiny[0, rows], out_ref[0, rows]) < 1e-12


def pin_u_closed_form(lib):
    g = np.random.default_rng(37)
    pars = [random_parent(g, 13, bmax=2), random_parent(g, 13, bmax=4)]
    pb = small_problem(63, pars, D=10, Hv=2, Hqk=1)
    out, err, u = oracle.verify(pb["parent"], pb["node_row"], np.zeros(2, np.int32), pb["q"], pb["k"],
                                pb["v"], pb["alpha"], pb["beta"], pb["pool"], pb["state_idx"], pb["Hqk"],
                                pb["Hv"], False, want_u=True, lib=lib)
    assert err == 0
    d = oracle.desc_build(pb["parent"], pb["node_row"], pb["R"], 1, lib=lib)
    for b in range(pb["B"]):
        rows = pb["node_row"][b]
        for h in range(pb["Hv"]):
            ops = [operands(pb, b, h, i) for i in range(pb["N"])]
            Q, K, V = (np.stack([o[c] for o in ops]) for c in range(3))
            al = np.array([o[3] for o in ops])
            be = np.array([o[4] for o in ops])
            S0 = pb["pool"][pb["state_idx"][b], h]
            _, U = cf.solve_tree(pars[b], al, be, Q, K, V, S0)
            assert relerr(u[b, rows, h], U) < 1e-11, "u differs from the solve of (I + G) U = R"
        # Eq. (10) with the oracle's own u == the oracle's replayed commit
        fr = int(np.argmax([len(a) for a in cf.ancestors(pars[b])]))
        pth = cf.ancestors(pars[b])[fr] + [fr]
        path = np.full((pb["B"], 13), -1, np.int32)
        path[:, :len(pth)] = pth
        plen = np.zeros(pb["B"], np.int32)
        plen[b] = len(pth)
        path_b = path.copy()
        if b == 0:
            path_b[1] = -1
        pool_new, _, err = oracle.commit(pb["parent"], pb["node_row"], d["status"], path_b, plen, pb["k"],
                                         pb["v"], pb["alpha"], pb["beta"], pb["pool"], pb["state_idx"],
                                         pb["Hqk"], pb["Hv"], False, lib=lib)
        assert err == 0
        for h in range(pb["Hv"]):
            ops = [operands(pb, b, h, i) for i in range(pb["N"])]
            K = np.stack([o[1] for o in ops])
            al = np.array([o[3] for o in ops])
            Snew = cf.commit_factorized(pars[b], al, pth, K, u[b, rows, h], pb["pool"][pb["state_idx"][b], h])
            assert relerr(pool_new[pb["state_idx"][b], h], Snew) < 1e-11


def pin_conv_publish(lib):
    """The conv history a commit publishes is what the causal conv of the
    token sequence needs next (LumoTree, Sec. V-A: the accepted path drives
    the convolution publication; Sec. V-C: windows continue from the prior
    history).  Step 1: a tree convolved over history h0, a root chain of it
    accepted (len 0, shorter than W-1, equal, longer).  Step 2: a chain tree
    convolved over the published history.  Every step-2 output must equal
    numpy.convolve over h0 ++ x of the accepted nodes ++ x of the chain."""
    g = np.random.default_rng(36)
    # a tree with a root path of 6 nodes (plus side branches)
    par1 = np.array([-1, 0, 1, 0, 2, 3, 4, 1, 6, 8, 5], np.int32)
    chain = [0, 1, 2, 4, 6, 8]  # root path of node 8 (parents 1->0, 2->1, 4->2, 6->4, 8->6)
    for j in range(1, len(chain)):
        assert par1[chain[j]] == chain[j - 1]
    N1, N2 = len(par1), 5
    par2 = np.arange(-1, N2 - 1, dtype=np.int32)
    C = 4
    for W in (2, 3, 4):
        H = W - 1
        lengths = [0, 1, 2, 3, 4, 6]
        B = len(lengths)
        R1, R2 = N1 + 2, N2 + 3
        rows1 = np.stack([g.permutation(R1)[:N1] for _ in range(B)]).astype(np.int32)
        rows2 = np.stack([g.permutation(R2)[:N2] for _ in range(B)]).astype(np.int32)
        x1 = g.standard_normal((B, R1, C))
        x2 = g.standard_normal((B, R2, C))
        P = B + 1
        h0 = g.standard_normal((P, H, C))
        w = g.standard_normal((C, W))
        sidx = g.permutation(P)[:B].astype(np.int32)
        path = np.full((B, len(chain)), -1, np.int32)
        for b, L in enumerate(lengths):
            path[b, :L] = chain[:L]
        plen = np.array(lengths, np.int32)
        # commit of step 1's accepted paths (state operands are irrelevant here)
        pb = small_problem(62 + W, [par1] * B, R=R1, D=4, Hv=1)
        d1 = oracle.desc_build(np.tile(par1, (B, 1)), rows1, R1, 1, lib=lib)
        _, h1, err = oracle.commit(np.tile(par1, (B, 1)), rows1, d1["status"], path, plen, pb["k"],
                                   pb["v"], pb["alpha"], pb["beta"], pb["pool"][:P], sidx, 1, 1,
                                   False, x=x1, hist=h0, W=W, lib=lib)
        assert err == 0
        d2 = oracle.desc_build(np.tile(par2, (B, 1)), rows2, R2, W, lib=lib)
        y2, err = oracle.conv(rows2, d2["conv_src"], d2["status"], x2, h1, sidx, w, None, 0, R2, C,
                              W, lib=lib)
        assert err == 0
        for b, L in enumerate(lengths):
            for c in range(C):
                seq = np.concatenate([h0[sidx[b], :, c], x1[b, rows1[b][chain[:L]], c],
                                      x2[b, rows2[b], c]])
                ref = _np_causal(seq, w[c])[L:]
                got = y2[b, rows2[b], c]
                assert np.max(np.abs(got - ref)) < 1e-12, (W, L, c)


ALL_PINS = [
    pin_chain_textbook, pin_paths_are_chains, pin_sibling_isolation, pin_commit_is_replay,
    pin_closed_form, pin_treewy_states, pin_nilpotent, pin_factorized_commit, pin_pure_decay,
    pin_delta_write, pin_conv_chain, pin_conv_tree_paths, pin_conv_w1, pin_desc_enumeration,
    pin_norm_flag, pin_norm_invariance, pin_conv_publish, pin_u_closed_form,
]


def failing_pins(lib):
    bad = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            bad.append(pin.__name__)
    return bad
