"""Malformed inputs: the oracle's error bits and the untouched outputs they
imply (the GPU path must reproduce both bit-exactly)."""
import numpy as np

import oracle
from oracle_pins import small_problem, random_parent


def test_desc_rejects_bad_parent_and_rows():
    par = np.array([[-1, 0, 1, 1], [-1, 0, 3, 1], [-1, -2, 0, 0]], np.int32)
    rows = np.array([[0, 1, 2, 3], [0, 1, 2, 3], [0, 1, 2, 3]], np.int32)
    d = oracle.desc_build(par, rows, 4, 4)
    assert d["status"].tolist() == [0, oracle.EV_PARENT, oracle.EV_PARENT]
    assert d["err"] == oracle.EV_PARENT
    assert (d["depth"][1:] == 0).all() and (d["anc"][1:] == 0).all() and (d["conv_src"][1:] == 0).all()
    rows2 = np.array([[0, 1, 1, 3], [0, 1, 2, 9], [0, 1, 2, -1]], np.int32)
    d = oracle.desc_build(par[:1].repeat(3, 0), rows2, 4, 1)
    assert d["status"].tolist() == [oracle.EV_ROW] * 3


def _commit(pb, path, plen, sidx=None):
    d = oracle.desc_build(pb["parent"], pb["node_row"], pb["R"], 1)
    return oracle.commit(pb["parent"], pb["node_row"], d["status"], path, plen, pb["k"],
                         pb["v"], pb["alpha"], pb["beta"], pb["pool"],
                         pb["state_idx"] if sidx is None else sidx, pb["Hqk"], pb["Hv"], False)


def test_commit_len0_is_identity_and_bad_paths_are_skipped():
    g = np.random.default_rng(1)
    pars = [random_parent(g, 8) for _ in range(4)]
    pb = small_problem(2, pars, D=6)
    B = 4
    path = np.full((B, 8), -1, np.int32)
    plen = np.zeros(B, np.int32)
    # b0: len 0; b1: starts at a non-root node; b2: skips a level; b3: len > Lmax
    path[1, :2] = [1, 2]
    plen[1] = 2
    chain = [0]
    n = int(np.argmax([len(a) for a in __import__("oracle.closed_form", fromlist=["x"]).ancestors(pars[2])]))
    from oracle.closed_form import ancestors
    full = ancestors(pars[2])[n] + [n]
    if len(full) >= 3:
        bad = [full[0], full[2]]
    else:
        bad = [full[-1], full[0]]
    path[2, :2] = bad
    plen[2] = 2
    plen[3] = 9
    pool_new, _, err = _commit(pb, path, plen)
    assert err == oracle.EV_PATH
    assert np.array_equal(pool_new, pb["pool"])


def test_commit_rejects_duplicate_and_out_of_range_slots():
    g = np.random.default_rng(3)
    pars = [random_parent(g, 6) for _ in range(3)]
    pb = small_problem(5, pars, D=6)
    path = np.zeros((3, 6), np.int32)
    plen = np.ones(3, np.int32)
    sidx = np.array([1, 1, 0], np.int32)
    pool_new, _, err = _commit(pb, path, plen, sidx)
    assert err == oracle.EV_STATE
    assert np.array_equal(pool_new[1], pb["pool"][1])
    assert not np.array_equal(pool_new[0], pb["pool"][0])  # request 2 committed
    sidx = np.array([0, 7, 2], np.int32)
    pool_new, _, err = _commit(pb, path, plen, sidx)
    assert err == oracle.EV_STATE
    # verify only checks the range (it never writes the pool)
    d = oracle.desc_build(pb["parent"], pb["node_row"], pb["R"], 1)
    out, err = oracle.verify(pb["parent"], pb["node_row"], d["status"], pb["q"], pb["k"], pb["v"],
                             pb["alpha"], pb["beta"], pb["pool"], np.array([1, 1, 0], np.int32),
                             1, 2, False)
    assert err == 0
    out, err = oracle.verify(pb["parent"], pb["node_row"], d["status"], pb["q"], pb["k"], pb["v"],
                             pb["alpha"], pb["beta"], pb["pool"], np.array([0, 9, 1], np.int32),
                             1, 2, False)
    assert err == oracle.EV_STATE
    assert np.isnan(out[1]).all()


def test_conv_history_publish():
    # W=4: last 3 of (hist ++ accepted rows)
    g = np.random.default_rng(9)
    par = np.array([[-1, 0, 1, 1, 2]], np.int32)
    rows = np.array([[4, 0, 2, 1, 3]], np.int32)
    B, R, C, W = 1, 6, 3, 4
    x = g.standard_normal((B, R, C))
    hist = g.standard_normal((2, W - 1, C))
    pb = small_problem(6, [par[0]], R=R, D=4, Hv=1)
    pb["node_row"] = rows
    d = oracle.desc_build(par, rows, R, 1)
    for L in range(0, 4):
        path = np.array([[0, 1, 2, -1]], np.int32)
        sidx = np.array([1], np.int32)
        _, hnew, err = oracle.commit(par, rows, d["status"], path, np.array([L], np.int32),
                                     pb["k"], pb["v"], pb["alpha"], pb["beta"], pb["pool"][:2],
                                     sidx, 1, 1, False, x=x, hist=hist, W=W)
        assert err == 0
        seq = list(hist[1]) + [x[0, rows[0, n]] for n in [0, 1, 2][:L]]
        assert np.array_equal(hnew[1], np.stack(seq[-3:]))
        assert np.array_equal(hnew[0], hist[0])
