"""Worked examples printed on the pages (structure only: the pages print no
numeric values for them).  Fixtures under tests/golden/ carry their citation."""
import json
import os

import numpy as np

import oracle
from oracle import closed_form as cf
from oracle_pins import small_problem, run_verify, chain_textbook, operands, relerr

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_bole_three_node_example():
    fx = _load("bole_three_node.json")
    par = np.array(fx["parent"], np.int32)
    assert cf.ancestors(par) == fx["strict_ancestors"]
    d = oracle.desc_build(par[None], np.arange(3, dtype=np.int32)[None], 3, 1)
    for i, anc in enumerate(fx["strict_ancestors"]):
        assert int(d["anc"][0, i]) == sum(1 << j for j in anc)
    pb = small_problem(3, [par], D=6, Hv=1)
    ops = [operands(pb, 0, 0, i) for i in range(3)]
    K = np.stack([o[1] for o in ops])
    al = np.array([o[3] for o in ops])
    be = np.array([o[4] for o in ops])
    G = cf.g_matrix(par, al, be, K)
    nz = sorted([list(map(int, ij)) for ij in zip(*np.nonzero(G))])
    assert nz == sorted(fx["G_nonzero_positions"])
    assert np.all(G @ G == 0.0) == fx["G_squared_is_zero"]
    assert np.allclose(np.linalg.inv(np.eye(3) + G), np.eye(3) - G, rtol=0, atol=1e-15)
    # S_3 from S_1, not S_2: node 2 (0-based) equals the chain 0 -> 2
    out, _, st = run_verify(pb, oracle.load())
    S_end, _ = chain_textbook(pb["pool"][pb["state_idx"][0], 0], [ops[0], ops[2]])
    assert relerr(st[0, 2, 0], S_end) < 1e-13


def test_packed_row_trap_example():
    fx = _load("packed_row_trap.json")
    par = np.array(fx["parent"], np.int32)[None]
    rows = np.array(fx["node_row"], np.int32)[None]
    d = oracle.desc_build(par, rows, fx["R"], fx["conv_W"])
    assert d["err"] == 0
    assert d["depth"][0].tolist() == fx["expected_depth"]
    assert [int(a) for a in d["anc"][0]] == fx["expected_anc_bits"]
    assert d["conv_src"][0].tolist() == fx["expected_conv_src_W4"]
    # the spine m -> a -> d publishes the state of running a then d, and d's
    # verify state is built from a (row 1), not from b (row 2, previous packed row)
    pb = small_problem(4, [fx["parent"]], R=fx["R"], D=6, Hv=1)
    pb["node_row"] = rows
    out, _, st = run_verify(pb, oracle.load())
    ops = [operands(pb, 0, 0, i) for i in range(4)]
    S0 = pb["pool"][pb["state_idx"][0], 0]
    S_ad, _ = chain_textbook(S0, [ops[0], ops[2]])
    S_bd, _ = chain_textbook(S0, [ops[1], ops[2]])
    assert relerr(st[0, 2, 0], S_ad) < 1e-13
    assert relerr(st[0, 2, 0], S_bd) > 1e-3
    path = np.array([fx["spine_path"]], np.int32)
    pool_new, _, err = oracle.commit(par, rows, d["status"], path, np.array([2], np.int32),
                                     pb["k"], pb["v"], pb["alpha"], pb["beta"], pb["pool"],
                                     pb["state_idx"], 1, 1, False)
    assert err == 0
    assert np.array_equal(pool_new[pb["state_idx"][0], 0], st[0, 2, 0])
