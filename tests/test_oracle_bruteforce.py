"""Brute force over every parent array of tiny trees (N <= 5: N! arrays; N = 6
under -m slow): descriptor vs explicit path enumeration, each path == its own
chain run, closed form, commit of every frontier."""
import itertools

import numpy as np
import pytest

import oracle
from oracle import closed_form as cf
from oracle_pins import small_problem, run_verify, operands, chain_textbook, relerr


def all_parents(N):
    choices = [range(-1, i) for i in range(N)]
    for combo in itertools.product(*choices):
        yield np.array(combo, np.int32)


def _check_tree(par, seed):
    N = len(par)
    pb = small_problem(seed, [par], D=4, Hv=1, Hqk=1)
    lib = oracle.load()
    d = oracle.desc_build(pb["parent"], pb["node_row"], pb["R"], 3)
    anc = cf.ancestors(par)
    for i in range(N):
        assert d["depth"][0, i] == len(anc[i]) + 1
        assert int(d["anc"][0, i]) == sum(1 << j for j in anc[i])
        seq = [-1, -2] + [int(pb["node_row"][0][j]) for j in anc[i]]
        assert list(d["conv_src"][0, i]) == seq[-2:]
    out, err, st = run_verify(pb, lib)
    assert err == 0
    ops = [operands(pb, 0, 0, i) for i in range(N)]
    S0 = pb["pool"][pb["state_idx"][0], 0]
    Q = np.stack([o[0] for o in ops]); K = np.stack([o[1] for o in ops]); V = np.stack([o[2] for o in ops])
    al = np.array([o[3] for o in ops]); be = np.array([o[4] for o in ops])
    O, U = cf.solve_tree(par, al, be, Q, K, V, S0)
    assert relerr(out[0, pb["node_row"][0], 0], O) < 1e-11
    for i in range(N):
        nodes = anc[i] + [i]
        S_end, outs = chain_textbook(S0, [ops[j] for j in nodes])
        assert relerr(st[0, i, 0], S_end) < 1e-12
        path = np.array([nodes + [-1] * (N - len(nodes))], np.int32)
        pool_new, _, err = oracle.commit(pb["parent"], pb["node_row"], d["status"], path,
                                         np.array([len(nodes)], np.int32), pb["k"], pb["v"],
                                         pb["alpha"], pb["beta"], pb["pool"], pb["state_idx"],
                                         1, 1, False)
        assert err == 0
        assert np.array_equal(pool_new[pb["state_idx"][0], 0], st[0, i, 0])


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5])
def test_all_trees(N):
    for t, par in enumerate(all_parents(N)):
        _check_tree(par, 1000 * N + t)


@pytest.mark.slow
def test_all_trees_n6():
    for t, par in enumerate(all_parents(6)):
        _check_tree(par, 6000 + t)
