"""GPU parity with raw gate inputs (GDN_F_RAW_GATES): alpha / beta hold the
raw per-node inputs a, b and gate_params the per-head A_log, dt_bias; the
kernels evaluate the gates themselves (fp32, hardware exp2 / log2), the
oracle evaluates them in fp64 (oracle/gates.py) and runs its usual
recurrence.  Same bars as the other parity tests: error bits and untouched
rows / slots bit-exact, outputs and committed states within 2e-3 (max
relative per row).  Covered: verify (matrix-core and vector-ALU kernels),
commit, the fused commit + verify, the one-launch layer step and the
layer-batched commit."""
import numpy as np
import pytest

import gdn_inputs as gi
from harness import (max_rel_rows, node_rows_mask, run_gpu, run_gpu_layer, run_gpu_two_steps,
                     run_oracle, run_oracle_two_steps, two_step_case)

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _g():
    import tree_speculative_verification_gdn_amd as g
    return g


def _raw_two_steps(c1, c2):
    r1 = gi.with_raw_gates(c1)
    return r1, gi.with_raw_gates(c2, r1["gate_params"])


def _cmp_single(case, gr, orr):
    assert gr["err"] == orr["err"]
    m = node_rows_mask(case)
    assert np.isnan(gr["out"][~m]).all()
    rel = max_rel_rows(gr["out"][m], orr["out"][m], 2)
    assert rel <= TOL, f"output max rel {rel:.3e}"
    used = case["state_idx"]
    rel = max_rel_rows(gr["pool"][used], orr["pool"][used], 2)
    assert rel <= TOL, f"state max rel {rel:.3e}"
    z = used[case["path_len"] == 0]
    assert np.array_equal(gr["pool"][z], case["pool"][z])


@pytest.mark.parametrize("valu", [False, True])
def test_verify_and_commit_tree27(valu):
    g = _g()
    case = gi.with_raw_gates(gi.make_case(gi.CONFIGS[3], seed=61, B=6))
    gr = run_gpu(case, flags=g.GDN_F_VALU if valu else 0)
    orr = run_oracle(case)
    _cmp_single(case, gr, orr)


def test_verify_and_commit_tree64():
    # two 32-row blocks: the wide-tree kernel with the gates evaluated in it
    case = gi.with_raw_gates(gi.make_case(gi.CONFIGS[5], seed=65, B=4))
    _cmp_single(case, run_gpu(case), run_oracle(case))


def test_verify_and_commit_f32_small():
    case = gi.with_raw_gates(gi.make_case(gi.CONFIGS[1], seed=62, B=3))
    _cmp_single(case, run_gpu(case), run_oracle(case))


def test_raw_gates_differ_from_taking_them_as_gates():
    # the flag is honoured: the same buffers read as activated gates give
    # another result (guards against the parameters being ignored)
    case = gi.with_raw_gates(gi.make_case(gi.CONFIGS[3], seed=63, B=2))
    plain = dict(case)
    del plain["gate_params"]
    plain["alpha"] = np.clip(case["alpha"], 0.0, 1.0)
    plain["beta"] = np.clip(case["beta"], 0.0, 1.0)
    a = run_gpu(case, commit=False)
    b = run_gpu(plain, commit=False)
    m = node_rows_mask(case)
    assert max_rel_rows(a["out"][m], b["out"][m], 2) > 1e-2


@pytest.mark.parametrize("cfg_id", [3, 2, 5])
def test_fused_commit_verify(cfg_id):
    c1, c2 = two_step_case(gi.CONFIGS[cfg_id], seed=64, B=5, extra_slots=1)
    r1, r2 = _raw_two_steps(c1, c2)
    gr = run_gpu_two_steps(r1, r2)
    orr = run_oracle_two_steps(r1, r2)
    assert gr["err"] == orr["err"]
    m = node_rows_mask(r2) & (orr["status2"] == 0)[:, None]
    assert max_rel_rows(gr["out"][m], orr["out"][m], 2) <= TOL
    used = r1["state_idx"]
    assert max_rel_rows(gr["pool"][used], orr["pool"][used], 2) <= TOL
    # the separate calls agree with the fused ones (fp32 rounding apart: the
    # fused replay runs on the matrix cores with a hi/lo split of the state)
    gs = run_gpu_two_steps(r1, r2, fused=False)
    assert max_rel_rows(gs["out"][m], gr["out"][m], 2) <= 1e-4
    assert max_rel_rows(gs["pool"][used], gr["pool"][used], 2) <= 1e-4


def test_layer_step_exact_conv():
    cfg = gi.CONFIGS[4].replace(act=0)
    c1, c2 = two_step_case(cfg, seed=65, B=5, extra_slots=1, conv_values="dyadic")
    r1, r2 = _raw_two_steps(c1, c2)
    gr = run_gpu_layer(r1, r2)
    orr = run_oracle_two_steps(r1, r2)
    assert gr["err"] == orr["err"] == 0
    m = node_rows_mask(r2)
    assert np.array_equal(gr["y2"][m], orr["y2"][m])
    assert max_rel_rows(gr["out"][m], orr["out"][m], 2) <= TOL
    used = r1["state_idx"]
    assert max_rel_rows(gr["pool"][used], orr["pool"][used], 2) <= TOL


def test_layer_step_long_paths():
    # whole-chain paths longer than one replay segment (the long-path kernel)
    cfg = gi.CONFIGS[2].replace(N=20, R=23, Hv=4, Hqk=2, conv_W=4, conv_C=1024, norm_qk=True, act=0)
    c1, c2 = two_step_case(cfg, seed=66, B=3, conv_values="dyadic")
    r1, r2 = _raw_two_steps(c1, c2)
    gr = run_gpu_layer(r1, r2)
    orr = run_oracle_two_steps(r1, r2)
    assert (gr["path_n"] == 20).all()
    m = node_rows_mask(r2)
    assert max_rel_rows(gr["out"][m], orr["out"][m], 2) <= TOL
    used = r1["state_idx"]
    assert max_rel_rows(gr["pool"][used], orr["pool"][used], 2) <= TOL


def test_commit_layers():
    import torch
    from harness import to_dev
    from test_gpu_commit_layers import layer_slice, layers_case, oracle_commit
    g = _g()
    cfg = gi.CONFIGS[3]
    lc = layers_case(cfg, seed=67, L=3, B=4, extra_slots=1)
    gps = []
    for l in range(3):
        r = gi.with_raw_gates(dict(layer_slice(lc, l), layer=l))
        lc["alpha"][l], lc["beta"][l] = r["alpha"], r["beta"]
        gps.append(r["gate_params"])
    gp = np.stack(gps)
    desc = g.TreeDesc(to_dev(lc["parent"]), to_dev(lc["node_row"]), cfg.R, 1, B=lc["B"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.gdn_tree_desc_build(desc, err)
    pool = to_dev(lc["pool"])
    g.gdn_tree_commit_layers(desc, to_dev(lc["path"]), to_dev(lc["path_len"]), to_dev(lc["k"]),
                             to_dev(lc["v"]), to_dev(lc["alpha"]), to_dev(lc["beta"]), pool,
                             to_dev(lc["state_idx"]), err, gate_params=to_dev(gp))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    gpool = pool.cpu().numpy()
    used = lc["state_idx"]
    for l in range(3):
        c = dict(layer_slice(lc, l), gate_params=gp[l])
        from harness import oracle_gates
        c["alpha"], c["beta"] = oracle_gates(c)
        op, _ = oracle_commit(c, False)
        assert max_rel_rows(gpool[l][used], op[used], 2) <= TOL, f"layer {l}"
