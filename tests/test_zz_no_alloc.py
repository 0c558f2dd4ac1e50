"""gdn_tree_attention_noalloc (the library's own scratch, nothing allocated)
against gdn_tree_attention (a caller workspace) through the C ABI, on two
calls in a row, the second with a smaller input, and against the fp64
oracle: outputs must agree bit for bit with the workspace call (the same
kernels on the same inputs) and within 2e-3 of the oracle."""
import numpy as np
import pytest

import gdn_inputs as gi
from harness import max_rel_rows, to_dev
from oracle.attention import tree_attention as oracle_tree_attention

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _run(c, splits, noalloc):
    import torch
    import tree_speculative_verification_gdn_amd as g
    B, N, Hq, D = c["B"], c["N"], c["Hq"], c["D"]
    desc = g.TreeDesc(to_dev(c["parent"]), to_dev(c["node_row"]), c["R"], 1, B=B)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.gdn_tree_desc_build(desc, err)
    out = torch.full((B, N, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    q, k, v, ctx = to_dev(c["q"]), to_dev(c["k"]), to_dev(c["v"]), to_dev(c["ctx"])
    if noalloc:
        code = g.gdn_tree_attention_noalloc(desc, q, k, v, ctx, out, err, splits=splits)
    else:
        nbytes = g.gdn_tree_attention_workspace_bytes(B, N, Hq, D, splits)
        ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
        code = g.gdn_tree_attention(desc, q, k, v, ctx, out, ws, err, splits=splits)
    torch.cuda.synchronize()
    return code, out.cpu().numpy(), int(err.item()), desc.status.cpu().numpy()


def test_noalloc_matches_workspace_call_on_two_calls():
    import tree_speculative_verification_gdn_amd as g
    big = gi.make_attention_case(31, B=3, N=27, R=32, Hq=16, Hkv=2, D=256, ctx=[900, 1700, 3000], S=3100,
                                 packing="bfs")
    small = gi.make_attention_case(32, B=1, N=9, R=12, Hq=4, Hkv=2, D=128, ctx=[45], S=64)
    for c, splits in ((big, 16), (small, 2)):  # the second call is smaller: stale scratch must not leak
        need = g.gdn_tree_attention_workspace_bytes(c["B"], c["N"], c["Hq"], c["D"], splits)
        assert need <= g.GDN_ATTN_NOALLOC_SCRATCH_BYTES
        code_w, out_w, err_w, st = _run(c, splits, noalloc=False)
        code_n, out_n, err_n, _ = _run(c, splits, noalloc=True)
        assert code_w == code_n == 0 and err_w == err_n == 0
        assert np.array_equal(out_n, out_w, equal_nan=True)
        ref = oracle_tree_attention(c["parent"], c["node_row"], st, c["q"], c["k"], c["v"], c["ctx"], c["R"],
                                    c["Hq"], c["Hkv"], 1.0 / np.sqrt(c["D"]))[0]
        assert max_rel_rows(out_n, ref, 1) <= TOL


def test_noalloc_refuses_past_its_scratch_and_launches_nothing():
    import torch
    import tree_speculative_verification_gdn_amd as g
    c = gi.make_attention_case(33, B=2, N=27, R=32, Hq=16, Hkv=2, D=256, ctx=[100, 200], S=300, packing="bfs")
    splits = 600
    assert g.gdn_tree_attention_workspace_bytes(2, 27, 16, 256, splits) > g.GDN_ATTN_NOALLOC_SCRATCH_BYTES
    desc = g.TreeDesc(to_dev(c["parent"]), to_dev(c["node_row"]), c["R"], 1, B=2)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.gdn_tree_desc_build(desc, err)
    out = torch.full((2, 27, 16, 256), float("nan"), dtype=torch.float32, device="cuda")
    code = g.gdn_tree_attention_noalloc(desc, to_dev(c["q"]), to_dev(c["k"]), to_dev(c["v"]), to_dev(c["ctx"]),
                                        out, err, splits=splits, raise_on_error=False)
    torch.cuda.synchronize()
    assert code == g.GDN_ERR_UNSUPPORTED
    assert torch.isnan(out).all().item() and int(err.item()) == 0
