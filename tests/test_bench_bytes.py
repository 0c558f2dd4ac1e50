"""The bench's byte model on the conv-fed 27-node workload (B = 128, 32 value
heads over 16 qk heads, d = 128, causal conv of width 4 over 8,192 channels).

Algorithmic bytes follow the state-streaming accounting of a GDN layer step
(TreeWY, Sec. 1 and the Bole review, Sec. 1: the fp32 state S is read once
and the committed state written once per request and head; LumoTree, Sec. V-A
and V-C: the conv input rows are read once, the conv history is read and
replaced): q/k/v count once, as the conv input x, and the conv output's round
trip through memory is never credited.  The expected figures below are
written out per tensor, with their shapes, independently of the bench's own
helper functions.
"""
import sys
from pathlib import Path

import numpy as np
import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import gdn_inputs as gi  # noqa: E402

import bench  # noqa: E402

B, N, D, HV, HQK, W = 128, 27, 128, 32, 16, 4
C = 2 * HQK * D + HV * D  # conv channels: q | k | v


def _cfg():
    cfg = gi.CONFIGS[4]
    assert (cfg.N, cfg.D, cfg.Hv, cfg.Hqk, cfg.conv_W, cfg.conv_C) == (N, D, HV, HQK, W, C)
    return cfg


def _paths(seed):
    rng = np.random.default_rng(seed)
    L = rng.integers(0, 7, size=B).astype(np.int32)  # accepted path lengths, 0 allowed
    L[:3] = [0, 1, 6]
    return L


def _expected_layer(L):
    state_tile = D * D * 4                                   # one head's fp32 state
    state_read = B * HV * state_tile                         # every request is verified
    state_write = int((L > 0).sum()) * HV * state_tile       # only requests with a path commit
    outputs = B * N * HV * D * 4                             # fp32 o_i
    gates = B * N * HV * (4 + 4)                             # alpha_i, beta_i
    path_rows = int(L.sum()) * (HQK * D + HV * D) * 2        # the path's k and v conv inputs (bf16)
    path_gates = int(L.sum()) * HV * (4 + 4)
    x_rows = B * N * C * 2                                   # the tree's conv input, once
    history = B * (W - 1) * C * 2 * 2                        # history read and written
    weights = C * W * 2
    new_hist_rows = int(np.minimum(L, W - 1).sum()) * C * 2  # accepted rows entering the history
    return (state_read + state_write + outputs + gates + path_rows + path_gates + x_rows + history + weights
            + new_hist_rows)


@pytest.mark.parametrize("seed", [0, 1])
def test_layer_step_bytes_follow_the_state_streaming_count(seed):
    cfg = _cfg()
    L = _paths(seed)
    cur = {"B": B, "path_len": _paths(seed + 100)}
    prev = {"B": B, "path_len": L, "path": np.zeros((B, 6), np.int32)}
    m = bench.byte_model(cfg, cur, prev, "layer")
    assert m["layer"] == _expected_layer(L)


def test_fused_form_moves_the_same_bytes_and_no_conv_output():
    cfg = _cfg()
    L = _paths(3)
    cur = {"B": B, "path_len": _paths(4)}
    prev = {"B": B, "path_len": L, "path": np.zeros((B, 6), np.int32)}
    layer = bench.byte_model(cfg, cur, prev, "layer")
    fused = bench.byte_model(cfg, cur, prev, "fused")
    # two launches (conv, then commit + verify) credit exactly the one-launch bytes:
    # the conv output y written by one and read by the other is not counted
    assert fused["conv"] + fused["commit_verify"] == layer["layer"]
    # the conv itself: its input rows, the history read and written, the weights
    # and the accepted rows entering the history (no output term)
    assert fused["conv"] == B * N * C * 2 + B * (W - 1) * C * 4 + C * W * 2 + int(np.minimum(L, W - 1).sum()) * C * 2


def test_separate_form_passes_over_the_state_three_times():
    cfg = _cfg()
    L = _paths(5)
    cur = {"B": B, "path_len": L, "path": np.zeros((B, 6), np.int32)}
    sep = bench.byte_model(cfg, cur, cur, "separate")
    state = B * HV * D * D * 4
    active = int((L > 0).sum()) * HV * D * D * 4
    # verify reads the state once (q/k/v come from the conv: not credited again)
    assert sep["verify"] == state + B * N * HV * 8 + B * N * HV * D * 4
    # the commit reads and writes the committed requests' states
    assert sep["commit"] == 2 * active + int(L.sum()) * ((HQK * D + HV * D) * 2 + HV * 8)
