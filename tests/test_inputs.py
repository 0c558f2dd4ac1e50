"""Seeded synthetic inputs: determinism, tree shape limits, row packing, path
draws, bf16 rounding (checked against torch's own float->bfloat16 cast)."""
import numpy as np
import torch

import gdn_inputs as gi


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1e-40, 3.4e38, -3.4e38, np.inf, -np.inf], np.float32)])
    # include exact halfway cases
    halves = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, halves])
    ours = gi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(gi.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_trees_respect_limits_and_are_seeded():
    for cid in (3, 5):
        cfg = gi.CONFIGS[cid]
        for b in range(20):
            par = gi.tree_for(cfg, 2026, b)
            assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, len(par)))
            ch = np.bincount(par[par >= 0], minlength=len(par))
            assert ch.max() <= cfg.bmax
            assert gi.path_lengths(par).max() <= cfg.depth_max + 1
            assert np.array_equal(par, gi.tree_for(cfg, 2026, b))
    assert gi.tree_for(gi.CONFIGS[1], 0, 0).tolist() == [-1, 0, 0, 1, 1, 2, 2]
    assert gi.tree_for(gi.CONFIGS[2], 0, 0).tolist() == list(range(-1, 7))


def test_case_layout_and_paths():
    cfg = gi.CONFIGS[3]
    c1 = gi.make_case(cfg, seed=7, B=4, extra_slots=2)
    c2 = gi.make_case(cfg, seed=7, B=4, extra_slots=2)
    for key in ("parent", "node_row", "q", "k", "v", "alpha", "beta", "pool", "state_idx", "path"):
        assert np.array_equal(c1[key], c2[key], equal_nan=True), key
    assert c1["q"].dtype == np.uint16 and c1["q"].shape == (4, 32, 16, 128)
    assert c1["v"].shape == (4, 32, 32, 128) and c1["pool"].shape == (6, 32, 128, 128)
    for b in range(4):
        rows = c1["node_row"][b]
        assert len(set(rows.tolist())) == cfg.N and rows.max() < cfg.R
        pad = np.setdiff1d(np.arange(cfg.R), rows)
        assert (c1["q"][b, pad] == gi.BF16_NAN).all()
        L = c1["path_len"][b]
        p = c1["path"][b, :L]
        assert c1["parent"][b, p[0]] == -1
        assert all(c1["parent"][b, p[j]] == p[j - 1] for j in range(1, L))
    unused = np.setdiff1d(np.arange(6), c1["state_idx"])
    assert np.isnan(c1["pool"][unused]).all()


def test_bfs_packing_trap():
    par = gi.tree_for(gi.CONFIGS[3], 2026, 0)
    rows = gi.bfs_rows(par)
    inv = np.argsort(rows)
    prev_is_parent = sum(1 for r in range(1, len(par)) if par[inv[r]] == inv[r - 1])
    assert prev_is_parent < len(par) // 2
