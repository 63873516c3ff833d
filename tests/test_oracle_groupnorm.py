"""Pins of the oracle's GroupNorm (CPU only): a hand-worked fixture, the
zero-mean / unit-variance invariant, direct loops, torch group_norm."""
import json
import os

import numpy as np
import torch

from oracle import edit_oracle as O


def test_groupnorm_worked(golden_dir):
    with open(os.path.join(golden_dir, "groupnorm_worked.json")) as f:
        g = json.load(f)
    grid = np.array(g["grid"], dtype=np.float64)[None]       # [1, 1, 2, 4]
    mean, var = O.group_norm_stats(grid, g["groups"])
    np.testing.assert_array_equal(mean[0], g["mean"])
    np.testing.assert_array_equal(var[0], g["var"])


def test_groupnorm_invariant():
    rng = np.random.default_rng(0)
    B, H, W, C, G = 3, 5, 7, 12, 4
    x = rng.standard_normal((B, H, W, C)) * 3.0 + 1.5
    y = O.group_norm(x, G, np.ones(C), np.zeros(C))
    _, var = O.group_norm_stats(x, G)
    v = y.reshape(B, H * W, G, C // G)
    np.testing.assert_allclose(v.mean(axis=(1, 3)), 0.0, atol=1e-12)
    np.testing.assert_allclose(v.var(axis=(1, 3)), var / (var + O.GN_EPS), rtol=1e-12)


def test_groupnorm_groups_are_consecutive_channels():
    x = np.zeros((1, 2, 2, 8))
    x[..., 0] = 4.0           # only channel 0 moves: only group 0 (channels 0,1) sees it
    mean, _ = O.group_norm_stats(x, 4)
    np.testing.assert_array_equal(mean[0], [2.0, 0, 0, 0])


def test_groupnorm_vs_loops_and_torch():
    rng = np.random.default_rng(1)
    B, H, W, C, G = 2, 3, 4, 6, 3
    x = rng.standard_normal((B, H, W, C))
    gamma = rng.standard_normal(C); beta = rng.standard_normal(C)
    y = O.group_norm(x, G, gamma, beta)
    cg = C // G
    ref = np.zeros_like(x)
    for b in range(B):
        for g in range(G):
            vals = [x[b, i, j, c] for i in range(H) for j in range(W) for c in range(g * cg, (g + 1) * cg)]
            m = sum(vals) / len(vals)
            v = sum((t - m) ** 2 for t in vals) / len(vals)
            for i in range(H):
                for j in range(W):
                    for c in range(g * cg, (g + 1) * cg):
                        ref[b, i, j, c] = (x[b, i, j, c] - m) / (v + O.GN_EPS) ** 0.5 * gamma[c] + beta[c]
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-11)
    t = torch.nn.functional.group_norm(torch.from_numpy(x).permute(0, 3, 1, 2), G,
                                       torch.from_numpy(gamma), torch.from_numpy(beta), eps=O.GN_EPS)
    np.testing.assert_allclose(y, t.permute(0, 2, 3, 1).numpy(), rtol=1e-10, atol=1e-10)
