"""Pins of the oracle's convolutions and reshapes (CPU only).

Against: hand-worked fixtures (tests/golden/conv3x3_worked.json,
dwconv_s2_worked.json), direct nested loops, and torch.nn.functional.conv2d
on the CPU as an independent implementation.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import edit_oracle as O


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_conv3x3_worked_examples(golden_dir):
    g = _load(golden_dir, "conv3x3_worked.json")
    inp = np.array(g["input"], dtype=np.float64)[None, :, :, None]
    for case in g["cases"]:
        w = np.array(case["w"], dtype=np.float64)[None, :, :, None]   # [Cout=1][3][3][Cin=1]
        out = O.conv3x3(inp, w, np.array([case["b"]], dtype=np.float64))
        np.testing.assert_array_equal(out[0, :, :, 0], np.array(case["out"]), err_msg=case["name"])


def test_dwconv_s2_worked_examples(golden_dir):
    g = _load(golden_dir, "dwconv_s2_worked.json")
    inp = np.array(g["input"], dtype=np.float64)[None, :, :, None]
    for case in g["cases"]:
        w = np.array(case["w"], dtype=np.float64)[:, :, None]          # [3][3][C=1]
        out = O.dwconv3x3_s2(inp, w, np.array([case["b"]], dtype=np.float64))
        np.testing.assert_array_equal(out[0, :, :, 0], np.array(case["out"]), err_msg=case["name"])


def _conv3x3_loops(g, w, b):
    B, H, W, Ci = g.shape
    Co = w.shape[0]
    out = np.zeros((B, H, W, Co))
    for bb in range(B):
        for y in range(H):
            for x in range(W):
                for o in range(Co):
                    acc = b[o]
                    for ky in range(3):
                        for kx in range(3):
                            yy, xx = y + ky - 1, x + kx - 1
                            if 0 <= yy < H and 0 <= xx < W:
                                for i in range(Ci):
                                    acc += w[o, ky, kx, i] * g[bb, yy, xx, i]
                    out[bb, y, x, o] = acc
    return out


def _dw_loops(g, w, b):
    B, H, W, C = g.shape
    Ho, Wo = (H + 1) // 2, (W + 1) // 2
    out = np.zeros((B, Ho, Wo, C))
    for bb in range(B):
        for y in range(Ho):
            for x in range(Wo):
                for c in range(C):
                    acc = b[c]
                    for ky in range(3):
                        for kx in range(3):
                            yy, xx = 2 * y + ky - 1, 2 * x + kx - 1
                            if 0 <= yy < H and 0 <= xx < W:
                                acc += w[ky, kx, c] * g[bb, yy, xx, c]
                    out[bb, y, x, c] = acc
    return out


@pytest.mark.parametrize("H,W", [(1, 1), (3, 5), (4, 4), (7, 2)])
def test_conv3x3_vs_loops(H, W):
    rng = np.random.default_rng(1)
    g = rng.standard_normal((2, H, W, 3))
    w = rng.standard_normal((2, 3, 3, 3))
    b = rng.standard_normal(2)
    np.testing.assert_allclose(O.conv3x3(g, w, b), _conv3x3_loops(g, w, b), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("H,W", [(1, 1), (2, 2), (3, 3), (5, 4), (7, 1), (16, 16)])
def test_dwconv_s2_vs_loops(H, W):
    rng = np.random.default_rng(2)
    g = rng.standard_normal((2, H, W, 3))
    w = rng.standard_normal((3, 3, 3))
    b = rng.standard_normal(3)
    out = O.dwconv3x3_s2(g, w, b)
    assert out.shape == (2, (H + 1) // 2, (W + 1) // 2, 3)
    np.testing.assert_allclose(out, _dw_loops(g, w, b), rtol=1e-12, atol=1e-12)


def test_dwconv_delta_kernel_is_subsampling():
    rng = np.random.default_rng(3)
    g = rng.standard_normal((1, 9, 6, 4))
    w = np.zeros((3, 3, 4)); w[1, 1, :] = 1.0
    out = O.dwconv3x3_s2(g, w, np.zeros(4))
    np.testing.assert_array_equal(out, g[:, ::2, ::2, :])


def test_conv3x3_identity_centre_tap_copies_channels():
    rng = np.random.default_rng(4)
    g = rng.standard_normal((1, 5, 3, 4))
    w = np.zeros((4, 3, 3, 4))
    for c in range(4):
        w[c, 1, 1, (c + 1) % 4] = 1.0        # output c <- input c+1: pins channel order
    out = O.conv3x3(g, w, np.zeros(4))
    np.testing.assert_array_equal(out, g[..., [1, 2, 3, 0]])


def test_conv_vs_torch_cpu():
    rng = np.random.default_rng(5)
    B, H, W, Ci, Co = 2, 7, 6, 8, 5
    g = rng.standard_normal((B, H, W, Ci))
    w = rng.standard_normal((Co, 3, 3, Ci))
    b = rng.standard_normal(Co)
    t = torch.nn.functional.conv2d(torch.from_numpy(g).permute(0, 3, 1, 2),
                                   torch.from_numpy(w).permute(0, 3, 1, 2),
                                   torch.from_numpy(b), stride=1, padding=1)
    np.testing.assert_allclose(O.conv3x3(g, w, b), t.permute(0, 2, 3, 1).numpy(), rtol=1e-10, atol=1e-10)
    # depthwise stride 2
    wd = rng.standard_normal((3, 3, Ci))
    bd = rng.standard_normal(Ci)
    t = torch.nn.functional.conv2d(torch.from_numpy(g).permute(0, 3, 1, 2),
                                   torch.from_numpy(wd).permute(2, 0, 1)[:, None],
                                   torch.from_numpy(bd), stride=2, padding=1, groups=Ci)
    np.testing.assert_allclose(O.dwconv3x3_s2(g, wd, bd), t.permute(0, 2, 3, 1).numpy(), rtol=1e-10, atol=1e-10)
    # 1x1
    w1 = rng.standard_normal((Co, Ci))
    t = torch.nn.functional.conv2d(torch.from_numpy(g).permute(0, 3, 1, 2),
                                   torch.from_numpy(w1)[:, :, None, None], torch.from_numpy(b))
    np.testing.assert_allclose(O.conv1x1(g, w1, b), t.permute(0, 2, 3, 1).numpy(), rtol=1e-10, atol=1e-10)


def test_token_grid_is_row_major():
    x = np.arange(2 * 6 * 3, dtype=np.float64).reshape(2, 6, 3)
    g = O.tokens_to_grid(x, 2, 3)
    # token n = y*W + x
    assert g[1, 1, 2, 0] == x[1, 1 * 3 + 2, 0]
    np.testing.assert_array_equal(O.grid_to_tokens(g), x)


def test_linear_vs_loops():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 3, 4)); w = rng.standard_normal((5, 4)); b = rng.standard_normal(5)
    ref = np.zeros((2, 3, 5))
    for i in range(2):
        for j in range(3):
            for o in range(5):
                ref[i, j, o] = b[o] + sum(w[o, k] * x[i, j, k] for k in range(4))
    np.testing.assert_allclose(O.linear(x, w, b), ref, rtol=1e-12, atol=1e-12)


def test_activations_special_values():
    x = np.array([-2.0, -0.0, 0.0, 3.0])
    np.testing.assert_array_equal(O.relu(x), [0, 0, 0, 3])
    np.testing.assert_array_equal(O.leaky_relu(x), [-0.02, 0, 0, 3])
