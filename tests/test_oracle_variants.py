"""Pins of the oracle's ablation variants (CPU only).

The notes' ablation table (section "Ablation: Query/Key/Value processing")
runs the layer with the query and key/value processing swapped:
(CF, SC, SC), (CF, CF, -), (-, SC, SC) and (CF, -, -). Each variant is
checked against something other than itself: the layer it must reproduce
when parameters make two forms coincide, the explicit N x N kernelised sum
over the uncompressed tokens, and torch.nn.functional on the CPU."""
import math

import numpy as np
import pytest
import torch

from oracle import edit_oracle as O
from seeded_inputs import make_inputs, make_shape

S_F32 = make_shape(B=2, H=5, W=6, C=32, heads=2, head_dim=16, reduction=4, gn_groups=2, x_std=1.0)


def _inp(seed=0, **kw):
    return make_inputs(S_F32, seed=seed, gn_affine_random=True, key_convfusion=True, **kw)


def test_main_row_is_the_layer():
    inp = _inp(1)
    a = O.edit_attn_variant_forward(inp["x"], inp["w"], S_F32, "convfusion", "compressed")
    np.testing.assert_array_equal(a, O.edit_attn_forward(inp["x"], inp["w"], S_F32))


@pytest.mark.parametrize("kv", ["compressed", "full", "key_convfusion"])
def test_linear_query_is_convfusion_with_a_silent_branch(kv):
    """With the 1x1 restore conv and its bias at zero, X + ConvFusion(X) = X,
    so the ConvFusion query is the plain query of the (-, ., .) rows."""
    inp = _inp(2)
    w0 = dict(inp["w"], w_cf2=np.zeros_like(inp["w"]["w_cf2"]), b_cf2=np.zeros_like(inp["w"]["b_cf2"]))
    a = O.edit_attn_variant_forward(inp["x"], inp["w"], S_F32, "linear", kv, inp["w_kcf"])
    b = O.edit_attn_variant_forward(inp["x"], w0, S_F32, "convfusion", kv, inp["w_kcf"])
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)
    # ... and differs from the ConvFusion query when the branch is live.
    c = O.edit_attn_variant_forward(inp["x"], inp["w"], S_F32, "convfusion", kv, inp["w_kcf"])
    assert np.abs(a - c).max() > 1e-5


def test_full_kv_against_explicit_kernel_sum():
    """(CF, -, -): y_i = sum_j (q_i . k_j) v_j / (sum_j q_i . k_j + eps) over
    all N tokens, every weight written out; K and V from torch's linear."""
    inp = _inp(3)
    x, w = inp["x"].astype(np.float64), inp["w"]
    tr = {}
    out = O.edit_attn_variant_forward(x, w, S_F32, "convfusion", "full", trace=tr)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    k = torch.relu(torch.nn.functional.linear(t(x), t(w["w_k"]), t(w["b_k"]))).numpy()
    v = torch.nn.functional.linear(t(x), t(w["w_v"]), t(w["b_v"])).numpy()
    np.testing.assert_allclose(tr["k"], k, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(tr["v"], v, rtol=1e-13, atol=1e-15)
    q = tr["q"]
    B, N, C = q.shape
    h, d = S_F32.heads, S_F32.head_dim
    y = np.zeros_like(q)
    for b in range(B):
        for hh in range(h):
            sl = slice(hh * d, (hh + 1) * d)
            wgt = q[b, :, sl] @ k[b, :, sl].T                       # [N, N] kernel weights
            y[b, :, sl] = (wgt @ v[b, :, sl]) / (wgt.sum(1, keepdims=True) + S_F32.eps)
    np.testing.assert_allclose(tr["y"], y, rtol=1e-12, atol=1e-14)
    ref = torch.nn.functional.linear(t(y), t(w["w_o"]), t(w["b_o"])).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    assert tr["k"].shape[1] == N          # the sums run over the uncompressed tokens


def test_key_convfusion_structure():
    inp = _inp(4)
    x, w, wk = inp["x"], inp["w"], inp["w_kcf"]
    # Same ConvFusion parameters and W_k = W_q: the keys are the queries.
    w_same = dict(w, w_k=w["w_q"], b_k=w["b_q"])
    wk_same = {n: w[n] for n in wk}
    tr = {}
    O.edit_attn_variant_forward(x, w_same, S_F32, "convfusion", "key_convfusion", wk_same, trace=tr)
    np.testing.assert_array_equal(tr["k"], tr["q"])
    np.testing.assert_array_equal(tr["xt_k"], tr["xt"])
    # A silent key branch (restore weights zero) gives the (CF, -, -) row.
    wk0 = dict(wk, w_cf2=np.zeros_like(wk["w_cf2"]), b_cf2=np.zeros_like(wk["b_cf2"]))
    a = O.edit_attn_variant_forward(x, w, S_F32, "convfusion", "key_convfusion", wk0)
    b = O.edit_attn_variant_forward(x, w, S_F32, "convfusion", "full")
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)
    # The key branch takes its own parameters: a live branch changes the keys.
    tr2 = {}
    O.edit_attn_variant_forward(x, w, S_F32, "convfusion", "key_convfusion", wk, trace=tr2)
    k_plain = np.maximum(x.astype(np.float64) @ w["w_k"].T.astype(np.float64) + w["b_k"], 0.0)
    assert np.abs(tr2["k"] - k_plain).max() > 1e-4
    # V is the uncompressed value Linear in this row.
    np.testing.assert_allclose(tr2["v"], x.astype(np.float64) @ w["w_v"].T.astype(np.float64) + w["b_v"],
                               rtol=1e-13, atol=1e-15)


def test_key_convfusion_keys_against_torch():
    """The key branch: Conv3x3 -> GN -> LeakyReLU -> Conv1x1 + X -> Linear_K -> ReLU,
    composed from torch.nn.functional (channels-first) as a third opinion."""
    inp = _inp(5)
    x, w, wk = inp["x"], inp["w"], inp["w_kcf"]
    tr = {}
    O.edit_attn_variant_forward(x, w, S_F32, "convfusion", "key_convfusion", wk, trace=tr)
    s = S_F32
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    g = t(x).reshape(s.B, s.H, s.W, s.C).permute(0, 3, 1, 2)
    xc = torch.nn.functional.conv2d(g, t(wk["w_cf1"]).permute(0, 3, 1, 2), t(wk["b_cf1"]), padding=1)
    a = torch.nn.functional.leaky_relu(
        torch.nn.functional.group_norm(xc, s.gn_groups, t(wk["gn_gamma"]), t(wk["gn_beta"]), eps=1e-5), 0.01)
    r = torch.nn.functional.conv2d(a, t(wk["w_cf2"])[:, :, None, None], t(wk["b_cf2"]))
    xt = (g + r).permute(0, 2, 3, 1).reshape(s.B, s.N, s.C)
    k = torch.relu(torch.nn.functional.linear(xt, t(w["w_k"]), t(w["b_k"])))
    np.testing.assert_allclose(tr["xt_k"], xt.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(tr["k"], k.numpy(), rtol=1e-12, atol=1e-13)


def test_unknown_variant_and_missing_weights_rejected():
    inp = _inp(6)
    with pytest.raises(ValueError):
        O.edit_attn_variant_forward(inp["x"], inp["w"], S_F32, "conv", "compressed")
    with pytest.raises(ValueError):
        O.edit_attn_variant_forward(inp["x"], inp["w"], S_F32, "convfusion", "key_convfusion")


def test_key_convfusion_draws_do_not_disturb_the_others():
    a = make_inputs(S_F32, seed=7)
    b = make_inputs(S_F32, seed=7, key_convfusion=True)
    np.testing.assert_array_equal(a["x"], b["x"])
    for n in a["w"]:
        np.testing.assert_array_equal(a["w"][n], b["w"][n])
    assert set(b["w_kcf"]) == {"w_cf1", "b_cf1", "gn_gamma", "gn_beta", "w_cf2", "b_cf2"}
    assert b["w_kcf"]["w_cf1"].shape == a["w"]["w_cf1"].shape
    assert math.isclose(float(np.std(b["w_kcf"]["w_cf1"])), 0.02, rel_tol=0.2)
