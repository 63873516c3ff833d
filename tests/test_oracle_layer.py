"""Pins of the composed oracle layers (CPU only).

* the whole EDiT layer and the hybrid against an independent composition of
  torch.nn.functional ops (conv2d, group_norm, leaky_relu, linear,
  scaled_dot_product_attention) in float64 on the CPU;
* the literal reading of the Spatial-Compressor equations (K and V sharing
  one phi_SC) gives K' = ReLU(V') exactly;
* zeroed ConvFusion convolutions leave X~ = X + b_cf2;
* test power: plausible mistakes move the bf16-gated error measures well past
  the 2e-2 tolerance, so the GPU parity gate would catch them.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import edit_oracle as O
from seeded_inputs import CONFIGS, make_inputs, make_shape
from tests._metrics import BF16_TOL, centred_rel_err, max_rel_err


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def torch_edit_layer(x, w, s):
    """Independent torch float64 CPU composition of the layer (NCHW convs)."""
    B, N, C = x.shape
    X = _t(x)
    img = X.reshape(B, s.H, s.W, C).permute(0, 3, 1, 2)
    xc = F.conv2d(img, _t(w["w_cf1"]).permute(0, 3, 1, 2), _t(w["b_cf1"]), padding=1)
    a = F.leaky_relu(F.group_norm(xc, s.gn_groups, _t(w["gn_gamma"]), _t(w["gn_beta"]), eps=1e-5), 0.01)
    r = F.conv2d(a, _t(w["w_cf2"])[:, :, None, None], _t(w["b_cf2"]))
    xt = X + r.permute(0, 2, 3, 1).reshape(B, N, C)
    q = F.relu(F.linear(xt, _t(w["w_q"]), _t(w["b_q"])))

    def sc(wl, bl, wd, bd):
        t = F.linear(X, _t(wl), _t(bl)).reshape(B, s.H, s.W, C).permute(0, 3, 1, 2)
        t = F.conv2d(t, _t(wd).permute(2, 0, 1)[:, None], _t(bd), stride=2, padding=1, groups=C)
        return t.permute(0, 2, 3, 1).reshape(B, -1, C)

    kc = F.relu(sc(w["w_k"], w["b_k"], w["dw_k"], w["db_k"]))
    vc = sc(w["w_v"], w["b_v"], w["dw_v"], w["db_v"])
    h, d = s.heads, C // s.heads
    Q = q.reshape(B, N, h, d).transpose(1, 2)
    K = kc.reshape(B, -1, h, d).transpose(1, 2)
    V = vc.reshape(B, -1, h, d).transpose(1, 2)
    kv = torch.einsum("bhjd,bhje->bhde", K, V)
    num = torch.einsum("bhnd,bhde->bhne", Q, kv)
    den = torch.einsum("bhnd,bhd->bhn", Q, K.sum(2))
    y = (num / (den[..., None] + s.eps)).transpose(1, 2).reshape(B, N, C)
    return q, kc, vc, y, F.linear(y, _t(w["w_o"]), _t(w["b_o"]))


SMALL = [
    make_shape(B=2, H=6, W=6, C=32, heads=4, head_dim=8, reduction=4, gn_groups=4, x_std=1.0),
    make_shape(B=1, H=7, W=5, C=48, heads=3, head_dim=16, reduction=4, gn_groups=3, x_std=1.0),
]


@pytest.mark.parametrize("s", SMALL + [CONFIGS["tiny"]])
def test_layer_vs_torch(s):
    inp = make_inputs(s, seed=11, gn_affine_random=True)
    tr = {}
    out = O.edit_attn_forward(inp["x"], inp["w"], s, tr)
    q, kc, vc, y, o = torch_edit_layer(inp["x"], inp["w"], s)
    for name, ref in [("q", q), ("kc", kc), ("vc", vc), ("y", y)]:
        np.testing.assert_allclose(tr[name], ref.numpy(), rtol=1e-9, atol=1e-12, err_msg=name)
    np.testing.assert_allclose(out, o.numpy(), rtol=1e-9, atol=1e-12)


def test_hybrid_vs_torch():
    s = make_shape(B=2, H=6, W=4, C=32, heads=2, head_dim=16, reduction=4, gn_groups=4, x_std=1.0, n_text=5)
    inp = make_inputs(s, seed=12)
    tr = {}
    out_i, out_t = O.mmedit_hybrid_forward(inp["x"], inp["x_txt"], inp["w"], inp["w_txt"], s, tr)
    q, kc, vc, ylin, _ = torch_edit_layer(inp["x"], inp["w"], s)
    wt = inp["w_txt"]
    xt = _t(inp["x_txt"])
    qt, kt, vt = (F.linear(xt, _t(wt[a]), _t(wt[b])) for a, b in [("w_q", "b_q"), ("w_k", "b_k"), ("w_v", "b_v")])
    B, C, h = 2, 32, 2

    def heads(t):
        return t.reshape(B, -1, h, C // h).transpose(1, 2)

    def merge(t):
        return t.transpose(1, 2).reshape(B, -1, C)

    eta = 24 / 29
    y_img = eta * ylin + (1 - eta) * merge(F.scaled_dot_product_attention(heads(q), heads(kt), heads(vt)))
    y_txt = merge(F.scaled_dot_product_attention(heads(qt), heads(torch.cat([kc, kt], 1)),
                                                 heads(torch.cat([vc, vt], 1))))
    np.testing.assert_allclose(out_i, F.linear(y_img, _t(inp["w"]["w_o"]), _t(inp["w"]["b_o"])).numpy(),
                               rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(out_t, F.linear(y_txt, _t(wt["w_o"]), _t(wt["b_o"])).numpy(), rtol=1e-9, atol=1e-12)


def test_literal_shared_phi_sc():
    """With K's and V's Linear and depthwise parameters equal, K' = ReLU(V')."""
    s = SMALL[0]
    inp = make_inputs(s, seed=13)
    w = dict(inp["w"])
    for a, b in [("w_k", "w_v"), ("b_k", "b_v"), ("dw_k", "dw_v"), ("db_k", "db_v")]:
        w[a] = w[b]
    kc, vc = O.spatial_compressor_kv(inp["x"], s.H, s.W, w)
    np.testing.assert_array_equal(kc, O.relu(vc))
    assert kc.shape[1] == 9          # 6x6 grid -> 3x3 compressed tokens


def test_zeroed_convfusion_branch():
    s = SMALL[1]
    inp = make_inputs(s, seed=14)
    w = dict(inp["w"])
    w["w_cf2"] = np.zeros_like(w["w_cf2"])
    tr = {}
    O.convfusion_query(inp["x"], s.H, s.W, w, s.gn_groups, tr)
    np.testing.assert_array_equal(tr["xt"], inp["x"].astype(np.float64) + w["b_cf2"])


# ---------------------------------------------------------------------------
# Test power of the bf16 gate
# ---------------------------------------------------------------------------

POWER = make_shape(B=1, H=16, W=16, C=128, heads=2, head_dim=64, reduction=4, gn_groups=8, x_std=1.0)


def _mutated(kind, x, w, s):
    w = dict(w)
    H, W = s.H, s.W
    if kind == "cf_branch_zeroed":
        w["w_cf2"] = np.zeros_like(w["w_cf2"]); w["b_cf2"] = np.zeros_like(w["b_cf2"])
        return O.edit_attn_forward(x, w, s, tr := {}), tr
    tr = {}
    q = O.convfusion_query(x, H, W, w, s.gn_groups, tr)
    k0 = O.linear(x, w["w_k"], w["b_k"]); v0 = O.linear(x, w["w_v"], w["b_v"])
    gk, gv = O.tokens_to_grid(k0, H, W), O.tokens_to_grid(v0, H, W)
    if kind == "relu_on_v_not_k":
        kc = O.dwconv3x3_s2(gk, w["dw_k"], w["db_k"]); vc = O.relu(O.dwconv3x3_s2(gv, w["dw_v"], w["db_v"]))
    elif kind == "subsample_not_conv":
        kc = O.relu(gk[:, ::2, ::2]); vc = gv[:, ::2, ::2]
    else:
        kc = O.relu(O.dwconv3x3_s2(gk, w["dw_k"], w["db_k"])); vc = O.dwconv3x3_s2(gv, w["dw_v"], w["db_v"])
    kc, vc = O.grid_to_tokens(kc), O.grid_to_tokens(vc)
    if kind == "head_split_transposed":
        perm = np.arange(s.C).reshape(s.head_dim, s.heads).T.reshape(-1)   # channel c = k*h + head
        y = O.linear_attention(q[..., perm], kc[..., perm], vc[..., perm], s.heads, s.eps)
        y = y[..., np.argsort(perm)]
    else:
        y = O.linear_attention(q, kc, vc, s.heads, s.eps)
    tr["y"] = y
    return O.linear(y, w["w_o"], w["b_o"]), tr


@pytest.mark.parametrize("kind", ["cf_branch_zeroed", "relu_on_v_not_k", "subsample_not_conv",
                                  "head_split_transposed"])
def test_bf16_gate_catches_mutation(kind):
    inp = make_inputs(POWER, seed=15)
    tr = {}
    ref = O.edit_attn_forward(inp["x"], inp["w"], POWER, tr)
    got, trm = _mutated(kind, inp["x"], inp["w"], POWER)
    errs = [max_rel_err(got, ref), centred_rel_err(got, ref),
            max_rel_err(trm["y"], tr["y"]), centred_rel_err(trm["y"], tr["y"])]
    assert max(errs) > 5 * BF16_TOL, (kind, errs)


def test_bf16_gate_catches_eta_forced_to_one():
    s = make_shape(B=1, H=8, W=8, C=64, heads=2, head_dim=32, reduction=4, gn_groups=4, x_std=1.0, n_text=20)
    inp = make_inputs(s, seed=16)
    tr = {}
    O.mmedit_hybrid_forward(inp["x"], inp["x_txt"], inp["w"], inp["w_txt"], s, tr)
    errs = [max_rel_err(tr["y_lin"], tr["y"]), centred_rel_err(tr["y_lin"], tr["y"])]
    assert max(errs) > 5 * BF16_TOL, errs
