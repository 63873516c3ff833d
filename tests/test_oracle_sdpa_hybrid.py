"""Pins of the oracle's softmax attention and the MM-EDiT hybrid (CPU only).

Against: hand-worked fixtures (sdpa_worked.json, hybrid_eta.json), a loop
softmax, torch scaled_dot_product_attention on the CPU, the decomposition
of a joint softmax into two blocks with exact per-row weights, and the
reduction of the hybrid to the plain EDiT layer when there is no text."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import edit_oracle as O
from seeded_inputs import make_inputs, make_shape


def test_sdpa_worked(golden_dir):
    with open(os.path.join(golden_dir, "sdpa_worked.json")) as f:
        g = json.load(f)
    firsts = {"0": 0.0, "ln2": math.log(2), "ln5": math.log(5)}
    k = np.zeros((1, 3, 4))
    k[0, :, 0] = [firsts[s] for s in g["k_first_component"]]
    out = O.sdpa(np.array(g["q"], float)[None], k, np.array(g["v"], float)[None], heads=1)
    np.testing.assert_allclose(out[0], g["out"], rtol=1e-14, atol=1e-14)


def test_eta_fixture(golden_dir):
    with open(os.path.join(golden_dir, "hybrid_eta.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert O.hybrid_eta(c["n_img"], c["n_txt"]) == float(Fraction(c["num"], c["den"]))


def test_sdpa_vs_loops_and_torch():
    rng = np.random.default_rng(0)
    B, heads, d, Nq, Nk = 2, 3, 8, 5, 7
    q = rng.standard_normal((B, Nq, heads * d)); k = rng.standard_normal((B, Nk, heads * d))
    v = rng.standard_normal((B, Nk, heads * d))
    out = O.sdpa(q, k, v, heads)
    for b in range(B):
        for h in range(heads):
            sl = slice(h * d, (h + 1) * d)
            for i in range(Nq):
                s = [float(q[b, i, sl] @ k[b, j, sl]) / math.sqrt(d) for j in range(Nk)]
                m = max(s)
                e = [math.exp(t - m) for t in s]
                tot = sum(e)
                ref = sum(e[j] / tot * v[b, j, sl] for j in range(Nk))
                np.testing.assert_allclose(out[b, i, sl], ref, rtol=1e-12, atol=1e-14)
    tq = torch.from_numpy(q).reshape(B, Nq, heads, d).transpose(1, 2)
    tk = torch.from_numpy(k).reshape(B, Nk, heads, d).transpose(1, 2)
    tv = torch.from_numpy(v).reshape(B, Nk, heads, d).transpose(1, 2)
    t = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).transpose(1, 2).reshape(B, Nq, heads * d)
    np.testing.assert_allclose(out, t.numpy(), rtol=1e-10, atol=1e-12)


def test_joint_softmax_decomposition():
    """softmax over [K1;K2] = eta_row * A(Q,K1,V1) + (1-eta_row) * A(Q,K2,V2),
    eta_row = (sum over block 1 of e^s) / (sum over both): the block form of
    the hybrid matrix holds exactly with per-row weights."""
    rng = np.random.default_rng(1)
    d = 6
    q = rng.standard_normal((1, 4, d)); k1 = rng.standard_normal((1, 5, d)); v1 = rng.standard_normal((1, 5, d))
    k2 = rng.standard_normal((1, 3, d)); v2 = rng.standard_normal((1, 3, d))
    joint = O.sdpa(q, np.concatenate([k1, k2], 1), np.concatenate([v1, v2], 1), 1)
    s1 = np.exp(q[0] @ k1[0].T / math.sqrt(d)).sum(1)
    s2 = np.exp(q[0] @ k2[0].T / math.sqrt(d)).sum(1)
    eta = (s1 / (s1 + s2))[:, None]
    np.testing.assert_allclose(joint[0], eta * O.sdpa(q, k1, v1, 1)[0] + (1 - eta) * O.sdpa(q, k2, v2, 1)[0],
                               rtol=1e-12, atol=1e-13)


def _small_shape(n_text):
    return make_shape(B=2, H=6, W=5, C=16, heads=2, head_dim=8, reduction=4, gn_groups=2, n_text=n_text, x_std=1.0)


def test_hybrid_without_text_is_edit():
    s = _small_shape(0)
    inp = make_inputs(s, seed=3, gn_affine_random=True)
    out_h, out_t = O.mmedit_hybrid_forward(inp["x"], None, inp["w"], None, s)
    assert out_t is None
    np.testing.assert_array_equal(out_h, O.edit_attn_forward(inp["x"], inp["w"], s))


def test_hybrid_rows_by_definition():
    """Image rows mix the linear result and text-key softmax by the token
    ratio; text rows attend jointly over compressed image keys and text keys."""
    s = _small_shape(4)
    inp = make_inputs(s, seed=4)
    tr = {}
    out_i, out_t = O.mmedit_hybrid_forward(inp["x"], inp["x_txt"], inp["w"], inp["w_txt"], s, tr)
    eta = 30 / 34
    wt = inp["w_txt"]
    qt = inp["x_txt"].astype(float) @ wt["w_q"].T.astype(float) + wt["b_q"]
    kt = inp["x_txt"].astype(float) @ wt["w_k"].T.astype(float) + wt["b_k"]
    vt = inp["x_txt"].astype(float) @ wt["w_v"].T.astype(float) + wt["b_v"]
    d = 8
    for b in range(2):
        for h in range(2):
            sl = slice(h * d, (h + 1) * d)
            # image row 7
            sc = np.exp(tr["q"][b, 7, sl] @ kt[b, :, sl].T / math.sqrt(d))
            sd = (sc[:, None] * vt[b, :, sl]).sum(0) / sc.sum()
            np.testing.assert_allclose(tr["y"][b, 7, sl], eta * tr["y_lin"][b, 7, sl] + (1 - eta) * sd, rtol=1e-12)
            # text row 2 over [K'_I ; K_T]
            keys = np.concatenate([tr["kc"][b, :, sl], kt[b, :, sl]])
            vals = np.concatenate([tr["vc"][b, :, sl], vt[b, :, sl]])
            assert keys.shape[0] == 3 * 3 + 4
            sc = np.exp(qt[b, 2, sl] @ keys.T / math.sqrt(d))
            np.testing.assert_allclose(tr["y_txt"][b, 2, sl], (sc[:, None] * vals).sum(0) / sc.sum(), rtol=1e-12)
    np.testing.assert_allclose(out_t, tr["y_txt"] @ wt["w_o"].T.astype(float) + wt["b_o"], rtol=1e-12)


# ---------------------------------------------------------------------------
# The hybrid's image rows with eta^Lin computed exactly (joint normaliser).
# ---------------------------------------------------------------------------

def _exact_rows_by_loops(q, kc, vc, kt, vt, heads, eps):
    """Every weight written out: image key j weighs Q_i . K'_j (the linear
    kernel, no S or z), text key t weighs exp(Q_i . K_t / sqrt(d)); one
    normaliser over both, plus eps (pure Python floats)."""
    B, N, C = q.shape
    d = C // heads
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(heads):
            sl = slice(h * d, (h + 1) * d)
            for i in range(N):
                num = [0.0] * d
                den = eps
                for j in range(kc.shape[1]):
                    wgt = sum(float(q[b, i, h * d + c]) * float(kc[b, j, h * d + c]) for c in range(d))
                    den += wgt
                    for c in range(d):
                        num[c] += wgt * float(vc[b, j, h * d + c])
                for t in range(kt.shape[1]):
                    s = sum(float(q[b, i, h * d + c]) * float(kt[b, t, h * d + c]) for c in range(d))
                    wgt = math.exp(s / math.sqrt(d))
                    den += wgt
                    for c in range(d):
                        num[c] += wgt * float(vt[b, t, h * d + c])
                out[b, i, sl] = [u / den for u in num]
    return out


def _feats(rng, B, N, Nc, NT, C):
    q = np.abs(rng.standard_normal((B, N, C)))          # ReLU'd queries
    kc = np.abs(rng.standard_normal((B, Nc, C)))        # ReLU'd compressed keys
    vc = rng.standard_normal((B, Nc, C))
    kt = rng.standard_normal((B, NT, C))
    vt = rng.standard_normal((B, NT, C))
    return q, kc, vc, kt, vt


def test_exact_rows_vs_explicit_weights():
    rng = np.random.default_rng(3)
    B, heads, d, N, Nc, NT, eps = 2, 2, 4, 5, 6, 3, 1e-6
    q, kc, vc, kt, vt = _feats(rng, B, N, Nc, NT, heads * d)
    S, z = O.kv_state(kc, vc, heads)
    got = O.hybrid_image_rows_exact(q, S, z, kt, vt, heads, eps)
    ref = _exact_rows_by_loops(q, kc, vc, kt, vt, heads, eps)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_exact_rows_are_the_hybrid_matrix_with_row_eta():
    """eta_i A^Lin + (1 - eta_i) A with the page's two blocks computed by the
    oracle's own linear attention and softmax attention, eta_i from the
    explicit weight masses."""
    rng = np.random.default_rng(4)
    B, heads, d, N, Nc, NT, eps = 1, 3, 8, 7, 9, 4, 1e-6
    q, kc, vc, kt, vt = _feats(rng, B, N, Nc, NT, heads * d)
    S, z = O.kv_state(kc, vc, heads)
    lin = O.linear_attention_apply(q, S, z, heads, eps)
    soft = O.sdpa(q, kt, vt, heads)
    got = O.hybrid_image_rows_exact(q, S, z, kt, vt, heads, eps)
    Q, Kc, Kt = O.split_heads(q, heads), O.split_heads(kc, heads), O.split_heads(kt, heads)
    lin_mass = (Q @ np.swapaxes(Kc, 2, 3)).sum(-1) + eps                 # [B, h, N]
    soft_mass = np.exp(Q @ np.swapaxes(Kt, 2, 3) / math.sqrt(d)).sum(-1)
    eta = O.merge_heads(np.repeat((lin_mass / (lin_mass + soft_mass))[..., None], d, axis=-1))
    np.testing.assert_allclose(got, eta * lin + (1 - eta) * soft, rtol=1e-12, atol=1e-14)
    den = O.linear_attention_denominator(q, z, heads, eps)
    np.testing.assert_allclose(den, lin_mass.transpose(0, 2, 1), rtol=1e-13)


def test_exact_rows_closed_forms():
    rng = np.random.default_rng(5)
    B, heads, d, N, Nc, NT = 1, 2, 4, 4, 5, 3
    q, kc, vc, kt, vt = _feats(rng, B, N, Nc, NT, heads * d)
    # Every value the same vector v: a convex combination returns v, up to the
    # eps share of the normaliser, which has the closed form below.
    v = rng.standard_normal(heads * d)
    vc[:] = v
    vt[:] = v
    S, z = O.kv_state(kc, vc, heads)
    eps = 0.25
    got = O.hybrid_image_rows_exact(q, S, z, kt, vt, heads, eps)
    den = O.linear_attention_denominator(q, z, heads, eps)                       # [B, N, h]
    Q, Kt = O.split_heads(q, heads), O.split_heads(kt, heads)
    soft = np.exp(Q @ np.swapaxes(Kt, 2, 3) / math.sqrt(d)).sum(-1).transpose(0, 2, 1)
    frac = (den - eps + soft) / (den + soft)                                      # [B, N, h]
    np.testing.assert_allclose(got, np.repeat(frac, d, axis=-1) * v, rtol=1e-13)
    # No text keys: the linear attention itself.
    got0 = O.hybrid_image_rows_exact(q, S, z, kt[:, :0], vt[:, :0], heads, 1e-6)
    np.testing.assert_allclose(got0, O.linear_attention_apply(q, S, z, heads, 1e-6), rtol=1e-14)


def test_exact_hybrid_layer_reduces_and_differs():
    s = make_shape(B=1, H=6, W=5, C=32, heads=2, head_dim=16, reduction=4, gn_groups=2, n_text=3, x_std=1.0)
    inp = make_inputs(s, seed=2)
    tr_r, tr_e = {}, {}
    o_r, t_r = O.mmedit_hybrid_forward(inp["x"], inp["x_txt"], inp["w"], inp["w_txt"], s, tr_r)
    o_e, t_e = O.mmedit_hybrid_forward(inp["x"], inp["x_txt"], inp["w"], inp["w_txt"], s, tr_e, eta="exact")
    # Text rows are exact in both modes.
    np.testing.assert_array_equal(t_r, t_e)
    # The image rows differ (the ratio is an approximation) ...
    assert np.abs(o_r - o_e).max() > 1e-6
    # ... and with no text both modes are the plain EDiT layer.
    s0 = make_shape(B=1, H=6, W=5, C=32, heads=2, head_dim=16, reduction=4, gn_groups=2, x_std=1.0)
    inp0 = make_inputs(s0, seed=2)
    e0, _ = O.mmedit_hybrid_forward(inp0["x"], None, inp0["w"], None, s0, eta="exact")
    np.testing.assert_array_equal(e0, O.edit_attn_forward(inp0["x"], inp0["w"], s0))
