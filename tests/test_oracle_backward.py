"""Pins of the oracle's backward pass (CPU only).

The backward is checked against three things other than itself:
- torch.autograd through an independent float64 forward written with
  torch.nn.functional (channels-first convolutions, group_norm, the linear
  attention formula with einsum), the same readings R1-R12;
- central finite differences of the oracle forward, coordinate by
  coordinate, for x and every parameter;
- the invariants of the GroupNorm gradient (orthogonal to the ones and to the
  normalised input within each sample and group)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import edit_backward as OB
from oracle import edit_oracle as O
from seeded_inputs import make_inputs, make_shape

S_TINY = make_shape(B=2, H=5, W=6, C=16, heads=2, head_dim=8, reduction=4, gn_groups=2, x_std=1.0, w_std=0.2)
S_MID = make_shape(B=1, H=7, W=8, C=32, heads=4, head_dim=8, reduction=4, gn_groups=4, x_std=1.0, w_std=0.1)


def _inp(s, seed):
    inp = make_inputs(s, seed=seed, gn_affine_random=True)
    rng = np.random.default_rng(1000 + seed)
    dout = rng.standard_normal((s.B, s.N, s.C))
    return inp, dout


def _kink(out, pre, mask):
    """out's values with the derivative `mask` (a tensor of slopes) in place
    of out's own: a straight-through branch choice."""
    return out if mask is None else out.detach() + (pre - pre.detach()) * mask


def torch_forward(x, w, s, masks=None):
    """The layer in float64 torch.nn.functional, channels-first, written
    independently of the oracle (same readings). masks (optional): per kink
    the slope its derivative takes ("q", "kc": 1 / 0; "act": 1 / 0.01), in
    the token-major shapes of the oracle's q, kc and cf_act."""
    B, H, W, C, h = s.B, s.H, s.W, s.C, s.heads
    d = C // h
    m = masks or {}
    cf = lambda t: None if t is None else t.reshape(B, H, W, -1).permute(0, 3, 1, 2)
    g = x.reshape(B, H, W, C).permute(0, 3, 1, 2)
    xc = F.conv2d(g, w["w_cf1"].permute(0, 3, 1, 2), w["b_cf1"], padding=1)
    gn = F.group_norm(xc, s.gn_groups, w["gn_gamma"], w["gn_beta"], eps=1e-5)
    a = _kink(F.leaky_relu(gn, 0.01), gn, cf(m.get("act")))
    r = F.conv2d(a, w["w_cf2"][:, :, None, None], w["b_cf2"])
    xt = (g + r).permute(0, 2, 3, 1).reshape(B, H * W, C)
    qp = F.linear(xt, w["w_q"], w["b_q"])
    q = _kink(F.relu(qp), qp, m.get("q"))
    k0 = F.linear(x, w["w_k"], w["b_k"]).reshape(B, H, W, C).permute(0, 3, 1, 2)
    v0 = F.linear(x, w["w_v"], w["b_v"]).reshape(B, H, W, C).permute(0, 3, 1, 2)
    kp = F.conv2d(k0, w["dw_k"].permute(2, 0, 1)[:, None], w["db_k"], stride=2, padding=1, groups=C)
    mk = m.get("kc")
    kc = _kink(F.relu(kp), kp, None if mk is None else mk.reshape(B, kp.shape[2], kp.shape[3], C).permute(0, 3, 1, 2))
    vc = F.conv2d(v0, w["dw_v"].permute(2, 0, 1)[:, None], w["db_v"], stride=2, padding=1, groups=C)
    kc = kc.permute(0, 2, 3, 1).reshape(B, -1, h, d)
    vc = vc.permute(0, 2, 3, 1).reshape(B, -1, h, d)
    Q = q.reshape(B, H * W, h, d)
    S = torch.einsum("bjha,bjhc->bhac", kc, vc)
    z = kc.sum(dim=1)                                               # [B, h, d]
    num = torch.einsum("bnha,bhac->bnhc", Q, S)
    den = torch.einsum("bnha,bha->bnh", Q, z) + s.eps
    y = (num / den[..., None]).reshape(B, H * W, C)
    return F.linear(y, w["w_o"], w["b_o"])


@pytest.mark.parametrize("s,seed", [(S_TINY, 0), (S_MID, 1)])
def test_backward_against_torch_autograd(s, seed):
    inp, dout = _inp(s, seed)
    dx, grads = OB.edit_attn_backward(inp["x"], inp["w"], s, dout)
    xt = torch.tensor(inp["x"], dtype=torch.float64, requires_grad=True)
    wt = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in inp["w"].items()}
    out = torch_forward(xt, wt, s)
    np.testing.assert_allclose(out.detach().numpy(), O.edit_attn_forward(inp["x"], inp["w"], s), rtol=1e-11,
                               atol=1e-12)
    (out * torch.from_numpy(dout)).sum().backward()

    def close(a, b, name):
        scale = max(np.abs(b).max(), 1e-300)
        assert np.abs(a - b).max() <= 1e-10 * scale, f"{name}: {np.abs(a - b).max() / scale:.3e}"
    close(dx, xt.grad.numpy(), "x")
    for n in OB.PARAM_NAMES:
        assert grads[n].shape == inp["w"][n].shape, n
        close(grads[n], wt[n].grad.numpy(), n)


@pytest.mark.parametrize("s,seed", [(S_TINY, 2), (S_MID, 4)])
def test_backward_with_kink_masks_against_torch_autograd(s, seed):
    """With masks given, the oracle backward is the gradient of the branch the
    masks name (R28): torch.autograd through a forward whose ReLU and
    LeakyReLU keep their values but take the masks' slopes. A fifth of the
    decisions are flipped against the oracle's own forward, so the masks,
    not the signs of the float64 forward, must decide."""
    inp, dout = _inp(s, seed)
    f = {}
    O.edit_attn_forward(inp["x"], inp["w"], s, f)
    rng = np.random.default_rng(2000 + seed)
    flip = lambda on: on ^ (rng.random(on.shape) < 0.2)
    masks = {"q": flip(f["q"] > 0), "kc": flip(f["kc"] > 0), "act": flip(f["cf_act"] >= 0)}
    dx, grads = OB.edit_attn_backward(inp["x"], inp["w"], s, dout, masks=masks)
    dx0, _ = OB.edit_attn_backward(inp["x"], inp["w"], s, dout)
    assert np.abs(dx - dx0).max() > 1e-3 * np.abs(dx0).max()       # the flips matter
    slopes = {"q": torch.from_numpy(masks["q"].astype(np.float64)),
              "kc": torch.from_numpy(masks["kc"].astype(np.float64)),
              "act": torch.from_numpy(np.where(masks["act"], 1.0, 0.01))}
    xt = torch.tensor(inp["x"], dtype=torch.float64, requires_grad=True)
    wt = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in inp["w"].items()}
    (torch_forward(xt, wt, s, slopes) * torch.from_numpy(dout)).sum().backward()
    for name, a, b in [("x", dx, xt.grad.numpy())] + [(n, grads[n], wt[n].grad.numpy()) for n in OB.PARAM_NAMES]:
        scale = max(np.abs(b).max(), 1e-300)
        assert np.abs(a - b).max() <= 1e-10 * scale, f"{name}: {np.abs(a - b).max() / scale:.3e}"


def test_backward_with_own_masks_is_unchanged():
    """Masks equal to the oracle's own kink decisions give its unmasked result bit for bit."""
    s = S_TINY
    inp, dout = _inp(s, 6)
    f = {}
    O.edit_attn_forward(inp["x"], inp["w"], s, f)
    masks = {"q": f["q"] > 0, "kc": f["kc"] > 0, "act": f["cf_act"] >= 0}
    dx, g = OB.edit_attn_backward(inp["x"], inp["w"], s, dout, masks=masks)
    dx0, g0 = OB.edit_attn_backward(inp["x"], inp["w"], s, dout)
    assert np.array_equal(dx, dx0)
    for n in OB.PARAM_NAMES:
        assert np.array_equal(g[n], g0[n]), n


def _loss(x, w, s, dout):
    return float((O.edit_attn_forward(x, w, s) * dout).sum())


def test_backward_against_finite_differences():
    """Central differences of the oracle forward at a few coordinates of x
    and of every parameter (step 1e-6; the data keep every ReLU and
    LeakyReLU input at least 1e-3 from its kink at these coordinates with
    overwhelming probability)."""
    s = S_TINY
    inp, dout = _inp(s, 3)
    x, w = inp["x"].astype(np.float64), {k: v.astype(np.float64) for k, v in inp["w"].items()}
    dx, grads = OB.edit_attn_backward(x, w, s, dout)
    rng = np.random.default_rng(7)
    h = 1e-6
    targets = [("x", x, dx)] + [(n, w[n], grads[n]) for n in OB.PARAM_NAMES]
    for name, arr, g in targets:
        for _ in range(3):
            idx = tuple(rng.integers(0, d) for d in arr.shape)
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(x, w, s, dout)
            arr[idx] = old - h
            lm = _loss(x, w, s, dout)
            arr[idx] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-5 * max(1.0, abs(g[idx])), (name, idx, fd, g[idx])


def test_group_norm_gradient_invariants():
    """With eps = 0 the output of GroupNorm is invariant to shifting and
    scaling the input within a (sample, group), so the input gradient is
    orthogonal to the ones and to the normalised input there."""
    rng = np.random.default_rng(11)
    g = rng.standard_normal((2, 4, 5, 12)) * 3 + 1
    gamma = rng.standard_normal(12)
    dout = rng.standard_normal(g.shape)
    dg, dgamma, dbeta = OB.group_norm_backward(g, 3, gamma, dout, eps=0.0)
    mean, var = O.group_norm_stats(g, 3)
    xhat = (g.reshape(2, 20, 3, 4) - mean[:, None, :, None]) / np.sqrt(var[:, None, :, None])
    dgr = dg.reshape(2, 20, 3, 4)
    assert np.abs(dgr.sum(axis=(1, 3))).max() < 1e-11
    assert np.abs((dgr * xhat).sum(axis=(1, 3))).max() < 1e-11
    np.testing.assert_allclose(dbeta, dout.sum(axis=(0, 1, 2)), rtol=1e-13)
    np.testing.assert_allclose(dgamma, (dout * xhat.reshape(g.shape)).sum(axis=(0, 1, 2)), rtol=1e-12)


def test_linear_attention_backward_finite_differences():
    rng = np.random.default_rng(5)
    B, N, h, d, eps = 1, 6, 2, 3, 1e-6
    q = rng.uniform(0.1, 1.0, (B, N, h * d))
    S = rng.standard_normal((B, h, d, d))
    z = rng.uniform(0.5, 1.5, (B, h, d))
    dy = rng.standard_normal((B, N, h * d))
    dq, dS, dz = OB.linear_attention_apply_backward(q, S, z, h, eps, dy)
    L = lambda q_, S_, z_: float((O.linear_attention_apply(q_, S_, z_, h, eps) * dy).sum())
    step = 1e-7
    for arr, g in ((q, dq), (S, dS), (z, dz)):
        for idx in np.ndindex(*arr.shape):
            old = arr[idx]
            arr[idx] = old + step
            lp = L(q, S, z)
            arr[idx] = old - step
            lm = L(q, S, z)
            arr[idx] = old
            assert abs((lp - lm) / (2 * step) - g[idx]) < 1e-6 * max(1.0, abs(g[idx]))
