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


def torch_forward(x, w, s, given=None):
    """The layer in float64 torch.nn.functional, channels-first, written
    independently of the oracle (same readings).

    given (optional): token-major arrays for some of the forward tensors
    (xc, cf_act, xt, q, k0, v0, kc, vc, S, z, y). Each given tensor replaces
    the computed one by value, while the gradient still flows through the
    computed one (a straight-through substitution), so every later step runs
    at the given values and its derivative is taken there; a ReLU or
    LeakyReLU whose output is given takes its branch from the given output's
    sign."""
    B, H, W, C, h = s.B, s.H, s.W, s.C, s.heads
    d = C // h
    gv = given or {}

    def T(a):
        return torch.from_numpy(np.asarray(a, dtype=np.float64))

    def cf(a):      # token-major [B, H*W or H'*W', ch] -> channels-first [B, ch, rows, cols]
        a = T(a)
        n = a.shape[1]
        rows = H if n == H * W else (H + 1) // 2
        return a.reshape(B, rows, n // rows, -1).permute(0, 3, 1, 2)

    def sub(name, t, to_layout=None):
        if name not in gv:
            return t
        v = to_layout(gv[name]) if to_layout else T(gv[name]).reshape(t.shape)
        return v + (t - t.detach())

    g = x.reshape(B, H, W, C).permute(0, 3, 1, 2)
    xc = sub("xc", F.conv2d(g, w["w_cf1"].permute(0, 3, 1, 2), w["b_cf1"], padding=1), cf)
    gn = F.group_norm(xc, s.gn_groups, w["gn_gamma"], w["gn_beta"], eps=1e-5)
    if "cf_act" in gv:
        a = torch.where(cf(gv["cf_act"]) >= 0, gn, 0.01 * gn)
    else:
        a = F.leaky_relu(gn, 0.01)
    a = sub("cf_act", a, cf)
    r = F.conv2d(a, w["w_cf2"][:, :, None, None], w["b_cf2"])
    xt = sub("xt", (g + r).permute(0, 2, 3, 1).reshape(B, H * W, C))
    qp = F.linear(xt, w["w_q"], w["b_q"])
    q = sub("q", qp * (T(gv["q"]) > 0) if "q" in gv else F.relu(qp))
    k0 = sub("k0", F.linear(x, w["w_k"], w["b_k"])).reshape(B, H, W, C).permute(0, 3, 1, 2)
    v0 = sub("v0", F.linear(x, w["w_v"], w["b_v"])).reshape(B, H, W, C).permute(0, 3, 1, 2)
    kp = F.conv2d(k0, w["dw_k"].permute(2, 0, 1)[:, None], w["db_k"], stride=2, padding=1, groups=C)
    kc = sub("kc", kp * (cf(gv["kc"]) > 0) if "kc" in gv else F.relu(kp), cf)
    vc = sub("vc", F.conv2d(v0, w["dw_v"].permute(2, 0, 1)[:, None], w["db_v"], stride=2, padding=1, groups=C), cf)
    kc = kc.permute(0, 2, 3, 1).reshape(B, -1, h, d)
    vc = vc.permute(0, 2, 3, 1).reshape(B, -1, h, d)
    Q = q.reshape(B, H * W, h, d)
    S = sub("S", torch.einsum("bjha,bjhc->bhac", kc, vc))
    z = sub("z", kc.sum(dim=1))                                     # [B, h, d]
    num = torch.einsum("bnha,bhac->bnhc", Q, S)
    den = torch.einsum("bnha,bha->bnh", Q, z) + s.eps
    y = sub("y", (num / den[..., None]).reshape(B, H * W, C))
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


def _perturbed_forward(inp, s, seed):
    """The oracle's forward tensors moved by relative noise of 1e-3, with a
    fifth of the ReLU / LeakyReLU outputs moved across their kink: a forward
    as another computation might store it."""
    f = {}
    O.edit_attn_forward(inp["x"], inp["w"], s, f)
    rng = np.random.default_rng(2000 + seed)
    given = {}
    for k in OB.FORWARD_KEYS:
        t = f[k] * (1 + 1e-3 * rng.standard_normal(f[k].shape))
        if k in ("q", "kc", "cf_act"):
            flip = rng.random(t.shape) < 0.2
            small = 1e-6 * np.abs(t).max()
            t = np.where(flip, np.where(t > 0, -small if k == "cf_act" else 0.0, small), t)
        given[k] = t
    return f, given


@pytest.mark.parametrize("s,seed", [(S_TINY, 2), (S_MID, 4)])
def test_backward_at_given_forward_against_torch_autograd(s, seed):
    """With a forward supplied, the oracle backward is the chain rule of every
    step evaluated at the supplied tensors (kink branches from their signs):
    torch.autograd through the straight-through forward above, on a forward
    perturbed away from the oracle's own (so the supplied tensors, not the
    float64 forward, must be what is used)."""
    inp, dout = _inp(s, seed)
    f, given = _perturbed_forward(inp, s, seed)
    dx, grads = OB.edit_attn_backward(inp["x"], inp["w"], s, dout, forward=given)
    dx0, _ = OB.edit_attn_backward(inp["x"], inp["w"], s, dout)
    assert np.abs(dx - dx0).max() > 1e-3 * np.abs(dx0).max()       # the supplied forward matters
    tg = dict(given)
    tg["xt"] = inp["x"] + O.linear(given["cf_act"], inp["w"]["w_cf2"], inp["w"]["b_cf2"])
    xt = torch.tensor(inp["x"], dtype=torch.float64, requires_grad=True)
    wt = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in inp["w"].items()}
    (torch_forward(xt, wt, s, tg) * torch.from_numpy(dout)).sum().backward()
    for name, a, b in [("x", dx, xt.grad.numpy())] + [(n, grads[n], wt[n].grad.numpy()) for n in OB.PARAM_NAMES]:
        scale = max(np.abs(b).max(), 1e-300)
        assert np.abs(a - b).max() <= 1e-10 * scale, f"{name}: {np.abs(a - b).max() / scale:.3e}"


def test_backward_at_own_forward_is_unchanged():
    """The oracle's own forward tensors, supplied, give its result (up to the
    restored stream's rounding, formed anew from cf_act)."""
    s = S_TINY
    inp, dout = _inp(s, 6)
    f = {}
    O.edit_attn_forward(inp["x"], inp["w"], s, f)
    dx, g = OB.edit_attn_backward(inp["x"], inp["w"], s, dout, forward={k: f[k] for k in OB.FORWARD_KEYS})
    dx0, g0 = OB.edit_attn_backward(inp["x"], inp["w"], s, dout)
    np.testing.assert_allclose(dx, dx0, rtol=0, atol=1e-13 * np.abs(dx0).max())
    for n in OB.PARAM_NAMES:
        np.testing.assert_allclose(g[n], g0[n], rtol=0, atol=1e-12 * np.abs(g0[n]).max(), err_msg=n)


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


def test_step_chain_is_exact_on_the_oracles_own_tensors():
    """The step-by-step comparison (tests/_bwd_steps.py) fed the oracle's own
    forward tensors and intermediate gradients as the "GPU" side agrees with
    itself at every step: the chain is wired like the backward."""
    from tests import _bwd_steps as BSt
    s = S_MID
    inp, dout = _inp(s, 8)
    tr = {}
    dx, grads = OB.edit_attn_backward(inp["x"], inp["w"], s, dout, trace=tr)
    f, C = tr["forward"], s.C
    fwd = {k: f[k] for k in OB.FORWARD_KEYS}
    x = np.asarray(inp["x"], np.float64)
    bwd = {"dy": tr["dy"], "dq_pre": tr["dq_pre"], "dS": tr["dS"], "dz": tr["dz"],
           "dkv": np.concatenate([OB.relu_backward(f["kc"], tr["dkc"]), tr["dvc"]], -1),
           "dk0v0": np.concatenate([tr["dk0"], tr["dv0"]], -1), "dxq": tr["dxt"],
           "dxkv": tr["dxt"] + tr["dk0"] @ inp["w"]["w_k"] + tr["dv0"] @ inp["w"]["w_v"],
           "dact": tr["dact"], "dxc": tr["dxc"]}
    pairs = BSt.step_pairs(s, x, inp["w"], dout, fwd, bwd, {"x": dx, **grads})
    assert set(BSt.BWD_TENSORS) | {"x"} | set(OB.PARAM_NAMES) == set(pairs)
    for k, (a, b) in pairs.items():
        scale = max(np.abs(b).max(), 1e-300)
        assert np.abs(np.asarray(a) - b).max() <= 1e-12 * scale, k
