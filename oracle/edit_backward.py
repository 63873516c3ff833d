"""CPU oracle of the EDiT layer's backward pass, in float64 numpy.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The HIP library never calls it and
shares no code, table or helper with it.

Source: the forward steps of the page "EDiT: Efficient Diffusion Transformers
with Linear Compressed Attention" (ICCV 2025 paper notes), as composed in
edit_oracle: sections "ConvFusion", "Spatial Compressor", "Linear-attention
formula", and the output Linear (R12). The page trains the layer by
distillation (section "训练策略", training strategy), which needs these gradients; it
writes no backward formulas itself, so every function below is the chain
rule applied to the forward definition it names: given the gradient of a
step's output (the upstream gradient), it returns the gradients of that
step's inputs and parameters. Sums over tokens run over every sample and
position, so a parameter's gradient is its total over the batch.

Pins live in tests/test_oracle_backward.py: torch.autograd through an
independent float64 torch.nn.functional forward, central finite differences
of the oracle forward, and the invariants of the GroupNorm gradient.
"""
from __future__ import annotations

import numpy as np

from . import edit_oracle as O

_f64 = O._f64


# ----------------------------------------------------------------------------
# Elementwise maps and the Linear
# ----------------------------------------------------------------------------

def relu_backward(out, dout):
    """ReLU: the gradient passes where the output is positive (the derivative
    at 0 is taken as 0, where ReLU's output is 0)."""
    return np.where(_f64(out) > 0, _f64(dout), 0.0)


def leaky_relu_backward(pre, dout, slope=O.LEAKY_SLOPE):
    """LeakyReLU (R5): slope 1 where the input is >= 0, `slope` below. The sign
    of the output equals the sign of the input, so `pre` may be either."""
    return np.where(_f64(pre) >= 0, _f64(dout), slope * _f64(dout))


def linear_backward(x, w, dout):
    """y = x W^T + b: dx = dy W, dW = sum_tokens dy^T x, db = sum_tokens dy."""
    x, w, dout = _f64(x), _f64(w), _f64(dout)
    C_in, C_out = x.shape[-1], dout.shape[-1]
    x2, d2 = x.reshape(-1, C_in), dout.reshape(-1, C_out)
    return dout @ w, d2.T @ x2, d2.sum(axis=0)


# ----------------------------------------------------------------------------
# Convolutions
# ----------------------------------------------------------------------------

def conv3x3_backward(g, w, dout):
    """Backward of edit_oracle.conv3x3 (dense 3x3, stride 1, zero pad 1).

    Tap (ky, kx) carries g[y+ky-1, x+kx-1] to out[y, x]: its input gradient is
    dout @ w[:, ky, kx, :] added back at the shifted position, its weight
    gradient the sum over positions of dout^T times the shifted window."""
    g, w, dout = _f64(g), _f64(w), _f64(dout)
    B, H, W, Cin = g.shape
    Cout = w.shape[0]
    pad = np.zeros((B, H + 2, W + 2, Cin))
    pad[:, 1:H + 1, 1:W + 1, :] = g
    dpad = np.zeros_like(pad)
    dw = np.zeros_like(w)
    d2 = dout.reshape(-1, Cout)
    for ky in range(3):
        for kx in range(3):
            window = pad[:, ky:ky + H, kx:kx + W, :]
            dpad[:, ky:ky + H, kx:kx + W, :] += dout @ w[:, ky, kx, :]
            dw[:, ky, kx, :] = d2.T @ window.reshape(-1, Cin)
    return dpad[:, 1:H + 1, 1:W + 1, :], dw, d2.sum(axis=0)


def dwconv3x3_s2_backward(g, w, dout):
    """Backward of edit_oracle.dwconv3x3_s2 (depthwise 3x3, stride 2, pad 1):
    tap (ky, kx) of output (y', x') read input (2y'+ky-1, 2x'+kx-1), so the
    input gradient scatters dout * w back there and the weight gradient sums
    dout times that input over the output positions."""
    g, w, dout = _f64(g), _f64(w), _f64(dout)
    B, H, W, C = g.shape
    Ho, Wo = dout.shape[1], dout.shape[2]
    pad = np.zeros((B, 2 * Ho + 2, 2 * Wo + 2, C))
    pad[:, 1:H + 1, 1:W + 1, :] = g
    dpad = np.zeros_like(pad)
    dw = np.zeros_like(w)
    for ky in range(3):
        for kx in range(3):
            window = pad[:, ky:ky + 2 * Ho:2, kx:kx + 2 * Wo:2, :]
            dpad[:, ky:ky + 2 * Ho:2, kx:kx + 2 * Wo:2, :] += dout * w[ky, kx, :]
            dw[ky, kx, :] = (dout * window).sum(axis=(0, 1, 2))
    return dpad[:, 1:H + 1, 1:W + 1, :], dw, dout.sum(axis=(0, 1, 2))


# ----------------------------------------------------------------------------
# GroupNorm
# ----------------------------------------------------------------------------

def group_norm_backward(g, groups, gamma, dout, eps=O.GN_EPS):
    """Backward of edit_oracle.group_norm (R4: statistics per sample and group
    over positions and the group's channels, biased variance).

    With xhat = (g - mean) / sqrt(var + eps) and out = gamma xhat + beta:
    dgamma = sum dout xhat, dbeta = sum dout, and with dxhat = dout gamma,
    dg = (dxhat - mean(dxhat) - xhat mean(dxhat xhat)) / sqrt(var + eps),
    the means over each (sample, group)."""
    g, dout, gamma = _f64(g), _f64(dout), _f64(gamma)
    B, H, W, C = g.shape
    cg = C // groups
    mean, var = O.group_norm_stats(g, groups)
    rstd = 1.0 / np.sqrt(var + eps)                                    # [B, G]
    mean_c = np.repeat(mean, cg, axis=1)[:, None, None, :]
    rstd_c = np.repeat(rstd, cg, axis=1)[:, None, None, :]
    xhat = (g - mean_c) * rstd_c
    dgamma = (dout * xhat).sum(axis=(0, 1, 2))
    dbeta = dout.sum(axis=(0, 1, 2))
    dxhat = (dout * gamma).reshape(B, H * W, groups, cg)
    xh = xhat.reshape(B, H * W, groups, cg)
    m1 = dxhat.mean(axis=(1, 3), keepdims=True)
    m2 = (dxhat * xh).mean(axis=(1, 3), keepdims=True)
    dg = (dxhat - m1 - xh * m2) * rstd[:, None, :, None]
    return dg.reshape(B, H, W, C), dgamma, dbeta


# ----------------------------------------------------------------------------
# Linear attention
# ----------------------------------------------------------------------------

def linear_attention_apply_backward(q, S, z, heads, eps, dy):
    """Backward of edit_oracle.linear_attention_apply, y_i = num_i / den_i with
    num_i = Q_i S and den_i = Q_i . z + eps per head (section "Linear-attention
    formula"): dnum = dy / den, dden = -(dy . num) / den^2, so
    dQ = dnum S^T + dden z, dS = sum_i Q_i^T dnum_i, dz = sum_i dden_i Q_i."""
    Q = O.split_heads(q, heads)
    dY = O.split_heads(dy, heads)
    S, z = _f64(S), _f64(z)
    num = Q @ S
    den = (Q * z[:, :, None, :]).sum(axis=-1) + eps                    # [B, h, N]
    dnum = dY / den[..., None]
    dden = -(dY * num).sum(axis=-1) / den ** 2
    dQ = dnum @ np.swapaxes(S, 2, 3) + dden[..., None] * z[:, :, None, :]
    dS = np.swapaxes(Q, 2, 3) @ dnum
    dz = (dden[..., None] * Q).sum(axis=2)
    return O.merge_heads(dQ), dS, dz


def kv_state_backward(kc, vc, dS, dz, heads):
    """Backward of edit_oracle.kv_state, S = sum_j K'_j^T V'_j and
    z = sum_j K'_j: dK'_j = V'_j dS^T + dz, dV'_j = K'_j dS."""
    K = O.split_heads(kc, heads)
    V = O.split_heads(vc, heads)
    dS, dz = _f64(dS), _f64(dz)
    dK = V @ np.swapaxes(dS, 2, 3) + dz[:, :, None, :]
    dV = K @ dS
    return O.merge_heads(dK), O.merge_heads(dV)


# ----------------------------------------------------------------------------
# The layer
# ----------------------------------------------------------------------------

PARAM_NAMES = ("w_cf1", "b_cf1", "gn_gamma", "gn_beta", "w_cf2", "b_cf2", "w_q", "b_q", "w_k", "b_k",
               "w_v", "b_v", "dw_k", "db_k", "dw_v", "db_v", "w_o", "b_o")


FORWARD_KEYS = ("xc", "cf_act", "q", "k0", "v0", "kc", "vc", "S", "z", "y")


def edit_attn_backward(x, w, shape, dout, trace=None, forward=None):
    """Gradients of sum(dout * edit_attn_forward(x, w, shape)) with respect to
    x and every parameter, in the forward's composition (the restored stream
    xt is formed, as the page writes it). Returns (dx, {name: gradient}) with
    each gradient in its parameter's shape; ``trace`` receives the
    intermediate gradients (dy, dq, dS, dz, dkc, dvc, dk0, dv0, dxt, dact,
    dxc).

    ``forward`` (optional) supplies the forward tensors every step's backward
    is evaluated at, instead of this function's own float64 forward: a dict
    with the token-major arrays FORWARD_KEYS (xc, cf_act, q, k0, v0, kc, vc,
    y as [B, tokens, channels]; S [B, h, d, d]; z [B, h, d]), e.g. those
    another computation of the same forward stored. Each step's chain rule
    then runs at that computation's values, kink decisions included (R28:
    the derivative at a kink follows the sign of the forward value there),
    and the restored stream is xt = x + cf_act W_cf2^T + b_cf2 from the given
    cf_act. With the float64 forward's own tensors the result is unchanged."""
    H, W, heads, G = shape.H, shape.W, shape.heads, shape.gn_groups
    x = _f64(x)
    f = {}
    if forward is None:
        O.edit_attn_forward(x, w, shape, f)
    else:
        missing = [k for k in FORWARD_KEYS if k not in forward]
        if missing:
            raise ValueError(f"forward lacks {missing}")
        f = {k: _f64(forward[k]) for k in FORWARD_KEYS}
        f["xt"] = x + O.linear(f["cf_act"], w["w_cf2"], w["b_cf2"])
    grid = lambda t: O.tokens_to_grid(t, H, W)
    tok = O.grid_to_tokens

    # output Linear
    dy, dw_o, db_o = linear_backward(f["y"], w["w_o"], dout)
    # linear attention (apply, then the per-head sums)
    dq, dS, dz = linear_attention_apply_backward(f["q"], f["S"], f["z"], heads, shape.eps, dy)
    dkc, dvc = kv_state_backward(f["kc"], f["vc"], dS, dz, heads)
    # Spatial Compressor: ReLU on the keys, depthwise stride-2 convs, Linears
    dkc_pre = relu_backward(f["kc"], dkc)
    dk0, ddw_k, ddb_k = dwconv3x3_s2_backward(grid(f["k0"]), w["dw_k"], O.tokens_to_grid(
        dkc_pre, (H + 1) // 2, (W + 1) // 2))
    dv0, ddw_v, ddb_v = dwconv3x3_s2_backward(grid(f["v0"]), w["dw_v"], O.tokens_to_grid(
        dvc, (H + 1) // 2, (W + 1) // 2))
    dk0, dv0 = tok(dk0), tok(dv0)
    dx_k, dw_k, db_k = linear_backward(x, w["w_k"], dk0)
    dx_v, dw_v, db_v = linear_backward(x, w["w_v"], dv0)
    # ConvFusion: outer ReLU, query Linear, residual + 1x1 restore,
    # LeakyReLU, GroupNorm, 3x3 conv
    dq_pre = relu_backward(f["q"], dq)
    dxt, dw_q, db_q = linear_backward(f["xt"], w["w_q"], dq_pre)
    dact, dw_cf2, db_cf2 = linear_backward(f["cf_act"], w["w_cf2"], dxt)
    da0 = leaky_relu_backward(f["cf_act"], dact)
    dxc, dgamma, dbeta = group_norm_backward(grid(f["xc"]), G, w["gn_gamma"], grid(da0))
    dx_c, dw_cf1, db_cf1 = conv3x3_backward(grid(x), w["w_cf1"], dxc)
    dx = dxt + tok(dx_c) + dx_k + dx_v
    grads = {"w_cf1": dw_cf1, "b_cf1": db_cf1, "gn_gamma": dgamma, "gn_beta": dbeta,
             "w_cf2": dw_cf2, "b_cf2": db_cf2, "w_q": dw_q, "b_q": db_q, "w_k": dw_k, "b_k": db_k,
             "w_v": dw_v, "b_v": db_v, "dw_k": ddw_k, "db_k": ddb_k, "dw_v": ddw_v, "db_v": ddb_v,
             "w_o": dw_o, "b_o": db_o}
    if trace is not None:
        trace.update(forward=f, dy=dy, dq=dq, dq_pre=dq_pre, dS=dS, dz=dz, dkc=dkc, dvc=dvc, dk0=dk0,
                     dv0=dv0, dxt=dxt, dact=dact, dxc=tok(dxc))
    return dx, grads
