"""CPU oracle of the EDiT linear compressed attention layer and its MM-EDiT
hybrid, in float64 numpy.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The HIP library never calls it and
shares no code, table or helper with it.

Source: the page "EDiT: Efficient Diffusion Transformers with Linear
Compressed Attention" (ICCV 2025 paper notes, arXiv 2503.16726), cited below
by its sections: "ConvFusion" (the Q^EDiT equation), "Spatial Compressor"
(the K^EDiT / V^EDiT equations and the depthwise stride-2 remark),
"Linear-attention formula" (the y_i equation), "MM-EDiT" (the A^Hybrid
matrix and the eta approximation under it) and "Ablation: Query/Key/Value
processing" (the table of Q/K/V variants).

Every step is written from its definition, in the order the page composes
them, with numpy's matmul as the only library primitive. Where the page
leaves a detail open, the reading taken is named at the function (R1..R16,
R23..R26);
the same readings are listed in the design notes of the repository.

Pins (what checks this code against something other than itself) live in
tests/test_oracle_*.py: brute-force loops and exact rational arithmetic on tiny
inputs, closed forms, invariants, hand-worked fixtures under tests/golden/,
and torch.nn.functional on the CPU as an independent third opinion. Every
function below has at least one such pin; none is "parity unpinned". The
composed layer cannot be pinned to the authors' own outputs (no code or
weights are published), only to the definitions.
"""
from __future__ import annotations

import numpy as np

GN_EPS = 1e-5          # R4: GroupNorm epsilon (the common default)
LEAKY_SLOPE = 0.01     # R5: LeakyReLU negative slope (the common default)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# Elementwise maps
# ----------------------------------------------------------------------------

def relu(x):
    """max(x, 0). ConvFusion's outer activation and the key feature map
    (sections "ConvFusion" and "Spatial Compressor")."""
    x = _f64(x)
    return np.where(x > 0, x, 0.0)


def leaky_relu(x, slope=LEAKY_SLOPE):
    """x for x >= 0, slope*x otherwise (section "ConvFusion"; R5: slope 0.01)."""
    x = _f64(x)
    return np.where(x >= 0, x, slope * x)


# ----------------------------------------------------------------------------
# Token grid and convolutions
# ----------------------------------------------------------------------------

def tokens_to_grid(x, H, W):
    """[B, H*W, C] -> [B, H, W, C]: token n sits at row n // W, column n % W
    (section "ConvFusion": the 1-D sequence is laid out as a 2-D image before
    any convolution; R7: row-major token order, channels last)."""
    x = _f64(x)
    B, N, C = x.shape
    assert N == H * W
    return x.reshape(B, H, W, C)


def grid_to_tokens(g):
    B, H, W, C = g.shape
    return g.reshape(B, H * W, C)


def linear(x, w, b):
    """y = x W^T + b over the last axis; W is [out][in]."""
    return _f64(x) @ _f64(w).T + _f64(b)


def conv3x3(g, w, b):
    """Dense 3x3 convolution, stride 1, zero padding 1, with bias.

    out[b, y, x, o] = b[o] + sum_{ky, kx, i} w[o, ky, kx, i] * g[b, y+ky-1, x+kx-1, i]
    (cross-correlation, the deep-learning convention; out-of-grid inputs read
    as zero). g is [B, H, W, Cin], w is [Cout, 3, 3, Cin].
    Section "ConvFusion": the first convolution is 3x3 and changes the channel
    count (R2: dense, stride 1, pad 1 so the residual shape matches)."""
    g, w, b = _f64(g), _f64(w), _f64(b)
    B, H, W, Cin = g.shape
    Cout = w.shape[0]
    assert w.shape == (Cout, 3, 3, Cin)
    pad = np.zeros((B, H + 2, W + 2, Cin))
    pad[:, 1:H + 1, 1:W + 1, :] = g
    out = np.broadcast_to(b, (B, H, W, Cout)).copy()
    for ky in range(3):
        for kx in range(3):
            window = pad[:, ky:ky + H, kx:kx + W, :]        # g[y+ky-1, x+kx-1]
            out += window @ w[:, ky, kx, :].T
    return out


def conv1x1(g, w, b):
    """1x1 convolution = a per-pixel Linear; w is [Cout][Cin]
    (section "ConvFusion": the second convolution, R3: with bias)."""
    return linear(g, w, b)


def dwconv3x3_s2(g, w, b):
    """Depthwise 3x3 convolution, stride 2, zero padding 1, with bias.

    out[b, y', x', c] = b[c] + sum_{ky, kx} w[ky, kx, c] * g[b, 2y'+ky-1, 2x'+kx-1, c]
    with out-of-grid inputs zero; output grid ceil(H/2) x ceil(W/2).
    Section "Spatial Compressor": 3x3 depthwise, stride 2, four times fewer
    tokens (R8: padding 1, ceiling for odd sizes). w is [3, 3, C]."""
    g, w, b = _f64(g), _f64(w), _f64(b)
    B, H, W, C = g.shape
    Ho, Wo = (H + 1) // 2, (W + 1) // 2
    pad = np.zeros((B, 2 * Ho + 2, 2 * Wo + 2, C))
    pad[:, 1:H + 1, 1:W + 1, :] = g
    out = np.broadcast_to(b, (B, Ho, Wo, C)).copy()
    for ky in range(3):
        for kx in range(3):
            # padded index of input row 2y'+ky-1 is 2y'+ky
            window = pad[:, ky:ky + 2 * Ho:2, kx:kx + 2 * Wo:2, :]
            out += window * w[ky, kx, :]
    return out


# ----------------------------------------------------------------------------
# GroupNorm
# ----------------------------------------------------------------------------

def group_norm_stats(g, groups):
    """Per (sample, group) mean and biased variance over every spatial
    position and the group's C/groups consecutive channels (R4).
    Returns (mean, var), each [B, groups]."""
    g = _f64(g)
    B, H, W, C = g.shape
    assert C % groups == 0
    v = g.reshape(B, H * W, groups, C // groups)
    mean = v.mean(axis=(1, 3))
    var = ((v - mean[:, None, :, None]) ** 2).mean(axis=(1, 3))
    return mean, var


def group_norm(g, groups, gamma, beta, eps=GN_EPS):
    """GroupNorm with per-channel affine (section "ConvFusion": GN after the
    compressing conv, for stability; R4)."""
    g = _f64(g)
    B, H, W, C = g.shape
    mean, var = group_norm_stats(g, groups)
    cg = C // groups
    mean_c = np.repeat(mean, cg, axis=1)[:, None, None, :]
    var_c = np.repeat(var, cg, axis=1)[:, None, None, :]
    return (g - mean_c) / np.sqrt(var_c + eps) * _f64(gamma) + _f64(beta)


# ----------------------------------------------------------------------------
# ConvFusion queries and Spatial-Compressor keys / values
# ----------------------------------------------------------------------------

def convfusion_query(x, H, W, w, groups, trace=None):
    """Q = ReLU(Linear_Q(X + Conv1x1(LeakyReLU(GN(Conv3x3(X)))))).

    Section "ConvFusion", the Q^EDiT equation, read inside out. R6: the
    outer Linear is the layer's query projection (W_q, b_q). Returns
    [B, N, C]; ``trace`` (a dict) receives the intermediates."""
    x = _f64(x)
    g = tokens_to_grid(x, H, W)
    xc = conv3x3(g, w["w_cf1"], w["b_cf1"])
    mean, var = group_norm_stats(xc, groups)
    a = leaky_relu(group_norm(xc, groups, w["gn_gamma"], w["gn_beta"]))
    xt = x + grid_to_tokens(conv1x1(a, w["w_cf2"], w["b_cf2"]))
    q = relu(linear(xt, w["w_q"], w["b_q"]))
    if trace is not None:
        trace.update(xc=grid_to_tokens(xc), gn_mean=mean, gn_var=var,
                     cf_act=grid_to_tokens(a), xt=xt, q=q)
    return q


def spatial_compressor_kv(x, H, W, w, trace=None):
    """K' = ReLU(DW(Linear_K(X))), V' = DW(Linear_V(X)).

    Section "Spatial Compressor": phi_SC(X) = Conv(Linear(X)), the key takes a
    ReLU and the value none. R1: K and V carry their own Linear and
    depthwise parameters. Returns ([B, N', C], [B, N', C])."""
    x = _f64(x)
    k0 = linear(x, w["w_k"], w["b_k"])
    v0 = linear(x, w["w_v"], w["b_v"])
    kc = relu(dwconv3x3_s2(tokens_to_grid(k0, H, W), w["dw_k"], w["db_k"]))
    vc = dwconv3x3_s2(tokens_to_grid(v0, H, W), w["dw_v"], w["db_v"])
    kc, vc = grid_to_tokens(kc), grid_to_tokens(vc)
    if trace is not None:
        trace.update(k0=k0, v0=v0, kc=kc, vc=vc)
    return kc, vc


# ----------------------------------------------------------------------------
# Linear attention
# ----------------------------------------------------------------------------

def split_heads(t, heads):
    """[B, N, C] -> [B, heads, N, d]; head h owns channels h*d .. h*d+d-1 (R10)."""
    t = _f64(t)
    B, N, C = t.shape
    d = C // heads
    return t.reshape(B, N, heads, d).transpose(0, 2, 1, 3)


def merge_heads(t):
    B, h, N, d = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, N, h * d)


def kv_state(kc, vc, heads):
    """Per (sample, head): S = sum_j K'_j^T V'_j (d x d) and z = sum_j K'_j (d).

    Section "Linear-attention formula": the two sums shared by every query
    (R9: over the compressed tokens). Returns S [B, h, d, d], z [B, h, d]."""
    K = split_heads(kc, heads)
    V = split_heads(vc, heads)
    S = np.swapaxes(K, 2, 3) @ V
    z = K.sum(axis=2)
    return S, z


def linear_attention_apply(q, S, z, heads, eps):
    """y_i = (Q_i S) / (Q_i . z + eps), per head (section "Linear-attention
    formula"; R11: eps in the denominator, no 1/sqrt(d) in this branch).
    Returns [B, N, C]."""
    Q = split_heads(q, heads)
    num = Q @ S                                   # [B, h, N, d]
    den = (Q * z[:, :, None, :]).sum(axis=-1)     # [B, h, N]
    return merge_heads(num / (den[..., None] + eps))


def linear_attention(q, kc, vc, heads, eps):
    S, z = kv_state(kc, vc, heads)
    return linear_attention_apply(q, S, z, heads, eps)


# ----------------------------------------------------------------------------
# EDiT layer
# ----------------------------------------------------------------------------

def edit_attn_forward(x, w, shape, trace=None):
    """The EDiT attention layer: ConvFusion queries, Spatial-Compressor keys
    and values, linear attention, then the output projection (R12).

    x is [B, H*W, C]; ``shape`` carries H, W, heads, gn_groups and eps.
    Returns [B, N, C]."""
    H, W, heads = shape.H, shape.W, shape.heads
    q = convfusion_query(x, H, W, w, shape.gn_groups, trace)
    kc, vc = spatial_compressor_kv(x, H, W, w, trace)
    S, z = kv_state(kc, vc, heads)
    y = linear_attention_apply(q, S, z, heads, shape.eps)
    out = linear(y, w["w_o"], w["b_o"])
    if trace is not None:
        trace.update(S=S, z=z, y=y, out=out)
    return out


# ----------------------------------------------------------------------------
# Ablation variants of the query / key / value processing
# ----------------------------------------------------------------------------

QUERY_MODES = ("convfusion", "linear")
KV_MODES = ("compressed", "full", "key_convfusion")


def edit_attn_variant_forward(x, w, shape, query="convfusion", kv="compressed", w_kcf=None, trace=None):
    """The EDiT layer with the query and key/value processing of the notes'
    ablation table (section "Ablation: Query/Key/Value processing", whose rows
    are (Q, K, V) = (CF, SC, SC), (CF, CF, -), (-, SC, SC) and (CF, -, -)).

    query="convfusion": Q = ReLU(Linear_Q(X + ConvFusion(X)))  (the layer's Q)
    query="linear":     Q = ReLU(Linear_Q(X))                   (R24)
    kv="compressed":    K' = ReLU(DW(Linear_K X)), V' = DW(Linear_V X)  (SC, SC)
    kv="full":          K = ReLU(Linear_K X), V = Linear_V X over all N tokens  (-, -; R25)
    kv="key_convfusion": K = ReLU(Linear_K(X + ConvFusion_K(X))) with the key
                        branch's own ConvFusion parameters ``w_kcf`` (w_cf1,
                        b_cf1, gn_gamma, gn_beta, w_cf2, b_cf2), V = Linear_V X
                        (CF, -; R26)
    The linear attention, its eps and the output projection are the layer's.
    ``trace`` receives q, k, v (the keys and values the sums run over), S, z,
    y, out, and for the key branch xc_k / xt_k."""
    if query not in QUERY_MODES or kv not in KV_MODES:
        raise ValueError(f"unknown variant ({query!r}, {kv!r})")
    H, W, heads, G = shape.H, shape.W, shape.heads, shape.gn_groups
    x = _f64(x)
    if query == "convfusion":
        q = convfusion_query(x, H, W, w, G, trace)
    else:
        q = relu(linear(x, w["w_q"], w["b_q"]))
    if kv == "compressed":
        k, v = spatial_compressor_kv(x, H, W, w, trace)
    elif kv == "full":
        k = relu(linear(x, w["w_k"], w["b_k"]))
        v = linear(x, w["w_v"], w["b_v"])
    else:
        if w_kcf is None:
            raise ValueError("kv='key_convfusion' needs the key ConvFusion parameters")
        wk = dict(w_kcf)
        wk["w_q"], wk["b_q"] = w["w_k"], w["b_k"]
        tk = {} if trace is not None else None
        k = convfusion_query(x, H, W, wk, G, tk)
        v = linear(x, w["w_v"], w["b_v"])
        if trace is not None:
            trace.update(xc_k=tk["xc"], cf_act_k=tk["cf_act"], xt_k=tk["xt"])
    S, z = kv_state(k, v, heads)
    y = linear_attention_apply(q, S, z, heads, shape.eps)
    out = linear(y, w["w_o"], w["b_o"])
    if trace is not None:
        trace.update(q=q, k=k, v=v, S=S, z=z, y=y, out=out)
    return out


# ----------------------------------------------------------------------------
# Scaled dot-product attention and the MM-EDiT hybrid
# ----------------------------------------------------------------------------

def softmax_rows(s):
    """Row softmax; the row maximum is subtracted first (an identity)."""
    s = _f64(s)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def sdpa(q, k, v, heads):
    """softmax(Q K^T / sqrt(d)) V per head, no mask (R15).
    q [B, Nq, C], k and v [B, Nk, C]; returns [B, Nq, C]."""
    Q, K, V = split_heads(q, heads), split_heads(k, heads), split_heads(v, heads)
    d = Q.shape[-1]
    P = softmax_rows(Q @ np.swapaxes(K, 2, 3) / np.sqrt(d))
    return merge_heads(P @ V)


def hybrid_eta(n_img, n_txt):
    """eta^Lin approximated by the token-count ratio N_I / (N_I + N_T)
    (section "MM-EDiT", the approximation under the hybrid matrix; R13: N_I
    counts the uncompressed image tokens)."""
    return n_img / (n_img + n_txt)


def linear_attention_denominator(q, z, heads, eps):
    """Q_i . z + eps per token and head: the normaliser of the linear block
    (section "Linear-attention formula"; R11). Returns [B, N, heads]."""
    Q = split_heads(q, heads)
    return (Q * z[:, :, None, :]).sum(axis=-1).transpose(0, 2, 1) + eps


def hybrid_image_rows_exact(q_i, S, z, k_t, v_t, heads, eps):
    """Image rows of the hybrid with eta^Lin computed instead of approximated.

    Section "MM-EDiT": the hybrid matrix weights the linear block A^Lin by
    eta^Lin and the image->text softmax block by 1 - eta^Lin; the page replaces
    eta^Lin by the token ratio to avoid a custom kernel. Computed exactly, the
    two blocks share one normaliser (R23):
        y_i = (Q_i S + sum_t exp(s_it) V_t) / (Q_i . z + eps + sum_t exp(s_it)),
        s_it = Q_i . K_t / sqrt(d),
    which is eta_i A^Lin_i + (1 - eta_i) A_i with
    eta_i = (Q_i . z + eps) / (Q_i . z + eps + sum_t exp(s_it)).
    q_i [B, N, C]; S [B, h, d, d]; z [B, h, d]; k_t, v_t [B, N_T, C]."""
    Q = split_heads(q_i, heads)
    Kt, Vt = split_heads(k_t, heads), split_heads(v_t, heads)
    d = Q.shape[-1]
    e = np.exp(Q @ np.swapaxes(Kt, 2, 3) / np.sqrt(d))     # [B, h, N, N_T]
    num = Q @ S + e @ Vt
    den = (Q * z[:, :, None, :]).sum(axis=-1) + eps + e.sum(axis=-1)
    return merge_heads(num / den[..., None])


def mmedit_hybrid_forward(x_img, x_txt, w, wt, shape, trace=None, eta="ratio"):
    """The MM-EDiT hybrid attention layer (section "MM-EDiT").

    Image rows:  eta * A^Lin(Q_I, K'_I, V'_I) + (1 - eta) * A(Q_I, K_T, V_T)
    Text rows:   exact softmax attention over the concatenated keys
                 [K'_I ; K_T] with values [V'_I ; V_T]  (R14)
    then separate image and text output projections (R12, R16).
    Q_I, K'_I, V'_I are the EDiT features of the image stream (R14); the
    text stream has its own Linear Q/K/V/O and no convolutions (R16).
    eta="ratio" takes the page's token-count ratio for eta^Lin (R13);
    eta="exact" computes it per row (hybrid_image_rows_exact, R23).
    Returns (out_img [B, N, C], out_txt [B, N_T, C])."""
    if eta not in ("ratio", "exact"):
        raise ValueError(f"eta must be 'ratio' or 'exact', not {eta!r}")
    H, W, heads = shape.H, shape.W, shape.heads
    x_img = _f64(x_img)
    n_img = H * W
    q_i = convfusion_query(x_img, H, W, w, shape.gn_groups, trace)
    kc, vc = spatial_compressor_kv(x_img, H, W, w, trace)
    S, z = kv_state(kc, vc, heads)
    y_lin = linear_attention_apply(q_i, S, z, heads, shape.eps)
    n_txt = 0 if x_txt is None else x_txt.shape[1]
    if n_txt == 0:
        y_img = y_lin
        y_txt = None
        out_txt = None
        q_t = k_t = v_t = None
    else:
        x_txt = _f64(x_txt)
        q_t = linear(x_txt, wt["w_q"], wt["b_q"])
        k_t = linear(x_txt, wt["w_k"], wt["b_k"])
        v_t = linear(x_txt, wt["w_v"], wt["b_v"])
        if eta == "exact":
            y_img = hybrid_image_rows_exact(q_i, S, z, k_t, v_t, heads, shape.eps)
        else:
            e_r = hybrid_eta(n_img, n_txt)
            y_img = e_r * y_lin + (1.0 - e_r) * sdpa(q_i, k_t, v_t, heads)
        y_txt = sdpa(q_t, np.concatenate([kc, k_t], axis=1),
                     np.concatenate([vc, v_t], axis=1), heads)
        out_txt = linear(y_txt, wt["w_o"], wt["b_o"])
    out_img = linear(y_img, w["w_o"], w["b_o"])
    if trace is not None:
        trace.update(S=S, z=z, y_lin=y_lin, y=y_img, y_txt=y_txt, q_t=q_t,
                     k_t=k_t, v_t=v_t, out=out_img, out_txt=out_txt,
                     lin_den=linear_attention_denominator(q_i, z, heads, shape.eps))
    return out_img, out_txt
