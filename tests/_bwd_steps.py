"""Step-by-step comparison of the GPU layer backward with the oracle (test
infrastructure).

Each chain-rule step of the backward is checked on its own: the oracle's
step function (oracle/edit_backward.py) receives the inputs that step had on
the GPU -- the forward tensors the GPU stored and the upstream gradient the
GPU's previous step stored -- and its result is compared with what the GPU
step wrote. So no step inherits the rounding of another, and every tensor
can be held to the plain max-relative gate even where a sum cancels (the key
bias gradients sum terms ~1000 times larger than the result).
"""
import numpy as np

from oracle import edit_backward as OB
from oracle import edit_oracle as O

BWD_TENSORS = ("dy", "dq_pre", "dS", "dz", "dkv", "dk0v0", "dxq", "dxkv", "dact", "dxc")


def read_forward(lca, s, fws, torch, T):
    """The forward tensors the oracle's backward steps are evaluated at."""
    lay = lca.edit_attn_workspace_layout(s, 0)
    B, N, Nc, C, Cr, h, d = s.B, s.N, s.Nc, s.C, s.Cr, s.heads, s.head_dim
    es = 2 if T == torch.bfloat16 else 4

    def v(name, shape, dt=T):
        n = int(np.prod(shape)) * (4 if dt == torch.float32 else es)
        return fws[lay[name]:lay[name] + n].view(dt).float().cpu().numpy().reshape(shape)
    kv0 = v("kv0", (B, N, 2 * C))
    return {"xc": v("xc", (B, N, Cr)), "cf_act": v("cf_act", (B, N, Cr)), "q": v("q", (B, N, C)),
            "k0": kv0[..., :C], "v0": kv0[..., C:], "kc": v("kc", (B, Nc, C)), "vc": v("vc", (B, Nc, C)),
            "S": v("S", (B, h, d, d), torch.float32), "z": v("z", (B, h, d), torch.float32), "y": v("y", (B, N, C))}


def read_backward(lca, s, bws, torch, T):
    """The backward's intermediate gradients from its workspace."""
    lay = lca.edit_attn_backward_workspace_layout(s)
    B, N, Nc, C, Cr, h, d = s.B, s.N, s.Nc, s.C, s.Cr, s.heads, s.head_dim
    es = 2 if T == torch.bfloat16 else 4

    def v(name, shape, dt=T):
        n = int(np.prod(shape)) * (4 if dt == torch.float32 else es)
        return bws[lay[name]:lay[name] + n].view(dt).float().cpu().numpy().reshape(shape)
    f32 = torch.float32
    return {"dy": v("dy", (B, N, C)), "dq_pre": v("dq_pre", (B, N, C)), "dS": v("dS", (B, h, d, d), f32),
            "dz": v("dz", (B, h, d), f32), "dkv": v("dkv", (B, Nc, 2 * C), f32), "dk0v0": v("dk0v0", (B, N, 2 * C)),
            "dxq": v("dxq", (B, N, C)), "dxkv": v("dxkv", (B, N, C)), "dact": v("dact", (B, N, Cr)),
            "dxc": v("dxc", (B, N, lay["dxc_ld"]))[..., :Cr]}


def step_pairs(s, x, w, dout, fwd, bwd, got):
    """(GPU, oracle) pairs of every backward step's outputs, the oracle step
    fed that step's GPU inputs. fwd: read_forward; bwd: read_backward; got:
    the GPU's dx ("x") and parameter gradients."""
    H, W, heads, C = s.H, s.W, s.heads, s.C
    x = np.asarray(x, np.float64)
    grid = lambda t: O.tokens_to_grid(t, H, W)
    cgrid = lambda t: O.tokens_to_grid(t, (H + 1) // 2, (W + 1) // 2)
    tok = O.grid_to_tokens
    p = {}
    # output Linear: dout, y -> dy, dW_o, db_o
    dy, p_wo, p_bo = OB.linear_backward(fwd["y"], w["w_o"], dout)
    p["dy"], p["w_o"], p["b_o"] = (bwd["dy"], dy), (got["w_o"], p_wo), (got["b_o"], p_bo)
    # linear-attention apply at q, S, z with the GPU's dy; the queries' ReLU
    dq, dS, dz = OB.linear_attention_apply_backward(fwd["q"], fwd["S"], fwd["z"], heads, s.eps, bwd["dy"])
    p["dq_pre"] = (bwd["dq_pre"], OB.relu_backward(fwd["q"], dq))
    p["dS"], p["dz"] = (bwd["dS"], dS), (bwd["dz"], dz)
    # the per-head sums S, z with the GPU's dS, dz; the keys' ReLU
    dkc, dvc = OB.kv_state_backward(fwd["kc"], fwd["vc"], bwd["dS"], bwd["dz"], heads)
    p["dkv"] = (bwd["dkv"], np.concatenate([OB.relu_backward(fwd["kc"], dkc), dvc], -1))
    # the depthwise stride-2 convs with the GPU's dkv
    dk0, dwk, dbk = OB.dwconv3x3_s2_backward(grid(fwd["k0"]), w["dw_k"], cgrid(bwd["dkv"][..., :C]))
    dv0, dwv, dbv = OB.dwconv3x3_s2_backward(grid(fwd["v0"]), w["dw_v"], cgrid(bwd["dkv"][..., C:]))
    dk0, dv0 = tok(dk0), tok(dv0)
    p["dk0v0"] = (bwd["dk0v0"], np.concatenate([dk0, dv0], -1))
    p["dw_k"], p["db_k"], p["dw_v"], p["db_v"] = (got["dw_k"], dwk), (got["db_k"], dbk), (got["dw_v"], dwv), \
        (got["db_v"], dbv)
    # the key / value Linears with the GPU's dk0 | dv0 (their bias gradients: sums of the step above)
    dxk, p_wk, _ = OB.linear_backward(x, w["w_k"], bwd["dk0v0"][..., :C])
    dxv, p_wv, _ = OB.linear_backward(x, w["w_v"], bwd["dk0v0"][..., C:])
    p["w_k"], p["w_v"] = (got["w_k"], p_wk), (got["w_v"], p_wv)
    p["b_k"], p["b_v"] = (got["b_k"], dk0.sum(axis=(0, 1))), (got["b_v"], dv0.sum(axis=(0, 1)))
    p["dxkv"] = (bwd["dxkv"], bwd["dxq"] + dxk + dxv)
    # the query Linear over the restored stream xt = x + act W_cf2^T + b_cf2, with the GPU's dq_pre
    xt = x + O.linear(fwd["cf_act"], w["w_cf2"], w["b_cf2"])
    dxt, p_wq, p_bq = OB.linear_backward(xt, w["w_q"], bwd["dq_pre"])
    p["dxq"], p["w_q"], p["b_q"] = (bwd["dxq"], dxt), (got["w_q"], p_wq), (got["b_q"], p_bq)
    # the 1x1 restore, with the GPU's dxt
    dact, p_w2, p_b2 = OB.linear_backward(fwd["cf_act"], w["w_cf2"], bwd["dxq"])
    p["dact"], p["w_cf2"], p["b_cf2"] = (bwd["dact"], dact), (got["w_cf2"], p_w2), (got["b_cf2"], p_b2)
    # LeakyReLU and GroupNorm, with the GPU's dact
    da0 = OB.leaky_relu_backward(fwd["cf_act"], bwd["dact"])
    dxc, dgam, dbet = OB.group_norm_backward(grid(fwd["xc"]), s.gn_groups, w["gn_gamma"], grid(da0))
    p["dxc"], p["gn_gamma"], p["gn_beta"] = (bwd["dxc"], tok(dxc)), (got["gn_gamma"], dgam), (got["gn_beta"], dbet)
    # the 3x3 conv with the GPU's dxc; dx adds the GPU's other input-gradient terms
    dxcv, p_w1, p_b1 = OB.conv3x3_backward(grid(x), w["w_cf1"], grid(bwd["dxc"]))
    p["x"], p["w_cf1"], p["b_cf1"] = (got["x"], tok(dxcv) + bwd["dxkv"]), (got["w_cf1"], p_w1), (got["b_cf1"], p_b1)
    return p
