"""Helpers of the GPU parity tests: move seeded inputs to the device, call
the library through its binding, and read back outputs and the
intermediates the workspace layout names (test infrastructure)."""
import numpy as np
import torch

import linear_compressed_attention_amd as lca

TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(TORCH_DTYPE[dtype])


def dev_weights(w, dtype):
    return {k: to_dev(v, dtype) for k, v in w.items()}


def poison(t):
    """Fill with all-ones bytes (NaN in bf16 and f32) so unwritten elements show."""
    t.view(torch.uint8).fill_(0xFF)


def _view(ws, off, shape, dtype):
    n = int(np.prod(shape))
    es = torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + n * es].view(dtype).view(*shape)


def read_intermediates(shape, ws, n_text=0):
    lay = lca.edit_attn_workspace_layout(shape, n_text)
    s = shape
    T = TORCH_DTYPE[s.dtype]
    f32 = torch.float32
    B, N, C, h, d = s.B, s.N, s.C, s.heads, s.head_dim
    out = {
        "xc": _view(ws, lay["xc"], (B, N, s.Cr), T),
        "gn_stat": _view(ws, lay["gn_stat"], (B, s.gn_groups, 2), f32),
        "cf_act": _view(ws, lay["cf_act"], (B, N, s.Cr), T),
        "q_fold_w": _view(ws, lay["q_fold_w"], (C, C + s.Cr), T),
        "q_fold_b": _view(ws, lay["q_fold_b"], (C,), T),
        "q": _view(ws, lay["q"], (B, N, C), T),
        "kv0": _view(ws, lay["kv0"], (B, N, 2 * C), T),
        "kc": _view(ws, lay["kc"], (B, s.Nc, C), T),
        "vc": _view(ws, lay["vc"], (B, s.Nc, C), T),
        "S": _view(ws, lay["S"], (B, h, d, d), f32),
        "z": _view(ws, lay["z"], (B, h, d), f32),
        "y": _view(ws, lay["y"], (B, N, C), T),
    }
    if n_text:
        out["qkv_t"] = _view(ws, lay["qkv_t"], (B, n_text, 3 * C), T)
        out["y_img"] = _view(ws, lay["y_img"], (B, N, C), T)
        out["y_txt"] = _view(ws, lay["y_txt"], (B, n_text, C), T)
    return {k: v.float().cpu().numpy() for k, v in out.items()}


def run_edit(shape, inp, stream=None, with_intermediates=True):
    x = to_dev(inp["x"], shape.dtype)
    w = dev_weights(inp["w"], shape.dtype)
    y = torch.empty_like(x)
    ws = torch.empty(lca.edit_attn_workspace_size(shape), dtype=torch.uint8, device="cuda")
    poison(y)
    poison(ws)
    lca.edit_attn_forward(shape, w, x, y, ws, stream)
    torch.cuda.synchronize()
    res = {"out": y.float().cpu().numpy()}
    if with_intermediates:
        res.update(read_intermediates(shape, ws))
    return res


def run_hybrid(shape, inp, n_text, with_intermediates=True, exact=False):
    x = to_dev(inp["x"], shape.dtype)
    w = dev_weights(inp["w"], shape.dtype)
    xt = to_dev(inp["x_txt"], shape.dtype) if n_text else None
    wt = dev_weights(inp["w_txt"], shape.dtype) if n_text else None
    y = torch.empty_like(x)
    yt = torch.empty_like(xt) if n_text else None
    ws = torch.empty(lca.mmedit_hybrid_workspace_size(shape, n_text), dtype=torch.uint8, device="cuda")
    poison(y)
    poison(ws)
    if yt is not None:
        poison(yt)
    fwd = lca.mmedit_hybrid_exact_forward if exact else lca.mmedit_hybrid_forward
    fwd(shape, n_text, w, wt, x, xt, y, yt, ws)
    torch.cuda.synchronize()
    res = {"out": y.float().cpu().numpy()}
    if yt is not None:
        res["out_txt"] = yt.float().cpu().numpy()
    if with_intermediates:
        res.update(read_intermediates(shape, ws, n_text))
        if exact and n_text:
            lay = lca.edit_attn_workspace_layout(shape, n_text)
            res["lin_den"] = _view(ws, lay["lin_den"], (shape.B, shape.N, shape.heads),
                                   torch.float32).cpu().numpy()
    return res


def restore_fold(w_lin, b_lin, w_cf2, b_cf2):
    """[W | W W_cf2] and b + W b_cf2 in float64 from the weights (the 1x1
    restore folded into the Linear that reads x + Conv1x1(act))."""
    import numpy as np
    W, W2 = np.asarray(w_lin, np.float64), np.asarray(w_cf2, np.float64)
    return (np.concatenate([W, W @ W2], axis=1),
            np.asarray(b_lin, np.float64) + W @ np.asarray(b_cf2, np.float64))


def oracle_views(tr, shape):
    """The oracle trace in the shapes of read_intermediates."""
    import numpy as np
    rstd = 1.0 / np.sqrt(tr["gn_var"] + 1e-5)
    return {
        "xc": tr["xc"], "gn_stat": np.stack([tr["gn_mean"], rstd], axis=-1), "cf_act": tr["cf_act"],
        "q": tr["q"],
        "kv0": np.concatenate([tr["k0"], tr["v0"]], axis=-1), "kc": tr["kc"], "vc": tr["vc"],
        "S": tr["S"], "z": tr["z"], "out": tr["out"],
    }


def run_variant(shape, inp, query, kv):
    """edit_attn_variant_forward; returns the output and the variant's intermediates."""
    x = to_dev(inp["x"], shape.dtype)
    w = dev_weights(inp["w"], shape.dtype)
    if query == "linear":
        for n in ("w_cf1", "b_cf1", "gn_gamma", "gn_beta", "w_cf2", "b_cf2"):
            w.pop(n)
    if kv != "compressed":
        for n in ("dw_k", "db_k", "dw_v", "db_v"):
            w.pop(n)
    kcf = dev_weights(inp["w_kcf"], shape.dtype) if kv == "key_convfusion" else None
    y = torch.empty_like(x)
    ws = torch.empty(lca.edit_attn_variant_workspace_size(shape, query, kv), dtype=torch.uint8, device="cuda")
    poison(y)
    poison(ws)
    lca.edit_attn_variant_forward(shape, query, kv, w, kcf, x, y, ws)
    torch.cuda.synchronize()
    lay = lca.edit_attn_variant_workspace_layout(shape, query, kv)
    s = shape
    T, f32 = TORCH_DTYPE[s.dtype], torch.float32
    B, N, C, h, d = s.B, s.N, s.C, s.heads, s.head_dim
    got = {"out": y, "q": _view(ws, lay["q"], (B, N, C), T), "S": _view(ws, lay["S"], (B, h, d, d), f32),
           "z": _view(ws, lay["z"], (B, h, d), f32), "y": _view(ws, lay["y"], (B, N, C), T)}
    if kv == "compressed":
        got["kc"] = _view(ws, lay["kc"], (B, s.Nc, C), T)
        got["vc"] = _view(ws, lay["vc"], (B, s.Nc, C), T)
    else:
        kv0 = _view(ws, lay["kv0"], (B, N, 2 * C), T)
        got["k"], got["v"] = kv0[..., :C], kv0[..., C:]
    if kv == "key_convfusion":
        got["cf_act_k"] = _view(ws, lay["cf_act_k"], (B, N, s.Cr), T)
        got["k_fold_w"] = _view(ws, lay["k_fold_w"], (C, C + s.Cr), T)
        got["k_fold_b"] = _view(ws, lay["k_fold_b"], (C,), T)
    if query == "convfusion":
        got["cf_act"] = _view(ws, lay["cf_act"], (B, N, s.Cr), T)
        got["q_fold_w"] = _view(ws, lay["q_fold_w"], (C, C + s.Cr), T)
        got["q_fold_b"] = _view(ws, lay["q_fold_b"], (C,), T)
    return {k: v.float().cpu().numpy() for k, v in got.items()}
