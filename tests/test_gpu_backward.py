"""GPU parity of the layer backward (edit_attn_backward) against the
float64 oracle backward, through the C ABI.

A forward fills the workspace, the backward reads it; dx and all 18
parameter gradients are compared with oracle.edit_backward on the same
seeded inputs and upstream gradient. Outputs and scratch are NaN-filled
first.

The backward passes three kinks (the queries' ReLU, the keys' ReLU, the
LeakyReLU after GroupNorm). Where a pre-activation lies within the GPU
forward's rounding of zero, the GPU and a float64 forward can fall on
opposite sides, and that gradient element then moves by a whole upstream
value (about 2-6% normwise in bf16 for every gradient behind a kink). The
oracle therefore takes its kink decisions from the GPU's own stored forward
values (q > 0, K' > 0, act >= 0, read from the forward workspace): both sides
then differentiate the same branch, and every tensor is gated max-relative,
max |g - o| / max |o| <= 1e-4 (fp32) and <= 2e-2 (bf16). The normwise error
against the oracle's own decisions is printed beside it as a diagnostic.
"""
import numpy as np
import pytest
import torch

from oracle import edit_backward as OB
from seeded_inputs import CONFIGS, make_inputs, make_shape
from seeded_inputs import round_to_bf16
from tests._metrics import BF16_TOL, F32_TOL, max_rel_err, norm_rel_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import linear_compressed_attention_amd as lca
    from tests import _gpu as G


SHAPES = {
    "f32_ragged": make_shape(B=2, H=13, W=11, C=128, heads=4, head_dim=32, reduction=4, gn_groups=4,
                             dtype="f32", x_std=1.0),
    "f32_d72": make_shape(B=1, H=9, W=14, C=288, heads=4, head_dim=72, reduction=4, gn_groups=4,
                          dtype="f32", x_std=1.0),
    "bf16_ragged_c384": make_shape(B=2, H=13, W=11, C=384, heads=4, head_dim=96, reduction=4, gn_groups=8,
                                   dtype="bf16", x_std=1.0),
    "bf16_c1152": make_shape(B=1, H=16, W=16, C=1152, heads=16, head_dim=72, reduction=4, gn_groups=32,
                             dtype="bf16", x_std=1.0),
    # the per-head kernels' extremes: one 16-wide K step (d = 8) and eight (d = 128), and an even count (d = 64)
    "f32_d8": make_shape(B=1, H=10, W=9, C=64, heads=8, head_dim=8, reduction=4, gn_groups=2, dtype="f32",
                         x_std=1.0),
    "f32_d64": make_shape(B=2, H=7, W=10, C=192, heads=3, head_dim=64, reduction=4, gn_groups=4, dtype="f32",
                          x_std=1.0),
    "f32_d128": make_shape(B=1, H=12, W=9, C=256, heads=2, head_dim=128, reduction=4, gn_groups=8, dtype="f32",
                           x_std=1.0),
    "bf16_d128": make_shape(B=1, H=12, W=10, C=256, heads=2, head_dim=128, reduction=4, gn_groups=8,
                            dtype="bf16", x_std=1.0),
}
F32_PIXART1024 = make_shape(B=2, H=64, W=64, C=1152, heads=16, head_dim=72, reduction=4, gn_groups=32,
                            dtype="f32", x_std=1.0)


def run_backward(s, inp, dout):
    """GPU forward + backward; returns the gradients and the kink decisions
    the GPU forward took (from its stored q, K' and act)."""
    x = G.to_dev(inp["x"], s.dtype)
    w = G.dev_weights(inp["w"], s.dtype)
    y = torch.empty_like(x)
    fws = torch.empty(lca.edit_attn_workspace_size(s), dtype=torch.uint8, device="cuda")
    G.poison(fws)
    lca.edit_attn_forward(s, w, x, y, fws)
    dy = G.to_dev(dout, s.dtype)
    dx = torch.empty_like(x)
    grads = {n: torch.empty_like(t) for n, t in w.items()}
    ws = torch.empty(lca.edit_attn_backward_workspace_size(s), dtype=torch.uint8, device="cuda")
    for t in [dx, ws] + list(grads.values()):
        G.poison(t)
    lca.edit_attn_backward(s, w, x, dy, fws, dx, grads, ws)
    torch.cuda.synchronize()
    out = {"x": dx.float().cpu().numpy()}
    out.update({n: t.float().cpu().numpy() for n, t in grads.items()})
    fwd = G.read_intermediates(s, fws)
    masks = {"q": fwd["q"] > 0, "kc": fwd["kc"] > 0, "act": fwd["cf_act"] >= 0}
    return out, masks


def check_backward(s, seed=0):
    inp = make_inputs(s, seed=seed, gn_affine_random=True)
    rng = np.random.default_rng(500 + seed)
    dout = rng.standard_normal((s.B, s.N, s.C)).astype(np.float32)
    if s.dtype == "bf16":
        dout = round_to_bf16(dout)
    print(f"\n[gpu-case] backward {s} seed={seed}", flush=True)
    got, masks = run_backward(s, inp, dout)
    dx, grads = OB.edit_attn_backward(inp["x"], inp["w"], s, dout, masks=masks)
    ref = {"x": dx, **grads}
    # diagnostic only: the oracle's own kink decisions
    tr = {}
    dx0, grads0 = OB.edit_attn_backward(inp["x"], inp["w"], s, dout, trace=tr)
    own = {"x": dx0, **grads0}
    f = tr["forward"]
    flips = {"q": int((masks["q"] != (f["q"] > 0)).sum()), "kc": int((masks["kc"] != (f["kc"] > 0)).sum()),
             "act": int((masks["act"] != (f["cf_act"] >= 0)).sum())}
    tol = F32_TOL if s.dtype == "f32" else BF16_TOL
    errs, bad = {}, {}
    for k, r in ref.items():
        g = got[k]
        assert g.shape == r.shape, (k, g.shape, r.shape)
        assert np.isfinite(g).all(), f"{k}: non-finite elements (unwritten or overflow)"
        e = max_rel_err(g, r)
        errs[k] = (e, norm_rel_err(g, own[k]))
        if not e <= tol:
            bad[k] = e
    print("kink decisions that differ from the float64 forward:", flips)
    print("max-rel (GPU kink decisions) / normwise (float64 decisions):",
          {k: f"{a:.2e}/{b:.2e}" for k, (a, b) in errs.items()}, flush=True)
    assert not bad, f"over tolerance {tol}: {bad}"
    return errs


@pytest.mark.parametrize("name", list(SHAPES))
def test_backward_small(name):
    check_backward(SHAPES[name], seed=1)


def test_backward_deterministic():
    s = SHAPES["bf16_ragged_c384"]
    inp = make_inputs(s, seed=4)
    dout = np.random.default_rng(4).standard_normal((s.B, s.N, s.C)).astype(np.float32)
    a, _ = run_backward(s, inp, dout)
    b, _ = run_backward(s, inp, dout)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_backward_f32_pixart1024_shape():
    check_backward(F32_PIXART1024)


def test_backward_pixart1024():
    check_backward(CONFIGS["pixart1024"])
