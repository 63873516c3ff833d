"""GPU parity of the layer backward (edit_attn_backward) against the
float64 oracle backward, through the C ABI.

A forward fills the workspace, the backward reads it; outputs and scratch are
NaN-filled first. Two comparisons per case:

- step by step (tests/_bwd_steps.py): every chain-rule step of the backward
  -- the output Linear, the linear-attention apply, the per-head sums, the
  depthwise convs, the key/value Linears, the query Linear and the 1x1
  restore, LeakyReLU + GroupNorm, the 3x3 conv -- is the oracle's step
  function fed the inputs that step had on the GPU (the forward tensors in
  the forward workspace, the upstream gradient the previous GPU step left in
  the backward workspace). Every intermediate gradient, dx and all 18
  parameter gradients are gated max-relative, max |g - o| / max |o| <= 1e-4
  (fp32) and <= 2e-2 (bf16). Fed the GPU's own inputs, no step inherits
  another's rounding, and both sides take the same kink decisions (R28);
- end to end: dx and the parameter gradients against the oracle's own
  float64 forward and backward, normwise ||g - o|| / ||o|| <= 1e-3 (fp32) and
  <= 1e-1 (bf16) (R29). In bf16 a pre-activation within rounding of zero can
  take the other side of its kink, and the key gradients cancel ~25-fold
  (dK' = V' dS^T + dz), so the bf16 forward's rounding alone moves some
  gradients by a few percent there.
"""
import numpy as np
import pytest
import torch

from oracle import edit_backward as OB
from seeded_inputs import CONFIGS, make_inputs, make_shape
from seeded_inputs import round_to_bf16
from tests._metrics import BF16_TOL, F32_TOL, max_rel_err, norm_rel_err
from tests import _bwd_steps as BS

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
    """GPU forward + backward; returns the gradients, the forward tensors the
    GPU stored and the backward's intermediate gradients."""
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
    T = G.TORCH_DTYPE[s.dtype]
    return out, BS.read_forward(lca, s, fws, torch, T), BS.read_backward(lca, s, ws, torch, T)


END_TO_END_NORMWISE = {"f32": 1e-3, "bf16": 1e-1}


def check_backward(s, seed=0):
    inp = make_inputs(s, seed=seed, gn_affine_random=True)
    rng = np.random.default_rng(500 + seed)
    dout = rng.standard_normal((s.B, s.N, s.C)).astype(np.float32)
    if s.dtype == "bf16":
        dout = round_to_bf16(dout)
    print(f"\n[gpu-case] backward {s} seed={seed}", flush=True)
    got, fwd, bwd = run_backward(s, inp, dout)
    tol = F32_TOL if s.dtype == "f32" else BF16_TOL
    bad = {}
    step = {}
    for k, (g, r) in BS.step_pairs(s, inp["x"], inp["w"], dout, fwd, bwd, got).items():
        assert g.shape == r.shape, (k, g.shape, r.shape)
        assert np.isfinite(g).all(), f"{k}: non-finite elements (unwritten or overflow)"
        step[k] = max_rel_err(g, r)
        if not step[k] <= tol:
            bad[k] = ("step max-rel", step[k])
    dx0, grads0 = OB.edit_attn_backward(inp["x"], inp["w"], s, dout)
    e2e = {}
    for k, r in {"x": dx0, **grads0}.items():
        e2e[k] = norm_rel_err(got[k], r)
        if not e2e[k] <= END_TO_END_NORMWISE[s.dtype]:
            bad[k] = ("end-to-end normwise", e2e[k])
    print("step max-rel:", {k: f"{v:.2e}" for k, v in step.items()}, flush=True)
    print("end-to-end normwise:", {k: f"{v:.2e}" for k, v in e2e.items()}, flush=True)
    assert not bad, f"over tolerance: {bad}"
    return step, e2e


@pytest.mark.parametrize("name", list(SHAPES))
def test_backward_small(name):
    check_backward(SHAPES[name], seed=1)


def test_backward_deterministic():
    s = SHAPES["bf16_ragged_c384"]
    inp = make_inputs(s, seed=4)
    dout = np.random.default_rng(4).standard_normal((s.B, s.N, s.C)).astype(np.float32)
    a = run_backward(s, inp, dout)[0]
    b = run_backward(s, inp, dout)[0]
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_backward_f32_pixart1024_shape():
    check_backward(F32_PIXART1024)


def test_backward_pixart1024():
    check_backward(CONFIGS["pixart1024"])
