"""edit_attn_forward_noalloc (the forward for callers that cannot allocate)
against edit_attn_forward, through the C ABI.

Two calls in a row on the shared static scratch, the second with a smaller
input than the first, each compared with edit_attn_forward's output on the
same inputs (its own workspace): bit for bit (both run the same kernels in
the same order per step), and within the parity gate of the oracle."""
import numpy as np
import pytest
import torch

from oracle import edit_oracle as O
from seeded_inputs import CONFIGS, make_inputs, make_shape
from tests._metrics import BF16_TOL, F32_TOL, max_rel_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import linear_compressed_attention_amd as lca
    from tests import _gpu as G

CASES = [
    CONFIGS["pixart1024"],                                        # 2 x 64x64 tokens, C = 1152 (95 MB of scratch)
    make_shape(B=2, H=13, W=11, C=384, heads=4, head_dim=96, reduction=4, gn_groups=8, dtype="bf16", x_std=1.0),
    make_shape(B=1, H=9, W=14, C=288, heads=4, head_dim=72, reduction=4, gn_groups=4, dtype="f32", x_std=1.0),
]


def _both(s, seed):
    inp = make_inputs(s, seed=seed)
    x = G.to_dev(inp["x"], s.dtype)
    w = G.dev_weights(inp["w"], s.dtype)
    y_ref = torch.empty_like(x)
    ws = torch.empty(lca.edit_attn_workspace_size(s), dtype=torch.uint8, device="cuda")
    lca.edit_attn_forward(s, w, x, y_ref, ws)
    y = torch.empty_like(x)
    G.poison(y)
    lca.edit_attn_forward_noalloc(s, w, x, y)
    torch.cuda.synchronize()
    return inp, y.float().cpu().numpy(), y_ref.float().cpu().numpy()


def test_noalloc_calls_in_a_row_match_the_forward():
    for i, s in enumerate(CASES):
        assert lca.edit_attn_workspace_size(s) <= lca.EDIT_NOALLOC_SCRATCH_BYTES
        print(f"\n[gpu-case] noalloc call {i}: {s}", flush=True)
        inp, got, ref = _both(s, seed=i)
        assert np.isfinite(got).all()
        assert np.array_equal(got, ref), max_rel_err(got, ref)
        if s.N <= 512:
            tol = BF16_TOL if s.dtype == "bf16" else F32_TOL
            assert max_rel_err(got, O.edit_attn_forward(inp["x"], inp["w"], s)) <= tol
