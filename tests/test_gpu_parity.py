"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Every intermediate the workspace layout names (xc, GN statistics, cf_act, the folded query weights, q,
kv0, kc, vc, S, z, y) and the output are compared element by element with
the float64 oracle on the same seeded inputs: max |g - o| / max |o| per
tensor <= 2e-2 for bf16, <= 1e-4 for fp32. Outputs and workspace are filled
with NaN bytes first, so an element a kernel fails to write shows up.
"""
import numpy as np
import pytest
import torch

from oracle import edit_oracle as O
from seeded_inputs import CONFIGS, make_inputs, make_shape
from tests._metrics import BF16_TOL, F32_TOL, centred_rel_err, max_rel_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import _gpu as G


def _tol(s):
    return BF16_TOL if s.dtype == "bf16" else F32_TOL


def _announce(tag):
    print(f"\n[gpu-case] {tag}", flush=True)


def check_edit(s, seed=0, gn_affine_random=False, x_std=None, centred=("q", "kc", "vc")):
    inp = make_inputs(s, seed=seed, gn_affine_random=gn_affine_random, x_std=x_std)
    _announce(f"edit {s} seed={seed}")
    got = G.run_edit(s, inp)
    tr = {}
    O.edit_attn_forward(inp["x"], inp["w"], s, tr)
    ref = G.oracle_views(tr, s)
    ref["y"] = tr["y"]
    ref["q_fold_w"], ref["q_fold_b"] = G.restore_fold(inp["w"]["w_q"], inp["w"]["b_q"], inp["w"]["w_cf2"],
                                                      inp["w"]["b_cf2"])
    tol = _tol(s)
    errs = {}
    for k, r in ref.items():
        g = got[k]
        assert np.isfinite(g).all(), f"{k}: non-finite elements (unwritten or overflow)"
        errs[k] = max_rel_err(g, r)
    for k in centred:
        errs[k + "_centred"] = centred_rel_err(got[k], ref[k])
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"over tolerance {tol}: {bad}"
    return got, tr


SMALL = {
    "f32_d32_ragged": make_shape(B=2, H=13, W=11, C=128, heads=4, head_dim=32, reduction=4, gn_groups=4,
                                 dtype="f32", x_std=1.0),
    "bf16_d64_ragged": make_shape(B=2, H=13, W=11, C=256, heads=4, head_dim=64, reduction=4, gn_groups=8,
                                  dtype="bf16", x_std=1.0),
    "bf16_d72_ragged": make_shape(B=1, H=21, W=19, C=288, heads=4, head_dim=72, reduction=4, gn_groups=8,
                                  dtype="bf16", x_std=1.0),
    "f32_d72": make_shape(B=1, H=9, W=14, C=288, heads=4, head_dim=72, reduction=4, gn_groups=4,
                          dtype="f32", x_std=1.0),
    "bf16_d8": make_shape(B=1, H=10, W=10, C=64, heads=8, head_dim=8, reduction=4, gn_groups=2,
                          dtype="bf16", x_std=1.0),
    "bf16_d128": make_shape(B=1, H=12, W=16, C=256, heads=2, head_dim=128, reduction=4, gn_groups=8,
                            dtype="bf16", x_std=1.0),
    # bf16 shapes whose GEMMs take the direct-to-LDS kernel at ragged token
    # counts: 256 x 96 conv tiles (C/r = 96) with 6 K steps per projection,
    # and 256 x 128 conv tiles (C/r = 128) with 72 conv K steps.
    "bf16_d96_conv96": make_shape(B=2, H=13, W=11, C=384, heads=4, head_dim=96, reduction=4, gn_groups=8,
                                  dtype="bf16", x_std=1.0),
    "bf16_d128_conv128": make_shape(B=1, H=9, W=7, C=512, heads=4, head_dim=128, reduction=4, gn_groups=8,
                                    dtype="bf16", x_std=1.0),
    # Token counts per sample that are multiples of 128, so the GroupNorm
    # restore also runs on the direct-to-LDS kernel: K = C/r = 96 (one and a
    # half K steps) and K = 288 (four and a half, the PixArt width).
    "bf16_gnrestore_k96": make_shape(B=2, H=16, W=8, C=384, heads=4, head_dim=96, reduction=4, gn_groups=8,
                                     dtype="bf16", x_std=1.0),
    "bf16_gnrestore_k288": make_shape(B=1, H=16, W=16, C=1152, heads=16, head_dim=72, reduction=4, gn_groups=32,
                                      dtype="bf16", x_std=1.0),
    # the halo-staged conv: 256-pixel tiles of whole rows (W = 32: eight rows, W = 64: four), two
    # samples, C/r = 96 (one column tile) and 288 (three)
    "bf16_halo_w32": make_shape(B=2, H=8, W=32, C=384, heads=4, head_dim=96, reduction=4, gn_groups=8,
                                dtype="bf16", x_std=1.0),
    "bf16_halo_w64_c1152": make_shape(B=2, H=4, W=64, C=1152, heads=16, head_dim=72, reduction=4, gn_groups=32,
                                      dtype="bf16", x_std=1.0),
    # the bf16 depthwise + state kernel's chunks are tiles of the compressed grid: 16 x 16 (19 x 21 compressed:
    # 2 x 2 chunks, three of them partial), one compressed row (64 x 4 and 1 x 256 tiles), one compressed
    # column (128 x 2 tiles)
    "bf16_tiles_19x21": make_shape(B=2, H=38, W=42, C=128, heads=2, head_dim=64, reduction=4, gn_groups=4,
                                   dtype="bf16", x_std=1.0),
    "bf16_1x5": make_shape(B=1, H=1, W=5, C=64, heads=2, head_dim=32, reduction=4, gn_groups=2,
                           dtype="bf16", x_std=1.0),
    "bf16_2x600": make_shape(B=1, H=2, W=600, C=64, heads=2, head_dim=32, reduction=4, gn_groups=2,
                             dtype="bf16", x_std=1.0),
    "bf16_600x2": make_shape(B=1, H=600, W=2, C=64, heads=2, head_dim=32, reduction=4, gn_groups=2,
                             dtype="bf16", x_std=1.0),
    "f32_1x1": make_shape(B=2, H=1, W=1, C=64, heads=2, head_dim=32, reduction=4, gn_groups=2,
                          dtype="f32", x_std=1.0),
    "f32_1x5": make_shape(B=1, H=1, W=5, C=64, heads=2, head_dim=32, reduction=4, gn_groups=2,
                          dtype="f32", x_std=1.0),
}


def test_tiny_config_f32():
    check_edit(CONFIGS["tiny"])


@pytest.mark.parametrize("name", list(SMALL))
def test_small_shapes(name):
    check_edit(SMALL[name], seed=1, gn_affine_random=True)


@pytest.mark.parametrize("name", ["pixart1024", "pixart2048", "pixart4096", "pixart8192"])
def test_pixart_full_size(name):
    check_edit(CONFIGS[name])


def test_pixart1024_shape_f32():
    """fp32 mode at the PixArt-1024 layer shape (2 x 64x64 tokens, C = 1152,
    16 heads x 72): every intermediate and the output within 1e-4."""
    s = make_shape(B=2, H=64, W=64, C=1152, heads=16, head_dim=72, reduction=4, gn_groups=32, dtype="f32",
                   x_std=1.0)
    check_edit(s, seed=0)


def check_hybrid(s, n_text, seed=0, exact=False):
    inp = make_inputs(s, seed=seed, n_text=n_text)
    _announce(f"hybrid {s} n_text={n_text} seed={seed} exact_eta={exact}")
    got = G.run_hybrid(s, inp, n_text, exact=exact)
    tr = {}
    out_i, out_t = O.mmedit_hybrid_forward(inp["x"], inp.get("x_txt"), inp["w"], inp.get("w_txt"), s, tr,
                                           eta="exact" if exact else "ratio")
    tol = _tol(s)
    pairs = {"out": (got["out"], out_i), "q": (got["q"], tr["q"]), "kc": (got["kc"], tr["kc"]),
             "vc": (got["vc"], tr["vc"])}
    # bf16 with head_dim <= 64 and the text keys in one split of 384: the image rows' softmax kernel forms the
    # linear part itself and y_lin is never written (y_img and out carry it); otherwise it is compared
    fused = s.dtype == "bf16" and s.head_dim <= 64 and 0 < n_text <= 384
    if not fused:
        pairs["y_lin"] = (got["y"], tr["y_lin"])
    if n_text:
        pairs.update({"out_txt": (got["out_txt"], out_t), "y_img": (got["y_img"], tr["y"]),
                      "y_txt": (got["y_txt"], tr["y_txt"]),
                      "qkv_t": (got["qkv_t"], np.concatenate([tr["q_t"], tr["k_t"], tr["v_t"]], -1))})
        if exact:
            pairs["lin_den"] = (got["lin_den"], tr["lin_den"])
    errs = {}
    for k, (g, r) in pairs.items():
        assert np.isfinite(g).all(), f"{k}: non-finite elements"
        errs[k] = max_rel_err(g, r)
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"over tolerance {tol}: {bad}"
    return got


HYB = {
    "f32_small": make_shape(B=2, H=9, W=7, C=128, heads=2, head_dim=64, reduction=4, gn_groups=4, dtype="f32",
                            x_std=1.0),
    "bf16_small": make_shape(B=2, H=12, W=10, C=192, heads=3, head_dim=64, reduction=4, gn_groups=4, dtype="bf16",
                             x_std=1.0),
    "bf16_d72": make_shape(B=1, H=8, W=8, C=288, heads=4, head_dim=72, reduction=4, gn_groups=4, dtype="bf16",
                           x_std=1.0),
    # narrower heads: the softmax blocks' two-query-tile waves at 2 and 3 head-dim steps of 16
    "bf16_d32": make_shape(B=2, H=10, W=12, C=128, heads=4, head_dim=32, reduction=4, gn_groups=4, dtype="bf16",
                           x_std=1.0),
    "bf16_d48": make_shape(B=1, H=16, W=14, C=192, heads=4, head_dim=48, reduction=4, gn_groups=4, dtype="bf16",
                           x_std=1.0),
    # enough keys that the softmax blocks split them (bf16: splits of 384 keys, so 300 text keys give the
    # text rows two splits over 256 + 300 keys, and 500 text keys split the image rows as well, both
    # problems writing partials in the one launch; fp32: the one-pass kernel's splits)
    "bf16_many_keys": make_shape(B=1, H=32, W=32, C=256, heads=4, head_dim=64, reduction=4, gn_groups=4,
                                 dtype="bf16", x_std=1.0),
    "f32_many_keys": make_shape(B=1, H=32, W=32, C=128, heads=2, head_dim=64, reduction=4, gn_groups=4,
                                dtype="f32", x_std=1.0),
    # a wider fp32 hybrid: 4096 image tokens, 16 heads
    "f32_many_queries": make_shape(B=1, H=64, W=64, C=1024, heads=16, head_dim=64, reduction=4, gn_groups=8,
                                   dtype="f32", x_std=1.0),
}


@pytest.mark.parametrize("name,n_text", [("f32_small", 37), ("bf16_small", 77), ("bf16_d72", 5), ("f32_small", 1),
                                         ("bf16_many_keys", 300), ("bf16_many_keys", 500), ("bf16_d72", 420),
                                         ("bf16_d32", 45), ("bf16_d48", 100), ("bf16_d48", 450),
                                         ("f32_many_keys", 300), ("f32_many_queries", 40)])
def test_hybrid_small(name, n_text):
    check_hybrid(HYB[name], n_text, seed=2)


def test_hybrid_sd35m_full_size():
    s = CONFIGS["sd35m_hybrid"]
    check_hybrid(s, s.n_text)


@pytest.mark.parametrize("name,n_text", [("f32_small", 37), ("bf16_small", 77), ("bf16_d72", 5),
                                         ("bf16_many_keys", 300), ("bf16_many_keys", 500), ("bf16_d72", 420),
                                         ("bf16_d32", 45), ("f32_many_keys", 300)])
def test_hybrid_exact_eta_small(name, n_text):
    check_hybrid(HYB[name], n_text, seed=6, exact=True)


def test_hybrid_exact_eta_sd35m_full_size():
    s = CONFIGS["sd35m_hybrid"]
    check_hybrid(s, s.n_text, exact=True)


@pytest.mark.parametrize("name", ["f32_small", "bf16_small"])
def test_hybrid_exact_eta_without_text_equals_edit(name):
    s = HYB[name]
    inp = make_inputs(s, seed=3)
    _announce(f"exact-eta hybrid n_text=0 vs edit {name}")
    a = G.run_hybrid(s, inp, 0, with_intermediates=False, exact=True)["out"]
    b = G.run_edit(s, inp, with_intermediates=False)["out"]
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("name", ["f32_small", "bf16_small"])
def test_hybrid_without_text_equals_edit(name):
    s = HYB[name]
    inp = make_inputs(s, seed=3)
    _announce(f"hybrid n_text=0 vs edit {name}")
    a = G.run_hybrid(s, inp, 0, with_intermediates=False)["out"]
    b = G.run_edit(s, inp, with_intermediates=False)["out"]
    np.testing.assert_array_equal(a, b)


def test_bitwise_deterministic():
    s = SMALL["bf16_d72_ragged"]
    inp = make_inputs(s, seed=4)
    _announce("determinism")
    a = G.run_edit(s, inp)
    b = G.run_edit(s, inp)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_timed_forward_matches_forward():
    import ctypes
    import linear_compressed_attention_amd as lca
    s = SMALL["bf16_d64_ragged"]
    inp = make_inputs(s, seed=5)
    _announce("timed forward")
    ref = G.run_edit(s, inp, with_intermediates=False)["out"]
    hip = ctypes.CDLL("libamdhip64.so.7")
    evs = []
    for _ in range(lca.EDIT_NUM_STEPS + 1):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    x = G.to_dev(inp["x"], s.dtype)
    w = G.dev_weights(inp["w"], s.dtype)
    y = torch.empty_like(x)
    ws = torch.empty(lca.edit_attn_workspace_size(s), dtype=torch.uint8, device="cuda")
    lca.edit_attn_forward_timed(s, w, x, y, ws, (ctypes.c_void_p * len(evs))(*evs))
    torch.cuda.synchronize()
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    for i in range(lca.EDIT_NUM_STEPS):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[i], evs[i + 1]) == 0
        assert ms.value >= 0.0
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))
    np.testing.assert_array_equal(y.float().cpu().numpy(), ref)


# ---------------------------------------------------------------------------
# Ablation variants of the query / key-value processing
# ---------------------------------------------------------------------------

VARIANTS = [("convfusion", "key_convfusion"), ("linear", "compressed"), ("convfusion", "full"),
            ("linear", "full"), ("linear", "key_convfusion")]


def check_variant(s, query, kv, seed=0):
    inp = make_inputs(s, seed=seed, gn_affine_random=True, key_convfusion=(kv == "key_convfusion"))
    _announce(f"variant ({query}, {kv}) {s} seed={seed}")
    got = G.run_variant(s, inp, query, kv)
    tr = {}
    out = O.edit_attn_variant_forward(inp["x"], inp["w"], s, query, kv, inp.get("w_kcf"), trace=tr)
    ref = {"out": out, "q": tr["q"], "S": tr["S"], "z": tr["z"], "y": tr["y"]}
    if kv == "compressed":
        ref.update(kc=tr["kc"], vc=tr["vc"])
    else:
        ref.update(k=tr["k"], v=tr["v"])
    if kv == "key_convfusion":
        ref["cf_act_k"] = tr["cf_act_k"]
        ref["k_fold_w"], ref["k_fold_b"] = G.restore_fold(inp["w"]["w_k"], inp["w"]["b_k"], inp["w_kcf"]["w_cf2"],
                                                          inp["w_kcf"]["b_cf2"])
    if query == "convfusion":
        ref["cf_act"] = tr["cf_act"]
        ref["q_fold_w"], ref["q_fold_b"] = G.restore_fold(inp["w"]["w_q"], inp["w"]["b_q"], inp["w"]["w_cf2"],
                                                          inp["w"]["b_cf2"])
    tol = _tol(s)
    errs = {}
    for k, r in ref.items():
        assert np.isfinite(got[k]).all(), f"{k}: non-finite elements"
        errs[k] = max_rel_err(got[k], r)
    for k in ("q", "k", "kc"):
        if k in ref:
            errs[k + "_centred"] = centred_rel_err(got[k], ref[k])
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"over tolerance {tol}: {bad}"


@pytest.mark.parametrize("query,kv", VARIANTS)
@pytest.mark.parametrize("name", ["f32_d32_ragged", "bf16_d96_conv96"])
def test_variants_small(name, query, kv):
    check_variant(SMALL[name], query, kv, seed=8)


@pytest.mark.parametrize("query,kv", [("convfusion", "key_convfusion"), ("linear", "compressed"),
                                      ("convfusion", "full")])
def test_variants_pixart1024(query, kv):
    check_variant(CONFIGS["pixart1024"], query, kv)


def test_variant_main_row_equals_layer():
    s = SMALL["bf16_d64_ragged"]
    inp = make_inputs(s, seed=9)
    _announce("variant (convfusion, compressed) vs edit")
    a = G.run_variant(s, inp, "convfusion", "compressed")["out"]
    b = G.run_edit(s, inp, with_intermediates=False)["out"]
    np.testing.assert_array_equal(a, b)
