"""Host-side checks of the C ABI (CPU only, no kernel runs): the library
loads, exports every function include/edit_attn.h declares, sizes its
workspace, and rejects bad arguments before touching a device."""
import ctypes
import subprocess

import pytest
import torch

import linear_compressed_attention_amd as lca
from seeded_inputs import CONFIGS, make_shape


def test_exports_every_header_symbol():
    names = lca.header_symbols()
    assert {"edit_attn_forward", "mmedit_hybrid_forward", "mmedit_hybrid_exact_forward", "edit_attn_workspace_size",
            "mmedit_hybrid_workspace_size", "edit_attn_workspace_layout", "edit_status_string",
            "edit_last_error"} <= set(names)
    lib = ctypes.CDLL(lca.lib_path())
    for n in names:
        assert hasattr(lib, n), n
    dyn = subprocess.run(["nm", "-D", "--defined-only", lca.lib_path()], capture_output=True, text=True).stdout
    for n in names:
        assert f" T {n}\n" in dyn, n


def test_library_has_gfx950_code_object():
    sec = subprocess.run(["objdump", "-h", lca.lib_path()], capture_output=True, text=True).stdout
    assert ".hip_fatbin" in sec
    with open(lca.lib_path(), "rb") as f:
        assert b"amdgcn-amd-amdhsa--gfx950" in f.read()


@pytest.mark.parametrize("name", list(CONFIGS))
def test_workspace_size_and_layout(name):
    s = CONFIGS[name]
    n = lca.mmedit_hybrid_workspace_size(s, s.n_text)
    lay = lca.edit_attn_workspace_layout(s, s.n_text)
    assert lay["total"] == n
    es = 2 if s.dtype == "bf16" else 4
    assert lay["y"] + s.B * s.N * s.C * es <= n
    offs = sorted(v for k, v in lay.items() if k != "total" and v)
    assert all(o % 256 == 0 for o in offs)
    if s.n_text == 0:
        assert lca.edit_attn_workspace_size(s) == n


BAD = [
    dict(C=60),                     # C != heads * head_dim
    dict(reduction=5),              # r does not divide C
    dict(gn_groups=5),              # G does not divide C/r
    dict(B=0), dict(H=-1), dict(heads=0),
]


@pytest.mark.parametrize("delta", BAD)
def test_bad_shapes_rejected(delta):
    base = dict(B=1, H=8, W=8, C=64, heads=2, head_dim=32, reduction=4, gn_groups=4, eps=1e-6, dtype="bf16")
    base.update(delta)
    with pytest.raises(lca.EditError) as e:
        lca.edit_attn_workspace_size(base)
    assert e.value.status == 1


def test_unsupported_shapes():
    base = dict(B=1, H=8, W=8, C=160, heads=1, head_dim=160, reduction=4, gn_groups=4, eps=1e-6, dtype="bf16")
    with pytest.raises(lca.EditError) as e:
        lca.edit_attn_workspace_size(base)
    assert e.value.status == 2 and "head_dim" in e.value.detail
    base = dict(B=1, H=8, W=8, C=36, heads=3, head_dim=12, reduction=4, gn_groups=3, eps=1e-6, dtype="bf16")
    with pytest.raises(lca.EditError) as e:
        lca.edit_attn_workspace_size(base)
    assert e.value.status == 2


def _fake_weights(base=0x100000):
    return {n: base + 0x1000 * i for i, n in enumerate(lca.IMAGE_WEIGHT_FIELDS)}


class _FakeWS:
    """A pointer/size pair standing in for a workspace tensor (never dereferenced)."""
    def __init__(self, ptr, n):
        self.ptr, self.n = ptr, n

    def data_ptr(self):
        return self.ptr

    def numel(self):
        return self.n

    def element_size(self):
        return 1


SHAPE = make_shape(B=1, H=8, W=8, C=64, heads=2, head_dim=32, reduction=4, gn_groups=4, dtype="bf16")


def _call(w=None, x=0x9000000, y=0xA000000, ws=None):
    ws = ws or _FakeWS(0xB000000, lca.edit_attn_workspace_size(SHAPE))
    lca.edit_attn_forward(SHAPE, w or _fake_weights(), x, y, ws, stream=0)


def test_argument_errors_before_any_launch():
    w = _fake_weights(); w["w_q"] = None
    with pytest.raises(lca.EditError) as e:
        _call(w=w)
    assert e.value.status == 1 and "w_q" in e.value.detail
    w = _fake_weights(); w["b_o"] += 8
    with pytest.raises(lca.EditError) as e:
        _call(w=w)
    assert e.value.status == 1 and "aligned" in e.value.detail
    with pytest.raises(lca.EditError) as e:
        _call(x=0)
    assert e.value.status == 1
    with pytest.raises(lca.EditError) as e:
        _call(ws=_FakeWS(0xB000000, 100))
    assert e.value.status == 3
    with pytest.raises(lca.EditError) as e:
        _call(ws=_FakeWS(0xB000010, 1 << 30))
    assert e.value.status == 1 and "256" in e.value.detail
    with pytest.raises(lca.EditError) as e:
        _call(y=0x9000000 + 64)
    assert e.value.status == 1 and "overlap" in e.value.detail


@pytest.mark.parametrize("fwd", ["mmedit_hybrid_forward", "mmedit_hybrid_exact_forward"])
def test_hybrid_argument_errors(fwd):
    f = getattr(lca, fwd)
    ws = _FakeWS(0xB000000, lca.mmedit_hybrid_workspace_size(SHAPE, 5))
    with pytest.raises(lca.EditError) as e:
        f(SHAPE, -1, _fake_weights(), None, 0x9000000, None, 0xA000000, None, ws, stream=0)
    assert e.value.status == 1
    with pytest.raises(lca.EditError) as e:
        f(SHAPE, 5, _fake_weights(), None, 0x9000000, 0x9800000, 0xA000000, 0xA800000, ws, stream=0)
    assert e.value.status == 1 and "text weights" in e.value.detail
    small = _FakeWS(0xB000000, lca.mmedit_hybrid_workspace_size(SHAPE, 5) - 256)
    with pytest.raises(lca.EditError) as e:
        f(SHAPE, 5, _fake_weights(), {n: 0x200000 + 0x1000 * i for i, n in enumerate(lca.TEXT_WEIGHT_FIELDS)},
          0x9000000, 0x9800000, 0xA000000, 0xA800000, small, stream=0)
    assert e.value.status == 3


def test_exact_eta_layout_has_the_normaliser():
    lay = lca.edit_attn_workspace_layout(SHAPE, 5)
    assert lay["lin_den"] > 0 and lay["lin_den"] % 256 == 0
    assert lca.edit_attn_workspace_layout(SHAPE, 0)["lin_den"] == 0


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device path")
def test_no_device_is_reported():
    with pytest.raises(lca.EditError) as e:
        _call()
    assert e.value.status == 4


def test_status_strings():
    assert lca.edit_status_string(0) == "EDIT_OK"
    assert "WORKSPACE" in lca.edit_status_string(3)


@pytest.mark.parametrize("query,kv", [("convfusion", "compressed"), ("convfusion", "full"),
                                      ("convfusion", "key_convfusion"), ("linear", "compressed"),
                                      ("linear", "full")])
def test_variant_layouts(query, kv):
    s = CONFIGS["pixart1024"]
    lay = lca.edit_attn_variant_workspace_layout(s, query, kv)
    assert lay["total"] == lca.edit_attn_variant_workspace_size(s, query, kv)
    assert (lay["q_fold_w"] > 0) == (query == "convfusion")
    assert (lay["kc"] > 0) == (kv == "compressed")
    assert (lay["k_fold_w"] > 0) == (kv == "key_convfusion")
    assert all(v % 256 == 0 for v in lay.values())
    if (query, kv) == ("convfusion", "compressed"):
        assert lay == lca.edit_attn_workspace_layout(s, 0)


def test_variant_argument_errors():
    ws = _FakeWS(0xB000000, lca.edit_attn_variant_workspace_size(SHAPE, "convfusion", "key_convfusion"))
    with pytest.raises(lca.EditError) as e:
        lca.edit_attn_variant_forward(SHAPE, 7, "compressed", _fake_weights(), None, 0x9000000, 0xA000000, ws,
                                      stream=0)
    assert e.value.status == 1 and "query mode" in e.value.detail
    with pytest.raises(lca.EditError) as e:
        lca.edit_attn_variant_forward(SHAPE, "convfusion", 5, _fake_weights(), None, 0x9000000, 0xA000000, ws,
                                      stream=0)
    assert e.value.status == 1 and "key/value mode" in e.value.detail
    with pytest.raises(lca.EditError) as e:
        lca.edit_attn_variant_forward(SHAPE, "convfusion", "key_convfusion", _fake_weights(), None, 0x9000000,
                                      0xA000000, ws, stream=0)
    assert e.value.status == 1 and "key ConvFusion" in e.value.detail
    w = _fake_weights()
    w["w_cf1"] = None
    with pytest.raises(lca.EditError) as e:
        lca.edit_attn_variant_forward(SHAPE, "convfusion", "full", w, None, 0x9000000, 0xA000000, ws, stream=0)
    assert e.value.status == 1 and "w_cf1" in e.value.detail


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device path")
def test_variant_unread_weights_may_be_null():
    """A plain query reads no ConvFusion parameters and uncompressed keys no
    depthwise ones: the arguments pass, and only the missing device is reported."""
    w = {n: p for n, p in _fake_weights().items()
         if n not in ("w_cf1", "b_cf1", "gn_gamma", "gn_beta", "w_cf2", "b_cf2", "dw_k", "db_k", "dw_v", "db_v")}
    ws = _FakeWS(0xB000000, lca.edit_attn_variant_workspace_size(SHAPE, "linear", "full"))
    with pytest.raises(lca.EditError) as e:
        lca.edit_attn_variant_forward(SHAPE, "linear", "full", w, None, 0x9000000, 0xA000000, ws, stream=0)
    assert e.value.status == 4


def _fake_grads(base=0x3000000):
    return {n: base + 0x10000 * i for i, n in enumerate(lca.IMAGE_WEIGHT_FIELDS)}


def _bwd_call(grads=None, w=None, x=0x9000000, dy=0x9800000, dx=0xA000000):
    fws = _FakeWS(0xB000000, lca.edit_attn_workspace_size(SHAPE))
    ws = _FakeWS(0xC000000, lca.edit_attn_backward_workspace_size(SHAPE))
    lca.edit_attn_backward(SHAPE, w or _fake_weights(), x, dy, fws, dx, grads or _fake_grads(), ws, stream=0)


@pytest.mark.parametrize("case", ["x", "dy", "dx", "weight", "fwd_ws", "ws", "other_grad", "dx_weight"])
def test_backward_gradient_overlaps_rejected(case):
    """Each gradient is an output sized from the shape (w_cf1: C/r x 9 x C, a Linear: C x C, ...): one that
    overlaps an input, another output or a workspace is rejected before anything is launched."""
    g = _fake_grads()
    kw = {}
    if case == "x":
        g["w_q"] = 0x9000000 + 0x100
    elif case == "dy":
        g["b_k"] = 0x9800000
    elif case == "dx":
        g["dw_v"] = 0xA000000 + 0x400
    elif case == "weight":
        g["w_cf1"] = _fake_weights()["w_o"] + 0x10    # within w_o's C x C bf16 elements
    elif case == "fwd_ws":
        g["gn_beta"] = 0xB000000 + 0x200
    elif case == "ws":
        g["b_o"] = 0xC000000 + 0x2000
    elif case == "other_grad":
        g["b_q"] = g["w_q"] + 64 * 64 * 2 - 16      # the last 16 bytes of w_q's gradient
    elif case == "dx_weight":
        kw["dx"] = _fake_weights()["w_k"]
    with pytest.raises(lca.EditError) as e:
        _bwd_call(grads=g, **kw)
    assert e.value.status == 1 and "overlaps" in e.value.detail, e.value.detail


def test_backward_gradients_just_apart_pass_the_checks():
    """Gradients that only touch end to start are accepted (the missing device is what is reported here)."""
    g = _fake_grads()
    g["b_q"] = g["w_q"] + 64 * 64 * 2                # right after w_q's gradient
    if torch.cuda.device_count() > 0:
        pytest.skip("checks the argument path up to the no-device report")
    with pytest.raises(lca.EditError) as e:
        _bwd_call(grads=g)
    assert e.value.status == 4, e.value.detail


def test_forward_output_overlapping_a_weight_rejected():
    with pytest.raises(lca.EditError) as e:
        _call(y=_fake_weights()["w_q"])
    assert e.value.status == 1 and "weight" in e.value.detail


def test_noalloc_rejects_a_shape_beyond_the_static_scratch():
    """edit_attn_forward_noalloc checks the shape's workspace against its static scratch before it
    touches a device (65536 tokens at C = 1152 need ~760 MB)."""
    s = CONFIGS["pixart4096"]
    assert lca.edit_attn_workspace_size(s) > lca.EDIT_NOALLOC_SCRATCH_BYTES
    with pytest.raises(lca.EditError) as e:
        lca.edit_attn_forward_noalloc(s, _fake_weights(), 0x10000000000, 0x20000000000, stream=0)
    assert e.value.status == 3 and "static scratch" in e.value.detail


def test_noalloc_argument_errors_before_any_launch():
    w = _fake_weights()
    w["w_k"] = None
    with pytest.raises(lca.EditError) as e:
        lca.edit_attn_forward_noalloc(SHAPE, w, 0x9000000, 0xA000000, stream=0)
    assert e.value.status == 1 and "w_k" in e.value.detail
    with pytest.raises(lca.EditError) as e:
        lca.edit_attn_forward_noalloc(SHAPE, _fake_weights(), 0x9000000, 0x9000000 + 64, stream=0)
    assert e.value.status == 1 and "overlap" in e.value.detail


def test_noalloc_scratch_bound_matches_the_header():
    import os
    import re
    with open(os.path.join(os.path.dirname(os.path.dirname(lca.lib_path())), "include", "edit_attn.h")) as f:
        m = re.search(r"#define EDIT_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == lca.EDIT_NOALLOC_SCRATCH_BYTES
    # the 128 x 128, C = 1152 bf16 layer fits
    assert lca.edit_attn_workspace_size(CONFIGS["pixart2048"]) <= lca.EDIT_NOALLOC_SCRATCH_BYTES
