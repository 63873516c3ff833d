"""Python binding of libedit_attn.so, the gfx950 EDiT linear compressed
attention layer and its MM-EDiT hybrid.

The functions carry the C ABI's names (include/edit_attn.h) and only marshal
arguments: torch tensors become device pointers, the current torch stream
becomes the hipStream_t. Every step of the layer runs in the library's HIP
kernels; there is no other code path. If the shared library is missing the
import of this package fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Mapping, Optional

__all__ = [
    "EDIT_F32", "EDIT_BF16", "EditError", "IMAGE_WEIGHT_FIELDS", "TEXT_WEIGHT_FIELDS", "LAYOUT_FIELDS",
    "edit_attn_workspace_size", "edit_attn_forward", "mmedit_hybrid_workspace_size",
    "mmedit_hybrid_forward", "mmedit_hybrid_exact_forward", "edit_attn_forward_timed", "edit_attn_workspace_layout", "EDIT_NUM_STEPS", "edit_status_string", "edit_last_error",
    "lib_path", "header_symbols", "QUERY_MODES", "KV_MODES", "KEY_CONVFUSION_FIELDS",
    "edit_attn_variant_workspace_size", "edit_attn_variant_workspace_layout", "edit_attn_variant_forward",
    "edit_attn_backward_workspace_size", "edit_attn_backward", "edit_attn_backward_workspace_layout",
    "BWD_LAYOUT_FIELDS", "edit_attn_forward_noalloc", "EDIT_NOALLOC_SCRATCH_BYTES",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_PKG)
_LIB_PATH = os.path.join(_PKG, "libedit_attn.so")

EDIT_F32, EDIT_BF16 = 0, 1
EDIT_NUM_STEPS = 9
_STATUS = {0: "EDIT_OK", 1: "EDIT_ERR_ARG", 2: "EDIT_ERR_UNSUPPORTED", 3: "EDIT_ERR_WORKSPACE", 4: "EDIT_ERR_HIP"}

IMAGE_WEIGHT_FIELDS = ("w_cf1", "b_cf1", "gn_gamma", "gn_beta", "w_cf2", "b_cf2", "w_q", "b_q", "w_k", "b_k",
                       "w_v", "b_v", "dw_k", "db_k", "dw_v", "db_v", "w_o", "b_o")
TEXT_WEIGHT_FIELDS = ("w_q", "b_q", "w_k", "b_k", "w_v", "b_v", "w_o", "b_o")
LAYOUT_FIELDS = ("xc", "gn_stat", "cf_act", "q_fold_w", "q_fold_b", "q", "kv0", "kc", "vc", "S", "z", "y", "qkv_t",
                 "y_img", "y_txt", "lin_den", "xc_k", "gn_stat_k", "cf_act_k", "k_fold_w", "k_fold_b", "total")
QUERY_MODES = {"convfusion": 0, "linear": 1}                      # edit_query_mode_t
KV_MODES = {"compressed": 0, "full": 1, "key_convfusion": 2}      # edit_kv_mode_t
KEY_CONVFUSION_FIELDS = ("w_cf1", "b_cf1", "gn_gamma", "gn_beta", "w_cf2", "b_cf2")


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "H", "W", "C", "heads", "head_dim", "reduction", "gn_groups")] + \
               [("eps", ctypes.c_float), ("dtype", ctypes.c_int)]


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in IMAGE_WEIGHT_FIELDS]


class _Grads(ctypes.Structure):          # edit_grads_t: one output per weight, same order
    _fields_ = [(n, ctypes.c_void_p) for n in IMAGE_WEIGHT_FIELDS]


class _TextWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in TEXT_WEIGHT_FIELDS]


class _Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in LAYOUT_FIELDS]


BWD_LAYOUT_FIELDS = ("dy", "dq_pre", "dS", "dz", "dkv", "dk0v0", "dxq", "dxkv", "dact", "dxc", "dxc_ld", "total")


class _BwdLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in BWD_LAYOUT_FIELDS]


class _Variant(ctypes.Structure):
    _fields_ = [("query", ctypes.c_int), ("kv", ctypes.c_int)]


class _ConvFusionWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in KEY_CONVFUSION_FIELDS]


class EditError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python linear_compressed_attention_amd/build.py` "
                          "(the HIP library is the only implementation of this package)")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER
    lib.edit_attn_workspace_size.argtypes = [P(_Shape)]
    lib.edit_attn_workspace_size.restype = ctypes.c_size_t
    lib.mmedit_hybrid_workspace_size.argtypes = [P(_Shape), ctypes.c_int]
    lib.mmedit_hybrid_workspace_size.restype = ctypes.c_size_t
    lib.edit_attn_forward.argtypes = [P(_Shape), P(_Weights), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]
    lib.edit_attn_forward.restype = ctypes.c_int
    lib.edit_attn_forward_noalloc.argtypes = [P(_Shape), P(_Weights), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]
    lib.edit_attn_forward_noalloc.restype = ctypes.c_int
    lib.mmedit_hybrid_forward.argtypes = [P(_Shape), ctypes.c_int, P(_Weights), P(_TextWeights), ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]
    lib.mmedit_hybrid_forward.restype = ctypes.c_int
    lib.mmedit_hybrid_exact_forward.argtypes = lib.mmedit_hybrid_forward.argtypes
    lib.mmedit_hybrid_exact_forward.restype = ctypes.c_int
    lib.edit_attn_variant_workspace_size.argtypes = [P(_Shape), P(_Variant)]
    lib.edit_attn_variant_workspace_size.restype = ctypes.c_size_t
    lib.edit_attn_variant_workspace_layout.argtypes = [P(_Shape), P(_Variant), P(_Layout)]
    lib.edit_attn_variant_workspace_layout.restype = ctypes.c_int
    lib.edit_attn_variant_forward.argtypes = [P(_Shape), P(_Variant), P(_Weights), P(_ConvFusionWeights),
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                              ctypes.c_void_p]
    lib.edit_attn_variant_forward.restype = ctypes.c_int
    lib.edit_attn_forward_timed.argtypes = [P(_Shape), P(_Weights), ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.edit_attn_forward_timed.restype = ctypes.c_int
    lib.edit_attn_workspace_layout.argtypes = [P(_Shape), ctypes.c_int, P(_Layout)]
    lib.edit_attn_workspace_layout.restype = ctypes.c_int
    lib.edit_attn_backward_workspace_size.argtypes = [P(_Shape)]
    lib.edit_attn_backward_workspace_size.restype = ctypes.c_size_t
    lib.edit_attn_backward.argtypes = [P(_Shape), P(_Weights), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p, P(_Grads), ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
    lib.edit_attn_backward.restype = ctypes.c_int
    lib.edit_attn_backward_workspace_layout.argtypes = [P(_Shape), P(_BwdLayout)]
    lib.edit_attn_backward_workspace_layout.restype = ctypes.c_int
    lib.edit_status_string.argtypes = [ctypes.c_int]
    lib.edit_status_string.restype = ctypes.c_char_p
    lib.edit_last_error.argtypes = []
    lib.edit_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib_path() -> str:
    return _LIB_PATH


def header_symbols():
    """Function names declared in include/edit_attn.h."""
    import re
    with open(os.path.join(_ROOT, "include", "edit_attn.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, re.M)))


def _get(obj, name):
    return obj[name] if isinstance(obj, Mapping) else getattr(obj, name)


def _shape(s) -> _Shape:
    dt = _get(s, "dtype")
    if isinstance(dt, str):
        dt = {"f32": EDIT_F32, "bf16": EDIT_BF16}[dt]
    return _Shape(*(int(_get(s, n)) for n in ("B", "H", "W", "C", "heads", "head_dim", "reduction", "gn_groups")),
                  float(_get(s, "eps")), int(dt))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != 0:
        raise EditError(status, _lib.edit_last_error().decode())


def edit_status_string(status: int) -> str:
    return _lib.edit_status_string(int(status)).decode()


def edit_last_error() -> str:
    return _lib.edit_last_error().decode()


def edit_attn_workspace_size(shape) -> int:
    """Workspace bytes of edit_attn_forward; raises EditError on a bad shape."""
    sh = _shape(shape)
    n = _lib.edit_attn_workspace_size(ctypes.byref(sh))
    if n == 0:
        _check(_lib.edit_attn_workspace_layout(ctypes.byref(sh), 0, ctypes.byref(_Layout())))
    return n


def mmedit_hybrid_workspace_size(shape, n_text: int) -> int:
    sh = _shape(shape)
    n = _lib.mmedit_hybrid_workspace_size(ctypes.byref(sh), int(n_text))
    if n == 0:
        _check(_lib.edit_attn_workspace_layout(ctypes.byref(sh), int(n_text), ctypes.byref(_Layout())))
    return n


def edit_attn_workspace_layout(shape, n_text: int = 0) -> dict:
    """Byte offsets of the intermediates inside the workspace."""
    lay = _Layout()
    _check(_lib.edit_attn_workspace_layout(ctypes.byref(_shape(shape)), int(n_text), ctypes.byref(lay)))
    return {n: getattr(lay, n) for n in LAYOUT_FIELDS}


def _weights(w) -> _Weights:
    return _Weights(*(_ptr(_get(w, n)) for n in IMAGE_WEIGHT_FIELDS))


def _text_weights(w) -> Optional[_TextWeights]:
    if w is None:
        return None
    return _TextWeights(*(_ptr(_get(w, n)) for n in TEXT_WEIGHT_FIELDS))


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def edit_attn_forward(shape, weights, x, y, workspace, stream=None) -> None:
    """EDiT layer forward on device tensors (enqueued on ``stream``, default:
    torch's current stream). ``weights`` maps the edit_weights_t field names
    to tensors; ``workspace`` is a byte tensor of edit_attn_workspace_size."""
    sh = _shape(shape)
    w = _weights(weights)
    _check(_lib.edit_attn_forward(ctypes.byref(sh), ctypes.byref(w), _ptr(x), _ptr(y), _ptr(workspace),
                                  _nbytes(workspace), _stream(stream)))


def edit_attn_backward_workspace_size(shape) -> int:
    """Scratch bytes edit_attn_backward needs beyond the forward's workspace."""
    return int(_lib.edit_attn_backward_workspace_size(ctypes.byref(_shape(shape))))


def edit_attn_forward_noalloc(shape, weights, x, y, stream=None) -> None:
    """edit_attn_forward without a workspace: the library's static per-device
    scratch (EDIT_NOALLOC_SCRATCH_BYTES) holds the intermediates and the call
    allocates nothing; overlapping calls on one device race."""
    sh = _shape(shape)
    w = _weights(weights)
    _check(_lib.edit_attn_forward_noalloc(ctypes.byref(sh), ctypes.byref(w), _ptr(x), _ptr(y), _stream(stream)))


EDIT_NOALLOC_SCRATCH_BYTES = 256 << 20


def edit_attn_backward_workspace_layout(shape) -> dict:
    """Byte offsets of the backward's intermediate gradients in its workspace
    (and dxc_ld, the dxc row length in elements)."""
    lay = _BwdLayout()
    _check(_lib.edit_attn_backward_workspace_layout(ctypes.byref(_shape(shape)), ctypes.byref(lay)))
    return {n: int(getattr(lay, n)) for n in BWD_LAYOUT_FIELDS}


def edit_attn_backward(shape, weights, x, dy, fwd_workspace, dx, grads, workspace, stream=None) -> None:
    """EDiT layer backward on device tensors: dx and the parameter gradients
    of sum(dy * y), reading the intermediates a preceding edit_attn_forward
    left in ``fwd_workspace`` (same shape, weights and x). ``grads`` maps the
    edit_weights_t field names to output tensors."""
    sh = _shape(shape)
    w = _weights(weights)
    missing = [n for n in IMAGE_WEIGHT_FIELDS if n not in grads]
    if missing:
        raise ValueError(f"grads lacks {missing}")
    g = _Grads(**{n: _ptr(grads[n]) for n in IMAGE_WEIGHT_FIELDS})
    _check(_lib.edit_attn_backward(ctypes.byref(sh), ctypes.byref(w), _ptr(x), _ptr(dy), _ptr(fwd_workspace),
                                   _nbytes(fwd_workspace), _ptr(dx), ctypes.byref(g), _ptr(workspace),
                                   _nbytes(workspace), _stream(stream)))


def edit_attn_forward_timed(shape, weights, x, y, workspace, events, stream=None) -> None:
    """edit_attn_forward that records ``events`` (EDIT_NUM_STEPS + 1 hipEvent_t
    handles, a ctypes array) before each step and after the last one."""
    if len(events) != EDIT_NUM_STEPS + 1:
        raise ValueError(f"need {EDIT_NUM_STEPS + 1} events")
    sh = _shape(shape)
    w = _weights(weights)
    _check(_lib.edit_attn_forward_timed(ctypes.byref(sh), ctypes.byref(w), _ptr(x), _ptr(y), _ptr(workspace),
                                        _nbytes(workspace), _stream(stream), ctypes.cast(events, ctypes.c_void_p)))


def _hybrid(fn, shape, n_text, img_weights, txt_weights, x_img, x_txt, y_img, y_txt, workspace, stream):
    sh = _shape(shape)
    w = _weights(img_weights)
    tw = _text_weights(txt_weights)
    _check(fn(ctypes.byref(sh), int(n_text), ctypes.byref(w), ctypes.byref(tw) if tw is not None else None,
              _ptr(x_img), _ptr(x_txt), _ptr(y_img), _ptr(y_txt), _ptr(workspace), _nbytes(workspace),
              _stream(stream)))


def mmedit_hybrid_forward(shape, n_text, img_weights, txt_weights, x_img, x_txt, y_img, y_txt, workspace,
                          stream=None) -> None:
    """MM-EDiT hybrid forward (image and text rows), eta = token ratio; see edit_attn.h."""
    _hybrid(_lib.mmedit_hybrid_forward, shape, n_text, img_weights, txt_weights, x_img, x_txt, y_img, y_txt,
            workspace, stream)


def mmedit_hybrid_exact_forward(shape, n_text, img_weights, txt_weights, x_img, x_txt, y_img, y_txt, workspace,
                                stream=None) -> None:
    """MM-EDiT hybrid forward with eta computed exactly per image row and head; see edit_attn.h."""
    _hybrid(_lib.mmedit_hybrid_exact_forward, shape, n_text, img_weights, txt_weights, x_img, x_txt, y_img,
            y_txt, workspace, stream)


def _variant(query, kv) -> _Variant:
    q = QUERY_MODES[query] if isinstance(query, str) else int(query)
    k = KV_MODES[kv] if isinstance(kv, str) else int(kv)
    return _Variant(q, k)


def _opt(w, n):
    """A weight the variant may not read: absent keys pass NULL."""
    if isinstance(w, Mapping):
        return _ptr(w.get(n))
    return _ptr(getattr(w, n, None))


def edit_attn_variant_workspace_size(shape, query, kv) -> int:
    """Workspace bytes of edit_attn_variant_forward; raises EditError on a bad shape or variant."""
    sh, v = _shape(shape), _variant(query, kv)
    n = _lib.edit_attn_variant_workspace_size(ctypes.byref(sh), ctypes.byref(v))
    if n == 0:
        _check(_lib.edit_attn_variant_workspace_layout(ctypes.byref(sh), ctypes.byref(v), ctypes.byref(_Layout())))
    return n


def edit_attn_variant_workspace_layout(shape, query, kv) -> dict:
    lay = _Layout()
    _check(_lib.edit_attn_variant_workspace_layout(ctypes.byref(_shape(shape)), ctypes.byref(_variant(query, kv)),
                                                   ctypes.byref(lay)))
    return {n: getattr(lay, n) for n in LAYOUT_FIELDS}


def edit_attn_variant_forward(shape, query, kv, weights, key_cf, x, y, workspace, stream=None) -> None:
    """EDiT layer forward in an ablation variant (query "convfusion" | "linear",
    kv "compressed" | "full" | "key_convfusion"); see edit_attn.h. Weights the
    variant does not read may be absent; ``key_cf`` maps KEY_CONVFUSION_FIELDS
    to tensors (key_convfusion only, else None)."""
    sh, v = _shape(shape), _variant(query, kv)
    w = _Weights(*(_opt(weights, n) for n in IMAGE_WEIGHT_FIELDS))
    kcf = None if key_cf is None else _ConvFusionWeights(*(_opt(key_cf, n) for n in KEY_CONVFUSION_FIELDS))
    _check(_lib.edit_attn_variant_forward(ctypes.byref(sh), ctypes.byref(v), ctypes.byref(w),
                                          ctypes.byref(kcf) if kcf is not None else None, _ptr(x), _ptr(y),
                                          _ptr(workspace), _nbytes(workspace), _stream(stream)))
