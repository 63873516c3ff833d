"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module holds the workload shapes and the random draws only: it computes
nothing of the attention layer itself. Both sides of every parity check take
their inputs from here, so they see identical numbers.

Workloads (stand-ins for the PixArt-Sigma and SD3.5-Medium latents the EDiT
notes evaluate on; no dataset or trained weight is involved):

* ``tiny``          fp32, 1 x 16x16 grid, C=64, 2 heads x 32, r=4, 8 GN groups,
                    X and every weight ~ N(0, 0.02^2).
* ``pixart1024``    bf16, 2 x 64x64,   C=1152, 16 heads x 72, r=4, 32 groups.
* ``pixart2048``    bf16, 1 x 128x128, same channels (16384 tokens).
* ``pixart4096``    bf16, 1 x 256x256, same channels (65536 tokens).
* ``pixart8192``    bf16, 1 x 512x512, same channels (262144 tokens): the
                    largest resolution of the notes' latency table.
* ``sd35m_hybrid``  bf16, 2 x 64x64 image grid + 333 text tokens, C=1536,
                    24 heads x 64, r=4, 32 groups.

For the bf16 workloads X (and the text tokens) ~ N(0, 1) and every Linear /
conv weight and bias ~ N(0, 0.02^2). GroupNorm's affine starts at gamma=1,
beta=0 unless ``gn_affine_random`` asks for N(1, 0.1^2) / N(0, 0.1^2).
Values of a bf16 workload are rounded to bf16 (round to nearest even) once,
here, and returned as float32 arrays that hold bf16-exact values.

Draw order is fixed: x, then the image weights in the order of
``IMAGE_WEIGHT_NAMES``, then (hybrid only) x_txt and ``TEXT_WEIGHT_NAMES``,
then (key-ConvFusion ablation only) ``KEY_CONVFUSION_NAMES``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "LayerShape", "CONFIGS", "IMAGE_WEIGHT_NAMES", "TEXT_WEIGHT_NAMES", "KEY_CONVFUSION_NAMES",
    "image_weight_shapes", "text_weight_shapes", "round_to_bf16",
    "make_inputs", "make_shape",
]


@dataclasses.dataclass(frozen=True)
class LayerShape:
    B: int
    H: int
    W: int
    C: int
    heads: int
    head_dim: int
    reduction: int
    gn_groups: int
    eps: float
    dtype: str              # "f32" or "bf16"
    n_text: int = 0         # text tokens of the hybrid layer (0 = plain EDiT)
    x_std: float = 1.0
    w_std: float = 0.02

    @property
    def N(self) -> int:
        return self.H * self.W

    @property
    def Cr(self) -> int:
        return self.C // self.reduction

    @property
    def Hc(self) -> int:
        return (self.H + 1) // 2

    @property
    def Wc(self) -> int:
        return (self.W + 1) // 2

    @property
    def Nc(self) -> int:
        return self.Hc * self.Wc


CONFIGS: Dict[str, LayerShape] = {
    "tiny": LayerShape(B=1, H=16, W=16, C=64, heads=2, head_dim=32, reduction=4,
                       gn_groups=8, eps=1e-6, dtype="f32", x_std=0.02),
    "pixart1024": LayerShape(B=2, H=64, W=64, C=1152, heads=16, head_dim=72,
                             reduction=4, gn_groups=32, eps=1e-6, dtype="bf16"),
    "pixart2048": LayerShape(B=1, H=128, W=128, C=1152, heads=16, head_dim=72,
                             reduction=4, gn_groups=32, eps=1e-6, dtype="bf16"),
    "pixart4096": LayerShape(B=1, H=256, W=256, C=1152, heads=16, head_dim=72,
                             reduction=4, gn_groups=32, eps=1e-6, dtype="bf16"),
    "pixart8192": LayerShape(B=1, H=512, W=512, C=1152, heads=16, head_dim=72,
                             reduction=4, gn_groups=32, eps=1e-6, dtype="bf16"),
    "sd35m_hybrid": LayerShape(B=2, H=64, W=64, C=1536, heads=24, head_dim=64,
                               reduction=4, gn_groups=32, eps=1e-6, dtype="bf16",
                               n_text=333),
}

IMAGE_WEIGHT_NAMES = (
    "w_cf1", "b_cf1", "gn_gamma", "gn_beta", "w_cf2", "b_cf2",
    "w_q", "b_q", "w_k", "b_k", "w_v", "b_v",
    "dw_k", "db_k", "dw_v", "db_v", "w_o", "b_o",
)
TEXT_WEIGHT_NAMES = ("w_q", "b_q", "w_k", "b_k", "w_v", "b_v", "w_o", "b_o")


def make_shape(**kw) -> LayerShape:
    """A LayerShape from keyword arguments (defaults: fp32, eps 1e-6)."""
    kw.setdefault("eps", 1e-6)
    kw.setdefault("dtype", "f32")
    return LayerShape(**kw)


def image_weight_shapes(s: LayerShape) -> Dict[str, tuple]:
    """Storage shapes of the image-stream parameters.

    Linear weights are [out][in]; the 3x3 compressing conv is [C'][3][3][C]
    (input channels innermost); the depthwise kernels are [3][3][C]."""
    C, Cr = s.C, s.Cr
    return {
        "w_cf1": (Cr, 3, 3, C), "b_cf1": (Cr,),
        "gn_gamma": (Cr,), "gn_beta": (Cr,),
        "w_cf2": (C, Cr), "b_cf2": (C,),
        "w_q": (C, C), "b_q": (C,),
        "w_k": (C, C), "b_k": (C,),
        "w_v": (C, C), "b_v": (C,),
        "dw_k": (3, 3, C), "db_k": (C,),
        "dw_v": (3, 3, C), "db_v": (C,),
        "w_o": (C, C), "b_o": (C,),
    }


def text_weight_shapes(s: LayerShape) -> Dict[str, tuple]:
    C = s.C
    return {"w_q": (C, C), "b_q": (C,), "w_k": (C, C), "b_k": (C,),
            "w_v": (C, C), "b_v": (C,), "w_o": (C, C), "b_o": (C,)}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def _draw(rng: np.random.Generator, shape, std: float, mean: float = 0.0) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float64) * std + mean).astype(np.float32)


KEY_CONVFUSION_NAMES = ("w_cf1", "b_cf1", "gn_gamma", "gn_beta", "w_cf2", "b_cf2")


def make_inputs(s: LayerShape, seed: int = 0, gn_affine_random: bool = False,
                x_std: Optional[float] = None, n_text: Optional[int] = None,
                key_convfusion: bool = False) -> dict:
    """Draw one workload's inputs.

    Returns ``{"x": [B, N, C], "w": {...}}`` and, when the layer has text
    tokens, ``"x_txt": [B, N_T, C]`` and ``"w_txt": {...}``. With
    ``key_convfusion`` also ``"w_kcf"``: a second set of ConvFusion
    parameters (``KEY_CONVFUSION_NAMES``, shapes as the image weights of the
    same names) for the ablation variant that passes the keys through
    ConvFusion, drawn last. All arrays are float32 (bf16-exact for a bf16
    workload) and C-contiguous.
    """
    rng = np.random.default_rng(seed)
    xs = s.x_std if x_std is None else x_std
    nt = s.n_text if n_text is None else n_text
    rnd = round_to_bf16 if s.dtype == "bf16" else (lambda a: a)

    out = {"x": rnd(_draw(rng, (s.B, s.N, s.C), xs))}
    w = {}
    for name, shp in image_weight_shapes(s).items():
        if name == "gn_gamma":
            w[name] = _draw(rng, shp, 0.1, 1.0) if gn_affine_random else np.ones(shp, np.float32)
        elif name == "gn_beta":
            w[name] = _draw(rng, shp, 0.1) if gn_affine_random else np.zeros(shp, np.float32)
        else:
            w[name] = _draw(rng, shp, s.w_std)
        w[name] = rnd(w[name])
    out["w"] = w
    if nt:
        out["x_txt"] = rnd(_draw(rng, (s.B, nt, s.C), 1.0))
        out["w_txt"] = {name: rnd(_draw(rng, shp, s.w_std))
                        for name, shp in text_weight_shapes(s).items()}
    if key_convfusion:
        shapes = image_weight_shapes(s)
        wk = {}
        for name in KEY_CONVFUSION_NAMES:
            if name == "gn_gamma":
                wk[name] = _draw(rng, shapes[name], 0.1, 1.0) if gn_affine_random else np.ones(shapes[name], np.float32)
            elif name == "gn_beta":
                wk[name] = _draw(rng, shapes[name], 0.1) if gn_affine_random else np.zeros(shapes[name], np.float32)
            else:
                wk[name] = _draw(rng, shapes[name], s.w_std)
            wk[name] = rnd(wk[name])
        out["w_kcf"] = wk
    return out
