"""Error measures shared by the tests (test infrastructure).

max_rel_err is the parity gate: max_i |g_i - o_i| / max_i |o_i| over one
tensor. centred_rel_err applies it after subtracting each tensor's mean over
the token axis, so a mistake in the token-dependent part of a linear-attention
output (which is close to a per-channel average) cannot hide under the mean.
"""
import numpy as np

BF16_TOL = 2e-2
F32_TOL = 1e-4


def max_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    scale = np.abs(ref).max()
    if scale == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / scale)


def centred_rel_err(got, ref, token_axis=-2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return max_rel_err(got - got.mean(axis=token_axis, keepdims=True),
                       ref - ref.mean(axis=token_axis, keepdims=True))


def norm_rel_err(got, ref):
    """||g - o|| / ||o|| (Frobenius) over one tensor: the gate for bf16
    gradients that pass a ReLU mask, where a pre-activation within bf16
    rounding of zero may fall on the other side of the kink than in float64
    and move one element by a whole upstream value."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    n = np.linalg.norm(ref)
    if n == 0:
        return float(np.linalg.norm(got))
    return float(np.linalg.norm(got - ref) / n)
