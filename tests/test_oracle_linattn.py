"""Pins of the oracle's linear attention (CPU only).

Against: the hand-worked fixture tests/golden/linattn_worked.json, the
explicit N x N kernelised sum in exact rational arithmetic, closed forms
(constant values, zero query) and invariants (token permutation, key scale,
head-to-channel map)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import edit_oracle as O


def test_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "linattn_worked.json")) as f:
        g = json.load(f)
    K = np.array(g["K"], float)[None]; V = np.array(g["V"], float)[None]; Q = np.array(g["Q"], float)[None]
    S, z = O.kv_state(K, V, heads=1)
    np.testing.assert_array_equal(S[0, 0], g["S"])
    np.testing.assert_array_equal(z[0, 0], g["z"])
    y = O.linear_attention_apply(Q, S, z, heads=1, eps=0.0)
    np.testing.assert_array_equal(y[0], g["Y"])


def _kernelised_exact(Q, K, V, eps):
    """y_i = sum_j (Q_i . K_j) V_j / (sum_j Q_i . K_j + eps), all in Fractions."""
    out = []
    for qi in Q:
        w = [sum(Fraction(int(a)) * Fraction(int(b)) for a, b in zip(qi, kj)) for kj in K]
        den = sum(w) + eps
        out.append([sum(wj * Fraction(int(vj[c])) for wj, vj in zip(w, V)) / den for c in range(V.shape[1])])
    return out


@pytest.mark.parametrize("n_q,n_k,d,seed", [(3, 5, 2, 0), (4, 7, 3, 1), (2, 9, 4, 2)])
def test_factored_equals_explicit_sum(n_q, n_k, d, seed):
    rng = np.random.default_rng(seed)
    Q = rng.integers(0, 5, (n_q, d)); Q[0, 0] += 1
    K = rng.integers(0, 4, (n_k, d)); K[0, :] += 1
    V = rng.integers(-6, 7, (n_k, d))
    eps = Fraction(1, 1000)
    exact = _kernelised_exact(Q, K, V, eps)
    y = O.linear_attention(Q[None].astype(float), K[None].astype(float), V[None].astype(float), 1, float(eps))
    for i in range(n_q):
        for c in range(d):
            assert abs(y[0, i, c] - float(exact[i][c])) <= 1e-12 * max(1.0, abs(float(exact[i][c])))


def test_multihead_explicit_sum():
    rng = np.random.default_rng(3)
    B, heads, d, N, Nk = 2, 3, 4, 5, 6
    q = rng.random((B, N, heads * d)); k = rng.random((B, Nk, heads * d)); v = rng.standard_normal((B, Nk, heads * d))
    y = O.linear_attention(q, k, v, heads, 1e-6)
    for b in range(B):
        for h in range(heads):
            sl = slice(h * d, (h + 1) * d)
            for i in range(N):
                w = np.array([q[b, i, sl] @ k[b, j, sl] for j in range(Nk)])
                ref = (w[:, None] * v[b, :, sl]).sum(0) / (w.sum() + 1e-6)
                np.testing.assert_allclose(y[b, i, sl], ref, rtol=1e-12)


def test_constant_values_closed_form():
    rng = np.random.default_rng(4)
    q = rng.random((1, 8, 6)); k = rng.random((1, 5, 6))
    vvec = rng.standard_normal(6)
    v = np.broadcast_to(vvec, (1, 5, 6)).copy()
    y = O.linear_attention(q, k, v, 2, 1e-6)
    S, z = O.kv_state(k, v, 2)
    for h in range(2):
        sl = slice(3 * h, 3 * h + 3)
        qz = q[0, :, sl] @ z[0, h]
        np.testing.assert_allclose(y[0, :, sl], vvec[sl][None] * (qz / (qz + 1e-6))[:, None], rtol=1e-12)


def test_zero_query_gives_zero():
    rng = np.random.default_rng(5)
    q = np.zeros((1, 3, 4)); k = rng.random((1, 5, 4)); v = rng.standard_normal((1, 5, 4))
    np.testing.assert_array_equal(O.linear_attention(q, k, v, 2, 1e-6), 0.0)


def test_permutation_and_scale_invariance():
    rng = np.random.default_rng(6)
    q = rng.random((1, 7, 8)); k = rng.random((1, 11, 8)); v = rng.standard_normal((1, 11, 8))
    y = O.linear_attention(q, k, v, 2, 0.0)
    p = rng.permutation(11)
    np.testing.assert_allclose(O.linear_attention(q, k[:, p], v[:, p], 2, 0.0), y, rtol=1e-12)
    np.testing.assert_allclose(O.linear_attention(q, 3.5 * k, v, 2, 0.0), y, rtol=1e-12)
    # convex hull: each output channel lies within that channel's value range
    for h in range(2):
        sl = slice(4 * h, 4 * h + 4)
        assert np.all(y[0, :, sl] <= v[0, :, sl].max(0) + 1e-12)
        assert np.all(y[0, :, sl] >= v[0, :, sl].min(0) - 1e-12)


def test_head_channel_map():
    """Head h owns channels h*d..h*d+d-1: silencing head 1's keys zeroes
    exactly its output slice."""
    rng = np.random.default_rng(7)
    q = rng.random((1, 4, 6)); k = rng.random((1, 5, 6)); v = rng.standard_normal((1, 5, 6))
    k[..., 3:] = 0.0
    y = O.linear_attention(q, k, v, 2, 1e-6)
    np.testing.assert_array_equal(y[0, :, 3:], 0.0)
    assert np.all(np.abs(y[0, :, :3]) > 0)
