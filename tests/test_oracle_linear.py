"""Pins of the linear-attention oracle (oracle/linear.py).

The oracle uses the associative form (V K_rot^T) Q_rot / den. These tests hold it to facts
that do not depend on that form: the N x N quadratic form and scalar loops give the same
numbers; with V = 1 and no rotation the output is exactly the normaliser's ratio (about 1);
the result is invariant to the scale of K and of Q, linear in V, and invariant to a joint
permutation of the key tokens; one token gives the closed form.
"""
import math

import numpy as np
import pytest
import torch

from oracle.linear import LINEAR_EPS, linear_attention, linear_attention_quadratic


def bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def widen(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def inputs(B=1, N=40, H=2, d=128, seed=0):
    """ReLU'd q, k (non-negative) and independent signed rotated rows, N(0, 1) values."""
    rng = np.random.default_rng(seed)
    q = bits(np.maximum(rng.standard_normal((B, N, H, d)), 0))
    k = bits(np.maximum(rng.standard_normal((B, N, H, d)), 0))
    qr = bits(rng.standard_normal((B, N, H, d)))
    kr = bits(rng.standard_normal((B, N, H, d)))
    v = bits(rng.standard_normal((B, N, H, d)))
    return q, k, qr, kr, v


def test_quadratic_form_agrees():
    x = inputs(B=2, N=37, H=3)
    a = linear_attention(*x)
    b = linear_attention_quadratic(*x)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_scalar_loops_tiny():
    q, k, qr, kr, v = inputs(N=4, H=1, d=128, seed=1)
    out = linear_attention(q, k, qr, kr, v)
    Q, K, QR, KR, V = (widen(t)[0, :, 0] for t in (q, k, qr, kr, v))
    for n in range(4):
        den = sum(sum(float(Q[n, c]) * float(K[m, c]) for c in range(128)) for m in range(4)) + LINEAR_EPS
        for i in (0, 5, 127):
            num = 0.0
            for m in range(4):
                w = sum(float(QR[n, c]) * float(KR[m, c]) for c in range(128))
                num += w * float(V[m, i])
            assert out[0, n, 0, i] == pytest.approx(num / den, rel=1e-12, abs=1e-13)


def test_unit_values_without_rotation_give_one():
    q, k, _, _, _ = inputs(N=50, seed=2)
    v = bits(np.ones((1, 50, 2, 128)))
    out = linear_attention(q, k, q, k, v)
    Q, K = widen(q), widen(k)
    den = np.einsum("bnhc,bmhc->bnh", Q, K)
    want = (den / (den + LINEAR_EPS))[..., None] * np.ones(128)
    np.testing.assert_allclose(out, want, rtol=1e-13)
    np.testing.assert_allclose(out, 1.0, rtol=1e-12)


def test_scale_invariance_of_keys_and_queries():
    q, k, qr, kr, v = inputs(N=30, seed=3)
    base = linear_attention(q, k, qr, kr, v)
    two = lambda b: bits(widen(b) * 2.0)       # exact in BF16
    quarter = lambda b: bits(widen(b) * 0.25)
    np.testing.assert_allclose(linear_attention(q, two(k), qr, two(kr), v), base, rtol=1e-12)
    np.testing.assert_allclose(linear_attention(quarter(q), k, quarter(qr), kr, v), base, rtol=1e-12)


def test_linear_in_values():
    q, k, qr, kr, _ = inputs(N=25, seed=4)
    rng = np.random.default_rng(5)
    v1 = rng.integers(-8, 8, (1, 25, 2, 128)).astype(np.float32)
    v2 = rng.integers(-8, 8, (1, 25, 2, 128)).astype(np.float32)
    a = linear_attention(q, k, qr, kr, bits(v1)) + linear_attention(q, k, qr, kr, bits(v2))
    b = linear_attention(q, k, qr, kr, bits(v1 + v2))     # small integers: exact in BF16
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_joint_key_permutation_and_query_selection():
    q, k, qr, kr, v = inputs(N=33, seed=6)
    base = linear_attention(q, k, qr, kr, v)
    perm = np.random.default_rng(7).permutation(33)
    # keys permuted together (q stays): the sums over m do not change
    moved = linear_attention(q, k[:, perm], qr, kr[:, perm], v[:, perm])
    np.testing.assert_allclose(moved, base, rtol=1e-12, atol=1e-13)
    toks = [0, 3, 32]
    np.testing.assert_allclose(linear_attention(q, k, qr, kr, v, tokens=toks), base[:, toks], rtol=1e-13, atol=1e-14)


def test_one_token_closed_form():
    q, k, qr, kr, v = inputs(N=1, H=1, seed=8)
    out = linear_attention(q, k, qr, kr, v)[0, 0, 0]
    Q, K, QR, KR, V = (widen(t)[0, 0, 0] for t in (q, k, qr, kr, v))
    want = (QR @ KR) * V / (Q @ K + LINEAR_EPS)
    np.testing.assert_allclose(out, want, rtol=1e-13)
    assert math.isfinite(float(out.sum()))
