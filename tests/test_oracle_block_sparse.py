"""Pins of the block-skip oracle (oracle/block_sparse.py).

The routing rule is a reading (the pages give only its knobs), so the pins hold the oracle to
that rule written differently (scalar loops over explicit sums), to closed forms whose kept
set and output follow by hand, and to the rule's structural facts: tau = inf is dense
attention, the argmax block and the sink blocks are always kept, kept sets grow with tau,
key order inside a block does not matter.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention_dense
from oracle import attention_varlen
from oracle.block_sparse import (KEY_BLOCK, QUERY_BLOCK, attention_kept, attention_kept_varlen, decision_margin,
                                 kept_pairs, pooled_means, proxy_logits, route_blocks, route_blocks_varlen,
                                 segment_tiles)


def bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def widen(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def randn_bits(shape, seed, scale=1.0):
    return bits(np.random.default_rng(seed).standard_normal(shape) * scale)


def test_pooled_means_ragged_block():
    x = np.arange(130 * 3, dtype=np.float64).reshape(130, 3)
    m = pooled_means(x, 64)
    assert m.shape == (3, 3)
    np.testing.assert_array_equal(m[2], x[128:130].mean(axis=0))
    np.testing.assert_array_equal(m[0], x[:64].sum(axis=0) / 64)


def test_rule_by_scalar_loops():
    """z, zmax and keep from explicit Python sums over a tiny case (2 query blocks, 5 key
    blocks with a ragged last one, d = 128)."""
    N, d, bm, bn = 20, 128, 8, 4
    q = randn_bits((1, 1, N, d), 1)
    k = randn_bits((1, 1, N, d), 2)
    s, tau = 0.088388, 0.05
    keep, z, zmax = route_blocks(q, k, s, tau, sink_tokens=0, bm=bm, bn=bn)
    Q, K = widen(q)[0, 0], widen(k)[0, 0]
    sf = float(np.float32(s))
    for I in range(math.ceil(N / bm)):
        rows = range(I * bm, min(N, (I + 1) * bm))
        qbar = [math.fsum(Q[r, c] for r in rows) / len(rows) for c in range(d)]
        zs = []
        for J in range(math.ceil(N / bn)):
            keys = range(J * bn, min(N, (J + 1) * bn))
            kbar = [math.fsum(K[j, c] for j in keys) / len(keys) for c in range(d)]
            zs.append(sf * math.fsum(qbar[c] * kbar[c] for c in range(d)))
        np.testing.assert_allclose(z[0, 0, I], zs, rtol=1e-12, atol=1e-14)
        assert zmax[0, 0, I] == pytest.approx(max(zs), rel=1e-12)
        want = [zz >= max(zs) - tau for zz in zs]
        # the sums agree to ~1e-15; no z of this seed sits that close to the threshold
        assert all(abs(zz - (max(zs) - tau)) > 1e-9 for zz in zs)
        assert list(keep[0, 0, I]) == want


def test_infinite_tau_is_dense_attention():
    q, k, v = (randn_bits((2, 2, 150, 128), s) for s in (3, 4, 5))
    keep, _, _ = route_blocks(q, k, 0.0883883, math.inf, bm=64, bn=32)
    assert keep.all()
    o, lse = attention_kept(q, k, v, 0.0883883, keep, bm=64, bn=32)
    o_ref, lse_ref = attention_dense(q, k, v, 0.0883883)
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13)


def test_argmax_and_sinks_always_kept_and_nested_in_tau():
    q = randn_bits((1, 3, 600, 128), 6)
    k = randn_bits((1, 3, 600, 128), 7)
    prev = None
    for tau in (0.0, 0.01, 0.05, 0.2, 1.0, math.inf):
        keep, z, zmax = route_blocks(q, k, 0.0883883, tau, sink_tokens=100)
        arg = z.argmax(axis=-1)
        assert np.take_along_axis(keep, arg[..., None], -1).all()
        assert keep[..., :2].all()                    # keys 0..99 lie in blocks 0 and 1
        if prev is not None:
            assert not (prev & ~keep).any()           # nothing dropped when tau grows
        prev = keep
    keep0, z0, zmax0 = route_blocks(q, k, 0.0883883, 0.0)
    assert (keep0.sum(axis=-1) >= 1).all()
    np.testing.assert_array_equal(keep0, z0 == zmax0[..., None])


def test_closed_form_kept_set_and_output():
    """Every query row is a*e0; key block J holds 64 copies of b_J*e0 (plus per-key values).
    Then z_J = s*a*b_J exactly, the kept set is {J : b_J >= max b - tau/(s a)}, and each
    row's output is sum_J n_J exp(x_J) vbar_J / sum_J n_J exp(x_J) with x_J = s*a*b_J."""
    N, d = 4 * KEY_BLOCK, 128
    a, s = 2.0, 0.125
    b = np.array([1.0, 3.0, 2.5, -4.0])
    q = np.zeros((1, 1, N, d))
    q[..., 0] = a
    k = np.zeros((1, 1, N, d))
    for J in range(4):
        k[0, 0, J * 64:(J + 1) * 64, 0] = b[J]
    rng = np.random.default_rng(8)
    v = rng.integers(-8, 9, (1, 1, N, d)).astype(np.float64)
    qb, kb, vb = bits(q), bits(k), bits(v)
    z = proxy_logits(qb, kb, s)
    np.testing.assert_array_equal(z[0, 0, 0], s * a * b)
    tau = s * a * 0.6                                 # keeps b = 3.0 and 2.5, drops 1.0 and -4.0
    keep, _, _ = route_blocks(qb, kb, s, tau)
    np.testing.assert_array_equal(keep[0, 0, 0], [False, True, True, False])
    o, lse = attention_kept(qb, kb, vb, s, keep)
    x = s * a * b[[1, 2]]
    w = 64 * np.exp(x)
    vbar = np.stack([v[0, 0, 64:128].mean(axis=0), v[0, 0, 128:192].mean(axis=0)])
    want = (w[:, None] * vbar).sum(axis=0) / w.sum()
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(want, (N, d)), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], math.log(w.sum()), rtol=1e-14)


def test_single_kept_key_gives_its_value():
    """N = 65: the last key block holds key 64 alone; with queries along it and tau = 0 only
    that block is kept (its mean is that key), so o = v_64 and lse = s q.k_64."""
    N, d = 65, 128
    k = np.zeros((1, 1, N, d))
    k[0, 0, :64, 1] = 1.0
    k[0, 0, 64, 0] = 4.0
    q = np.zeros((1, 1, N, d))
    q[..., 0] = 1.0
    v = np.random.default_rng(9).integers(-5, 6, (1, 1, N, d)).astype(np.float64)
    qb, kb, vb = bits(q), bits(k), bits(v)
    keep, _, _ = route_blocks(qb, kb, 0.5, 0.0)
    np.testing.assert_array_equal(keep[0, 0, 0], [False, True])
    o, lse = attention_kept(qb, kb, vb, 0.5, keep)
    np.testing.assert_array_equal(o[0, 0], np.broadcast_to(v[0, 0, 64], (N, d)))
    np.testing.assert_allclose(lse[0, 0], 0.5 * 4.0)


def test_key_order_inside_a_block_is_irrelevant():
    q, k, v = (randn_bits((1, 2, 300, 128), s) for s in (10, 11, 12))
    keep, z, _ = route_blocks(q, k, 0.0883883, 0.03)
    perm = np.arange(300)
    rng = np.random.default_rng(13)
    for J in range(0, 300, 64):
        seg = perm[J:J + 64].copy()
        rng.shuffle(seg)
        perm[J:J + 64] = seg
    keep2, z2, _ = route_blocks(q, k[:, :, perm], 0.0883883, 0.03)
    np.testing.assert_allclose(z2, z, rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(keep2, keep)
    o1, l1 = attention_kept(q, k, v, 0.0883883, keep)
    o2, l2 = attention_kept(q, k[:, :, perm], v[:, :, perm], 0.0883883, keep)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, l1, rtol=1e-13)


def test_kept_attention_by_scalar_loops_and_empty_block():
    """A hand-picked kept set (not from the rule, as a caller of the hook may give) against
    math.exp / math.fsum loops; a query block with nothing kept gets o = 0, lse = -inf."""
    N, d, bm, bn = 12, 128, 4, 4
    q, k, v = (randn_bits((1, 1, N, d), s) for s in (14, 15, 16))
    keep = np.array([[[[True, False, True], [False, True, False], [False, False, False]]]])
    o, lse = attention_kept(q, k, v, 0.3, keep, bm=bm, bn=bn)
    Q, K, V = widen(q)[0, 0], widen(k)[0, 0], widen(v)[0, 0]
    s = float(np.float32(0.3))
    for i in range(8):
        keys = [j for j in range(N) if keep[0, 0, i // bm, j // bn]]
        x = [s * math.fsum(Q[i, c] * K[j, c] for c in range(d)) for j in keys]
        m = max(x)
        p = [math.exp(t - m) for t in x]
        l = math.fsum(p)
        for c in (0, 77, 127):
            assert o[0, 0, i, c] == pytest.approx(math.fsum(pj * V[j, c] for pj, j in zip(p, keys)) / l,
                                                  rel=1e-12, abs=1e-14)
        assert lse[0, 0, i] == pytest.approx(m + math.log(l), rel=1e-13)
    assert np.all(o[0, 0, 8:] == 0) and np.all(np.isneginf(lse[0, 0, 8:]))


def test_kept_pairs_and_margin():
    keep = np.ones((1, 1, 2, 3), bool)
    assert kept_pairs(keep, 300, bm=256, bn=128) == 300 * 300
    keep[0, 0, 1, 2] = False                          # rows 256..299 x keys 256..299
    assert kept_pairs(keep, 300, bm=256, bn=128) == 300 * 300 - 44 * 44
    q = randn_bits((1, 1, 300, 128), 17)
    k = randn_bits((1, 1, 300, 128), 18)
    mg = decision_margin(q, k, 0.0883883, 0.1)
    z = proxy_logits(q, k, 0.0883883)
    assert mg.shape == z.shape and (mg > 0).all()
    # the band is far below the spread of z (it only absorbs FP32 rounding)
    assert mg.max() < 5e-3 * (z.max() - z.min())


def test_default_blocks_are_the_kernel_tiles():
    assert (QUERY_BLOCK, KEY_BLOCK) == (256, 64)


def test_segment_tile_numbering():
    cu = [0, 300, 300, 301, 1000]
    np.testing.assert_array_equal(segment_tiles(cu, 256), [0, 2, 2, 3, 6])
    np.testing.assert_array_equal(segment_tiles(cu, 64), [0, 5, 5, 6, 17])


def test_varlen_routing_is_per_segment_dense_routing():
    """A packed batch of segments routes and attends exactly as each segment alone would: the
    varlen oracle on [a | b] equals the dense oracle on a and on b."""
    rng = np.random.default_rng(21)
    lens = [300, 1, 0, 520]
    T, H, d = sum(lens), 2, 128
    q, k, v = (bits(rng.standard_normal((T, H, d))) for _ in range(3))
    cu = np.concatenate([[0], np.cumsum(lens)])
    routes = route_blocks_varlen(q, k, cu, 0.0883883, 0.01, sink_tokens=64)
    assert routes[2] is None
    keeps = [None if r is None else r[0] for r in routes]
    o, lse = attention_kept_varlen(q, k, v, cu, 0.0883883, keeps)
    for s, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        if e == a:
            continue
        dq, dk, dv = (np.ascontiguousarray(x[a:e].transpose(1, 0, 2))[None] for x in (q, k, v))
        keep, z, zmax = route_blocks(dq, dk, 0.0883883, 0.01, sink_tokens=64)
        np.testing.assert_array_equal(keeps[s], keep[0])
        od, ld = attention_kept(dq, dk, dv, 0.0883883, keep)
        np.testing.assert_allclose(o[a:e], od[0].transpose(1, 0, 2), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse[:, a:e], ld[0], rtol=1e-13)
    # a length-1 segment keeps its only tile and returns its own value
    np.testing.assert_array_equal(o[300], widen(v[300]))


def test_varlen_infinite_tau_is_varlen_attention():
    rng = np.random.default_rng(22)
    lens = [129, 64, 7]
    T = sum(lens)
    q, k, v = (bits(rng.standard_normal((T, 3, 128))) for _ in range(3))
    cu = np.concatenate([[0], np.cumsum(lens)])
    keeps = [r[0] for r in route_blocks_varlen(q, k, cu, 0.0883883, math.inf)]
    assert all(kp.all() for kp in keeps)
    o, lse = attention_kept_varlen(q, k, v, cu, 0.0883883, keeps)
    o_ref, lse_ref = attention_varlen(q, k, v, cu, 0.0883883)
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13)
    rows = np.array([0, 128, 129, 3 * T - 1])
    o_r, lse_r = attention_kept_varlen(q, k, v, cu, 0.0883883, keeps, rows=rows)
    np.testing.assert_allclose(o_r, o.transpose(1, 0, 2).reshape(-1, 128)[rows], rtol=1e-12, atol=1e-15)
