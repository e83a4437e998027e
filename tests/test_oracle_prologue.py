"""Pins of the prologue oracle (oracle/prologue.py) and of the BF16 rounding helpers.

Each test fixes a fact the mathematics or an independent routine determines, so that a
plausible slip in the oracle (a wrong eps, a swapped sin sign, pairs taken non-interleaved,
a wrong axis split or frequency exponent, a transposed layout) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (bf16_faithful, bf16_round_f64, bf16_spacing, grid_positions, pair_frequencies,
                    qk_norm_rope, v_head_major)

EPS = 1e-6
EPS32 = float(np.float32(EPS))


def bits(x):
    """float -> bfloat16 bit patterns via torch (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def widen(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_bits(shape, seed=0, scale=1.0):
    return bits(np.random.default_rng(seed).standard_normal(shape) * scale)


# ---------------------------------------------------------------- BF16 rounding helper
def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-3,
                        rng.standard_normal(2000) * 300.0])
    ref = widen(bits(y.astype(np.float32)))   # float32 first: y has > 24 bits, check ties below
    got = bf16_round_f64(y.astype(np.float32).astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa is 1.0
    assert bf16_round_f64(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert bf16_round_f64(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert bf16_round_f64(np.array([-(1.0 + 2.0 ** -8)]))[0] == -1.0
    assert bf16_spacing(np.array([1.0, 1.99, 2.0, 0.75]))[0] == 2.0 ** -7
    assert list(bf16_spacing(np.array([1.99, 2.0, 0.75]))) == [2.0 ** -7, 2.0 ** -6, 2.0 ** -8]


def test_bf16_faithful_accepts_neighbours_only():
    exact = np.array([1.0 + 2.0 ** -9, 3.0])
    lo = np.array([1.0, 3.0])
    hi = np.array([1.0 + 2.0 ** -7, 3.0])
    assert bf16_faithful(lo, exact)["ok"] and bf16_faithful(hi, exact)["ok"]
    assert not bf16_faithful(np.array([1.0 + 2.0 ** -6, 3.0]), exact)["ok"]
    assert bf16_faithful(lo, exact)["rne_frac"] == 1.0 and bf16_faithful(hi, exact)["rne_frac"] == 0.5


# ---------------------------------------------------------------- prologue oracle
def test_grid_positions_raster_order():
    pos = grid_positions((3, 4, 5), 60)
    assert pos[0].tolist() == [0, 0, 0]
    assert pos[1].tolist() == [0, 0, 1]
    assert pos[5].tolist() == [0, 1, 0]
    assert pos[20].tolist() == [1, 0, 0]
    assert pos[59].tolist() == [2, 3, 4]


def test_pair_frequencies_split_and_exponents():
    axis, freq = pair_frequencies(10000.0)
    assert axis.tolist() == [0] * 22 + [1] * 21 + [2] * 21
    assert freq[0] == 1.0 and freq[22] == 1.0 and freq[43] == 1.0
    assert freq[21] == pytest.approx(10000.0 ** (-21 / 22), rel=1e-15)
    assert freq[42] == pytest.approx(1e-4 ** (20 / 21), rel=1e-15)
    assert freq[1] == pytest.approx(math.exp(-math.log(10000.0) / 22), rel=1e-15)


def test_rms_of_every_row_is_closed_form():
    """Rotation keeps the row norm, so every output row has RMS sqrt(ms / (ms + eps))."""
    xb = rand_bits((2, 12, 3, 128), seed=2, scale=0.01)    # small rows: eps matters
    out = qk_norm_rope(xb, (2, 2, 3), eps=EPS)
    x = widen(xb)
    ms = np.mean(x * x, axis=-1)                              # [B, N, H]
    want = np.sqrt(ms / (ms + EPS32)).transpose(0, 2, 1)      # [B, H, N]
    got = np.sqrt(np.mean(out * out, axis=-1))
    np.testing.assert_allclose(got, want, rtol=1e-13)
    assert np.all(want < 0.99995)                             # eps did change these rows


def test_token_zero_is_not_rotated():
    """At position (0, 0, 0) every angle is 0: the row keeps its direction."""
    xb = rand_bits((1, 6, 2, 128), seed=3)
    out = qk_norm_rope(xb, (1, 2, 3))
    x = widen(xb)
    for h in range(2):
        a, b = out[0, h, 0], x[0, 0, h]
        cos = a @ b / (np.linalg.norm(a) * np.linalg.norm(b))
        assert cos == pytest.approx(1.0, abs=1e-14)


@pytest.mark.parametrize("axis,token", [(0, 12), (1, 4), (2, 1)])   # grid (3, 3, 4): one step on t / h / w
def test_one_step_on_one_axis_turns_exactly_that_axis(axis, token):
    """Constant rows (RMSNorm output y on every channel): after one position step on one axis,
    pair i of that axis reads y (cos f - sin f, sin f + cos f) with f its frequency; pairs of
    the other axes are untouched."""
    grid = (3, 3, 4)
    assert grid_positions(grid, 36)[token].tolist() == [1 if a == axis else 0 for a in range(3)]
    x = np.full((1, 36, 1, 128), 0.75)
    out = qk_norm_rope(bits(x), grid)[0, 0, token]
    y = 0.75 / math.sqrt(0.75 ** 2 + EPS32)
    ax, freq = pair_frequencies()
    for i in range(64):
        f = freq[i] if ax[i] == axis else 0.0
        assert out[2 * i] == pytest.approx(y * (math.cos(f) - math.sin(f)), abs=1e-14)
        assert out[2 * i + 1] == pytest.approx(y * (math.sin(f) + math.cos(f)), abs=1e-14)
    # a printed value: the first pair of the turned axis turns by one radian
    first = {0: 0, 1: 22, 2: 43}[axis]
    assert out[2 * first] == pytest.approx(y * (0.5403023058681398 - 0.8414709848078965), abs=1e-14)


def test_angles_grow_linearly_with_position():
    """atan2 of a rotated pair over its unrotated one is pos * freq (mod 2 pi), per axis."""
    grid = (5, 6, 7)
    n = 5 * 6 * 7
    xb = rand_bits((1, n, 1, 128), seed=4)
    out = qk_norm_rope(xb, grid)[0, 0]
    x = widen(xb)[0, :, 0]
    pos = grid_positions(grid, n)
    ax, freq = pair_frequencies()
    rot = np.arctan2(out[:, 1::2], out[:, 0::2]) - np.arctan2(x[:, 1::2], x[:, 0::2])
    want = pos[:, ax] * freq
    d = np.angle(np.exp(1j * (rot - want)))
    assert np.max(np.abs(d)) < 1e-10


def test_relative_position_property():
    """<R(q, p), R(k, p')> is unchanged when both positions move by the same amount."""
    grid = (4, 5, 6)
    n = 120
    qb = rand_bits((1, n, 1, 128), seed=5)
    kb = rand_bits((1, n, 1, 128), seed=6)
    # the same q and k rows at every token, so only positions differ
    qb[:] = qb[:, :1]
    kb[:] = kb[:, :1]
    q = qk_norm_rope(qb, grid)[0, 0]
    k = qk_norm_rope(kb, grid)[0, 0]
    pos = grid_positions(grid, n)
    idx = {tuple(p): i for i, p in enumerate(pos.tolist())}
    for (p1, p2, delta) in [((0, 0, 0), (1, 2, 3), (2, 1, 1)), ((1, 4, 0), (0, 1, 5), (2, 0, 0)),
                            ((2, 2, 2), (2, 2, 2), (1, 2, 3))]:
        a = q[idx[p1]] @ k[idx[p2]]
        s1 = tuple(x + d for x, d in zip(p1, delta))
        s2 = tuple(x + d for x, d in zip(p2, delta))
        b = q[idx[s1]] @ k[idx[s2]]
        assert a == pytest.approx(b, abs=1e-12)


def test_layout_and_heads():
    """Output [b, h, n] comes from input [b, n, h]: permuting input heads permutes output heads."""
    xb = rand_bits((2, 6, 4, 128), seed=7)
    out = qk_norm_rope(xb, (1, 2, 3))
    perm = [2, 0, 3, 1]
    out_p = qk_norm_rope(xb[:, :, perm], (1, 2, 3))
    assert np.array_equal(out_p, out[:, perm])
    assert out.shape == (2, 4, 6, 128)


def test_weight_applies_before_the_rotation():
    """With a per-channel weight w, a position-0 row is RMSNorm(x) * w; at other positions the
    weighted pairs are rotated (the pair norm of y*w is kept)."""
    xb = rand_bits((1, 6, 1, 128), seed=8)
    w = np.linspace(0.5, 1.5, 128)
    out = qk_norm_rope(xb, (1, 2, 3), weight=w)[0, 0]
    base = qk_norm_rope(xb, (1, 2, 3))[0, 0]
    np.testing.assert_allclose(out[0], base[0] * w, rtol=1e-14)
    x = widen(xb)[0, :, 0]
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS32) * w
    pn_in = np.hypot(y[:, 0::2], y[:, 1::2])
    pn_out = np.hypot(out[:, 0::2], out[:, 1::2])
    np.testing.assert_allclose(pn_out, pn_in, rtol=1e-13)


def test_brute_force_tiny():
    """Scalar loops with math.cos/sin over a 1x2x3 grid, 2 heads, d = 128."""
    grid = (1, 2, 3)
    xb = rand_bits((1, 6, 2, 128), seed=9)
    x = widen(xb)
    out = qk_norm_rope(xb, grid, eps=EPS, theta=10000.0)
    split = [("t", 22), ("h", 21), ("w", 21)]
    for n in range(6):
        t, hh, ww = 0, n // 3, n % 3
        p = {"t": t, "h": hh, "w": ww}
        for h in range(2):
            row = [float(v) for v in x[0, n, h]]
            ms = sum(v * v for v in row) / 128.0
            r = 1.0 / math.sqrt(ms + EPS32)
            y = [v * r for v in row]
            i = 0
            for name, cnt in split:
                for k in range(cnt):
                    phi = p[name] * 10000.0 ** (-k / cnt)
                    a, b = y[2 * i], y[2 * i + 1]
                    assert out[0, h, n, 2 * i] == pytest.approx(a * math.cos(phi) - b * math.sin(phi), abs=1e-13)
                    assert out[0, h, n, 2 * i + 1] == pytest.approx(a * math.sin(phi) + b * math.cos(phi), abs=1e-13)
                    i += 1


def test_v_is_only_relaid():
    vb = rand_bits((2, 5, 3, 128), seed=10)
    out = v_head_major(vb)
    assert out.dtype == np.uint16 and out.shape == (2, 3, 5, 128)
    for b in range(2):
        for n in range(5):
            for h in range(3):
                assert np.array_equal(out[b, h, n], vb[b, n, h])


def test_selected_tokens_match_the_full_evaluation():
    xb = rand_bits((2, 60, 3, 128), seed=11)
    full = qk_norm_rope(xb, (3, 4, 5))
    toks = [0, 7, 19, 20, 59]
    assert np.array_equal(qk_norm_rope(xb, (3, 4, 5), tokens=toks), full[:, :, toks])


# ---------------------------------------------------------------- packed prologue (RMSNorm only)
def test_qk_norm_brute_force_tiny():
    """Scalar loops over a 3-token, 2-head packed batch: y = x / sqrt(mean x^2 + eps) * w."""
    from oracle import qk_norm
    xb = rand_bits((3, 2, 128), seed=21)
    w = np.random.default_rng(22).uniform(0.5, 1.5, 128)
    out = qk_norm(xb, weight=w, eps=EPS)
    x = widen(xb)
    for t in range(3):
        for h in range(2):
            row = [float(v) for v in x[t, h]]
            r = 1.0 / math.sqrt(math.fsum(v * v for v in row) / 128.0 + EPS32)
            for c in (0, 1, 64, 127):
                assert out[t, h, c] == pytest.approx(row[c] * r * w[c], rel=1e-14, abs=1e-300)


def test_qk_norm_closed_forms():
    """RMS of each output row is sqrt(ms / (ms + eps)) without a weight; a row of +-a gives
    +-a / sqrt(a^2 + eps); the weight scales each channel; rows are independent."""
    from oracle import qk_norm
    xb = rand_bits((5, 3, 128), seed=23, scale=3.0)
    x = widen(xb)
    y = qk_norm(xb, eps=EPS)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(ms / (ms + EPS32)), rtol=1e-13)
    a = 0.375                                          # exact in BF16
    row = np.where(np.arange(128) % 3 == 0, -a, a)
    yb = qk_norm(bits(row[None, None, :]), eps=EPS)[0, 0]
    np.testing.assert_allclose(yb, row / math.sqrt(a * a + EPS32), rtol=1e-15)
    w = np.linspace(0.25, 2.0, 128)
    np.testing.assert_allclose(qk_norm(xb, weight=w, eps=EPS), y * w, rtol=1e-15)
    x2 = xb.copy()
    x2[2, 1] = bits(np.full(128, 7.0))
    y2 = qk_norm(x2, eps=EPS)
    mask = np.ones((5, 3), bool)
    mask[2, 1] = False
    np.testing.assert_array_equal(y2[mask], y[mask])


def test_qk_norm_is_the_unrotated_prologue_of_token_zero():
    """Position 0 turns no pair, so token 0 of the 3-D prologue is the plain RMSNorm."""
    from oracle import qk_norm
    xb = rand_bits((1, 6, 4, 128), seed=24)
    dense = qk_norm_rope(xb, (1, 2, 3), eps=EPS)        # [1, H, N, d]
    packed = qk_norm(xb[0], eps=EPS)                    # the same rows seen as THD [N, H, d]
    np.testing.assert_allclose(packed[0], dense[0, :, 0], rtol=1e-15, atol=1e-300)
    assert not np.allclose(packed[1], dense[0, :, 1])   # later tokens are rotated there


def test_qk_norm_selected_tokens():
    from oracle import qk_norm
    xb = rand_bits((40, 2, 128), seed=25)
    toks = np.array([0, 7, 39])
    np.testing.assert_array_equal(qk_norm(xb, eps=EPS, tokens=toks), qk_norm(xb, eps=EPS)[toks])
