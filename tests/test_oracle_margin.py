"""Pins of the FP32 decision band of block-skip routing (oracle.block_sparse.proxy_error,
block_mean_error, decision_margin).

The GPU evaluates the routing proxies z_IJ = s * qbar_I . kbar_J in binary32, so a tile whose
exact z lies within binary32 rounding of the threshold may be kept or dropped either way; the
GPU tests accept a differing decision only inside the band. A band that is too narrow fails
correct kernels, one that is too wide hides routing bugs. Both sides are pinned here:

  * the band holds: binary32 replays of the rule in four evaluation orders (the routing kernel's
    own -- 16 row lanes of strided rows added in lane order, one division, a fused
    multiply-add chain over the 128 channels, one scaling -- and sequential, pairwise and
    reversed row sums with fused or unfused products) never leave it, on Gaussian, RMSNorm'd,
    cancellation-heavy and exponent-spread inputs, and replayed decisions differ from the exact
    ones only inside it;
  * the band is tight: on inputs shaped like the workloads it is at most 100 times the largest
    replayed error, and on inputs built to push one evaluation order to its worst case the
    replayed error reaches a large part of it (the dot chain and the block sums separately).

The replays use numpy binary32 arithmetic (correctly rounded +, *, /) and an exactly rounded
fused multiply-add (pinned against rational arithmetic below).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.attention import bf16_bits_to_f64
from oracle.block_sparse import block_mean_error, decision_margin, proxy_error, proxy_logits, route_blocks
from workloads import random_dense
from workloads.synth import rmsnorm_rows

f32, f64 = np.float32, np.float64
S128 = 1 / math.sqrt(128)


def bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------- binary32 replays

def fma32(a, b, c):
    """round_to_nearest_even(a*b + c) for binary32 arrays: the product is exact in binary64,
    TwoSum gives the exact residual of the binary64 sum, and the one case where rounding that
    sum to binary32 differs from rounding the exact value -- the sum sitting exactly on a
    binary32 midpoint with a nonzero residual -- is corrected toward the residual."""
    a, b, c = (np.asarray(x, f32) for x in (a, b, c))
    p = a.astype(f64) * b.astype(f64)
    c64 = c.astype(f64)
    s = p + c64
    bb = s - p
    err = (p - (s - bb)) + (c64 - bb)
    r = s.astype(f32)
    r64 = r.astype(f64)
    other = np.where(s > r64, np.nextafter(r, f32(np.inf)), np.nextafter(r, f32(-np.inf)))
    o64 = other.astype(f64)
    mid = (s != r64) & (s == (r64 + o64) / 2) & (err != 0) & (np.sign(err) == np.sign(o64 - r64))
    return np.where(mid, other, r)


def pool32(x, block, order):
    """binary32 means of the row blocks of x (float64 holding BF16 values) in a given order."""
    n, d = x.shape
    out = []
    for j in range(-(-n // block)):
        xb = x[j * block:(j + 1) * block].astype(f32)
        m = xb.shape[0]
        s = np.zeros(d, f32)
        if order == "kernel":          # 16 row lanes over rows rl, rl+16, ...; lanes added in order
            for rl in range(16):
                acc = np.zeros(d, f32)
                for r in range(rl, m, 16):
                    acc = acc + xb[r]
                s = s + acc
        elif order == "seq":
            for r in range(m):
                s = s + xb[r]
        elif order == "rev":
            for r in range(m - 1, -1, -1):
                s = s + xb[r]
        elif order == "pairwise":      # numpy's own blocked pairwise reduction
            s = xb.sum(axis=0, dtype=f32)
        out.append(s / f32(m))
    return np.array(out, f32).reshape(-1, d)


def z32(qb, kb, scale, fused):
    """binary32 proxies from binary32 means: a chain over the channels, then one scaling."""
    ntq, ntk = qb.shape[0], kb.shape[0]
    z = np.zeros((ntq, ntk), f32)
    for c in range(qb.shape[1]):
        a = np.broadcast_to(qb[:, c:c + 1], (ntq, ntk))
        b = np.broadcast_to(kb[None, :, c], (ntq, ntk))
        z = fma32(a, b, z) if fused else (a * b).astype(f32) + z
    return (z * f32(scale)).astype(f32)


ORDERS = [("kernel", True), ("seq", False), ("pairwise", True), ("rev", False)]


def replay(q_bits, k_bits, scale, order, fused):
    B, H, N, _ = q_bits.shape
    out = np.empty((B, H, -(-N // 256), -(-N // 64)))
    for b in range(B):
        for h in range(H):
            out[b, h] = z32(pool32(bf16_bits_to_f64(q_bits[b, h]), 256, order),
                            pool32(bf16_bits_to_f64(k_bits[b, h]), 64, order), float(f32(scale)), fused)
    return out


# ----------------------------------------------------------------- the replay's own pin

def test_fma32_is_exactly_rounded():
    rng = np.random.default_rng(3)
    a = (rng.standard_normal(4000) * 2.0 ** rng.integers(-20, 20, 4000)).astype(f32)
    b = (rng.standard_normal(4000) * 2.0 ** rng.integers(-20, 20, 4000)).astype(f32)
    c = (rng.standard_normal(4000) * 2.0 ** rng.integers(-40, 40, 4000)).astype(f32)
    # a*b = 1 + 2^-11 + 2^-24 sits exactly on the binary32 midpoint above 1 + 2^-11; c = +-2^-60
    # is lost in the binary64 sum, so only the residual decides: up for +, down (to even) for -,
    # and a plain tie (c = 0) goes to even
    a[:12] = b[:12] = f32(1.0 + 2.0 ** -12)
    c[:4], c[4:8], c[8:12] = f32(2.0 ** -60), f32(-(2.0 ** -60)), f32(0.0)
    got = fma32(a, b, c)
    for i in range(a.size):
        exact = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        lo = f32(float(exact))
        cand = [lo, np.nextafter(lo, f32(-np.inf)), np.nextafter(lo, f32(np.inf))]
        dist = [abs(Fraction(float(x)) - exact) for x in cand]
        best = min(dist)
        ties = [x for x, dd in zip(cand, dist) if dd == best]
        want = ties[0] if len(ties) == 1 else [x for x in ties if (int(np.asarray(x).view(np.uint32)) & 1) == 0][0]
        assert got[i] == want, (i, a[i], b[i], c[i], got[i], want)
    assert got[0] == np.nextafter(f32(1.0 + 2.0 ** -11), f32(2.0))
    assert got[4] == got[8] == f32(1.0 + 2.0 ** -11)


# ----------------------------------------------------------------- the band holds

def test_block_mean_error_holds_in_any_order():
    rng = np.random.default_rng(11)
    cases = [rng.standard_normal((256, 16)),
             rng.standard_normal((64, 16)) * 2.0 ** rng.integers(-20, 21, (64, 1)),
             np.concatenate([np.full((31, 16), 256.0), rng.standard_normal((33, 16)) * 1e-4]),
             rng.standard_normal((37, 16)) * 1e3]
    for x in cases:
        x = bf16_bits_to_f64(bits(x))
        bound = block_mean_error(x, x.shape[0])[0]
        exact = x.mean(axis=0)
        for order in ("kernel", "seq", "rev", "pairwise"):
            assert np.all(np.abs(pool32(x, x.shape[0], order)[0] - exact) <= bound), order
        for _ in range(20):                     # random association trees
            vals = [v for v in x.astype(f32)]
            while len(vals) > 1:
                i = int(rng.integers(0, len(vals) - 1))
                vals[i:i + 2] = [vals[i] + vals[i + 1]]
            assert np.all(np.abs((vals[0] / f32(x.shape[0])).astype(f64) - exact) <= bound)


def _inputs():
    rng = np.random.default_rng(5)
    N = 1000
    out = {"normal": random_dense(1, 2, N, seed=5)[:2],
           "normal_x30": random_dense(1, 1, N, seed=6, std=30.0)[:2],
           "rmsnorm": tuple(bits(rmsnorm_rows(rng.standard_normal((1, 1, N, 128)).astype(f32))) for _ in range(2))}
    sign = np.where(np.arange(N) % 2 == 0, 1.0, -1.0)[None, None, :, None]
    out["cancelling"] = (bits(rng.standard_normal((1, 1, N, 128)) * sign + 1e-3 * rng.standard_normal((1, 1, N, 128))),
                         bits(rng.standard_normal((1, 1, N, 128)) * sign + 1e-2))
    out["exponent_spread"] = tuple(bits(rng.standard_normal((1, 1, N, 128)) * 2.0 ** rng.integers(-14, 15, (1, 1, N, 1)))
                                   for _ in range(2))
    return out


INPUTS = _inputs()
WORKLOAD_LIKE = ("normal", "normal_x30", "rmsnorm", "cancelling")


@pytest.mark.parametrize("name", list(INPUTS))
def test_replays_stay_inside_the_bound(name):
    q, k = INPUTS[name]
    e = proxy_error(q, k, S128)
    z = proxy_logits(q, k, S128)
    worst = 0.0
    for order, fused in ORDERS:
        err = np.abs(replay(q, k, S128, order, fused) - z)
        assert np.all(err <= e), (name, order, float((err / e).max()))
        worst = max(worst, float(err.max()))
    if name in WORKLOAD_LIKE:
        # tight: within 100x of what a binary32 evaluation actually does on such inputs
        assert e.max() <= 100 * worst, (name, e.max(), worst)
    print(f"[band] {name}: bound max {e.max():.3e}, replayed error max {worst:.3e}, ratio {e.max() / worst:.1f}")


@pytest.mark.parametrize("tau", [0.0, 0.004, 0.008, 0.02])
def test_replayed_decisions_differ_only_inside_the_band(tau):
    q, k = INPUTS["normal"]
    keep, z, zmax = route_blocks(q, k, S128, tau)
    mg = decision_margin(q, k, S128, tau)
    inside = np.abs(z - (zmax[..., None] - tau)) <= mg
    for order, fused in ORDERS:
        zr = replay(q, k, S128, order, fused)
        thr = (zr.max(axis=-1) - f32(tau)).astype(f32)[..., None]   # the kernel forms max - tau in binary32
        diff = (zr >= thr) != keep
        assert not (diff & ~inside).any(), (order, tau)


def test_masked_margin_equals_the_full_one():
    q, k = INPUTS["normal"]
    full = decision_margin(q, k, S128, 0.008)
    mask = np.zeros(full.shape, bool)
    mask[0, 1, 2, [0, 5, 15]] = True
    mask[0, 0, 3, 7] = True
    part = decision_margin(q, k, S128, 0.008, mask=mask)
    np.testing.assert_array_equal(part[mask], full[mask])
    assert np.isnan(part[~mask]).all()
    pe = proxy_error(q, k, S128, pairs=np.nonzero(mask))
    np.testing.assert_array_equal(pe, proxy_error(q, k, S128)[mask])


# ----------------------------------------------------------------- the band is not loose

def test_dot_chain_worst_case_reaches_the_bound():
    """Equal rows make the block means exact; then q = (1, 2^-12, ...), k = (1, 0.8125 2^-12, ...)
    put every later product at 0.41 units in the last place of the partial sum 1, so each step
    of the chain rounds it away the same way."""
    q = np.full((1, 1, 512, 128), 2.0 ** -12)
    k = np.full((1, 1, 512, 128), 0.8125 * 2.0 ** -12)
    q[..., 0] = k[..., 0] = 1.0
    q, k = bits(q), bits(k)
    e = proxy_error(q, k, 1.0)
    mg = decision_margin(q, k, 1.0, 0.0)
    err = np.abs(replay(q, k, 1.0, "kernel", True) - proxy_logits(q, k, 1.0))
    assert np.all(err <= e)
    assert err.min() >= 0.5 * e.max()
    assert err.min() >= 0.25 * mg.max()
    print(f"[band] dot worst case: error {err.max():.3e}, bound {e.max():.3e}, margin {mg.max():.3e}")


def test_block_sum_worst_case_reaches_the_bound():
    """Key blocks of 31 rows of 256 (sum 7936, just under 2^13, so the grid g of the bound is
    2^-11 = the spacing of the partial sums) followed by 33 rows of 0.4921875 g: added in row
    order after the large ones, each small value is rounded away."""
    N = 256
    k = np.zeros((1, 1, N, 128))
    for t in range(N // 64):
        k[0, 0, 64 * t:64 * t + 31, 0] = 256.0
        k[0, 0, 64 * t + 31:64 * t + 64, 0] = 0.4921875 * 2.0 ** -11
    q = np.zeros((1, 1, N, 128))
    q[..., 0] = 1.0
    q, k = bits(q), bits(k)
    e = proxy_error(q, k, 1.0)
    mg = decision_margin(q, k, 1.0, 0.0)
    err = np.abs(replay(q, k, 1.0, "seq", False) - proxy_logits(q, k, 1.0))
    assert np.all(err <= e)
    assert err.min() >= 0.4 * e.max()
    assert err.min() >= 0.2 * mg.max()
    print(f"[band] block-sum worst case: error {err.max():.3e}, bound {e.max():.3e}, margin {mg.max():.3e}")


def test_a_planted_slip_is_caught():
    """Mistakes a band could hide: dropping one row of a 256-row query block moves z by far more
    than the band on Gaussian inputs, so a GPU kernel with that slip would be caught wherever it
    moves a tile across the threshold."""
    q, k = INPUTS["normal"]
    z = proxy_logits(q, k, S128)
    qs = q.copy()
    qs[:, :, 255] = bits(np.zeros(128))         # a pooling that loses row 255 of block 0
    moved = np.abs(proxy_logits(qs, k, S128)[:, :, 0] - z[:, :, 0])
    assert np.median(moved) > 20 * decision_margin(q, k, S128, 0.008)[:, :, 0].max()
