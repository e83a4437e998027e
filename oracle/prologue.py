"""FP64 CPU oracle for the attention prologue: per-head RMSNorm and interleaved 3-D RoPE on Q
and K, V passed through, all written in the attention kernel's [B, H, N, d] layout.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or call this module. The product path never does, and this module
imports nothing from it.

What is computed, for one token n of batch b and head h (x = the BF16 input row, widened
exactly; d = 128):

    ms      = (1/d) sum_c x_c^2
    y_c     = x_c / sqrt(ms + eps) * w_c                (w = 1 when no weight is given)
    for each interleaved pair i (channels 2i, 2i+1), on axis a(i) with index k(i) < P_a:
        phi = pos_a(n) * theta^(-k / P_a)
        out_2i   = y_2i cos(phi) - y_2i+1 sin(phi)
        out_2i+1 = y_2i sin(phi) + y_2i+1 cos(phi)
    the 64 pairs are split over the axes (t, h, w) as (22, 21, 21), in that order, and
    pos(n) = (n // (Hp*Wp), (n // Wp) % Hp, n % Wp) for a token grid (F, Hp, Wp).

Sources: page "PR #35728 report", section "key source excerpts" (``sana_video.py``
``forward``): the projected Q and K each go through an RMSNorm (``norm_q``, ``norm_k``), are
viewed as [B, N, H, D], and get an interleaved rotary embedding (Q and K only; V is only
reshaped); page "[sglang] SANA-Video 2.0 anchor attention ... FP32 upcast", introduction:
Q/K/V reach the attention already BF16 after RMSNorm and RoPE; page "PR #35728 report",
related context: a fused 3-D RoPE kernel for the LTX-2.5 decoder. The pages give no eps, no
theta, no axis split and no position order: per-head normalisation, eps = 1e-6, theta =
10000, the (22, 21, 21) split and the raster order are readings (listed with the others).
The rotation of a pair is the complex product (y_2i + i y_2i+1) e^{i phi}.

Inputs are BF16 bit patterns (uint16) in token-major [B, N, H, d] order, as the QKV
projection produces them. The result is float64, unrounded; comparisons decide the BF16
rounding (see ``compare.bf16_faithful``).
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64

AXIS_PAIRS = (22, 21, 21)


def grid_positions(grid, n_tokens: int) -> np.ndarray:
    """[N, 3] int64 (t, h, w) of raster-ordered tokens on a (F, Hp, Wp) grid."""
    _, hp, wp = (int(g) for g in grid)
    n = np.arange(n_tokens, dtype=np.int64)
    return np.stack([n // (hp * wp), (n // wp) % hp, n % wp], axis=1)


def pair_frequencies(theta: float = 10000.0, axis_pairs=AXIS_PAIRS):
    """(axis [64], frequency [64]) of the interleaved pairs: pair i of axis a at index k turns
    by theta^(-k/P_a) radians per position step."""
    axis, freq = [], []
    for a, p in enumerate(axis_pairs):
        for k in range(p):
            axis.append(a)
            freq.append(float(theta) ** (-k / p))
    return np.array(axis, dtype=np.int64), np.array(freq, dtype=np.float64)


def qk_norm_rope(x_bits, grid, weight=None, eps: float = 1e-6, theta: float = 10000.0,
                 axis_pairs=AXIS_PAIRS, tokens=None) -> np.ndarray:
    """RMSNorm over each head row, then interleaved 3-D RoPE; [B, N, H, d] uint16 ->
    [B, H, N, d] float64. With `tokens` (indices into N), only those tokens are evaluated
    (each token depends on its own rows and position only) and the result is
    [B, H, len(tokens), d]."""
    x_bits = np.asarray(x_bits, np.uint16)
    B, N, H, d = x_bits.shape
    assert d == 2 * sum(axis_pairs)
    assert N == int(np.prod(grid)), "the grid must cover the tokens"
    toks = np.arange(N) if tokens is None else np.asarray(tokens, np.int64)
    x = bf16_bits_to_f64(x_bits[:, toks])
    w = np.ones(d) if weight is None else np.asarray(weight, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + float(np.float32(eps))) * w
    axis, freq = pair_frequencies(theta, axis_pairs)
    pos = grid_positions(grid, N)[toks].astype(np.float64)    # [n, 3]
    phi = pos[:, axis] * freq                                  # [n, 64]
    c = np.cos(phi)[None, :, None, :]
    s = np.sin(phi)[None, :, None, :]
    ye, yo = y[..., 0::2], y[..., 1::2]
    out = np.empty_like(y)
    out[..., 0::2] = ye * c - yo * s
    out[..., 1::2] = ye * s + yo * c
    return np.ascontiguousarray(out.transpose(0, 2, 1, 3))


def qk_norm(x_bits, weight=None, eps: float = 1e-6, tokens=None) -> np.ndarray:
    """Per-head RMSNorm of packed (THD) rows, [T, H, d] uint16 -> [T, H, d] float64 (or the
    rows of `tokens` only): y_c = x_c / sqrt(mean_c x^2 + eps) * w_c.

    The prologue of the packed (varlen) path. Page "PR #35728 report", key source excerpts:
    the projected Q and K go through an RMSNorm before attention; page "PR #33702 report",
    motivation: packed tokens reach the varlen forward in the THD layout, which is the
    projection's own token-major layout. The pages give no positions for packed segments, so
    no rotation is applied here (the packed workload's recipe is RMSNorm only); eps and the
    per-head reading as for qk_norm_rope."""
    x_bits = np.asarray(x_bits, np.uint16)
    toks = slice(None) if tokens is None else np.asarray(tokens, np.int64)
    x = bf16_bits_to_f64(x_bits[toks])
    w = np.ones(x.shape[-1]) if weight is None else np.asarray(weight, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(np.float32(eps))) * w


def v_head_major(v_bits) -> np.ndarray:
    """V is not transformed, only laid out [B, N, H, d] -> [B, H, N, d] (uint16, exact)."""
    return np.ascontiguousarray(np.asarray(v_bits, np.uint16).transpose(0, 2, 1, 3))
