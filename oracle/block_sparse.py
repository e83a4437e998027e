"""FP64 CPU oracle for block-skip attention: key blocks routed per query block by a threshold
on pooled proxy logits, then exact softmax attention over the kept keys.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or call this module. The product path never does, and this module
imports nothing from it.

Source: page "PR #33702 report" (the Sol-Attn backend for MiniMax-H3), motivation and
breakdown: a training-free sparse attention that, inside the online-softmax pass, routes KV
blocks by a threshold and so skips much of the work without building a full proxy score map;
its knobs are a threshold ``tau`` (with a threshold type), ``sink_tokens``, and a dense guard
(``dense_steps`` first denoising steps and ``dense_layers`` stay dense); head size 128 only,
BF16 only. The page gives no formula for the proxy or the threshold. The rule here is a
reading of it (stated once, used by both sides):

    query block I  = BM = 256 consecutive query rows of one (batch, head)
    key block J    = BN = 64 consecutive keys of the same (batch, head)
    qbar_I, kbar_J = the means of the valid rows of the blocks (BF16 inputs widened exactly)
    z_IJ           = s * qbar_I . kbar_J            (s = the FP32 scale argument)
    keep(I, J)     = z_IJ >= max_J' z_IJ' - tau   or   J * BN < sink_tokens

    for a query row i of block I, the kept keys are the union of the kept blocks J, and
    x_ij, m_i, p_ij, l_i, o_i, lse_i are the plain softmax-attention definitions over them.

``tau = +inf`` keeps every block and gives dense attention. The block of the largest proxy
is always kept, so no row is left without keys.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import attention_rows, bf16_bits_to_f64, scale_as_used

QUERY_BLOCK = 256
KEY_BLOCK = 64


def pooled_means(x: np.ndarray, block: int) -> np.ndarray:
    """Means of consecutive row blocks of float64 x [N, d] -> [ceil(N/block), d]; the last
    block averages only its valid rows."""
    n = x.shape[0]
    nb = -(-n // block)
    out = np.empty((nb, x.shape[1]))
    for j in range(nb):
        out[j] = x[j * block:(j + 1) * block].mean(axis=0)
    return out


def proxy_logits(q_bits, k_bits, scale: float, bm: int = QUERY_BLOCK, bn: int = KEY_BLOCK) -> np.ndarray:
    """z [B, H, ntq, ntk] float64 for dense [B, H, N, d] BF16 bits."""
    B, H, N, _ = q_bits.shape
    s = scale_as_used(scale)
    ntq, ntk = -(-N // bm), -(-N // bn)
    z = np.empty((B, H, ntq, ntk))
    for b in range(B):
        for h in range(H):
            qb = pooled_means(bf16_bits_to_f64(q_bits[b, h]), bm)
            kb = pooled_means(bf16_bits_to_f64(k_bits[b, h]), bn)
            z[b, h] = s * (qb @ kb.T)
    return z


def route_blocks(q_bits, k_bits, scale: float, tau: float, sink_tokens: int = 0,
                 bm: int = QUERY_BLOCK, bn: int = KEY_BLOCK):
    """The kept blocks: (keep [B, H, ntq, ntk] bool, z [B, H, ntq, ntk], zmax [B, H, ntq])."""
    z = proxy_logits(q_bits, k_bits, scale, bm, bn)
    zmax = z.max(axis=-1)
    keep = z >= zmax[..., None] - float(tau)
    nsink = -(-int(sink_tokens) // bn) if sink_tokens > 0 else 0
    keep[..., :min(nsink, z.shape[-1])] = True
    return keep, z, zmax


def kept_keys(keep_row: np.ndarray, n: int, bn: int = KEY_BLOCK) -> np.ndarray:
    """Key indices (ascending) of the kept blocks of one query block."""
    blocks = np.nonzero(keep_row)[0]
    if blocks.size == 0:
        return np.zeros(0, np.int64)
    return np.concatenate([np.arange(j * bn, min((j + 1) * bn, n)) for j in blocks])


def attention_kept(q_bits, k_bits, v_bits, scale: float, keep, rows=None,
                   bm: int = QUERY_BLOCK, bn: int = KEY_BLOCK):
    """Softmax attention of dense [B, H, N, d] BF16 inputs where the rows of query block I see
    only the keys of its kept blocks (keep [B, H, ntq, ntk] bool).

    rows=None: o [B, H, N, d], lse [B, H, N]; rows = flat indices (b*H + h)*N + n: o [len, d],
    lse [len] in the order given. A row whose block keeps nothing gets o = 0, lse = -inf.
    """
    B, H, N, d = q_bits.shape
    keep = np.asarray(keep, bool)
    flat = np.arange(B * H * N) if rows is None else np.asarray(rows, np.int64)
    o = np.zeros((flat.size, d))
    lse = np.full(flat.size, -np.inf)
    bh_of, n_of = flat // N, flat % N
    for bh in np.unique(bh_of):
        b, h = divmod(int(bh), H)
        sel_bh = np.nonzero(bh_of == bh)[0]
        qb = n_of[sel_bh] // bm
        for I in np.unique(qb):
            sel = sel_bh[qb == I]
            keys = kept_keys(keep[b, h, I], N, bn)
            if keys.size == 0:
                continue
            o[sel], lse[sel] = attention_rows(bf16_bits_to_f64(q_bits[b, h, n_of[sel]]),
                                              bf16_bits_to_f64(k_bits[b, h, keys]),
                                              bf16_bits_to_f64(v_bits[b, h, keys]), scale)
    if rows is None:
        return o.reshape(B, H, N, d), lse.reshape(B, H, N)
    return o, lse


def kept_pairs(keep, N: int, bm: int = QUERY_BLOCK, bn: int = KEY_BLOCK) -> int:
    """Number of (query row, key) pairs the kept blocks cover: the work of the sparse pass."""
    keep = np.asarray(keep, bool)
    ntq, ntk = keep.shape[-2:]
    rows = np.minimum(bm, N - bm * np.arange(ntq))
    keys = np.minimum(bn, N - bn * np.arange(ntk))
    return int((keep.astype(np.int64) * rows[:, None] * keys[None, :]).sum())


U32 = 2.0 ** -24          # unit roundoff of binary32, round to nearest
F32_TINY = 2.0 ** -149    # spacing of the binary32 subnormals


def _pow2_at_least(x: np.ndarray) -> np.ndarray:
    """Smallest power of two >= x (x > 0), exactly (frexp, no logarithms)."""
    f, e = np.frexp(x)
    return np.ldexp(1.0, np.where(f == 0.5, e - 1, e).astype(np.int64))


def block_mean_error(x: np.ndarray, block: int) -> np.ndarray:
    """[ceil(N/block), d]: bound on |mean_fp32 - mean| for the per-channel mean of each row block
    of x (float64 [N, d] holding BF16 values exactly), where mean_fp32 adds the block's m values
    in binary32 in ANY order (any tree of round-to-nearest additions) and divides once by m.

    The sum part rests on two facts of round-to-nearest arithmetic. (1) If every leaf is a
    multiple of a power of two g and the leaves' magnitudes add up to at most 2^24 g, every
    partial sum is a multiple of g of at most 2^24 g, hence a binary32 number, so each addition
    is exact and the whole tree is exact. (2) Rounded addition is monotone in each operand, so
    the tree's result is monotone in each leaf. With S the sum of |x| and g the smallest power
    of two with S + m g <= 2^24 g, rounding every leaf that is not a multiple of g down (up) to
    one gives a tree that is exact by (1) and, by (2), a lower (upper) bound of the computed
    sum; the exact sum lies between the two as well. So the computed sum is off by at most g
    times the number of leaves that are not multiples of g. For BF16 inputs of unit size that
    number is nearly always zero: their 8 significant bits sit far above g.

    The classical bound of a tree of m - 1 additions, (m - 1) u S (1 + m u), holds as well;
    the smaller of the two is taken. The division adds one rounding, at most u times the
    computed mean.
    """
    n, d = x.shape
    nb = -(-n // block)
    out = np.empty((nb, d))
    for j in range(nb):
        xb = x[j * block:(j + 1) * block]
        m = xb.shape[0]
        S = np.abs(xb).sum(axis=0) * (1.0 + 2.0 ** -40)      # float64 sum: inflate past its own rounding
        g = np.maximum(_pow2_at_least(np.maximum(S, F32_TINY) / (2.0 ** 24 - m)), F32_TINY)
        fine = (np.fmod(xb, g) != 0).sum(axis=0)
        e_sum = np.minimum(g * fine, (m - 1) * U32 * S * (1.0 + m * U32))
        out[j] = e_sum / m + U32 * (np.abs(xb.sum(axis=0)) + e_sum) / m
    return out


def _chain_bound(qb, kb, eq, ek) -> tuple:
    """Error bound and |exact| of the dot products qbar_I . kbar_J for paired rows
    (qb, kb, eq, ek: [P, d]), evaluated in binary32 from computed means qb + dq, kb + dk
    (|dq| <= eq, |dk| <= ek) as a chain over the channels in index order, z_c = z_{c-1} +
    q_c k_c, fused (one rounding per step) or not (two). Running error analysis: step c errs by
    at most u |z_c| (+ u |q_c k_c| unfused), and |z_c| is at most the exact partial sum plus
    the input perturbation so far, times (1 + u)^c. A step whose computed product is exactly
    zero (both bounds zero) leaves z unchanged and is not charged."""
    d = qb.shape[-1]
    p = qb * kb
    dp = eq * np.abs(kb) + np.abs(qb) * ek + eq * ek                # input perturbation per term
    live = (np.abs(p) + dp) > 0
    Z = np.abs(np.cumsum(p, axis=-1)) + np.cumsum(dp, axis=-1)
    run = U32 * (1.0 + 2.0 * d * U32) * (live * (Z + np.abs(p) + dp)).sum(axis=-1)
    return dp.sum(axis=-1) + run, np.abs(p.sum(axis=-1))


def proxy_error(q_bits, k_bits, scale: float, pairs=None, bm: int = QUERY_BLOCK, bn: int = KEY_BLOCK):
    """Bound on |z_fp32 - z| for the proxies of dense [B, H, N, d] BF16 inputs, where z_fp32 is
    a binary32 evaluation of the rule: the block means as block_mean_error allows (any order,
    one division), the dot product as a chain over the channels in index order (fused or not,
    _chain_bound), then one multiplication by the FP32 scale (one more rounding).

    pairs=None: [B, H, ntq, ntk] for every pair. pairs = (b, h, I, J) index arrays: the bound of
    those pairs only, in that order (cheap at any N)."""
    B, H, N, d = q_bits.shape
    s = abs(scale_as_used(scale))
    ntq, ntk = -(-N // bm), -(-N // bn)
    slack = 2.0 ** -40                       # the float64 reference's own rounding
    if pairs is None:
        grid = np.meshgrid(np.arange(B), np.arange(H), np.arange(ntq), np.arange(ntk), indexing="ij")
        return proxy_error(q_bits, k_bits, scale, tuple(g.ravel() for g in grid), bm, bn).reshape(B, H, ntq, ntk)
    b_, h_, I_, J_ = (np.asarray(a, np.int64) for a in pairs)
    out = np.empty(b_.size)
    for bh in np.unique(b_ * H + h_):
        b, h = divmod(int(bh), H)
        sel = np.nonzero(b_ * H + h_ == bh)[0]
        q = bf16_bits_to_f64(q_bits[b, h])
        k = bf16_bits_to_f64(k_bits[b, h])
        qb, kb = pooled_means(q, bm), pooled_means(k, bn)
        eq, ek = block_mean_error(q, bm), block_mean_error(k, bn)
        for lo in range(0, sel.size, 4096):
            cut = sel[lo:lo + 4096]
            I, J = I_[cut], J_[cut]
            e_dot, zabs = _chain_bound(qb[I], kb[J], eq[I], ek[J])
            mag = (np.abs(qb[I]) * np.abs(kb[J])).sum(axis=-1)
            out[cut] = s * e_dot + U32 * s * (zabs + e_dot) + slack * s * mag
    return out


def decision_margin(q_bits, k_bits, scale: float, tau: float, mask=None, bm: int = QUERY_BLOCK,
                    bn: int = KEY_BLOCK) -> np.ndarray:
    """[B, H, ntq, ntk]: half-width of the band around the threshold inside which a binary32
    evaluation of the rule (proxy_error) may keep or drop a tile differently from the exact
    one: J may go either way only if |z_IJ - (zmax_I - tau)| <= margin_IJ.

    margin_IJ = e_IJ + E_I + u (|zmax_I| + E_I + tau), with e the proxy bound of the pair and
    E_I the bound of the computed row maximum: the computed max is the computed z of some tile
    J', which can exceed zmax only by e_IJ' for a tile with z_IJ' + e_IJ' >= zmax, and is at
    least z_IJ* - e_IJ* for the exact argmax J*. The candidates J' are found with the cheap
    order-free bound s (d + 2) u sum_c |qbar||kbar| plus the input perturbation, which is at
    least e. The subtraction of tau adds one rounding.

    mask=None: every entry. mask = bool [B, H, ntq, ntk]: the band at the marked entries only
    (NaN elsewhere), for large inputs where only a few entries need it."""
    B, H, N, d = q_bits.shape
    s = abs(scale_as_used(scale))
    t = 0.0 if math.isinf(tau) else abs(float(tau))
    ntq, ntk = -(-N // bm), -(-N // bn)
    mask = np.ones((B, H, ntq, ntk), bool) if mask is None else np.asarray(mask, bool)
    out = np.full((B, H, ntq, ntk), np.nan)
    for b, h in sorted({(int(b), int(h)) for b, h in zip(*np.nonzero(mask.any(axis=(2, 3))))}):
        q = bf16_bits_to_f64(q_bits[b, h])
        k = bf16_bits_to_f64(k_bits[b, h])
        qb, kb = pooled_means(q, bm), pooled_means(k, bn)
        eq, ek = block_mean_error(q, bm), block_mean_error(k, bn)
        z = scale_as_used(scale) * (qb @ kb.T)
        zmax = z.max(axis=1)
        for I in np.nonzero(mask[b, h].any(axis=1))[0]:
            crude = s * ((d + 2) * U32 * 1.01 * ((np.abs(qb[I]) + eq[I]) @ (np.abs(kb) + ek).T)
                         + eq[I] @ np.abs(kb).T + np.abs(qb[I]) @ ek.T + eq[I] @ ek.T)
            cand = np.nonzero(z[I] >= zmax[I] - crude)[0]
            want = np.nonzero(mask[b, h, I])[0]
            Js = np.concatenate([cand, want])
            e = proxy_error(q_bits, k_bits, scale, (np.full(Js.size, b), np.full(Js.size, h),
                                                    np.full(Js.size, I), Js), bm, bn)
            E = e[:cand.size].max()
            out[b, h, I, want] = e[cand.size:] + E + U32 * (abs(zmax[I]) + E + t)
    return out


# ---------------------------------------------------------------- packed (varlen) batches
# Page "PR #33702 report", motivation: the backend serves the packed varlen forward (THD
# layout, attention confined to each segment). Routing and attention are the rule above
# applied to each segment [cu[s], cu[s+1]) on its own: its query tiles are 256 of its rows,
# its key tiles 64 of its keys, counted from the segment start.

def segment_tiles(cu_seqlens, block: int) -> np.ndarray:
    """Offsets of each segment's first tile in the numbering segment by segment, tile by
    tile ([nseg + 1]; the last entry is the total number of tiles)."""
    cu = np.asarray(cu_seqlens, np.int64)
    counts = -(-(cu[1:] - cu[:-1]) // block)
    return np.concatenate([[0], np.cumsum(counts)])


def route_blocks_varlen(q_bits, k_bits, cu_seqlens, scale: float, tau: float, sink_tokens: int = 0,
                        bm: int = QUERY_BLOCK, bn: int = KEY_BLOCK):
    """Per segment s (empty ones skipped): (keep [H, ntq_s, ntk_s], z, zmax [H, ntq_s]) for THD
    [T, H, d] BF16 bits, as route_blocks on the segment seen as a [1, H, len, d] batch."""
    cu = np.asarray(cu_seqlens, np.int64)
    out = []
    for s in range(cu.size - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            out.append(None)
            continue
        qs = np.ascontiguousarray(np.asarray(q_bits)[a:e].transpose(1, 0, 2))[None]
        ks = np.ascontiguousarray(np.asarray(k_bits)[a:e].transpose(1, 0, 2))[None]
        keep, z, zmax = route_blocks(qs, ks, scale, tau, sink_tokens, bm, bn)
        out.append((keep[0], z[0], zmax[0]))
    return out


def attention_kept_varlen(q_bits, k_bits, v_bits, cu_seqlens, scale: float, keeps, rows=None,
                          bm: int = QUERY_BLOCK, bn: int = KEY_BLOCK):
    """Attention of THD [T, H, d] BF16 inputs where query tile i of segment s sees only the key
    tiles keeps[s][h, i] marks (keeps[s] bool [H, ntq_s, ntk_s], None for empty segments).

    rows=None: o [T, H, d], lse [H, T]; rows = flat indices h*T + t: o [len, d], lse [len]."""
    T, H, d = np.asarray(q_bits).shape
    cu = np.asarray(cu_seqlens, np.int64)
    flat = np.arange(H * T) if rows is None else np.asarray(rows, np.int64)
    o = np.zeros((flat.size, d))
    lse = np.full(flat.size, -np.inf)
    h_of, t_of = flat // T, flat % T
    seg_of = np.searchsorted(cu, t_of, side="right") - 1
    for s in np.unique(seg_of):
        a, e = int(cu[s]), int(cu[s + 1])
        sel_s = np.nonzero(seg_of == s)[0]
        for h in np.unique(h_of[sel_s]):
            sel_h = sel_s[h_of[sel_s] == h]
            qi = (t_of[sel_h] - a) // bm
            for i in np.unique(qi):
                sel = sel_h[qi == i]
                keys = a + kept_keys(keeps[s][h, i], e - a, bn)
                if keys.size == 0:
                    continue
                o[sel], lse[sel] = attention_rows(bf16_bits_to_f64(np.asarray(q_bits)[t_of[sel], h]),
                                                  bf16_bits_to_f64(np.asarray(k_bits)[keys, h]),
                                                  bf16_bits_to_f64(np.asarray(v_bits)[keys, h]), scale)
    if rows is None:
        return o.reshape(H, T, d).transpose(1, 0, 2), lse.reshape(H, T)
    return o, lse
