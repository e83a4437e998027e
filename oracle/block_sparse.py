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


def decision_margin(q_bits, k_bits, scale: float, tau: float, bm: int = QUERY_BLOCK,
                    bn: int = KEY_BLOCK) -> np.ndarray:
    """[B, H, ntq, ntk]: half-width of the band around the threshold inside which an FP32
    evaluation of the rule (block sums and the d-term dot product in FP32, any order) may
    decide differently from the exact one.

    With u = 2^-24, A_I and B_J the per-channel means of |q| over block I and of |k| over
    block J: an FP32 block mean is off by at most (rows + 1) u times the mean magnitude of its
    channel (a sum of `rows` terms, then one scaling), and a dot product of d terms by at most
    (d + 1) u times the sum of the magnitudes of its products. So an FP32 z_IJ is off by at
    most s u [(bm + 1) A_I.|kbar_J| + (bn + 1) |qbar_I|.B_J + (d + 3) |qbar_I|.|kbar_J|]
    (the last term also covers the scaling by s and the cross terms). z_IJ and the block
    maximum both carry such an error, and forming zmax - tau adds one rounding."""
    B, H, N, d = q_bits.shape
    s = abs(scale_as_used(scale))
    u = 2.0 ** -24
    t = 0.0 if math.isinf(tau) else abs(float(tau))
    ntq, ntk = -(-N // bm), -(-N // bn)
    out = np.empty((B, H, ntq, ntk))
    for b in range(B):
        for h in range(H):
            q = bf16_bits_to_f64(q_bits[b, h])
            k = bf16_bits_to_f64(k_bits[b, h])
            A, Bk = pooled_means(np.abs(q), bm), pooled_means(np.abs(k), bn)
            qb, kb = pooled_means(q, bm), pooled_means(k, bn)
            e = s * u * ((bm + 1) * (A @ np.abs(kb).T) + (bn + 1) * (np.abs(qb) @ Bk.T)
                         + (d + 3) * (np.abs(qb) @ np.abs(kb).T))
            zmax = (scale_as_used(scale) * (qb @ kb.T)).max(axis=1)
            out[b, h] = e + e.max(axis=1, keepdims=True) + 2 * u * (np.abs(zmax)[:, None] + t)
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
