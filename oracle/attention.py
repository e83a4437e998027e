"""FP64 CPU oracle for the non-causal scaled-dot-product attention forward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import or call this module. The product path (the HIP library and its
Python binding) never does, and this module imports nothing from it.

What is computed is the plain definition of softmax attention, written out in float64:
for one (batch, head) -- or one (segment, head) of a packed batch -- and every checked
query row i over the keys j of its own sequence,

    x_ij  = s * sum_c q_ic k_jc          (s = the FP32 scale argument, widened exactly)
    m_i   = max_j x_ij
    p_ij  = exp(x_ij - m_i)
    l_i   = sum_j p_ij
    o_i   = (sum_j p_ij v_j) / l_i
    lse_i = m_i + ln l_i                 (natural log of the scaled logits)

Sources: page "[sglang] SANA-Video 2.0 anchor attention ... FP32 upcast" (blog on PR #49219),
section "code analysis" item 1: the fast path is ``scaled_dot_product_attention(q, k, v,
dropout_p=0.0)`` on equal-shape 4-D BF16 tensors, i.e. non-causal, no mask, no dropout,
default scale 1/sqrt(d); the "lessons" list in the same page: flash attention accumulates
QK^T, softmax and PV in FP32 from BF16 inputs. Page "PR #33702 report", motivation and
breakdown item 2: packed tokens go through a varlen forward whose attention is confined to
each sequence (THD layout), head size 128. Subtracting m_i is the usual exact rewrite that
keeps exp() finite; it does not change o or lse.

The oracle does not model any rounding of the fast kernel (BF16 probabilities, BF16
output); comparisons absorb that with stated tolerances.

Inputs are BF16 bit patterns (uint16); ``bf16_bits_to_f64`` widens them exactly.
Row blocks bound memory: a block of R rows holds an R x N float64 logit matrix.
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 128


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns: the 16 bits are the top half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def scale_as_used(scale: float) -> float:
    """The kernel receives the scale as an FP32 argument; the oracle uses that same value."""
    return float(np.float32(scale))


def softmax_probabilities(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """p_ij = exp(x_ij - m_i) / l_i for float64 q [Nq,d], k [Nk,d] (small cases only)."""
    x = scale_as_used(scale) * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    p = np.exp(x - x.max(axis=1, keepdims=True))
    return p / p.sum(axis=1, keepdims=True)


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   block: int = ROW_BLOCK):
    """Attention of float64 query rows q [R,d] over one sequence k, v [Nk,d].

    Returns (o [R,d] float64, lse [R] float64).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = scale_as_used(scale)
    o = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.empty(q.shape[0], dtype=np.float64)
    kt = np.ascontiguousarray(k.T)
    for i0 in range(0, q.shape[0], block):
        x = s * (q[i0:i0 + block] @ kt)
        m = x.max(axis=1, keepdims=True)
        p = np.exp(x - m)
        l = p.sum(axis=1, keepdims=True)
        o[i0:i0 + block] = (p @ v) / l
        lse[i0:i0 + block] = m[:, 0] + np.log(l[:, 0])
    return o, lse


def attention_dense(q_bits, k_bits, v_bits, scale: float, rows=None):
    """Dense [B,H,N,d] attention from BF16 bits.

    rows=None: returns o [B,H,N,d] and lse [B,H,N] (float64).
    rows=flat indices r = (b*H + h)*N + n: returns o [len(rows), d] and lse [len(rows)],
    in the order given.
    """
    B, H, N, d = q_bits.shape
    if rows is None:
        o = np.empty((B, H, N, d), dtype=np.float64)
        lse = np.empty((B, H, N), dtype=np.float64)
        for b in range(B):
            for h in range(H):
                o[b, h], lse[b, h] = attention_rows(bf16_bits_to_f64(q_bits[b, h]),
                                                    bf16_bits_to_f64(k_bits[b, h]),
                                                    bf16_bits_to_f64(v_bits[b, h]), scale)
        return o, lse
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    bh_of = rows // N
    for bh in np.unique(bh_of):
        sel = np.nonzero(bh_of == bh)[0]
        b, h = divmod(int(bh), H)
        n = rows[sel] - bh * N
        o[sel], lse[sel] = attention_rows(bf16_bits_to_f64(q_bits[b, h, n]),
                                          bf16_bits_to_f64(k_bits[b, h]),
                                          bf16_bits_to_f64(v_bits[b, h]), scale)
    return o, lse


def attention_varlen(q_bits, k_bits, v_bits, cu_seqlens, scale: float, rows=None):
    """Packed THD [T,H,d] attention confined to the segments [cu[s], cu[s+1]).

    rows=None: returns o [T,H,d] and lse [H,T] (float64).
    rows=flat indices r = h*T + t: returns o [len(rows), d] and lse [len(rows)].
    """
    T, H, d = q_bits.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if rows is None:
        o = np.empty((T, H, d), dtype=np.float64)
        lse = np.empty((H, T), dtype=np.float64)
        for s in range(cu.size - 1):
            a, e = int(cu[s]), int(cu[s + 1])
            if e == a:
                continue
            for h in range(H):
                o[a:e, h], lse[h, a:e] = attention_rows(bf16_bits_to_f64(q_bits[a:e, h]),
                                                        bf16_bits_to_f64(k_bits[a:e, h]),
                                                        bf16_bits_to_f64(v_bits[a:e, h]), scale)
        return o, lse
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    h_of, t_of = rows // T, rows % T
    seg_of = np.searchsorted(cu, t_of, side="right") - 1
    for key in np.unique(seg_of * H + h_of):
        s, h = divmod(int(key), H)
        sel = np.nonzero((seg_of == s) & (h_of == h))[0]
        a, e = int(cu[s]), int(cu[s + 1])
        o[sel], lse[sel] = attention_rows(bf16_bits_to_f64(q_bits[t_of[sel], h]),
                                          bf16_bits_to_f64(k_bits[a:e, h]),
                                          bf16_bits_to_f64(v_bits[a:e, h]), scale)
    return o, lse
