"""FP64 CPU oracle for the SANA-Video linear attention (ReLU feature map, rotated Q/K in the
numerator, un-rotated Q/K in the normaliser).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or call this module. The product path never does, and this module
imports nothing from it.

What is computed, per batch b and head h, over the N tokens of the sequence (rows of the
token-major [B, N, H, d] inputs; q, k are the ReLU-activated rows, q_rot, k_rot the same
rows after the rotary embedding, v the values; all BF16, widened exactly):

    ksum      = sum_m k_m                           [d]
    den_n     = q_n . ksum + eps                    (eps = 1e-15)
    kv        = sum_m v_m k_rot_m^T                 [d, d]   (kv[i, j] = sum_m v_mi k_rot_mj)
    out_n     = (kv q_rot_n) / den_n                [d]

which is the associative form of out_n = sum_m (q_rot_n . k_rot_m) v_m / sum_m (q_n . k_m).

Sources: page "PR #35728 report", section "key source excerpts": ``sana_video.py``
``forward`` (ReLU on the normalised Q and K, interleaved rotary embedding, permute to
[B, H, D, N], normaliser 1 / (K.sum(-1)^T Q + 1e-15) from the un-rotated K and Q, then
(V K_rot^T) Q_rot times the normaliser, flattened back to [B, N, H*D]); the site file
``try_sana_video_linear_attention``: the first product with BF16 inputs and FP32
accumulation/output, the second in FP32; section "risks": the BF16-input path differs from
the FP32 chain by about 1e-2. The page computes the normaliser in the activation dtype;
here it is exact (FP64), a reading listed with the others.

Inputs are BF16 bit patterns (uint16), token-major [B, N, H, d]; the result is float64
[B, N, H, d].
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64

LINEAR_EPS = 1e-15


def linear_attention(q_bits, k_bits, qr_bits, kr_bits, v_bits, eps: float = LINEAR_EPS,
                     tokens=None) -> np.ndarray:
    """SANA-Video linear attention, float64 [B, N, H, d] (or [B, len(tokens), H, d] for the
    selected query tokens; the key-side sums always run over all N tokens)."""
    k = bf16_bits_to_f64(k_bits)
    kr = bf16_bits_to_f64(kr_bits)
    v = bf16_bits_to_f64(v_bits)
    B, N, H, d = k.shape
    toks = np.arange(N) if tokens is None else np.asarray(tokens, np.int64)
    q = bf16_bits_to_f64(np.asarray(q_bits, np.uint16)[:, toks])
    qr = bf16_bits_to_f64(np.asarray(qr_bits, np.uint16)[:, toks])
    out = np.empty((B, len(toks), H, d))
    for b in range(B):
        for h in range(H):
            ksum = k[b, :, h].sum(axis=0)                 # [d]
            den = q[b, :, h] @ ksum + eps                 # [n]
            kv = v[b, :, h].T @ kr[b, :, h]               # [d, d]
            out[b, :, h] = (qr[b, :, h] @ kv.T) / den[:, None]
    return out


def linear_attention_quadratic(q_bits, k_bits, qr_bits, kr_bits, v_bits, eps: float = LINEAR_EPS):
    """The same result through the N x N form (small N only): out_n = sum_m (q_rot_n .
    k_rot_m) v_m / (sum_m q_n . k_m + eps)."""
    q, k, qr, kr, v = (bf16_bits_to_f64(x) for x in (q_bits, k_bits, qr_bits, kr_bits, v_bits))
    B, N, H, d = q.shape
    out = np.empty((B, N, H, d))
    for b in range(B):
        for h in range(H):
            a = qr[b, :, h] @ kr[b, :, h].T               # [N, N]
            den = (q[b, :, h] @ k[b, :, h].T).sum(axis=1) + eps
            out[b, :, h] = (a @ v[b, :, h]) / den[:, None]
    return out
