"""Seeded synthetic inputs for the attention forward: shapes, value recipes, BF16 encoding.

This module is the one piece shared by the FP64 oracle side and the HIP side. It holds
no attention arithmetic: it only draws random numbers, applies the input transforms that
sit *before* attention in a video DiT (per-head RMSNorm, interleaved 3-D RoPE, outlier
channels) and rounds the result to BF16 bit patterns (uint16) once.

Sources for the recipes:
  * Page "[sglang] SANA-Video 2.0 anchor attention ... FP32 upcast" (blog on PR #49219),
    introduction: Q/K/V reach the anchor-layer attention already cast to BF16 after RMSNorm
    and RoPE. Page "PR #35728 report", key source excerpts (``sana_video.py`` ``forward``):
    RMSNorm on Q and K and an interleaved rotary embedding on Q and K only.
  * Shapes, head counts, the 480p/720p token grids, the packed segment lengths and the
    stress recipe are the five synthetic workloads of this package. The pages print no
    values, so everything below the shape level (RMSNorm eps and weight, RoPE base and
    axis split, the outlier-channel draw) is a chosen reading, not a page fact.

Seeding: ``numpy.random.Generator(PCG64)`` children of ``SeedSequence([20261202, cfg_index])``,
one independent stream per (tensor, batch, head), so heads can be generated in parallel and
any head can be regenerated alone.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 20261202
HEAD_DIM = 128
RMS_EPS = 1e-6
ROPE_THETA = 10000.0
ROPE_AXIS_PAIRS = (22, 21, 21)  # (t, h, w) pairs of the 64 interleaved pairs at d=128
OUTLIER_CHANNELS = 4
OUTLIER_FACTOR = 16.0

# stream slots under the per-config SeedSequence
_Q, _K, _V, _OUTLIER, _ROWS, _RAGGED = range(6)


@dataclass(frozen=True)
class Workload:
    """One synthetic attention workload.

    kind     : "dense" ([B,H,N,d] contiguous) or "varlen" (THD [T,H,d] + cu_seqlens)
    qk       : value recipe for Q and K: "normal" | "rmsnorm" | "rmsnorm_rope" | "outliers"
    grid     : (frames, patches_h, patches_w) token grid for RoPE positions (raster order)
    seqlens  : varlen segment lengths
    ragged   : extra varlen call of the stress recipe (segment lengths), first segments
               reuse the dense batches bit for bit
    sample_rows : number of seeded query rows the oracle checks at full size (0 = all)
    """

    name: str
    index: int
    kind: str
    H: int
    qk: str
    B: int = 1
    N: int = 0
    d: int = HEAD_DIM
    grid: tuple | None = None
    seqlens: tuple | None = None
    ragged: tuple | None = None
    sample_rows: int = 0
    description: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens)) if self.kind == "varlen" else self.B * self.N

    def flops(self) -> float:
        """Attention work counted as 4*B*H*N^2*d (varlen: sum over segments of 4*H*n^2*d)."""
        if self.kind == "varlen":
            return float(sum(4.0 * self.H * n * n * self.d for n in self.seqlens))
        return 4.0 * self.B * self.H * float(self.N) ** 2 * self.d


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_dense", 0, "dense", H=2, B=1, N=256, qk="normal",
                 description="tiny dense attention B=1 H=2 N=256 d=128, Q/K/V ~ N(0,1)"),
        Workload("video_480p", 1, "dense", H=16, B=1, N=32760, qk="rmsnorm_rope", grid=(21, 30, 52),
                 sample_rows=512,
                 description="480p-like video self-attention B=1 H=16 N=32760 (21x30x52) d=128"),
        Workload("video_720p", 2, "dense", H=16, B=1, N=180320, qk="rmsnorm_rope", grid=(49, 46, 80),
                 sample_rows=512,
                 description="720p-like video self-attention B=1 H=16 N=180320 (49x46x80) d=128"),
        Workload("packed_varlen", 3, "varlen", H=24, qk="rmsnorm", seqlens=(30000, 6000, 2048),
                 sample_rows=512,
                 description="packed varlen attention T=38048 in segments 30000/6000/2048, H=24 d=128"),
        Workload("numerics_stress", 4, "dense", H=16, B=2, N=8192, qk="outliers",
                 ragged=(8192, 8192, 1, 127), sample_rows=1024,
                 description="numerics stress B=2 H=16 N=8192 d=128, 4 outlier channels x16 in Q and K"),
    )
}


# ----------------------------------------------------------------------------------------
# BF16 encoding (IEEE-754 binary32 -> bfloat16, round to nearest, ties to even)
# ----------------------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returns the uint16 bit patterns.

    bfloat16 keeps the top 16 bits of binary32. Rounding adds 0x7FFF plus the lowest kept
    bit (the ties-to-even bias) to the 32-bit pattern before truncating. NaN payloads are
    replaced by the quiet NaN of the same sign; overflow past the largest finite bfloat16
    correctly rounds to infinity.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    out = t.astype(np.uint16)
    if not np.isnan(u.view(np.float32)).any():
        return out
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16) | np.uint16(0x7FC0)
    return out


# ----------------------------------------------------------------------------------------
# Input transforms (FP32, applied before the single BF16 rounding)
# ----------------------------------------------------------------------------------------
def rmsnorm_rows(x: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Per-row RMSNorm over the last axis with unit weight, in float32."""
    x = x.astype(np.float32, copy=False)
    ms = np.mean(np.square(x, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
    return x * (np.float32(1.0) / np.sqrt(ms + np.float32(eps)))


def rope_positions(grid: tuple, n_tokens: int) -> np.ndarray:
    """(t, h, w) integer positions for raster-ordered tokens n -> (n // (Hp*Wp), (n // Wp) % Hp, n % Wp)."""
    _, hp, wp = grid
    n = np.arange(n_tokens, dtype=np.int64)
    return np.stack([n // (hp * wp), (n // wp) % hp, n % wp], axis=1)


def rope_tables(grid: tuple, n_tokens: int, d: int = HEAD_DIM):
    """cos/sin tables [N, d/2] (float32) for interleaved 3-D RoPE.

    The d/2 rotation pairs are split over the (t, h, w) axes as ROPE_AXIS_PAIRS; within an
    axis with P pairs, pair k turns by position * THETA^(-k/P).
    """
    assert sum(ROPE_AXIS_PAIRS) == d // 2
    pos = rope_positions(grid, n_tokens).astype(np.float64)
    angles = []
    for axis, npairs in enumerate(ROPE_AXIS_PAIRS):
        freq = ROPE_THETA ** (-np.arange(npairs, dtype=np.float64) / npairs)
        angles.append(pos[:, axis:axis + 1] * freq[None, :])
    ang = np.concatenate(angles, axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope_interleaved(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs (x[2i], x[2i+1]) of each row by the row's angles, float32."""
    x = x.astype(np.float32, copy=False)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out


# ----------------------------------------------------------------------------------------
# Generation
# ----------------------------------------------------------------------------------------
def _seed_children(w: Workload):
    return np.random.SeedSequence([ROOT_SEED, w.index]).spawn(6)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _head_block(w: Workload, role: int, ss: np.random.SeedSequence, n_tokens: int,
                outlier_ch: np.ndarray | None, rope: tuple | None) -> np.ndarray:
    """One head's [n_tokens, d] block of Q (role 0), K (1) or V (2) as BF16 bits."""
    rng = np.random.Generator(np.random.PCG64(ss))
    x = rng.standard_normal((n_tokens, w.d), dtype=np.float32)
    if role in (_Q, _K):
        if w.qk in ("rmsnorm", "rmsnorm_rope"):
            x = rmsnorm_rows(x)
        if w.qk == "rmsnorm_rope":
            x = rope_interleaved(x, *rope)
        if w.qk == "outliers":
            x[:, outlier_ch] *= np.float32(OUTLIER_FACTOR)
    return f32_to_bf16_bits(x)


def outlier_channels(w: Workload) -> np.ndarray:
    """[B*H, 4] seeded outlier channel indices (stress recipe), the same for Q and K."""
    rng = np.random.Generator(np.random.PCG64(_seed_children(w)[_OUTLIER]))
    return np.stack([rng.choice(w.d, OUTLIER_CHANNELS, replace=False) for _ in range(w.B * w.H)])


def make_dense(w: Workload, threads: int | None = None):
    """BF16 bit patterns q, k, v as uint16 arrays [B, H, N, d] (contiguous)."""
    assert w.kind == "dense"
    kids = _seed_children(w)
    rope = rope_tables(w.grid, w.N, w.d) if w.qk == "rmsnorm_rope" else None
    och = outlier_channels(w) if w.qk == "outliers" else None
    out = [np.empty((w.B, w.H, w.N, w.d), dtype=np.uint16) for _ in range(3)]
    jobs = []
    for role in (_Q, _K, _V):
        per_head = kids[role].spawn(w.B * w.H)
        for bh in range(w.B * w.H):
            jobs.append((role, bh, per_head[bh]))

    def run(job):
        role, bh, ss = job
        blk = _head_block(w, role, ss, w.N, None if och is None else och[bh], rope)
        out[role][bh // w.H, bh % w.H] = blk

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(run, jobs))
    return tuple(out)


def make_varlen(w: Workload, threads: int | None = None):
    """THD inputs for the packed workload: q, k, v uint16 [T, H, d] and cu_seqlens int32 [nseg+1]."""
    assert w.kind == "varlen"
    kids = _seed_children(w)
    T = w.total_tokens
    out = [np.empty((T, w.H, w.d), dtype=np.uint16) for _ in range(3)]
    jobs = []
    for role in (_Q, _K, _V):
        per_head = kids[role].spawn(w.H)
        for h in range(w.H):
            jobs.append((role, h, per_head[h]))

    def run(job):
        role, h, ss = job
        out[role][:, h, :] = _head_block(w, role, ss, T, None, None)

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(run, jobs))
    cu = np.zeros(len(w.seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(w.seqlens)
    return out[0], out[1], out[2], cu


PROJ_ROOT = 7   # SeedSequence key of the projected-input streams (apart from the workload indices)


def make_projected(B: int, grid: tuple, H: int, seed: int = 0, with_v: bool = True,
                   threads: int | None = None, d: int = HEAD_DIM, chunk: int = 4096):
    """Raw projected Q, K (and V) as the QKV projection hands them to the prologue: BF16 bit
    patterns [B, N, H, d] (token-major), N = prod(grid). Every row is N(0, 1) times its own
    log-normal scale (sigma 0.5), so rows differ in RMS the way projection outputs do; one
    independent PCG64 stream per (tensor, batch, block of `chunk` tokens)."""
    N = int(np.prod(grid))
    roles = 3 if with_v else 2
    nchunk = (N + chunk - 1) // chunk
    kids = np.random.SeedSequence([ROOT_SEED, PROJ_ROOT, seed]).spawn(roles)
    out = [np.empty((B, N, H, d), dtype=np.uint16) for _ in range(roles)]
    jobs = [(r, i, ss) for r in range(roles) for i, ss in enumerate(kids[r].spawn(B * nchunk))]

    def run(job):
        r, i, ss = job
        b, c = divmod(i, nchunk)
        n0, n1 = c * chunk, min(N, (c + 1) * chunk)
        rng = np.random.Generator(np.random.PCG64(ss))
        x = rng.standard_normal((n1 - n0, H, d), dtype=np.float32)
        x *= rng.lognormal(0.0, 0.5, size=(n1 - n0, H, 1)).astype(np.float32)
        out[r][b, n0:n1] = f32_to_bf16_bits(x)

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(run, jobs))
    return tuple(out)


def make_linear_inputs(B: int, grid: tuple, H: int, seed: int = 0, threads: int | None = None,
                       d: int = HEAD_DIM, chunk: int = 4096):
    """Inputs of the SANA-Video linear attention: q, k = ReLU(RMSNorm(x)) rounded to BF16, and
    q_rot, k_rot = the interleaved 3-D RoPE of those BF16 rows (FP32, rounded once); v plain.
    x are the projected rows of make_projected. All BF16 bit patterns [B, N, H, d] (token-major)."""
    xq, xk, xv = make_projected(B, grid, H, seed=seed, threads=threads, d=d)
    N = int(np.prod(grid))
    cos, sin = rope_tables(grid, N, d)                        # [N, d/2]
    out = [np.empty_like(xq) for _ in range(4)]

    def run(job):
        which, b, n0 = job
        n1 = min(N, n0 + chunk)
        x = xq if which == 0 else xk
        f = ((x[b, n0:n1].astype(np.uint32) << 16).view(np.float32))       # [n, H, d]
        act = np.maximum(rmsnorm_rows(f), np.float32(0.0))
        act_bits = f32_to_bf16_bits(act)
        act_r = (act_bits.astype(np.uint32) << 16).view(np.float32)
        rot = rope_interleaved(act_r, cos[n0:n1, None, :], sin[n0:n1, None, :])
        out[2 * which][b, n0:n1] = act_bits
        out[2 * which + 1][b, n0:n1] = f32_to_bf16_bits(rot)

    jobs = [(which, b, n0) for which in (0, 1) for b in range(B) for n0 in range(0, N, chunk)]
    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(run, jobs))
    q, q_rot, k, k_rot = out
    return q, k, q_rot, k_rot, xv


def make_ragged(w: Workload, dense=None, threads: int | None = None):
    """Varlen call of the stress recipe: segments w.ragged, THD [T, H, d].

    The first B segments are the dense batches (each [H, N, d] transposed to [N, H, d]) bit
    for bit; the remaining segments are fresh draws of the same recipe (outlier channels of
    batch 0). Returns q, k, v uint16 [T, H, d] and cu_seqlens int32.
    """
    assert w.ragged is not None
    if dense is None:
        dense = make_dense(w, threads)
    lens = list(w.ragged)
    assert lens[: w.B] == [w.N] * w.B
    extra = sum(lens[w.B:])
    T = sum(lens)
    och = outlier_channels(w)
    kids = _seed_children(w)[_RAGGED].spawn(3)
    out = []
    for role in (_Q, _K, _V):
        a = np.empty((T, w.H, w.d), dtype=np.uint16)
        for b in range(w.B):
            a[b * w.N:(b + 1) * w.N] = dense[role][b].transpose(1, 0, 2)
        per_head = kids[role].spawn(w.H)
        for h in range(w.H):
            a[w.B * w.N:, h, :] = _head_block(w, role, per_head[h], extra, och[h], None)
        out.append(a)
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    return out[0], out[1], out[2], cu


def sample_rows(w: Workload, n_rows: int | None = None) -> np.ndarray:
    """Seeded, sorted, distinct flat query-row indices.

    Dense: indices into B*H*N (row = (b*H + h)*N + n). Varlen: indices into H*T
    (row = h*T + token), matching the LSE layouts.
    """
    n_rows = n_rows or w.sample_rows
    total = w.B * w.H * w.N if w.kind == "dense" else w.H * w.total_tokens
    rng = np.random.Generator(np.random.PCG64(_seed_children(w)[_ROWS]))
    return np.sort(rng.choice(total, min(n_rows, total), replace=False))


def random_dense(B: int, H: int, N: int, d: int = HEAD_DIM, seed: int = 0, std: float = 1.0):
    """Small ad-hoc dense case: N(0, std^2) Q/K/V as BF16 bits [B,H,N,d] (tests, edge cases)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, 1000 + seed])))
    return tuple(f32_to_bf16_bits(rng.standard_normal((B, H, N, d), dtype=np.float32) * np.float32(std))
                 for _ in range(3))


def random_varlen(seqlens, H: int, d: int = HEAD_DIM, seed: int = 0, std: float = 1.0):
    """Small ad-hoc varlen case: THD [T,H,d] BF16 bits and int32 cu_seqlens."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, 2000 + seed])))
    T = int(sum(seqlens))
    q, k, v = (f32_to_bf16_bits(rng.standard_normal((T, H, d), dtype=np.float32) * np.float32(std))
               for _ in range(3))
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    return q, k, v, cu
