"""GPU parity of the attention prologue (attn_qk_prologue: per-head RMSNorm + interleaved 3-D
RoPE, BF16, token-major -> head-major) against the FP64 oracle of oracle/prologue.py.

The bar: every Q/K output element within one BF16 spacing of the exact value (or 2^-18
absolute, for values produced by cancellation), and almost all of them equal to the
nearest-even rounding of the exact value; V bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, bf16_faithful, qk_norm_rope, v_head_major
from workloads import make_projected

from gpu_util import bits_of, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vd():
    import video_diffusion_dit_amd as m
    m.load_library()
    return m


def check_qk(got_bits, exact, label, rne_min=0.995):
    m = bf16_faithful(bf16_bits_to_f64(got_bits), exact)
    print(f"[prologue] {label}: err/limit={m['max_err_over_limit']:.3f} rne={m['rne_frac']:.5f} n={m['n_elems']}",
          flush=True)
    assert m["ok"] and m["rne_frac"] >= rne_min, (label, m)
    return m


@pytest.mark.parametrize("B,grid,H,weighted", [
    (1, (1, 1, 1), 1, False),        # one token at position 0
    (2, (3, 4, 5), 3, False),
    (1, (2, 3, 7), 16, True),        # 42 tokens: a partial last workgroup
    (3, (1, 1, 7), 5, True),         # H not a multiple of the 4 rows a group keeps in flight
    (1, (4, 6, 9), 24, False),
])
def test_small_shapes_in_full(vd, B, grid, H, weighted):
    xq, xk, xv = make_projected(B, grid, H, seed=B * 100 + H)
    wq = wk = None
    if weighted:
        rng = np.random.default_rng(H)
        wq = torch.from_numpy(rng.uniform(0.5, 1.5, 128).astype(np.float32)).to("cuda:0")
        wk = torch.from_numpy(rng.uniform(0.5, 1.5, 128).astype(np.float32)).to("cuda:0")
    q, k, v = vd.qk_prologue(dev(xq), dev(xk), dev(xv), grid=grid, weight_q=wq, weight_k=wk)
    torch.cuda.synchronize()
    wq_h = None if wq is None else wq.cpu().numpy()
    wk_h = None if wk is None else wk.cpu().numpy()
    check_qk(bits_of(q), qk_norm_rope(xq, grid, weight=wq_h), f"q B{B} grid{grid} H{H}")
    check_qk(bits_of(k), qk_norm_rope(xk, grid, weight=wk_h), f"k B{B} grid{grid} H{H}")
    assert np.array_equal(bits_of(v), v_head_major(xv))


def test_without_v_and_zero_rows(vd):
    grid = (2, 2, 2)
    xq, xk = make_projected(1, grid, 4, seed=5, with_v=False)
    xq[0, 3, 1] = 0                  # an all-zero row: normalised to zero, no NaN
    q, k = vd.qk_prologue(dev(xq), dev(xk), grid=grid)
    torch.cuda.synchronize()
    qb = bits_of(q)
    assert np.all(bf16_bits_to_f64(qb[0, 1, 3]) == 0.0)
    check_qk(qb, qk_norm_rope(xq, grid), "q with a zero row")
    check_qk(bits_of(k), qk_norm_rope(xk, grid), "k")


def test_deterministic(vd):
    grid = (3, 5, 7)
    xq, xk, xv = [dev(a) for a in make_projected(2, grid, 8, seed=6)]
    a = [bits_of(t) for t in vd.qk_prologue(xq, xk, xv, grid=grid)]
    b = [bits_of(t) for t in vd.qk_prologue(xq, xk, xv, grid=grid)]
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_preallocated_outputs_and_theta(vd):
    grid = (2, 3, 4)
    xq, xk, xv = make_projected(1, grid, 2, seed=7)
    out = tuple(torch.full((1, 2, 24, 128), 7.0, dtype=torch.bfloat16, device="cuda:0") for _ in range(3))
    res = vd.qk_prologue(dev(xq), dev(xk), dev(xv), grid=grid, theta=500.0, eps=1e-5, out=out)
    torch.cuda.synchronize()
    assert all(r is o for r, o in zip(res, out))
    check_qk(bits_of(out[0]), qk_norm_rope(xq, grid, theta=500.0, eps=1e-5), "q theta=500 eps=1e-5")
    assert np.array_equal(bits_of(out[2]), v_head_major(xv))


def test_video_720p_shape_sampled_tokens(vd):
    """The 720p grid (49 x 46 x 80 = 180320 tokens), 16 heads, in one call as the bench times
    it; the oracle checks 2048 seeded tokens plus the first and last 64 (all heads)."""
    grid = (49, 46, 80)
    N = 49 * 46 * 80
    xq, xk, xv = make_projected(1, grid, 16, seed=720)
    q, k, v = vd.qk_prologue(dev(xq), dev(xk), dev(xv), grid=grid)
    torch.cuda.synchronize()
    rng = np.random.default_rng(720)
    toks = np.unique(np.concatenate([rng.choice(N, 2048, replace=False), np.arange(64), np.arange(N - 64, N)]))
    for name, x, t in (("q", xq, q), ("k", xk, k)):
        check_qk(bits_of(t)[:, :, toks], qk_norm_rope(x, grid, tokens=toks), f"{name} 720p sampled")
    assert np.array_equal(bits_of(v)[:, :, toks], v_head_major(xv[:, toks]))


def test_video_720p_two_heads_sampled_tokens(vd):
    """One GPU's share of an 8-way head split at 720p (2 heads): each 16-lane group takes a
    token of its own. 2048 seeded tokens plus the first and last 64 against the oracle."""
    grid = (49, 46, 80)
    N = 49 * 46 * 80
    xq, xk, xv = make_projected(1, grid, 2, seed=7202)
    q, k, v = vd.qk_prologue(dev(xq), dev(xk), dev(xv), grid=grid)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7202)
    toks = np.unique(np.concatenate([rng.choice(N, 2048, replace=False), np.arange(64), np.arange(N - 64, N)]))
    for name, x, t in (("q", xq, q), ("k", xk, k)):
        check_qk(bits_of(t)[:, :, toks], qk_norm_rope(x, grid, tokens=toks), f"{name} 720p H2 sampled")
    assert np.array_equal(bits_of(v), v_head_major(xv))


# ---- the packed (varlen) prologue: per-head RMSNorm of THD rows, no re-layout, no rotation

def thd_rows(T, H, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    f = (rng.standard_normal((T, H, 128)) * scale).astype(np.float32)
    t = torch.from_numpy(f).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("T,H,weighted,in_place", [
    (1, 1, False, False),         # 2 rows: one group, half empty
    (5, 3, True, False),          # 30 rows: the last group straddles Q and K
    (257, 24, False, True),       # in place
    (1000, 2, True, True),
])
def test_packed_norm_in_full(vd, T, H, weighted, in_place):
    from oracle import qk_norm
    xq, xk = thd_rows(T, H, seed=T + H), thd_rows(T, H, seed=T + H + 1, scale=3.0)
    wq = wk = None
    if weighted:
        rng = np.random.default_rng(H)
        wq = torch.from_numpy(rng.uniform(0.5, 1.5, 128).astype(np.float32)).to("cuda:0")
        wk = torch.from_numpy(rng.uniform(0.5, 1.5, 128).astype(np.float32)).to("cuda:0")
    dq, dk = dev(xq), dev(xk)
    q, k = vd.qk_norm_packed(dq, dk, weight_q=wq, weight_k=wk, in_place=in_place)
    torch.cuda.synchronize()
    if in_place:
        assert q.data_ptr() == dq.data_ptr() and k.data_ptr() == dk.data_ptr()
    wq_h = None if wq is None else wq.cpu().numpy()
    wk_h = None if wk is None else wk.cpu().numpy()
    check_qk(bits_of(q), qk_norm(xq, weight=wq_h), f"packed q T{T} H{H}")
    check_qk(bits_of(k), qk_norm(xk, weight=wk_h), f"packed k T{T} H{H}")


def test_packed_norm_workload_size(vd):
    """The packed workload's token count and heads (38048 x 24), seeded tokens checked,
    including the first and the last."""
    from oracle import qk_norm
    from workloads import WORKLOADS
    w = WORKLOADS["packed_varlen"]
    T = w.total_tokens
    xq, xk = thd_rows(T, w.H, seed=31), thd_rows(T, w.H, seed=32)
    q, k = vd.qk_norm_packed(dev(xq), dev(xk))
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(33).choice(T, 256, replace=False)]))
    check_qk(bits_of(q)[toks], qk_norm(xq, tokens=toks), f"packed q {T}x{w.H} ({toks.size} tokens)")
    check_qk(bits_of(k)[toks], qk_norm(xk, tokens=toks), f"packed k {T}x{w.H} ({toks.size} tokens)")
