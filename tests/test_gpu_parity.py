"""GPU parity of the HIP attention forward against the FP64 oracle (small and edge cases).

Every case compares element by element with the oracle on the same seeded BF16 inputs;
the bar is relative L2 <= 5e-3, max-abs <= 2e-2 on the BF16 output and |dLSE| <= 1e-3.
Exact (bit-level) checks are used where the arithmetic is exact: length-1 sequences,
uniform weights over two keys (output rounding), determinism, segment isolation and
varlen-vs-dense equivalence.
"""
import math

import numpy as np
import pytest

from oracle import attention_dense, attention_varlen, bf16_bits_to_f64
from workloads import WORKLOADS, f32_to_bf16_bits, make_dense, random_dense, random_varlen

from gpu_util import cut_tiles, split_plan

pytestmark = pytest.mark.gpu

SCALE = 1 / math.sqrt(128)


@pytest.fixture(scope="module")
def attn():
    import torch  # noqa: F401
    import video_diffusion_dit_amd as m
    m.load_library()
    return m


def run_dense(attn, qb, kb, vb, scale=SCALE, lse=True):
    from gpu_util import dev
    import torch
    q, k, v = dev(qb), dev(kb), dev(vb)
    res = attn.attn_fwd(q, k, v, scale=scale, return_lse=lse)
    torch.cuda.synchronize()
    return res


def run_varlen(attn, qb, kb, vb, cu, scale=SCALE, lse=True):
    from gpu_util import dev, dev_i32
    import torch
    q, k, v = dev(qb), dev(kb), dev(vb)
    res = attn.attn_fwd_varlen(q, k, v, dev_i32(cu), scale=scale, return_lse=lse,
                               cu_seqlens_host=[int(x) for x in cu])
    torch.cuda.synchronize()
    return res


def test_tiny_config_full(attn):
    from gpu_util import check, f64_of
    w = WORKLOADS["tiny_dense"]
    qb, kb, vb = make_dense(w)
    o, lse = run_dense(attn, qb, kb, vb, w.scale)
    o_ref, lse_ref = attention_dense(qb, kb, vb, w.scale)
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, "tiny_dense")


@pytest.mark.parametrize("B,H,N", [(1, 1, 1), (1, 1, 2), (1, 1, 7), (1, 2, 63), (1, 2, 64), (1, 1, 65),
                                   (1, 1, 127), (1, 1, 128), (1, 1, 129), (2, 3, 191), (1, 2, 300),
                                   (1, 1, 1000), (3, 1, 517)])
def test_dense_shapes_full(attn, B, H, N):
    from gpu_util import check, f64_of
    qb, kb, vb = random_dense(B, H, N, seed=B * 100000 + H * 1000 + N)
    o, lse = run_dense(attn, qb, kb, vb)
    o_ref, lse_ref = attention_dense(qb, kb, vb, SCALE)
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, f"dense B={B} H={H} N={N}")


@pytest.mark.parametrize("scale", [0.0, 0.02, 0.25, -0.09])
def test_dense_other_scales(attn, scale):
    from gpu_util import check, f64_of
    qb, kb, vb = random_dense(1, 2, 333, seed=77)
    o, lse = run_dense(attn, qb, kb, vb, scale)
    o_ref, lse_ref = attention_dense(qb, kb, vb, scale)
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, f"scale={scale}")


def test_lse_optional_and_every_output_written(attn):
    import torch
    from gpu_util import bits_of, dev
    qb, kb, vb = random_dense(1, 2, 200, seed=5)
    q, k, v = dev(qb), dev(kb), dev(vb)
    out = torch.full_like(q, float("nan"))
    attn.attn_fwd(q, k, v, out=out)
    o2, _ = attn.attn_fwd(q, k, v, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert np.array_equal(bits_of(out), bits_of(o2))


def test_length_one_is_exact(attn):
    from gpu_util import bits_of
    qb, kb, vb = random_dense(2, 4, 1, seed=11)
    o, lse = run_dense(attn, qb, kb, vb)
    assert np.array_equal(bits_of(o), vb)
    _, lse_ref = attention_dense(qb, kb, vb, SCALE)
    assert np.max(np.abs(lse.cpu().numpy() - lse_ref)) <= 1e-3


def test_uniform_two_keys_output_rounding_is_rne(attn):
    # q = 0: both probabilities are exactly 1, l = 2, o = (v0 + v1)/2 exactly in FP32, so the
    # output bits must be round-to-nearest-even of that value (many exact ties occur).
    from gpu_util import bits_of
    H = 64
    _, kb, vb = random_dense(1, H, 2, seed=12)
    qb = np.zeros_like(kb)
    o, lse = run_dense(attn, qb, kb, vb)
    v = bf16_bits_to_f64(vb)[0]                         # [H, 2, 128]
    mean = (v[:, 0] + v[:, 1]) / 2
    exact_in_f32 = mean.astype(np.float32).astype(np.float64) == mean
    want = f32_to_bf16_bits(mean.astype(np.float32))
    got = bits_of(o)[0]                                 # [H, 2, 128]: both query rows equal
    for row in range(2):
        assert np.array_equal(got[:, row][exact_in_f32], want[exact_in_f32])
    assert exact_in_f32.mean() > 0.99
    assert np.max(np.abs(lse.cpu().numpy() - math.log(2))) <= 1e-6


def test_zero_query_mean_and_constant_value(attn):
    from gpu_util import check, f64_of
    _, kb, vb = random_dense(1, 2, 777, seed=13)
    qb = np.zeros_like(kb)
    o, lse = run_dense(attn, qb, kb, vb)
    o_ref, lse_ref = attention_dense(qb, kb, vb, SCALE)
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, "q=0")
    assert np.max(np.abs(lse.cpu().numpy() - math.log(777))) <= 1e-5
    # constant V: o = c up to the BF16 probability rounding (l sums FP32 probabilities)
    qb2, kb2, _ = random_dense(1, 2, 777, seed=14, std=3.0)
    c = f32_to_bf16_bits(np.linspace(-2, 2, 128, dtype=np.float32))
    vb2 = np.broadcast_to(c, kb2.shape).copy()
    o2, _ = run_dense(attn, qb2, kb2, vb2)
    dev = np.abs(f64_of(o2) - bf16_bits_to_f64(c))
    assert np.max(dev / np.maximum(np.abs(bf16_bits_to_f64(c)), 1e-30)) <= 2 ** -7


def test_one_hot_huge_logits(attn):
    # one key dominates by a logit of ~1000: exp without a max would overflow FP32
    from gpu_util import check, f64_of
    N = 300
    qf = np.zeros((1, 1, N, 128), np.float32)
    kf = np.zeros((1, 1, N, 128), np.float32)
    qf[0, 0, :, 0] = 96.0
    kf[0, 0, 5, 0] = 96.0
    kf[0, 0, :, 1] = 1.0
    rng = np.random.default_rng(3)
    vf = rng.standard_normal((1, 1, N, 128)).astype(np.float32)
    qb, kb, vb = f32_to_bf16_bits(qf), f32_to_bf16_bits(kf), f32_to_bf16_bits(vf)
    o, lse = run_dense(attn, qb, kb, vb, 0.125)
    o_ref, lse_ref = attention_dense(qb, kb, vb, 0.125)
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, "one-hot x~1152")


def test_deterministic(attn):
    from gpu_util import bits_of
    qb, kb, vb = random_dense(2, 4, 1500, seed=15, std=2.0)
    o1, l1 = run_dense(attn, qb, kb, vb)
    o2, l2 = run_dense(attn, qb, kb, vb)
    assert np.array_equal(bits_of(o1), bits_of(o2))
    assert np.array_equal(l1.cpu().numpy().view(np.uint32), l2.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("lens", [[5, 0, 17, 1, 33], [129, 128, 127, 1, 0, 64, 300], [1000], [1] * 40])
def test_varlen_full(attn, lens):
    from gpu_util import check, f64_of
    q, k, v, cu = random_varlen(lens, H=3, seed=len(lens))
    o, lse = run_varlen(attn, q, k, v, cu)
    o_ref, lse_ref = attention_varlen(q, k, v, cu, SCALE)
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, f"varlen {lens[:8]}")


def test_varlen_many_sorted_segments(attn):
    # 3000 segments: the schedule builder sorts them (below its limit) and every one of its 16
    # waves carries a share of the prefix of query tiles
    from gpu_util import check, f64_of
    lens = [int(x) for x in np.random.default_rng(5).integers(0, 300, 3000)]
    q, k, v, cu = random_varlen(lens, H=1, seed=25)
    o, lse = run_varlen(attn, q, k, v, cu)
    o_ref, lse_ref = attention_varlen(q, k, v, cu, SCALE)
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, "varlen 3000 sorted segments")


def test_varlen_many_segments_beyond_sort_limit(attn):
    from gpu_util import check, f64_of
    rng = np.random.default_rng(21)
    lens = list(rng.integers(0, 4, 9000))
    q, k, v, cu = random_varlen(lens, H=1, seed=22)
    o, lse = run_varlen(attn, q, k, v, cu)
    o_ref, lse_ref = attention_varlen(q, k, v, cu, SCALE)
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, "varlen 9000 segments")


def test_varlen_single_segment_equals_dense(attn):
    from gpu_util import bits_of
    q, k, v, cu = random_varlen([700], H=4, seed=23)
    ov, lv = run_varlen(attn, q, k, v, cu)
    qd, kd, vd = (np.ascontiguousarray(t.transpose(1, 0, 2))[None] for t in (q, k, v))
    od, ld = run_dense(attn, qd, kd, vd)
    assert np.array_equal(bits_of(ov).transpose(1, 0, 2), bits_of(od)[0])
    assert np.array_equal(lv.cpu().numpy(), ld.cpu().numpy()[0])


def test_varlen_segment_isolation(attn):
    from gpu_util import bits_of
    lens = [300, 65, 1, 200]
    q, k, v, cu = random_varlen(lens, H=2, seed=24)
    o1, l1 = run_varlen(attn, q, k, v, cu)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    a, e = cu[1], cu[2]
    for t in (q2, k2, v2):
        t[a:e] ^= np.uint16(0x0041)
    o2, l2 = run_varlen(attn, q2, k2, v2, cu)
    b1, b2 = bits_of(o1), bits_of(o2)
    L1, L2 = l1.cpu().numpy(), l2.cpu().numpy()
    for s in (0, 2, 3):
        x, y = cu[s], cu[s + 1]
        assert np.array_equal(b1[x:y], b2[x:y])
        assert np.array_equal(L1[:, x:y], L2[:, x:y])
    assert not np.array_equal(b1[a:e], b2[a:e])


def test_varlen_empty_batch_is_noop(attn):
    import torch
    from gpu_util import dev_i32
    z = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda:0")
    out = attn.attn_fwd_varlen(z, z, z, dev_i32([0, 0, 0]))
    torch.cuda.synchronize()
    assert out.shape == (0, 2, 128)


# ---- split-KV (attn_fwd_splitkv): the last, partly filled round of query tiles is cut over keys

@pytest.mark.parametrize("B,H,N,slots", [
    (1, 3, 4133, 7),      # 51 tiles: 42 whole, the last 9 cut over 7 workgroups; ragged last key tile
    (2, 2, 3000, 5),      # 48 tiles: the last 8 over 5 workgroups
    (1, 1, 8192, 64),     # 32 tiles, 64 workgroups: every tile cut in two
    (1, 1, 8192, 200),    # shares of 20.48 key tiles: tiles cut in up to 8 pieces
    (1, 2, 1100, 3),      # 10 tiles over 3 slots, 18 key tiles each (just above the minimum)
])
def test_splitkv_against_oracle_and_unsplit(attn, B, H, N, slots):
    import torch
    from gpu_util import bits_of, check, dev, f64_of
    D, R, G, ntk = split_plan(B, H, N, slots)
    assert G > 0 and attn.splitkv_workspace_bytes(B, H, N, slots=slots) > 0
    qb, kb, vb = random_dense(B, H, N, seed=9000 + N + slots)
    q, k, v = dev(qb), dev(kb), dev(vb)
    o, lse = attn.attn_fwd(q, k, v, scale=SCALE, return_lse=True, slots=slots)
    o_plain, lse_plain = attn.attn_fwd(q, k, v, scale=SCALE, return_lse=True, split_kv=False)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_dense(qb, kb, vb, SCALE)
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, f"splitkv B={B} H={H} N={N} slots={slots}")
    # query tiles computed whole are the plain kernel's rows, bit for bit; cut ones differ
    # only by rounding (their probabilities are BF16 relative to each piece's reference)
    cut = cut_tiles(B, H, N, slots)
    assert cut
    ntq = -(-N // 256)
    ob, opb = bits_of(o).reshape(B * H, N, 128), bits_of(o_plain).reshape(B * H, N, 128)
    lb, lpb = lse.cpu().numpy().reshape(B * H, N), lse_plain.cpu().numpy().reshape(B * H, N)
    for t in range(B * H * ntq):
        bh, qt = divmod(t, ntq)
        rows = slice(qt * 256, min(N, (qt + 1) * 256))
        if t not in cut:
            assert np.array_equal(ob[bh, rows], opb[bh, rows]), t
            assert np.array_equal(lb[bh, rows], lpb[bh, rows]), t


def test_splitkv_deterministic_and_no_split_is_plain(attn):
    import torch
    from gpu_util import bits_of, dev
    qb, kb, vb = random_dense(1, 1, 8192, seed=31)
    q, k, v = dev(qb), dev(kb), dev(vb)
    a = attn.attn_fwd(q, k, v, slots=200)
    b = attn.attn_fwd(q, k, v, slots=200)
    c = attn.attn_fwd(q, k, v, slots=16)          # 32 tiles, 16 slots: whole rounds, no cut
    d = attn.attn_fwd(q, k, v, split_kv=False)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(a), bits_of(b))
    assert np.array_equal(bits_of(c), bits_of(d))
    assert not np.array_equal(bits_of(a), bits_of(d))   # cut tiles do differ in rounding



@pytest.mark.parametrize("log2_scale", [-64, 60])
def test_value_magnitude_range(attn, log2_scale):
    # V scaled by an exact power of two, far from N(0,1): 2^-64 stays inside the range where the
    # accumulated sum(p v) is a normal FP32 number (the probabilities after an exact-path move
    # are 2^-48, so |v| >= 2^-78 is needed), 2^60 inside the overflow bound (accepted
    # probabilities <= 2^24, so N * 2^24 * max|v| < 2^128). Scaling V only scales every product
    # and sum, so the output divided back must match the unscaled call, which meets the bar
    # against the oracle; the LSE does not depend on V.
    from gpu_util import check, f64_of
    qb, kb, _ = random_dense(1, 2, 1000, seed=21, std=2.0)     # peaked rows: many exact-path moves
    _, _, vb = random_dense(1, 2, 1000, seed=22)                # V ~ N(0, 1)
    vf = bf16_bits_to_f64(vb) * 2.0 ** log2_scale
    vb_s = f32_to_bf16_bits(vf.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f64(vb_s), vf)       # the scaling is exact in BF16
    o, lse = run_dense(attn, qb, kb, vb)
    o_ref, lse_ref = attention_dense(qb, kb, vb, SCALE)
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, "V ~ N(0,1), peaked rows")
    o_s, lse_s = run_dense(attn, qb, kb, vb_s)
    back = f64_of(o_s) * 2.0 ** -log2_scale
    assert np.linalg.norm(back - f64_of(o)) <= 1e-6 * np.linalg.norm(f64_of(o)), log2_scale
    assert np.max(np.abs(lse_s.cpu().numpy() - lse.cpu().numpy())) <= 1e-6


def dominated_inputs(N, H=2, seed=31, vmax=7.0):
    from gpu_util import dominated_dense
    return dominated_dense(N, H, seed, vmax)


@pytest.mark.parametrize("split", [True, False])
def test_dominated_rows_dense(attn, split):
    from gpu_util import check, dev, f64_of
    import torch
    qb, kb, vb = dominated_inputs(700)
    q, k, v = dev(qb), dev(kb), dev(vb)
    print(f"[case] dominated rows dense N=700 split={split}", flush=True)
    o, lse = attn.attn_fwd(q, k, v, scale=SCALE, return_lse=True, split_kv=split)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_dense(qb, kb, vb, SCALE)
    assert np.abs(o_ref).max() > 4.0          # outputs in the binade where the bar is tight
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, f"dominated rows dense split={split}")


@pytest.mark.parametrize("split", [True, False])
def test_dominated_rows_varlen(attn, split):
    from gpu_util import check, dev, dev_i32, f64_of
    import torch
    lens = (700, 257, 1, 1300)
    T = sum(lens)
    qb, kb, vb = dominated_inputs(T, seed=41)
    q, k, v = (np.ascontiguousarray(x[0].transpose(1, 0, 2)) for x in (qb, kb, vb))   # THD
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    print(f"[case] dominated rows varlen lens={lens} split={split}", flush=True)
    o, lse = attn.attn_fwd_varlen(dev(q), dev(k), dev(v), dev_i32(cu), scale=SCALE, return_lse=True,
                                  cu_seqlens_host=[int(x) for x in cu], split_kv=split, slots=64 if split else 0)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_varlen(q, k, v, cu, SCALE)
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, f"dominated rows varlen split={split}")
