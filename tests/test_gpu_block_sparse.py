"""GPU parity of block-skip attention (attn_block_route + attn_fwd_block_sparse) against the
FP64 oracle of oracle/block_sparse.py.

Routing: the kept tiles must equal the oracle's except where the oracle's z lies within the
FP32 decision band around the threshold (oracle.block_sparse.decision_margin, pinned against
binary32 replays of the rule in tests/test_oracle_margin.py), such tiles must stay rare, and
the lists must be well formed (ascending, counted, padded). Attention: the oracle's exact softmax over
the tiles the GPU kept, with the dense bar (rel-L2 <= 5e-3, max-abs <= 2e-2, |dLSE| <= 1e-3).
With every tile listed the output must equal the dense kernel's bit for bit.
"""
import math

import numpy as np
import pytest
import torch

from oracle.block_sparse import attention_kept, decision_margin, route_blocks
from workloads import WORKLOADS, make_dense, random_dense

from gpu_util import bits_of, check, dev, dev_i32, device_normal_bf16, f64_of

pytestmark = pytest.mark.gpu

SCALE = 1 / math.sqrt(128)


@pytest.fixture(scope="module")
def vd():
    import video_diffusion_dit_amd as m
    m.load_library()
    return m


def lists_to_keep(kv_idx, kv_cnt, ntk):
    """[B,H,ntq,stride] / [B,H,ntq] int32 (host) -> keep [B,H,ntq,ntk], after checking that
    every list is strictly ascending inside [0, ntk) and padded with ntk."""
    B, H, ntq, stride = kv_idx.shape
    keep = np.zeros((B, H, ntq, ntk), bool)
    for b in range(B):
        for h in range(H):
            for i in range(ntq):
                c = int(kv_cnt[b, h, i])
                assert 1 <= c <= ntk
                row = kv_idx[b, h, i]
                ids = row[:c]
                assert np.all(np.diff(ids) > 0) and ids[0] >= 0 and ids[-1] < ntk, (b, h, i, ids)
                assert np.all(row[c:c + 8] == ntk)
                keep[b, h, i, ids] = True
    return keep


def in_band_budget(n_tiles):
    """Disagreements allowed inside the FP32 band: the band is about 1e-7 wide against a proxy
    spread near 1e-2, so on these inputs a tile lands in it about once per 10^4-10^5 tiles."""
    return 2 + n_tiles // 10000


def check_route(keep_gpu, q, k, tau, sink):
    keep, z, zmax = route_blocks(q, k, SCALE, tau, sink_tokens=sink)
    diff = keep_gpu != keep
    if diff.any():
        band = np.abs(z - (zmax[..., None] - tau)) <= decision_margin(q, k, SCALE, tau, mask=diff)
        assert not (diff & ~band).any(), f"{int((diff & ~band).sum())} tiles routed differently outside the band"
    assert int(diff.sum()) <= in_band_budget(diff.size), int(diff.sum())
    print(f"[route] tau={tau} sink={sink}: density {keep_gpu.mean():.4f}, "
          f"{int(diff.sum())} tiles inside the FP32 band differ", flush=True)
    return keep


def route(vd, q, k, tau, sink=0):
    kv_idx, kv_cnt = vd.block_route(dev(q), dev(k), tau=tau, sink_tokens=sink, scale=SCALE)
    torch.cuda.synchronize()
    return kv_idx, kv_cnt


@pytest.mark.parametrize("B,H,N,tau,sink", [
    (2, 3, 1000, 0.0, 0),        # ragged query and key tiles; only the best tile
    (2, 3, 1000, 0.008, 0),      # z spreads about 0.008 on these inputs
    (1, 2, 1000, 0.005, 100),    # sink tiles 0 and 1
    (1, 2, 4096, 0.01, 64),      # whole tiles only
    (1, 1, 65, 0.01, 0),         # a 1-key last tile
    (1, 1, 1, 0.0, 0),           # one token
    (1, 2, 700, math.inf, 0),    # everything kept
])
def test_route_and_attention_small(vd, B, H, N, tau, sink):
    q, k, v = random_dense(B, H, N, seed=N + H)
    kv_idx, kv_cnt = route(vd, q, k, tau, sink)
    ntk = -(-N // 64)
    keep_gpu = lists_to_keep(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), ntk)
    check_route(keep_gpu, q, k, tau, sink)
    if sink:
        assert keep_gpu[..., :-(-sink // 64)].all()
    out, lse = vd.attn_fwd_block_sparse(dev(q), dev(k), dev(v), kv_idx, kv_cnt, scale=SCALE, return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_kept(q, k, v, SCALE, keep_gpu)
    check(f64_of(out), o_ref, lse.cpu().numpy().astype(np.float64), lse_ref,
          label=f"block-sparse B{B} H{H} N{N} tau={tau} sink={sink}")


@pytest.mark.parametrize("B,H,N", [(1, 2, 1000), (2, 1, 4096), (1, 1, 1), (1, 3, 257)])
def test_every_tile_listed_equals_dense_bits(vd, B, H, N):
    """tau = inf lists every tile in order: the tile-list loop must then do exactly what the
    range loop does (the dense kernel without split-KV)."""
    q, k, v = random_dense(B, H, N, seed=7 * N)
    kv_idx, kv_cnt = route(vd, q, k, math.inf)
    assert (kv_cnt.cpu().numpy() == -(-N // 64)).all()
    out, lse = vd.attn_fwd_block_sparse(dev(q), dev(k), dev(v), kv_idx, kv_cnt, scale=SCALE, return_lse=True)
    ref, lse_ref = vd.attn_fwd(dev(q), dev(k), dev(v), scale=SCALE, return_lse=True, split_kv=False)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out), bits_of(ref))
    assert np.array_equal(lse.cpu().numpy(), lse_ref.cpu().numpy())


def custom_lists(B, H, N, rows_of):
    """kv_idx/kv_cnt from a function (b, h, query tile) -> list of tile indices; padding ntk."""
    ntq, ntk = -(-N // 256), -(-N // 64)
    stride = ntk + 8
    idx = np.full((B, H, ntq, stride), ntk, np.int32)
    cnt = np.zeros((B, H, ntq), np.int32)
    keep = np.zeros((B, H, ntq, ntk), bool)
    for b in range(B):
        for h in range(H):
            for i in range(ntq):
                ids = rows_of(b, h, i, ntk)
                cnt[b, h, i] = len(ids)
                idx[b, h, i, :len(ids)] = ids
                keep[b, h, i, [j for j in ids if 0 <= j < ntk]] = True
    return idx, cnt, keep


@pytest.mark.parametrize("name,rows_of", [
    ("last tile only", lambda b, h, i, ntk: [ntk - 1]),
    ("first and last", lambda b, h, i, ntk: [0, ntk - 1]),
    ("every third", lambda b, h, i, ntk: list(range(i % 3, ntk, 3))),
    ("two runs", lambda b, h, i, ntk: [0, 1, 2] + list(range(ntk // 2, ntk // 2 + 5))),
    ("per-head pattern", lambda b, h, i, ntk: list(range(h, ntk, 2 + h))),
])
def test_hook_with_caller_lists(vd, name, rows_of):
    B, H, N = 1, 3, 1500
    q, k, v = random_dense(B, H, N, seed=31)
    idx, cnt, keep = custom_lists(B, H, N, rows_of)
    out, lse = vd.attn_fwd_block_sparse(dev(q), dev(k), dev(v), dev_i32(idx), dev_i32(cnt), scale=SCALE,
                                        return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_kept(q, k, v, SCALE, keep)
    check(f64_of(out), o_ref, lse.cpu().numpy().astype(np.float64), lse_ref, label=f"hook: {name}")


def test_hook_dominated_rows(vd):
    """The tile-list loop carries the same normaliser correction: rows that one key dominates
    (K = Q, large V), each query tile's list holding its own diagonal key tiles plus every third
    other tile, meet the bar against the oracle over the kept tiles."""
    from gpu_util import dominated_dense
    B, H, N = 1, 2, 1500
    q, k, v = dominated_dense(N, H, seed=51)
    idx, cnt, keep = custom_lists(B, H, N, lambda b, h, i, ntk: sorted(
        set(range(4 * i, min(4 * i + 4, ntk))) | set(range(i % 3, ntk, 3))))
    out, lse = vd.attn_fwd_block_sparse(dev(q), dev(k), dev(v), dev_i32(idx), dev_i32(cnt), scale=SCALE,
                                        return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_kept(q, k, v, SCALE, keep)
    assert np.abs(o_ref).max() > 4.0
    check(f64_of(out), o_ref, lse.cpu().numpy().astype(np.float64), lse_ref, label="hook: dominated rows")


def test_hook_empty_tile_and_clamped_counts(vd):
    """kv_cnt <= 0 gives O = 0 and LSE = -inf for that query tile; a count above ntk is read
    as ntk; other tiles are unaffected."""
    B, H, N = 1, 2, 600
    q, k, v = random_dense(B, H, N, seed=41)
    ntk = -(-N // 64)
    idx, cnt, keep = custom_lists(B, H, N, lambda b, h, i, n: list(range(n)))
    cnt[0, 0, 1] = 0
    cnt[0, 1, 0] = -3
    cnt[0, 1, 2] = 10 * ntk               # clamped to ntk: all tiles, which the list holds
    keep[0, 0, 1] = False
    keep[0, 1, 0] = False
    out, lse = vd.attn_fwd_block_sparse(dev(q), dev(k), dev(v), dev_i32(idx), dev_i32(cnt), scale=SCALE,
                                        return_lse=True)
    torch.cuda.synchronize()
    o = f64_of(out)
    l = lse.cpu().numpy()
    assert np.all(o[0, 0, 256:512] == 0) and np.all(np.isneginf(l[0, 0, 256:512]))
    assert np.all(o[0, 1, 0:256] == 0) and np.all(np.isneginf(l[0, 1, 0:256]))
    o_ref, lse_ref = attention_kept(q, k, v, SCALE, keep)
    live = np.ones((B, H, N), bool)
    live[0, 0, 256:512] = False
    live[0, 1, 0:256] = False
    check(o[live], o_ref[live], l[live].astype(np.float64), lse_ref[live], label="hook with empty tiles")


def test_deterministic(vd):
    q, k, v = random_dense(1, 4, 3000, seed=51)
    a = vd.block_skip_attention(dev(q), dev(k), dev(v), tau=0.01, sink_tokens=64, scale=SCALE)
    b = vd.block_skip_attention(dev(q), dev(k), dev(v), tau=0.01, sink_tokens=64, scale=SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(a), bits_of(b))


def check_order(order, cnt, n, max_cnt, group=None):
    """order (host): its first n entries are a permutation of the n items; within each run of
    `group` entries (all n when None) the entries are that run's own items, longest list
    first. The counting sort bins counts into 4096 bins, one count per bin while
    max_cnt <= 4095; above that, neighbouring counts may share a bin and keep any order."""
    o = order[:n]
    assert np.array_equal(np.sort(o), np.arange(n))
    group = group or n
    for lo in range(0, n, group):
        run = o[lo:lo + group]
        assert np.array_equal(np.sort(run), np.arange(lo, min(lo + group, n)))
        c = np.clip(cnt.reshape(-1)[run].astype(np.int64), 0, max_cnt)
        if max_cnt <= 4095:
            assert np.all(np.diff(c) <= 0)
        else:
            assert np.all(np.diff((max_cnt - c) * 4095 // max_cnt) >= 0)


@pytest.mark.parametrize("B,H,N,tau", [
    (2, 3, 3000, 0.01),
    (1, 2, 700, math.inf),      # every list full: all counts equal
    (1, 1, 1, 0.0),             # one item
])
def test_dispatch_order(vd, B, H, N, tau):
    """The dispatch order: per (b, h), its query tiles sorted by count, longest first; the
    lists are the same with and without it, and so are the outputs, bit for bit."""
    q, k, v = random_dense(B, H, N, seed=N + 7 * H)
    kv_idx, kv_cnt = route(vd, q, k, tau)
    idx2, cnt2, order = vd.block_route(dev(q), dev(k), tau=tau, scale=SCALE, with_order=True)
    torch.cuda.synchronize()
    ntk = -(-N // 64)
    # lists are written up to their count plus 8 padding entries; compare that part
    assert np.array_equal(cnt2.cpu().numpy(), kv_cnt.cpu().numpy())
    assert np.array_equal(lists_to_keep(idx2.cpu().numpy(), cnt2.cpu().numpy(), ntk),
                          lists_to_keep(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), ntk))
    check_order(order.cpu().numpy(), kv_cnt.cpu().numpy(), kv_cnt.numel(), ntk, group=-(-N // 256))
    a, la = vd.attn_fwd_block_sparse(dev(q), dev(k), dev(v), kv_idx, kv_cnt, scale=SCALE, return_lse=True)
    b, lb = vd.attn_fwd_block_sparse(dev(q), dev(k), dev(v), kv_idx, kv_cnt, scale=SCALE, return_lse=True,
                                     order=order)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(a), bits_of(b))
    assert np.array_equal(la.cpu().numpy(), lb.cpu().numpy())


def test_long_sequence_routes_one_query_tile_per_workgroup(vd):
    """N = 260000: 4063 key tiles, more proxies than four query tiles' worth fit in a
    workgroup's LDS, so the routing takes one query tile per workgroup. Routing against the
    oracle over every tile; attention on 128 seeded rows and the last 32."""
    N = 260000
    q, k, v = random_dense(1, 1, N, seed=260)
    kv_idx, kv_cnt = route(vd, q, k, 0.01)
    keep_gpu = lists_to_keep(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), -(-N // 64))
    check_route(keep_gpu, q, k, 0.01, 0)
    out, lse = vd.attn_fwd_block_sparse(dev(q), dev(k), dev(v), kv_idx, kv_cnt, scale=SCALE, return_lse=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(26).choice(N, 128, replace=False), np.arange(N - 32, N)]))
    o_ref, lse_ref = attention_kept(q, k, v, SCALE, keep_gpu, rows=rows)
    check(f64_of(out).reshape(-1, 128)[rows], o_ref, lse.cpu().numpy().reshape(-1)[rows].astype(np.float64),
          lse_ref, label="block-sparse N=260000 tau=0.01 sampled rows")


@pytest.mark.parametrize("N", [1300, 245760, 245761])
def test_route_query_tiles_per_workgroup(vd, N):
    """The routing groups 4 query tiles per workgroup while their proxies fit in LDS (up to
    3840 key tiles, N = 245760), then 1: both sides of the bound, and a last group of 2 query
    tiles (N = 1300), routed against the oracle over every tile."""
    q, k, _ = random_dense(1, 1, N, seed=N % 1000 + 3)
    kv_idx, kv_cnt = route(vd, q, k, 0.01)
    keep_gpu = lists_to_keep(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), -(-N // 64))
    check_route(keep_gpu, q, k, 0.01, 0)


@pytest.fixture(scope="module")
def video_720p():
    return make_dense(WORKLOADS["video_720p"])


def test_video_720p_routing_and_sampled_rows(vd, video_720p):
    """The 720p grid (B=1, H=16, N=180320) at the timed setting tau = 0.02, in the timed
    launch (longest-first order per head): routing against the oracle over every (head, query tile,
    key tile), the order against the counts, attention on 384 seeded rows plus the last 64
    rows of head 15."""
    q, k, v = video_720p
    tau = 0.02
    kv_idx, kv_cnt, order = vd.block_route(dev(q), dev(k), tau=tau, scale=SCALE, with_order=True)
    torch.cuda.synchronize()
    N = q.shape[2]
    ntk = -(-N // 64)
    keep_gpu = lists_to_keep(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), ntk)
    check_route(keep_gpu, q, k, tau, 0)
    check_order(order.cpu().numpy(), kv_cnt.cpu().numpy(), kv_cnt.numel(), ntk, group=-(-N // 256))
    out, lse = vd.attn_fwd_block_sparse(dev(q), dev(k), dev(v), kv_idx, kv_cnt, scale=SCALE, return_lse=True,
                                        order=order)
    torch.cuda.synchronize()
    rng = np.random.default_rng(720)
    rows = np.unique(np.concatenate([rng.choice(16 * N, 384, replace=False), 15 * N + np.arange(N - 64, N)]))
    o_ref, lse_ref = attention_kept(q, k, v, SCALE, keep_gpu, rows=rows)
    o = f64_of(out).reshape(-1, 128)[rows]
    l = lse.cpu().numpy().reshape(-1)[rows].astype(np.float64)
    check(o, o_ref, l, lse_ref, label="block-sparse video_720p tau=0.02 sampled rows")


# ---------------------------------------------------------------- packed (varlen) batches
from oracle.block_sparse import attention_kept_varlen, route_blocks_varlen  # noqa: E402
from workloads import make_varlen, random_varlen  # noqa: E402


def varlen_keeps(vd, kv_idx, kv_cnt, cu, H):
    """Host lists -> per-segment keep [H, ntq_s, ntk_s] (None for empty segments), after
    checking every list is ascending inside the segment's key tiles and padded."""
    offs = vd.varlen_tile_offsets(list(cu))
    out = []
    for s in range(len(cu) - 1):
        n = int(cu[s + 1] - cu[s])
        if n == 0:
            out.append(None)
            continue
        ntq, ntk = -(-n // 256), -(-n // 64)
        keep = np.zeros((H, ntq, ntk), bool)
        for i in range(ntq):
            for h in range(H):
                c = int(kv_cnt[offs[s] + i, h])
                ids = kv_idx[offs[s] + i, h, :c]
                assert 1 <= c <= ntk and np.all(np.diff(ids) > 0) and ids[0] >= 0 and ids[-1] < ntk
                assert np.all(kv_idx[offs[s] + i, h, c:c + 8] == ntk)
                keep[h, i, ids] = True
        out.append(keep)
    return out


def check_route_varlen(keeps, q, k, cu, tau, sink):
    ref = route_blocks_varlen(q, k, cu, SCALE, tau, sink)
    n_diff = n_tiles = 0
    for s, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        if ref[s] is None:
            assert keeps[s] is None
            continue
        keep, z, zmax = ref[s]
        diff = keeps[s] != keep
        if diff.any():
            qs = np.ascontiguousarray(q[a:e].transpose(1, 0, 2))[None]
            ks = np.ascontiguousarray(k[a:e].transpose(1, 0, 2))[None]
            band = np.abs(z - (zmax[..., None] - tau)) <= decision_margin(qs, ks, SCALE, tau, mask=diff[None])[0]
            assert not (diff & ~band).any()
            n_diff += int(diff.sum())
        n_tiles += diff.size
    assert n_diff <= in_band_budget(n_tiles), n_diff
    print(f"[route varlen] tau={tau} sink={sink}: {n_diff} tiles inside the FP32 band differ", flush=True)


def run_varlen_route(vd, q, k, cu, tau, sink=0):
    cu_d = dev_i32(cu)
    kv_idx, kv_cnt = vd.block_route_varlen(dev(q), dev(k), cu_d, tau=tau, sink_tokens=sink, scale=SCALE)
    torch.cuda.synchronize()
    return cu_d, kv_idx, kv_cnt


@pytest.mark.parametrize("lens,H,tau,sink", [
    ((300, 1, 0, 520, 64), 3, 0.0, 0),      # a length-1 and an empty segment
    ((300, 1, 0, 520, 64), 3, 0.01, 100),
    ((1000,), 2, 0.008, 0),                  # one segment: the dense case
    ((256, 257, 511), 2, math.inf, 0),
])
def test_varlen_route_and_attention_small(vd, lens, H, tau, sink):
    q, k, v, cu = random_varlen(lens, H, seed=sum(lens) + H)
    cu_d, kv_idx, kv_cnt = run_varlen_route(vd, q, k, cu, tau, sink)
    keeps = varlen_keeps(vd, kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), cu, H)
    check_route_varlen(keeps, q, k, cu, tau, sink)
    out, lse = vd.attn_fwd_block_sparse_varlen(dev(q), dev(k), dev(v), cu_d, kv_idx, kv_cnt, scale=SCALE,
                                               return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_kept_varlen(q, k, v, cu, SCALE, keeps)
    check(f64_of(out), o_ref, lse.cpu().numpy().astype(np.float64), lse_ref,
          label=f"block-sparse varlen {lens} H{H} tau={tau} sink={sink}")


def test_varlen_route_at_the_routing_limit(vd):
    """A packed batch of T = 983040 tokens, route_max_tiles (15360) key tiles, the most the
    routing takes: one segment of 900000 tokens and one of 83040, one head. Each query tile's
    proxies fill the routing workgroup's LDS allowance (60 KiB), and the key means are read at
    the largest tile stride. Routing against the oracle over every tile of both segments."""
    lens, H = (900000, 83040), 1
    q, k, _, cu = random_varlen(lens, H, seed=983)
    _, kv_idx, kv_cnt = run_varlen_route(vd, q, k, cu, 0.01)
    keeps = varlen_keeps(vd, kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), cu, H)
    check_route_varlen(keeps, q, k, cu, 0.01, 0)


def test_varlen_every_tile_listed_equals_varlen_bits(vd):
    q, k, v, cu = random_varlen((700, 1, 64, 300), 3, seed=77)
    cu_d, kv_idx, kv_cnt = run_varlen_route(vd, q, k, cu, math.inf)
    out, lse = vd.attn_fwd_block_sparse_varlen(dev(q), dev(k), dev(v), cu_d, kv_idx, kv_cnt, scale=SCALE,
                                               return_lse=True)
    ref, lse_ref = vd.attn_fwd_varlen(dev(q), dev(k), dev(v), cu_d, scale=SCALE, return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out), bits_of(ref))
    assert np.array_equal(lse.cpu().numpy(), lse_ref.cpu().numpy())


def test_varlen_dispatch_order(vd):
    """Packed order: its first (query tiles x H) entries are a permutation of the items sorted
    by count; the outputs with and without it are equal bit for bit."""
    lens, H = (300, 1, 0, 520, 64, 1100), 3
    q, k, v, cu = random_varlen(lens, H, seed=91)
    cu_d, kv_idx, kv_cnt = run_varlen_route(vd, q, k, cu, 0.01)
    idx2, cnt2, order = vd.block_route_varlen(dev(q), dev(k), cu_d, tau=0.01, scale=SCALE, with_order=True)
    torch.cuda.synchronize()
    n = sum(-(-n_ // 256) for n_ in lens) * H
    # the first n rows are written, each up to its count plus 8 padding entries
    assert np.array_equal(cnt2.cpu().numpy().reshape(-1)[:n], kv_cnt.cpu().numpy().reshape(-1)[:n])
    for a_, b_ in zip(varlen_keeps(vd, idx2.cpu().numpy(), cnt2.cpu().numpy(), cu, H),
                      varlen_keeps(vd, kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), cu, H)):
        assert (a_ is None and b_ is None) or np.array_equal(a_, b_)
    check_order(order.cpu().numpy(), kv_cnt.cpu().numpy(), n, -(-int(cu[-1]) // 64))
    a, la = vd.attn_fwd_block_sparse_varlen(dev(q), dev(k), dev(v), cu_d, kv_idx, kv_cnt, scale=SCALE,
                                            return_lse=True)
    b, lb = vd.attn_fwd_block_sparse_varlen(dev(q), dev(k), dev(v), cu_d, kv_idx, kv_cnt, scale=SCALE,
                                            return_lse=True, order=order)
    c, lc = vd.block_skip_attention_varlen(dev(q), dev(k), dev(v), cu_d, tau=0.01, scale=SCALE, return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(a), bits_of(b)) and np.array_equal(bits_of(a), bits_of(c))
    assert np.array_equal(la.cpu().numpy(), lb.cpu().numpy()) and np.array_equal(la.cpu().numpy(), lc.cpu().numpy())


def test_varlen_hook_with_caller_lists(vd):
    """Caller lists: each tile keeps its segment's last key tile and tile 0; one tile keeps
    nothing (O = 0, LSE = -inf)."""
    lens, H = (600, 70, 300), 2
    q, k, v, cu = random_varlen(lens, H, seed=88)
    T = int(cu[-1])
    (G, _, stride), _ = vd.varlen_list_shapes(len(lens), T, H)
    offs = vd.varlen_tile_offsets(list(cu))
    idx = np.full((G, H, stride), 0, np.int32)
    cnt = np.zeros((G, H), np.int32)
    keeps = []
    for s, n in enumerate(lens):
        ntq, ntk = -(-n // 256), -(-n // 64)
        keep = np.zeros((H, ntq, ntk), bool)
        for i in range(ntq):
            for h in range(H):
                ids = sorted({0, ntk - 1})
                idx[offs[s] + i, h, :len(ids)] = ids
                idx[offs[s] + i, h, len(ids):] = ntk
                cnt[offs[s] + i, h] = len(ids)
                keep[h, i, ids] = True
        keeps.append(keep)
    cnt[offs[0] + 1, 1] = 0            # rows 256..511 of segment 0, head 1
    keeps[0][1, 1] = False
    out, lse = vd.attn_fwd_block_sparse_varlen(dev(q), dev(k), dev(v), dev_i32(cu), dev_i32(idx), dev_i32(cnt),
                                               scale=SCALE, return_lse=True)
    torch.cuda.synchronize()
    o, l = f64_of(out), lse.cpu().numpy()
    assert np.all(o[256:512, 1] == 0) and np.all(np.isneginf(l[1, 256:512]))
    o_ref, lse_ref = attention_kept_varlen(q, k, v, cu, SCALE, keeps)
    live = np.ones((T, H), bool)
    live[256:512, 1] = False
    check(o[live], o_ref[live], l.T[live].astype(np.float64), lse_ref.T[live], label="varlen hook")


def test_packed_varlen_workload_sampled(vd):
    """The packed workload (segments 30000 / 6000 / 2048, H = 24) at tau = 0.02, in the timed
    launch (longest-first order): routing of every tile against the oracle, attention on 384
    seeded rows plus the last 16 rows."""
    w = WORKLOADS["packed_varlen"]
    q, k, v, cu = make_varlen(w)
    T, H = q.shape[0], q.shape[1]
    cu_d = dev_i32(cu)
    kv_idx, kv_cnt, order = vd.block_route_varlen(dev(q), dev(k), cu_d, tau=0.02, scale=SCALE, with_order=True)
    torch.cuda.synchronize()
    keeps = varlen_keeps(vd, kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), cu, H)
    check_route_varlen(keeps, q, k, cu, 0.02, 0)
    n = sum(-(-int(n_) // 256) for n_ in np.diff(cu)) * H
    check_order(order.cpu().numpy(), kv_cnt.cpu().numpy(), n, -(-T // 64))
    out, lse = vd.attn_fwd_block_sparse_varlen(dev(q), dev(k), dev(v), cu_d, kv_idx, kv_cnt, scale=SCALE,
                                               return_lse=True, order=order)
    torch.cuda.synchronize()
    rng = np.random.default_rng(38)
    rows = np.unique(np.concatenate([rng.choice(H * T, 384, replace=False), (H - 1) * T + np.arange(T - 16, T)]))
    o_ref, lse_ref = attention_kept_varlen(q, k, v, cu, SCALE, keeps, rows=rows)
    o = f64_of(out).transpose(1, 0, 2).reshape(-1, 128)[rows]
    check(o, o_ref, lse.cpu().numpy().reshape(-1)[rows].astype(np.float64), lse_ref,
          label="block-sparse packed_varlen tau=0.02 sampled rows")


# ---------------------------------------------------------------- the largest sequences
from oracle import attention_dense  # noqa: E402


def kept_rows(ids, n):
    """Key rows of the listed 64-key tiles of a sequence of n keys, in tile order."""
    return np.concatenate([np.arange(64 * t, min(64 * t + 64, n)) for t in ids])


def test_hook_at_the_largest_sequence(vd):
    """N = 8388607, the longest sequence the kernels address (its K/V rows span N * 256 B =
    2^31 - 256 bytes): caller lists that reach the last, ragged key tile (63 keys, 2 GiB into
    the sequence) from query tiles at both ends. Each listed tile's rows against the oracle
    over its listed keys (dense attention over those keys); unlisted tiles give O = 0."""
    N = 8388607
    ntq, ntk = -(-N // 256), -(-N // 64)
    q, k, v = (device_normal_bf16((1, 1, N, 128), seed=s) for s in (801, 802, 803))
    stride = vd.block_list_stride(N)
    kv_idx = torch.full((1, 1, ntq, stride), ntk, dtype=torch.int32, device="cuda:0")
    kv_cnt = torch.zeros((1, 1, ntq), dtype=torch.int32, device="cuda:0")
    lists = {0: [0, 65536, ntk - 2, ntk - 1], 1: [ntk - 1], ntq // 2: [1, 2, 3, 100000], ntq - 1: [0, ntk - 1]}
    for i, ids in lists.items():
        kv_idx[0, 0, i, :len(ids)] = torch.tensor(ids, dtype=torch.int32)
        kv_cnt[0, 0, i] = len(ids)
    print(f"[max] dense hook N={N}: {ntq} query tiles, lists {lists}", flush=True)
    out, lse = vd.attn_fwd_block_sparse(q, k, v, kv_idx, kv_cnt, scale=SCALE, return_lse=True)
    torch.cuda.synchronize()
    del kv_idx
    for i, ids in lists.items():
        r0, r1 = 256 * i, min(256 * i + 256, N)
        keys = torch.from_numpy(kept_rows(ids, N)).to("cuda:0")
        qb = bits_of(q[0, 0, r0:r1])[None, None]
        kb, vb = bits_of(k[0, 0, keys])[None, None], bits_of(v[0, 0, keys])[None, None]
        o_ref, lse_ref = attention_dense(qb, kb, vb, SCALE)
        check(f64_of(out[0, 0, r0:r1]), o_ref[0, 0], lse[0, 0, r0:r1].cpu().numpy().astype(np.float64),
              lse_ref[0, 0], label=f"block-sparse N={N} query tile {i} keys {ids}")
    idle = out[0, 0, 256 * 2:256 * 40]
    assert bool((idle == 0).all()) and bool(torch.isneginf(lse[0, 0, 256 * 2:256 * 40]).all())
    del q, k, v, out, lse
    torch.cuda.empty_cache()


def test_varlen_hook_at_the_largest_batch(vd):
    """T = 4194303 tokens, H = 2: the largest packed batch the kernels address (T * H * 256 B =
    2^31 - 512 bytes). Segment 0 (4194003 tokens) lists its last, ragged key tile (19 keys,
    2 GiB into the tensor) from both of its ends; segment 1 (300 tokens) lists every tile.
    Checked against the oracle over the listed keys; unlisted tiles give O = 0."""
    H, T = 2, 4194303
    cu = [0, T - 300, T]
    q, k, v = (device_normal_bf16((T, H, 128), seed=s) for s in (811, 812, 813))
    (G, _, stride), _ = vd.varlen_list_shapes(2, T, H)
    offs = vd.varlen_tile_offsets(cu)
    n0 = cu[1]
    ntq0, ntk0 = -(-n0 // 256), -(-n0 // 64)
    kv_idx = torch.full((G, H, stride), 0, dtype=torch.int32, device="cuda:0")
    kv_cnt = torch.zeros((G, H), dtype=torch.int32, device="cuda:0")
    lists = {(0, 0, 0): [0, ntk0 - 1], (0, 0, 1): [32000, ntk0 - 1],
             (0, ntq0 - 1, 0): [ntk0 - 2, ntk0 - 1], (0, ntq0 - 1, 1): [ntk0 - 1],
             (1, 0, 0): [0, 1, 2, 3, 4], (1, 0, 1): [0, 1, 2, 3, 4], (1, 1, 0): [0, 1, 2, 3, 4],
             (1, 1, 1): [0, 1, 2, 3, 4]}
    for (s_, i, h), ids in lists.items():
        ntk_s = -(-(cu[s_ + 1] - cu[s_]) // 64)
        kv_idx[offs[s_] + i, h, :len(ids)] = torch.tensor(ids, dtype=torch.int32)
        kv_idx[offs[s_] + i, h, len(ids):len(ids) + 8] = ntk_s
        kv_cnt[offs[s_] + i, h] = len(ids)
    print(f"[max] varlen hook T={T} H={H} cu={cu}: lists {lists}", flush=True)
    cu_d = dev_i32(cu)
    out, lse = vd.attn_fwd_block_sparse_varlen(q, k, v, cu_d, kv_idx, kv_cnt, scale=SCALE, return_lse=True)
    torch.cuda.synchronize()
    del kv_idx
    for (s_, i, h), ids in lists.items():
        a, n = cu[s_], cu[s_ + 1] - cu[s_]
        r0, r1 = a + 256 * i, a + min(256 * i + 256, n)
        keys = torch.from_numpy(a + kept_rows(ids, n)).to("cuda:0")
        qb = bits_of(q[r0:r1, h])[None, None]
        kb, vb = bits_of(k[keys, h])[None, None], bits_of(v[keys, h])[None, None]
        o_ref, lse_ref = attention_dense(qb, kb, vb, SCALE)
        check(f64_of(out[r0:r1, h]), o_ref[0, 0], lse[h, r0:r1].cpu().numpy().astype(np.float64), lse_ref[0, 0],
              label=f"block-sparse varlen T={T} segment {s_} tile {i} head {h} keys {ids}")
    idle = out[256:256 * 40]
    assert bool((idle == 0).all()) and bool(torch.isneginf(lse[:, 256:256 * 40]).all())
    del q, k, v, out, lse
    torch.cuda.empty_cache()
