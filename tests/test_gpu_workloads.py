"""GPU parity on the five synthetic workloads at their full sizes, in the same launch
configuration the bench times. The FP64 oracle checks seeded samples of query rows (every
row would take minutes to hours on the host) plus every row of each ragged query tail.
"""
import math

import numpy as np
import pytest

from oracle import attention_dense, attention_varlen
from workloads import WORKLOADS, make_dense, make_ragged, make_varlen, sample_rows

pytestmark = pytest.mark.gpu

TAIL = 130  # rows at the end of a sequence: covers the last (ragged) query tile


@pytest.fixture(scope="module")
def attn():
    import video_diffusion_dit_amd as m
    m.load_library()
    return m


def dense_rows_with_tails(w, rows):
    extra = []
    for bh in (0, w.B * w.H - 1):
        extra += list(range(bh * w.N + w.N - min(TAIL, w.N), bh * w.N + w.N))
    return np.unique(np.concatenate([rows, np.array(extra, dtype=np.int64)]))


def varlen_rows_with_tails(w, rows, cu, T):
    extra = []
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        for h in (0, w.H - 1):
            extra += [h * T + t for t in range(max(a, e - TAIL), e)]
    return np.unique(np.concatenate([rows, np.array(extra, dtype=np.int64)]))


def run_dense_check(attn, w, label, split_kv=True, cut_rows=False):
    """The bench's launch (split-KV on the device's compute units by default) on the workload's
    full tensors, checked on its seeded row sample plus the ragged tails; with cut_rows, also
    the first and last row and two seeded rows of every query tile the split plan cuts."""
    import torch
    from gpu_util import check, cut_tile_rows, dev, device_slots, f64_of, split_plan
    print(f"[case] {label}: generating {w.description}", flush=True)
    qb, kb, vb = make_dense(w)
    q, k, v = dev(qb), dev(kb), dev(vb)
    print(f"[case] {label}: launching", flush=True)
    o, lse = attn.attn_fwd(q, k, v, scale=w.scale, return_lse=True, split_kv=split_kv)
    torch.cuda.synchronize()
    rows = dense_rows_with_tails(w, sample_rows(w))
    if cut_rows:
        slots = device_slots()
        D, R, G, _ = split_plan(w.B, w.H, w.N, slots)
        extra = cut_tile_rows(w.B, w.H, w.N, slots, seed=w.index)
        assert extra.size > 0, "the plan cuts no tile at this size"
        print(f"[case] {label}: {slots} slots, {R} tiles over {G} split workgroups, "
              f"{extra.size} rows in cut tiles", flush=True)
        rows = np.unique(np.concatenate([rows, extra]))
    o_ref, lse_ref = attention_dense(qb, kb, vb, w.scale, rows=rows)
    og = f64_of(o).reshape(-1, w.d)[rows]
    lg = lse.cpu().numpy().reshape(-1)[rows].astype(np.float64)
    check(og, o_ref, lg, lse_ref, f"{label} ({rows.size} rows)")
    return qb, kb, vb, o, lse


def test_video_480p_sampled(attn):
    run_dense_check(attn, WORKLOADS["video_480p"], "video_480p")


def test_packed_varlen_sampled(attn):
    import torch
    from gpu_util import check, dev, dev_i32, f64_of
    w = WORKLOADS["packed_varlen"]
    q, k, v, cu = make_varlen(w)
    T = w.total_tokens
    o, lse = attn.attn_fwd_varlen(dev(q), dev(k), dev(v), dev_i32(cu), scale=w.scale, return_lse=True,
                                  cu_seqlens_host=[int(x) for x in cu])
    torch.cuda.synchronize()
    rows = varlen_rows_with_tails(w, sample_rows(w), cu, T)
    o_ref, lse_ref = attention_varlen(q, k, v, cu, w.scale, rows=rows)
    og = f64_of(o)                                   # [T, H, d]
    h_of, t_of = rows // T, rows % T
    lg = lse.cpu().numpy()[h_of, t_of].astype(np.float64)
    check(og[t_of, h_of], o_ref, lg, lse_ref, f"packed_varlen ({rows.size} rows)")


def test_numerics_stress_dense_and_ragged(attn):
    import torch
    from gpu_util import bits_of, check, dev, dev_i32, f64_of
    w = WORKLOADS["numerics_stress"]
    # the plain dense path (no key split), whose rows the varlen call must reproduce bit for bit
    dense = run_dense_check(attn, w, "numerics_stress dense", split_kv=False)
    qb, kb, vb, o_dense, lse_dense = dense
    # realised logit range of the recipe, for the record
    qf = (qb[0, 0, :64].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    kf = (kb[0, 0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    x = w.scale * qf @ kf.T
    print(f"[stress] logit range head 0 (64 rows): [{x.min():.1f}, {x.max():.1f}]", flush=True)
    q, k, v, cu = make_ragged(w, (qb, kb, vb))
    T = int(cu[-1])
    o, lse = attn.attn_fwd_varlen(dev(q), dev(k), dev(v), dev_i32(cu), scale=w.scale, return_lse=True,
                                  cu_seqlens_host=[int(c) for c in cu])
    torch.cuda.synchronize()
    # the two 8192-token segments are the dense batches: identical bits
    ob = bits_of(o)
    od = bits_of(o_dense)
    for b in range(w.B):
        assert np.array_equal(ob[b * w.N:(b + 1) * w.N].transpose(1, 0, 2), od[b])
        assert np.array_equal(lse.cpu().numpy()[:, b * w.N:(b + 1) * w.N], lse_dense.cpu().numpy()[b])
    # the ragged segments (length 1 and 127) in full, against the oracle
    a = w.B * w.N
    o_ref, lse_ref = attention_varlen(q[a:], k[a:], v[a:], cu[w.B:] - a, w.scale)
    check(f64_of(o)[a:], o_ref, lse.cpu().numpy()[:, a:], lse_ref, "numerics_stress ragged 1+127")
    assert np.array_equal(ob[a], v[a])                 # length-1 segment: o = v exactly


def test_video_720p_sampled(attn):
    run_dense_check(attn, WORKLOADS["video_720p"], "video_720p", cut_rows=True)


def test_video_720p_one_gpu_share(attn):
    """One GPU's share of an 8-way head split of the 720p call: B=1, H=2, N=180320 (the first
    two heads, same values). 1410 query tiles are 5.5 rounds of 256 workgroups, so the split
    plan cuts its last 386 tiles; every cut tile is checked."""
    import dataclasses
    w = WORKLOADS["video_720p"]
    share = dataclasses.replace(w, name="video_720p_h2", H=2,
                                description=w.description.replace("H=16", "H=2"))
    run_dense_check(attn, share, "video_720p H=2 share", cut_rows=True)
