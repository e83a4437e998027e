"""GPU parity of split-KV for packed batches (attn_fwd_varlen_splitkv) against the FP64 oracle.

The plan is made on the device from the segment lengths; tests/gpu_util.varlen_plan restates it
to know which items (segment query tile, head) are cut. Every case is checked against the
oracle; items the plan leaves whole must equal the plain attn_fwd_varlen call bit for bit, cut
items may differ only by rounding (each piece takes its BF16 probabilities against its own
reference). Small cases are checked in full; the full-size packed workload and one GPU's share
of the 720p call as a packed batch (one 180320-token segment, H = 2) on seeded rows plus rows
of every cut item, in the launch configuration the bench times.
"""
import math

import numpy as np
import pytest

from oracle import attention_varlen
from workloads import WORKLOADS, make_dense, make_varlen, random_varlen, sample_rows

from gpu_util import bits_of, check, dev, dev_i32, f64_of, varlen_cut_rows, varlen_plan

pytestmark = pytest.mark.gpu

SCALE = 1 / math.sqrt(128)


@pytest.fixture(scope="module")
def vd():
    import video_diffusion_dit_amd as m
    m.load_library()
    return m


def run_both(vd, q, k, v, cu, slots):
    import torch
    cu_d = dev_i32(cu)
    host = [int(x) for x in cu]
    qd, kd, vd_ = dev(q), dev(k), dev(v)
    o, lse = vd.attn_fwd_varlen(qd, kd, vd_, cu_d, scale=SCALE, return_lse=True, cu_seqlens_host=host, slots=slots)
    o_plain, lse_plain = vd.attn_fwd_varlen(qd, kd, vd_, cu_d, scale=SCALE, return_lse=True, cu_seqlens_host=host,
                                            split_kv=False)
    torch.cuda.synchronize()
    return o, lse, o_plain, lse_plain


def uncut_items_equal(o, lse, o_plain, lse_plain, lens, H, slots):
    """Items the plan keeps whole are the plain call's rows bit for bit; returns the cut set."""
    entries, D, G, cut = varlen_plan(lens, H, slots)
    starts = np.concatenate([[0], np.cumsum(lens)])
    ob, opb = bits_of(o), bits_of(o_plain)
    lb, lpb = lse.cpu().numpy(), lse_plain.cpu().numpy()
    for it in range(len(entries) * H):
        if it in cut:
            continue
        s, i, _ = entries[it // H]
        h = it % H
        rows = slice(int(starts[s]) + i * 256, int(starts[s]) + min(lens[s], (i + 1) * 256))
        assert np.array_equal(ob[rows, h], opb[rows, h]), it
        assert np.array_equal(lb[h, rows], lpb[h, rows]), it
    return cut


@pytest.mark.parametrize("lens,H,slots", [
    ((4133,), 3, 7),                  # one segment: 49 items whole, 2 cut over 7 workgroups
    ((4133, 700, 64), 2, 9),          # cut items in two segments, a ragged last key tile
    ((5000, 1100, 300, 1), 2, 11),    # a length-1 segment left whole
    ((2500, 2500, 900, 130), 3, 13),  # equal segments, the cut ones the shorter
    ((6000, 257, 1), 1, 40),          # fewer items than slots: every item split, some into several pieces
    ((3000, 1000, 50, 1), 2, 16),
])
def test_varlen_splitkv_against_oracle_and_unsplit(vd, lens, H, slots):
    q, k, v, cu = random_varlen(lens, H, seed=sum(lens) + H + slots)
    print(f"[case] varlen split lens={lens} H={H} slots={slots}", flush=True)
    o, lse, o_plain, lse_plain = run_both(vd, q, k, v, cu, slots)
    o_ref, lse_ref = attention_varlen(q, k, v, cu, SCALE)
    check(f64_of(o), o_ref, lse.cpu().numpy(), lse_ref, f"varlen splitkv lens={lens} H={H} slots={slots}")
    cut = uncut_items_equal(o, lse, o_plain, lse_plain, list(lens), H, slots)
    assert cut, "the plan cuts no item here"


def test_varlen_splitkv_without_a_useful_split_is_the_plain_call(vd):
    # the stress recipe's ragged call: four whole rounds of equal items, then 32 tiny ones --
    # splitting them would not shorten the tail, so nothing is split
    lens = (8192, 8192, 1, 127)
    assert varlen_plan(lens, 16, 256)[2] == 0
    q, k, v, cu = random_varlen(lens, 16, seed=5)
    o, lse, o_plain, lse_plain = run_both(vd, q, k, v, cu, 256)
    assert np.array_equal(bits_of(o), bits_of(o_plain))
    assert np.array_equal(lse.cpu().numpy().view(np.uint32), lse_plain.cpu().numpy().view(np.uint32))


def test_varlen_splitkv_deterministic(vd):
    import torch
    lens = (6000, 257, 1)
    q, k, v, cu = random_varlen(lens, 1, seed=6)
    qd, kd, vd_, cu_d = dev(q), dev(k), dev(v), dev_i32(cu)
    host = [int(x) for x in cu]
    a = vd.attn_fwd_varlen(qd, kd, vd_, cu_d, cu_seqlens_host=host, slots=40)
    b = vd.attn_fwd_varlen(qd, kd, vd_, cu_d, cu_seqlens_host=host, slots=40)
    c = vd.attn_fwd_varlen(qd, kd, vd_, cu_d, cu_seqlens_host=host, slots=1)       # no split
    d = vd.attn_fwd_varlen(qd, kd, vd_, cu_d, cu_seqlens_host=host, split_kv=False)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(a), bits_of(b))
    assert np.array_equal(bits_of(c), bits_of(d))
    assert not np.array_equal(bits_of(a), bits_of(d))


def check_full_size(vd, q, k, v, cu, H, label, rows):
    import torch
    from gpu_util import device_slots
    slots = device_slots()
    lens = [int(b - a) for a, b in zip(cu[:-1], cu[1:])]
    entries, D, G, cut = varlen_plan(lens, H, slots)
    extra = varlen_cut_rows(lens, H, slots, seed=len(lens))
    print(f"[case] {label}: {slots} slots, {len(entries) * H} items, {D} whole, {len(cut)} cut over {G} "
          f"workgroups, {extra.size} rows in cut items", flush=True)
    assert cut
    o, lse, o_plain, lse_plain = run_both(vd, q, k, v, cu, 0)
    T = int(cu[-1])
    rows = np.unique(np.concatenate([rows, extra]))
    o_ref, lse_ref = attention_varlen(q, k, v, cu, SCALE, rows=rows)
    h_of, t_of = rows // T, rows % T
    check(f64_of(o)[t_of, h_of], o_ref, lse.cpu().numpy()[h_of, t_of].astype(np.float64), lse_ref,
          f"{label} ({rows.size} rows)")
    uncut_items_equal(o, lse, o_plain, lse_plain, lens, H, slots)


def test_packed_varlen_workload_split(vd):
    w = WORKLOADS["packed_varlen"]
    q, k, v, cu = make_varlen(w)
    check_full_size(vd, q, k, v, cu, w.H, "packed_varlen split", sample_rows(w))


def test_one_long_segment_h2_split(vd):
    """One GPU's share of the 720p call as a packed batch: one 180320-token segment, H = 2
    (1410 items, 5.5 rounds of 256 workgroups): the last 130 items are cut over 256 workgroups."""
    import dataclasses
    w = dataclasses.replace(WORKLOADS["video_720p"], H=2)
    qb, kb, vb = make_dense(w)
    q, k, v = (np.ascontiguousarray(x[0].transpose(1, 0, 2)) for x in (qb, kb, vb))   # [N, 2, 128] THD
    cu = np.array([0, w.N], dtype=np.int32)
    rows = np.random.default_rng(7).choice(2 * w.N, 512, replace=False)
    check_full_size(vd, q, k, v, cu, 2, "one 180320-token segment H=2 split", rows)
