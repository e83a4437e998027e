"""GPU test of attn_fwd_varlen_noalloc, the entry point for callers that cannot allocate: its
output must equal attn_fwd_varlen's (the same kernels, the schedule in the library's fixed
scratch instead of a workspace) bit for bit, on two calls in a row where the second is smaller
than the first, so a stale schedule left in the shared scratch would show. Both are also held
to the FP64 oracle's bar. Called through the C ABI (ctypes), arguments marshalled by hand."""
import math

import numpy as np
import pytest

from oracle import attention_varlen
from workloads import random_varlen

pytestmark = pytest.mark.gpu

SCALE = 1 / math.sqrt(128)


@pytest.fixture(scope="module")
def lib():
    import video_diffusion_dit_amd as m
    return m.load_library()


def call_both(lib, lens, H, seed):
    import torch
    from gpu_util import bits_of, check, dev, dev_i32, f64_of
    import video_diffusion_dit_amd.attention as A
    q, k, v, cu = random_varlen(lens, H, seed=seed)
    qd, kd, vd_, cud = dev(q), dev(k), dev(v), dev_i32(cu)
    T, nseg = int(cu[-1]), len(lens)
    print(f"[case] no-alloc varlen lens={lens} H={H}", flush=True)
    out_a = torch.full_like(qd, float("nan"))
    lse_a = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.attn_fwd_varlen_noalloc(qd.data_ptr(), kd.data_ptr(),
                                     vd_.data_ptr(), out_a.data_ptr(), lse_a.data_ptr(), cud.data_ptr(),
                                     nseg, H, T, 128, SCALE, stream)
    assert st == 0, lib.attn_last_error()
    out_b = torch.full_like(qd, float("nan"))
    lse_b = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda:0")
    nbytes = int(lib.attn_fwd_varlen_workspace_bytes(nseg, H, T))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    st = lib.attn_fwd_varlen(qd.data_ptr(), kd.data_ptr(), vd_.data_ptr(), out_b.data_ptr(), lse_b.data_ptr(),
                             cud.data_ptr(), nseg, H, T, 128, SCALE, ws.data_ptr(), nbytes, stream)
    assert st == 0, lib.attn_last_error()
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out_a), bits_of(out_b))
    assert np.array_equal(lse_a.cpu().numpy().view(np.uint32), lse_b.cpu().numpy().view(np.uint32))
    o_ref, lse_ref = attention_varlen(q, k, v, cu, SCALE)
    check(f64_of(out_a), o_ref, lse_a.cpu().numpy(), lse_ref, f"no-alloc varlen lens={lens} H={H}")


def test_no_alloc_matches_workspace_call_twice(lib):
    # first call: 1207 segments, so the schedule fills about 15 KB of the scratch
    call_both(lib, (1500, 1, 0, 700, 257, 64, 900) + (3,) * 1200, 3, seed=71)
    # second call, smaller: a few short segments; whatever the first left in the scratch
    call_both(lib, (130, 5), 2, seed=72)


def test_no_alloc_binding_matches_and_rejects_oversize(lib):
    import torch
    import video_diffusion_dit_amd as vd
    from gpu_util import bits_of, dev, dev_i32
    q, k, v, cu = random_varlen((300, 40), 2, seed=73)
    qd, kd, vd_, cud = dev(q), dev(k), dev(v), dev_i32(cu)
    out = torch.empty_like(qd)
    vd.attn_fwd_varlen_noalloc(qd, kd, vd_, cud, out)
    ref = vd.attn_fwd_varlen(qd, kd, vd_, cud, cu_seqlens_host=[int(x) for x in cu])
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out), bits_of(ref))
    # a schedule larger than the fixed scratch is refused before any launch
    n = 60000
    cu_big = dev_i32(np.arange(n + 1, dtype=np.int32))
    x = torch.zeros((n, 1, 128), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        vd.attn_fwd_varlen_noalloc(x, x.clone(), x.clone(), cu_big, torch.empty_like(x))
