"""The C ABI without a GPU: every symbol of include/attn.h is exported, and argument
validation answers on the host before any HIP call (so these run on any machine).

Fake device addresses below are never dereferenced: each call is rejected by validation.
"""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, -1, -2, -3, -4


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


@pytest.fixture(scope="module")
def lib():
    from video_diffusion_dit_amd.build import LIB_PATH, build
    path = os.environ.get("ATTN_BOUNDARY_LIB")   # another build of the same sources (the sanitized one)
    if path is None:
        path = LIB_PATH
        if not os.path.exists(LIB_PATH):
            build()
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp]
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, sz, vp]
    lib.attn_fwd_varlen_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp]
    lib.attn_qk_norm_packed.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, vp]
    lib.attn_fwd_varlen_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.attn_fwd_varlen_splitkv_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_fwd_varlen_splitkv_workspace_bytes.restype = sz
    lib.attn_fwd_varlen_workspace_bytes.argtypes = [i32, i32, i32]
    lib.attn_fwd_varlen_workspace_bytes.restype = sz
    lib.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.attn_fwd_splitkv_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_fwd_splitkv_workspace_bytes.restype = sz
    lib.attn_qk_prologue.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                     f32, f32, vp]
    lib.attn_linear_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, sz, vp]
    lib.attn_linear_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.attn_linear_workspace_bytes.restype = sz
    lib.attn_block_list_stride.argtypes = [i32]
    lib.attn_block_route_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.attn_block_route_workspace_bytes.restype = sz
    lib.attn_block_route.argtypes = [vp, vp, i32, i32, i32, i32, f32, f32, i32, vp, vp, vp, vp, sz, vp]
    lib.attn_fwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp]
    lib.attn_block_skip_use_dense.argtypes = [i32, i32, i32, ctypes.c_char_p]
    lib.attn_block_varlen_tiles.argtypes = [i32, i32]
    lib.attn_block_route_varlen_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.attn_block_route_varlen_workspace_bytes.restype = sz
    lib.attn_block_route_varlen.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, f32, i32, vp, vp, vp, vp, sz, vp]
    lib.attn_fwd_block_sparse_varlen_workspace_bytes.argtypes = [i32, i32, i32]
    lib.attn_fwd_block_sparse_varlen_workspace_bytes.restype = sz
    lib.attn_fwd_block_sparse_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, sz,
                                                 vp]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.restype = ctypes.c_char_p
    return lib


def test_header_declares_the_expected_api():
    fns = header_functions()
    for name in ("attn_fwd", "attn_fwd_varlen", "attn_fwd_varlen_workspace_bytes",
                 "attn_fwd_splitkv", "attn_fwd_splitkv_workspace_bytes", "attn_qk_prologue",
                 "attn_linear_fwd", "attn_linear_workspace_bytes", "attn_block_list_stride",
                 "attn_block_route", "attn_block_route_workspace_bytes", "attn_fwd_block_sparse",
                 "attn_block_skip_use_dense", "attn_block_varlen_tiles", "attn_block_route_varlen",
                 "attn_block_route_varlen_workspace_bytes", "attn_fwd_block_sparse_varlen",
                 "attn_fwd_block_sparse_varlen_workspace_bytes", "attn_fwd_varlen_noalloc",
                 "attn_fwd_varlen_splitkv", "attn_fwd_varlen_splitkv_workspace_bytes", "attn_qk_norm_packed",
                 "attn_status_string", "attn_last_error", "attn_tile_rows", "attn_tile_keys"):
        assert name in fns, fns


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), f"libattn.so does not export {name}"


# fake, never-dereferenced device addresses (distinct, far apart)
Q, K, V, O, L, CU, WS = (0x10000000 * (i + 1) for i in range(7))
MiB = 1 << 20


def dense(lib, q=Q, k=K, v=V, o=O, lse=None, B=1, H=2, N=256, d=128, scale=0.088):
    return lib.attn_fwd(q, k, v, o, lse, B, H, N, d, scale, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(o=None), INVALID),
    (dict(B=0), INVALID), (dict(H=0), INVALID), (dict(N=0), INVALID), (dict(N=-5), INVALID),
    (dict(d=64), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(d=0), INVALID),
    (dict(scale=math.nan), INVALID), (dict(scale=math.inf), INVALID),
    (dict(o=Q), INVALID), (dict(o=K + 64), INVALID),                         # out aliases q / k
    (dict(lse=O + 1024), INVALID),                                           # lse inside out
    (dict(B=1 << 20, H=1 << 20, N=1 << 20), UNSUPPORTED),                    # beyond index range
    (dict(B=1, H=1, N=8388608), UNSUPPORTED),                                # K/V rows past 2^31 - 1 bytes
])
def test_dense_validation(lib, kw, code):
    assert dense(lib, **kw) == code
    if code != OK:
        assert lib.attn_last_error().decode()


def varlen(lib, cu=CU, nseg=3, H=2, T=300, d=128, scale=0.088, ws=WS, wsb=None, lse=None, o=O):
    if wsb is None:
        wsb = lib.attn_fwd_varlen_workspace_bytes(nseg, H, T)
    return lib.attn_fwd_varlen(Q, K, V, o, lse, cu, nseg, H, T, d, scale, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(nseg=0), INVALID), (dict(T=-1), INVALID), (dict(cu=None), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(H=0), INVALID), (dict(scale=-math.inf), INVALID),
    (dict(ws=None), WORKSPACE), (dict(wsb=16), WORKSPACE), (dict(ws=WS + 8), WORKSPACE),
    (dict(o=V), INVALID), (dict(ws=O), INVALID),
    (dict(T=0), OK),                                                       # empty batch: no-op, no launch
    (dict(T=0, d=64), UNSUPPORTED), (dict(T=0, H=0), INVALID),
    (dict(T=4194304, H=2), UNSUPPORTED),                                   # T * H * 256 = 2^31 bytes
])
def test_varlen_validation(lib, kw, code):
    assert varlen(lib, **kw) == code


def varlen_noalloc(lib, cu=CU, nseg=3, H=2, T=300, d=128, scale=0.088, lse=None, o=O):
    return lib.attn_fwd_varlen_noalloc(Q, K, V, o, lse, cu, nseg, H, T, d, scale, None)


@pytest.mark.parametrize("kw,code", [
    (dict(nseg=0), INVALID), (dict(T=-1), INVALID), (dict(cu=None), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(H=0), INVALID), (dict(scale=math.nan), INVALID),
    (dict(o=V), INVALID), (dict(lse=O + 64), INVALID),
    (dict(T=0), OK),                                                       # empty batch: no-op, no launch
    (dict(T=4194304, H=2), UNSUPPORTED),                                   # T * H * 256 = 2^31 bytes
    (dict(nseg=60000, T=60000), UNSUPPORTED),                              # schedule beyond the fixed scratch
])
def test_varlen_noalloc_validation(lib, kw, code):
    assert varlen_noalloc(lib, **kw) == code
    if code == UNSUPPORTED and kw.get("nseg") == 60000:
        assert "scratch" in lib.attn_last_error().decode()


def test_noalloc_scratch_covers_every_nseg_up_to_16384(lib):
    # the header's promise: the schedule of nseg <= 16384 segments fits the fixed scratch at
    # any total_tokens the kernels accept (T * H <= 8388607, so T <= 8388607)
    text = open(HEADER).read()
    limit = int(text.split("#define ATTN_NOALLOC_SCRATCH_BYTES")[1].split()[0])
    assert lib.attn_fwd_varlen_workspace_bytes(16384, 1, 8388607) <= limit
    assert lib.attn_fwd_varlen_workspace_bytes(60000, 1, 60000) > limit


def test_workspace_query(lib):
    f = lib.attn_fwd_varlen_workspace_bytes
    assert f(0, 1, 10) == 0 and f(1, 0, 10) == 0 and f(1, 1, -1) == 0
    a, b = f(3, 24, 38048), f(3, 24, 80000)
    assert 0 < a < b and a % 256 == 0
    assert f(1000, 24, 38048) > a


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, 7):
        assert lib.attn_status_string(code).decode()
    assert dense(lib, d=64) == UNSUPPORTED
    assert "128" in lib.attn_last_error().decode()


def test_tile_shape_exports(lib):
    assert lib.attn_tile_rows() % 32 == 0 and lib.attn_tile_rows() >= 64
    assert lib.attn_tile_keys() in (32, 64, 128)


def test_python_cu_seqlens_validation():
    from video_diffusion_dit_amd import check_cu_seqlens
    assert check_cu_seqlens([0, 3, 3, 10], 10) == [0, 3, 3, 10]
    for bad, T in (([1, 3], 3), ([0, 5, 4, 9], 9), ([0, 4], 5), ([0], 0)):
        with pytest.raises(ValueError):
            check_cu_seqlens(bad, T)


def test_python_guards_without_gpu():
    import torch
    from video_diffusion_dit_amd import attn_fwd, try_attn_fwd
    q = torch.zeros(1, 1, 4, 128, dtype=torch.bfloat16)
    assert try_attn_fwd(q, q, q) is None                     # not on a GPU: caller falls back
    with pytest.raises(TypeError):
        attn_fwd(q.float(), q.float(), q.float())            # non-BF16 is a TypeError
    with pytest.raises(ValueError):
        attn_fwd(q, q, q)                                     # CPU tensors are rejected


# One partial result: 256 query rows x (128 O values + m_ref + l, padded to 132 floats).
PART_BYTES = 256 * 132 * 4


@pytest.mark.parametrize("B,H,N,slots,G", [
    (1, 16, 180320, 256, 256),    # 11280 tiles = 44 rounds + 16: the last 272 over 256 workgroups
    (1, 2, 180320, 256, 256),     # 1410 tiles = 5 rounds + 130
    (1, 1, 8192, 64, 64),         # 32 tiles < 64 slots: each cut in two (64 key tiles a share)
    (1, 1, 8192, 200, 200),       # shares of 20.48 key tiles: tiles cut into up to 8 pieces
    (1, 1, 8192, 1000, 256),      # shares never shorter than 16 key tiles: at most 128*32/16
])
def test_splitkv_workspace_plan(lib, B, H, N, slots, G):
    assert lib.attn_fwd_splitkv_workspace_bytes(B, H, N, 128, slots) == 2 * G * PART_BYTES


@pytest.mark.parametrize("B,H,N,slots", [
    (1, 16, 32768, 256),          # 2048 tiles: whole rounds, nothing to cut
    (4, 64, 512, 7),              # 8 key tiles per sequence: too short to cut
    (1, 1, 8192, 1),              # one slot
    (1, 1, 8192, 16),             # 32 tiles, 16 slots: two whole rounds
    (1, 1, 8192, 65537),          # beyond ATTN_MAX_SLOTS
    (0, 1, 8192, 64), (1, 0, 8192, 64), (1, 1, 0, 64),
])
def test_splitkv_no_workspace(lib, B, H, N, slots):
    assert lib.attn_fwd_splitkv_workspace_bytes(B, H, N, 128, slots) == 0
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 1, 8192, 64, 64) == 0      # d != 128


def splitkv(lib, q=Q, o=O, N=8192, d=128, slots=64, ws=WS, wsb=None, lse=None):
    if wsb is None:
        wsb = lib.attn_fwd_splitkv_workspace_bytes(1, 1, N, 128, slots)
    return lib.attn_fwd_splitkv(q, K, V, o, lse, 1, 1, N, d, 0.088, slots, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(d=64), UNSUPPORTED), (dict(slots=65537), INVALID),
    (dict(ws=None), WORKSPACE), (dict(wsb=1024), WORKSPACE), (dict(ws=WS + 16), WORKSPACE),
    (dict(ws=O), INVALID), (dict(o=K), INVALID),
    (dict(N=8388608), UNSUPPORTED),                                  # K/V rows past 2^31 - 1 bytes
])
def test_splitkv_validation(lib, kw, code):
    assert splitkv(lib, **kw) == code
    assert lib.attn_last_error().decode()


def test_python_splitkv_workspace_matches_c(lib):
    from video_diffusion_dit_amd import splitkv_workspace_bytes
    assert splitkv_workspace_bytes(1, 16, 180320, slots=256) == 2 * 256 * PART_BYTES
    assert splitkv_workspace_bytes(1, 16, 32768, slots=256) == 0


# ---------------------------------------------------------------- prologue
XQ, XK, XV, PQ, PK, PV, WQ, WK = (0x200000000 * (i + 1) for i in range(8))


def prologue(lib, xq=XQ, xk=XK, xv=XV, q=PQ, k=PK, v=PV, wq=None, wk=None, B=1, N=60, H=4, d=128,
             F=3, gh=4, gw=5, eps=1e-6, theta=10000.0):
    return lib.attn_qk_prologue(xq, xk, xv, q, k, v, wq, wk, B, N, H, d, F, gh, gw, eps, theta, None)


@pytest.mark.parametrize("kw,code", [
    (dict(xq=None), INVALID), (dict(k=None), INVALID), (dict(xv=None), INVALID), (dict(v=None), INVALID),
    (dict(B=0), INVALID), (dict(H=0), INVALID), (dict(N=0), INVALID), (dict(d=0), INVALID),
    (dict(d=64), UNSUPPORTED), (dict(gw=6), INVALID), (dict(F=0, N=0), INVALID), (dict(gh=-4, gw=-5), INVALID),
    (dict(eps=-1e-6), INVALID), (dict(eps=math.nan), INVALID), (dict(theta=0.0), INVALID),
    (dict(theta=math.inf), INVALID),
    (dict(q=XK), INVALID), (dict(v=XQ + 256), INVALID),                  # an output over an input
    (dict(k=PQ + 1024), INVALID),                                          # outputs overlap
    (dict(wq=PV + 64), INVALID),                                           # weight inside an output
    (dict(B=1 << 20, N=1 << 20, F=1 << 10, gh=1 << 10, gw=1), UNSUPPORTED),
])
def test_prologue_validation(lib, kw, code):
    assert prologue(lib, **kw) == code
    assert lib.attn_last_error().decode()


def qk_norm_packed(lib, xq=XQ, xk=XK, q=PQ, k=PK, wq=None, wk=None, T=300, H=4, d=128, eps=1e-6):
    return lib.attn_qk_norm_packed(xq, xk, q, k, wq, wk, T, H, d, eps, None)


@pytest.mark.parametrize("kw,code", [
    (dict(xq=None), INVALID), (dict(k=None), INVALID), (dict(T=-1), INVALID), (dict(H=0), INVALID),
    (dict(d=0), INVALID), (dict(d=64), UNSUPPORTED), (dict(eps=-1.0), INVALID), (dict(eps=math.inf), INVALID),
    (dict(T=0), OK),                                                       # empty batch: no-op
    (dict(q=XQ + 256), INVALID),                                           # partial overlap with its input
    (dict(q=XK), INVALID), (dict(k=XQ), INVALID), (dict(k=PQ + 512), INVALID),
    (dict(wk=PK + 64), INVALID),                                           # weight inside an output
    (dict(T=1 << 24, H=1 << 10), UNSUPPORTED),                             # more rows than one launch indexes
])
def test_qk_norm_packed_validation(lib, kw, code):
    assert qk_norm_packed(lib, **kw) == code


def test_varlen_splitkv_validation(lib):
    wsb = lib.attn_fwd_varlen_splitkv_workspace_bytes(3, 2, 300, 128, 16)
    assert wsb >= lib.attn_fwd_varlen_workspace_bytes(3, 2, 300)
    assert lib.attn_fwd_varlen_splitkv_workspace_bytes(3, 2, 300, 128, 1) == lib.attn_fwd_varlen_workspace_bytes(3, 2, 300)
    assert lib.attn_fwd_varlen_splitkv_workspace_bytes(3, 2, 300, 64, 16) == 0
    call = lambda **kw: lib.attn_fwd_varlen_splitkv(Q, K, V, kw.get("o", O), None, kw.get("cu", CU), 3, 2, 300,
                                                    kw.get("d", 128), 0.088, kw.get("slots", 16), kw.get("ws", WS),
                                                    kw.get("wsb", wsb), None)
    assert call(cu=None) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(slots=1 << 20) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(wsb=wsb - 1) == WORKSPACE
    assert call(ws=WS + 8) == WORKSPACE
    assert call(o=V) == INVALID


def test_python_prologue_guards_without_gpu():
    import torch
    import video_diffusion_dit_amd as vd
    x = torch.zeros((1, 6, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        vd.qk_prologue(x.float(), x, grid=(1, 2, 3))
    with pytest.raises(ValueError):
        vd.qk_prologue(x, x, grid=(1, 2, 3))          # CPU tensors


# ---------------------------------------------------------------- linear attention
LQ, LK, LQR, LKR, LV, LO, LWS = (0x4000000000 * (i + 1) for i in range(7))


def linear(lib, q=LQ, k=LK, qr=LQR, kr=LKR, v=LV, o=LO, B=1, N=300, H=2, d=128, eps=1e-15, ws=LWS, wsb=None):
    if wsb is None:
        wsb = lib.attn_linear_workspace_bytes(B, N, H, 128)
    return lib.attn_linear_fwd(q, k, qr, kr, v, o, B, N, H, d, eps, ws, wsb, None)


def test_linear_workspace_query(lib):
    f = lib.attn_linear_workspace_bytes
    # per head: one chunk partial (128*128 + 128 floats) per chunk, then kv as three BF16
    # terms and ksum (FP32), each region 256-byte aligned. The chunk is the shortest multiple of
    # 64 tokens (256 to 4096) whose B*H*chunks workgroups fit whole rounds of 3 per compute
    # unit; without a GPU the query assumes 256 compute units (768 slots).
    a = lambda x: (x + 255) // 256 * 256
    one, terms, ks = (128 * 128 + 128) * 4, 3 * 128 * 128 * 2, 128 * 4

    def expect(B, N, H, chunks):
        return a(B * H * chunks * one) + a(B * H * terms) + a(B * H * ks)
    assert f(1, 300, 2, 128) == expect(1, 300, 2, 2)              # 256-token chunks: 4 groups
    assert f(1, 180320, 16, 128) == expect(1, 180320, 16, 48)     # 3776: 768 groups, one round
    assert f(1, 180320, 2, 128) == expect(1, 180320, 2, 353)      # 512: 706 groups
    assert f(1, 180320, 4, 128) == expect(1, 180320, 4, 188)      # 960: 752 groups
    assert f(1, 180320, 8, 128) == expect(1, 180320, 8, 94)       # 1920: 752 groups
    assert f(1, 32760, 16, 128) == expect(1, 32760, 16, 47)       # 704: 752 groups
    assert f(1, 32760, 2, 128) == expect(1, 32760, 2, 128)        # 86 -> 256 (the floor): 256 groups
    assert f(4, 180320, 16, 128) == expect(4, 180320, 16, 48)     # 4096 needs 45 chunks a head: four rounds, 3776
    assert f(0, 300, 2, 128) == 0 and f(1, 300, 2, 64) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(kr=None), INVALID), (dict(o=None), INVALID),
    (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(H=0), INVALID), (dict(d=0), INVALID),
    (dict(d=64), UNSUPPORTED), (dict(eps=-1.0), INVALID), (dict(eps=math.inf), INVALID),
    (dict(o=LV + 128), INVALID),                                     # out overlaps v
    (dict(ws=None), WORKSPACE), (dict(wsb=1024), WORKSPACE), (dict(ws=LWS + 8), WORKSPACE),
    (dict(ws=LO), INVALID),                                          # workspace over out
    (dict(N=1 << 20, H=1024), UNSUPPORTED),                          # a (b, h) slice past 2 GiB
])
def test_linear_validation(lib, kw, code):
    assert linear(lib, **kw) == code
    assert lib.attn_last_error().decode()


# ---------------------------------------------------------------- block-skip attention
SQ, SK, SV, SO, SL, SI, SC, SW, SR = (0x8000000000 * (i + 1) for i in range(9))


def route(lib, q=SQ, k=SK, B=1, H=2, N=1000, d=128, scale=0.088, tau=0.1, sink=0, idx=SI, cnt=SC, order=SR, ws=SW,
          wsb=None):
    if wsb is None:
        wsb = lib.attn_block_route_workspace_bytes(B, H, N, 128)
    return lib.attn_block_route(q, k, B, H, N, d, scale, tau, sink, idx, cnt, order, ws, wsb, None)


def sparse(lib, q=SQ, k=SK, v=SV, o=SO, lse=SL, idx=SI, cnt=SC, order=SR, B=1, H=2, N=1000, d=128, scale=0.088):
    return lib.attn_fwd_block_sparse(q, k, v, o, lse, idx, cnt, order, B, H, N, d, scale, None)


def test_block_list_stride_and_route_workspace(lib):
    assert lib.attn_block_list_stride(1) == 1 + 8
    assert lib.attn_block_list_stride(64) == 1 + 8 and lib.attn_block_list_stride(65) == 2 + 8
    assert lib.attn_block_list_stride(180320) == 2818 + 8
    assert lib.attn_block_list_stride(0) == 0
    # pooled query tiles (FP32 [B*H][ceil(N/256)][128], 256-byte aligned), then pooled key tiles
    # (FP32 [B*H][32][ceil(N/64)][4])
    a = lambda x: (x + 255) // 256 * 256
    assert lib.attn_block_route_workspace_bytes(2, 3, 1000, 128) == a(6 * 4 * 512) + 6 * 16 * 512
    assert lib.attn_block_route_workspace_bytes(1, 2, 1000, 64) == 0
    assert lib.attn_block_route_workspace_bytes(0, 2, 1000, 128) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(cnt=None), INVALID), (dict(idx=None), INVALID),
    (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(d=64), UNSUPPORTED),
    (dict(scale=math.inf), INVALID), (dict(tau=-0.5), INVALID), (dict(tau=math.nan), INVALID),
    (dict(sink=-1), INVALID),
    (dict(N=983041), UNSUPPORTED),                                   # more key tiles than routing holds
    (dict(ws=None), WORKSPACE), (dict(wsb=100), WORKSPACE), (dict(ws=SW + 4), WORKSPACE),
    (dict(idx=SQ + 64), INVALID),                                    # list over q
    (dict(cnt=SI + 64), INVALID),                                    # counts inside the lists
    (dict(ws=SC), INVALID),                                          # workspace over the counts
    (dict(order=SC + 4), INVALID),                                   # order over the counts
])
def test_route_validation(lib, kw, code):
    assert route(lib, **kw) == code
    assert lib.attn_last_error().decode()


def test_route_accepts_infinite_tau_on_the_host(lib):
    # tau = +inf is valid (keeps every tile); with a null stream and fake pointers the call
    # would launch, so only the validation order is checked: a later error still wins
    assert route(lib, tau=math.inf, ws=None) == WORKSPACE


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(idx=None), INVALID), (dict(cnt=None), INVALID),
    (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(H=0), INVALID), (dict(d=64), UNSUPPORTED),
    (dict(scale=math.nan), INVALID), (dict(o=SV + 256), INVALID),   # out over v
    (dict(o=SI), INVALID), (dict(lse=SC), INVALID),                  # outputs over the lists
    (dict(o=SR), INVALID),                                           # out over the order
    (dict(B=1, H=1, N=8388608), UNSUPPORTED),                        # K/V rows past 2^31 - 1 bytes
])
def test_block_sparse_validation(lib, kw, code):
    assert sparse(lib, **kw) == code
    assert lib.attn_last_error().decode()


@pytest.mark.parametrize("step,layer,steps,layers,want", [
    (0, 7, 2, None, 1), (1, 7, 2, b"", 1), (2, 7, 2, b"", 0), (5, 3, 0, b"3", 1),
    (5, 3, 0, b"0-2,4", 0), (5, 4, 0, b"0-2,4", 1), (5, 12, 1, b" 0 - 2 , 9-12 ", 1),
    (5, 13, 1, b"0-2,9-12", 0),
    (5, 1, 0, b"2-1", INVALID), (5, 1, 0, b"1,", INVALID), (5, 1, 0, b"a", INVALID),
    (5, 1, 0, b"1;2", INVALID), (5, 1, 0, b"-1", INVALID), (-1, 1, 0, b"", INVALID),
    (1, -1, 0, b"", INVALID), (1, 1, -2, b"", INVALID), (5, 1, 0, b"99999999999", INVALID),
])
def test_dense_guard(lib, step, layer, steps, layers, want):
    assert lib.attn_block_skip_use_dense(step, layer, steps, layers) == want


def test_python_block_skip_guards_without_gpu():
    import torch
    import video_diffusion_dit_amd as vd
    x = torch.zeros((1, 2, 300, 128), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        vd.block_route(x.float(), x, tau=0.1)
    with pytest.raises(ValueError):
        vd.block_route(x, x, tau=0.1)                 # CPU tensors
    with pytest.raises(ValueError):
        vd.attn_fwd_block_sparse(x, x, x, torch.zeros(1, dtype=torch.int32), torch.zeros(1, dtype=torch.int32))
    assert vd.block_skip_use_dense(0, 0, 1, "") and not vd.block_skip_use_dense(1, 3, 1, "0-2")
    with pytest.raises(ValueError):
        vd.block_skip_use_dense(1, 3, 1, "3-")


# ---------------------------------------------------------------- packed block-skip
VQ, VK, VV, VO, VL, VI, VC, VW, VCU, VR = (0x10000000000 * (i + 1) for i in range(10))


def route_v(lib, q=VQ, k=VK, cu=VCU, nseg=3, H=2, T=1000, d=128, scale=0.088, tau=0.01, sink=0, idx=VI, cnt=VC,
            order=VR, ws=VW, wsb=None):
    if wsb is None:
        wsb = lib.attn_block_route_varlen_workspace_bytes(nseg, H, T, 128)
    return lib.attn_block_route_varlen(q, k, cu, nseg, H, T, d, scale, tau, sink, idx, cnt, order, ws, wsb, None)


def sparse_v(lib, q=VQ, k=VK, v=VV, o=VO, lse=VL, cu=VCU, idx=VI, cnt=VC, order=VR, nseg=3, H=2, T=1000, d=128,
             scale=0.088, ws=VW, wsb=None):
    if wsb is None:
        wsb = lib.attn_fwd_block_sparse_varlen_workspace_bytes(nseg, H, T)
    return lib.attn_fwd_block_sparse_varlen(q, k, v, o, lse, cu, idx, cnt, order, nseg, H, T, d, scale, ws, wsb, None)


def test_varlen_block_sizes(lib):
    assert lib.attn_block_varlen_tiles(3, 38048) == 38048 // 256 + 3
    assert lib.attn_block_varlen_tiles(0, 100) == 0
    a = lambda x: (x + 255) // 256 * 256
    # tile offsets (two int arrays of nseg + 1, then an item count), pooled query tiles,
    # pooled key tiles
    assert lib.attn_block_route_varlen_workspace_bytes(3, 2, 1000, 128) == \
        2 * a(4 * 4) + 256 + a((1000 // 256 + 3) * 2 * 512) + (1000 // 64 + 3) * 2 * 512
    assert lib.attn_block_route_varlen_workspace_bytes(3, 2, 1000, 64) == 0
    assert lib.attn_fwd_block_sparse_varlen_workspace_bytes(3, 2, 1000) == \
        lib.attn_fwd_varlen_workspace_bytes(3, 2, 1000) + 2 * a(4 * 4) + 256


@pytest.mark.parametrize("kw,code", [
    (dict(nseg=0), INVALID), (dict(H=0), INVALID), (dict(T=-1), INVALID), (dict(d=64), UNSUPPORTED),
    (dict(tau=-1.0), INVALID), (dict(sink=-2), INVALID), (dict(scale=math.nan), INVALID),
    (dict(q=None), INVALID), (dict(cu=None), INVALID), (dict(cnt=None), INVALID),
    (dict(T=983041), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(wsb=8), WORKSPACE), (dict(ws=VW + 8), WORKSPACE),
    (dict(idx=VQ + 256), INVALID), (dict(ws=VC), INVALID), (dict(cnt=VCU), INVALID),
    (dict(order=VI + 8), INVALID),
])
def test_route_varlen_validation(lib, kw, code):
    assert route_v(lib, **kw) == code
    assert lib.attn_last_error().decode()


def test_varlen_empty_batch_is_a_no_op(lib):
    assert route_v(lib, T=0, q=None, k=None, cu=None, idx=None, cnt=None, order=None, ws=None) == OK
    assert sparse_v(lib, T=0, q=None, k=None, v=None, o=None, cu=None, idx=None, cnt=None, order=None,
                    ws=None) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(nseg=0), INVALID), (dict(H=0), INVALID), (dict(d=64), UNSUPPORTED), (dict(scale=math.inf), INVALID),
    (dict(v=None), INVALID), (dict(cu=None), INVALID), (dict(idx=None), INVALID),
    (dict(ws=None), WORKSPACE), (dict(wsb=64), WORKSPACE),
    (dict(o=VQ), INVALID), (dict(o=VI), INVALID), (dict(lse=VC), INVALID), (dict(ws=VCU), INVALID),
    (dict(ws=VR), INVALID),
    (dict(T=4194304, H=2), UNSUPPORTED),                             # T * H * 256 = 2^31 bytes
])
def test_block_sparse_varlen_validation(lib, kw, code):
    assert sparse_v(lib, **kw) == code
    assert lib.attn_last_error().decode()
