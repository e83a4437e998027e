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
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp]
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, sz, vp]
    lib.attn_fwd_varlen_workspace_bytes.argtypes = [i32, i32, i32]
    lib.attn_fwd_varlen_workspace_bytes.restype = sz
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.restype = ctypes.c_char_p
    return lib


def test_header_declares_the_expected_api():
    fns = header_functions()
    for name in ("attn_fwd", "attn_fwd_varlen", "attn_fwd_varlen_workspace_bytes",
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
])
def test_varlen_validation(lib, kw, code):
    assert varlen(lib, **kw) == code


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
