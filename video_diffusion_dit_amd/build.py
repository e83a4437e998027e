"""Build libattn.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: ``python -m video_diffusion_dit_amd.build`` (or ``__graft_entry__.build()``).
The library lands in ``video_diffusion_dit_amd/lib/libattn.so``; nothing is installed.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libattn.so")
SOURCES = ["attn_fwd_gfx950.hip", "block_route_gfx950.hip", "prologue_gfx950.hip", "linear_gfx950.hip",
           "attn_api.cpp"]
ARCH = "gfx950"

# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 in the device code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def write_key_loop() -> list:
    """Regenerate csrc/key_loop_gfx950.inc and csrc/key_loop_idx_gfx950.inc (the
    hand-scheduled key loop over a tile range and over a tile list) from their generator."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("gen_key_loop", os.path.join(CSRC, "gen_key_loop.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    for path, indexed in ((gen.OUT, False), (gen.OUT_IDX, True)):
        text = gen.render(indexed)
        old = open(path).read() if os.path.exists(path) else None
        if text != old:
            with open(path, "w") as f:
                f.write(text)
    return [gen.OUT, gen.OUT_IDX]


def build(verbose: bool = False) -> str:
    """Regenerate the key loop, then compile every source for gfx950 into LIB_PATH; always
    recompiles."""
    write_key_loop()
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
