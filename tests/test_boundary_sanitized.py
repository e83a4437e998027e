"""The C-ABI validation layer under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The library's host code (argument checks, overlap and size arithmetic with its overflow
guards, the dense_layers parser, workspace plans) is rebuilt from the same sources with the
sanitizers on the host side only (each -fsanitize after -Xarch_host; the gfx950 device code is
compiled as usual), and the whole C-ABI matrix of tests/test_boundary.py runs against it in a
child process with the sanitizer runtime preloaded. Any report (out-of-bounds access, signed
overflow, misaligned access, use of an uninitialised shift, ...) aborts the child: the test
fails with the report. No GPU is used: launches fail on the host as they do without a device.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(asan_runtime() is None, reason="clang ASan runtime not installed")
def test_boundary_matrix_under_asan_and_ubsan(tmp_path):
    from video_diffusion_dit_amd.build import CSRC, HIPCC_FLAGS, SOURCES, hipcc, write_key_loop
    write_key_loop()
    lib = str(tmp_path / "libattn_sanitized.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan", "-g"]
    cmd = [hipcc(), *HIPCC_FLAGS, *san, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", lib,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ATTN_BOUNDARY_LIB=lib, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_boundary.py"), "-q",
                          "-m", "not gpu", "-k", "not python", "-p", "no:cacheprovider"],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = run.stdout[-4000:] + run.stderr[-4000:]
    assert run.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    print(run.stdout.strip().splitlines()[-1])
