"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU.

tests/sanitize/api_host_check.hip is linked with the library's own api.hip, both built for the
host only (no device code) with the two sanitizers on the host pass. The check stands in for
the kernel launchers and the HIP runtime calls: its launchers touch every byte the real
kernels would, on buffers and workspaces of exactly the sizes the API asks for, and it
checks that the named workspace regions do not overlap. It drives every host-side error path,
valid calls of every entry point over a range of shapes and tile heights, and the size queries
at the ends of their ranges. Any sanitizer report aborts it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_ffn_ids_amd", "csrc")
CHECK = os.path.join(ROOT, "tests", "sanitize", "api_host_check.hip")


def _tool(name):
    for cand in (shutil.which(name), f"/opt/rocm/bin/{name}", f"/opt/rocm/llvm/bin/{name}"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip(f"{name} not found")


def test_api_host_code_under_asan_and_ubsan(tmp_path):
    hipcc, clang = _tool("hipcc"), _tool("clang++")
    # the sanitizers go on the host pass only (there is no device pass in a host-only build)
    common = ["-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in (os.path.join(CSRC, "api.hip"), CHECK):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([hipcc, *common, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    exe = str(tmp_path / "api_host_check")
    r = subprocess.run([clang, "-fsanitize=address,undefined", *objs, "-o", exe, "-lpthread"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert "0 failures" in out, out[-6000:]
