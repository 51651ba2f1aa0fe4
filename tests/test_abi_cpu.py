"""The C ABI without a GPU: the library loads, exports exactly what include/moe.h
declares, and rejects bad arguments on the host before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

from mixture_experts_ffn_ids_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_layer_calls():
    names = declared_functions()
    for n in ("moe_dispatch", "moe_grouped_swiglu", "moe_combine", "moe_dispatch_workspace_size",
              "moe_swiglu_workspace_size", "moe_quantize_rows", "moe_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_no_undeclared_exports():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if re.search(r" T moe_", ln)}
    assert exported == set(declared_functions())


def test_status_strings():
    L = _lib.lib()
    for code in range(9):
        assert L.moe_status_string(code)
    assert L.moe_status_string(4) == b"workspace too small"


NULL = None


def test_dispatch_validation_on_host():
    L = _lib.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.cast(buf, ctypes.c_void_p)
    # K > E, K < 1, E < 1, N < 0, E beyond the limit
    assert L.moe_dispatch(p, 4, 9, 8, p, p, p, p, p, 1 << 16, 0, NULL) == 2
    assert L.moe_dispatch(p, 4, 0, 8, p, p, p, p, p, 1 << 16, 0, NULL) == 2
    assert L.moe_dispatch(p, 4, 1, 0, p, p, p, p, p, 1 << 16, 0, NULL) == 2
    assert L.moe_dispatch(p, -1, 2, 8, p, p, p, p, p, 1 << 16, 0, NULL) == 2
    assert L.moe_dispatch(p, 4, 2, 8193, p, p, p, p, p, 1 << 16, 0, NULL) == 2
    # null pointers
    assert L.moe_dispatch(NULL, 4, 2, 8, p, p, p, p, p, 1 << 16, 0, NULL) == 1
    assert L.moe_dispatch(p, 4, 2, 8, NULL, p, p, p, p, 1 << 16, 0, NULL) == 1
    # misaligned int32 array
    mis = ctypes.c_void_p(p.value + 2)
    assert L.moe_dispatch(mis, 4, 2, 8, p, p, p, p, p, 1 << 16, 0, NULL) == 3
    # workspace too small
    need = L.moe_dispatch_workspace_size(4, 2, 8)
    assert need > 0
    assert L.moe_dispatch(p, 4, 2, 8, p, p, p, p, p, need - 1, 0, NULL) == 4


def test_swiglu_and_combine_validation_on_host():
    L = _lib.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.cast(buf, ctypes.c_void_p)
    args = [p] * 7   # six weight/scale arrays and y_sorted
    # d, d_ff not multiples of 128
    assert L.moe_grouped_swiglu(p, 4, 2, 8, 100, 128, p, p, *args, p, 1 << 16, 0, NULL) == 2
    assert L.moe_grouped_swiglu(p, 4, 2, 8, 128, 0, p, p, *args, p, 1 << 16, 0, NULL) == 2
    # N = 0 is a no-op even with null pointers
    assert L.moe_grouped_swiglu(NULL, 0, 2, 8, 128, 128, *([NULL] * 9), NULL, 0, 0, NULL) == 0
    # null weight
    a2 = list(args)
    a2[2] = NULL
    assert L.moe_grouped_swiglu(p, 4, 2, 8, 128, 128, p, p, *a2, p, 1 << 16, 0, NULL) == 1
    # misaligned bf16 x
    mis = ctypes.c_void_p(p.value + 8)
    assert L.moe_grouped_swiglu(mis, 4, 2, 8, 128, 128, p, p, *args, p, 1 << 16, 0, NULL) == 3
    need = L.moe_swiglu_workspace_size(4, 2, 8, 128, 128)
    assert L.moe_grouped_swiglu(p, 4, 2, 8, 128, 128, p, p, *args, p, need - 1, 0, NULL) == 4
    # combine
    assert L.moe_combine(p, p, p, NULL, 4, 2, 130, p, NULL) == 2
    assert L.moe_combine(p, p, p, NULL, 4, 65, 128, p, NULL) == 2
    assert L.moe_combine(NULL, p, p, NULL, 4, 2, 128, p, NULL) == 1
    assert L.moe_combine(p, p, p, NULL, 0, 2, 128, NULL, NULL) == 0
    # quantize
    assert L.moe_quantize_rows(p, 3, 96, p, p, NULL) == 2
    assert L.moe_quantize_rows(NULL, 3, 128, p, p, NULL) == 1
    assert L.moe_quantize_rows(p, 0, 128, NULL, NULL, NULL) == 0


def test_workspace_sizes_scale_with_shapes():
    L = _lib.lib()
    small = L.moe_swiglu_workspace_size(16, 8, 384, 7168, 2048)
    big = L.moe_swiglu_workspace_size(8192, 8, 384, 7168, 2048)
    # x_q (N*d) + h_q (N*K*d_ff) dominate
    assert big >= 8192 * 7168 + 8192 * 8 * 2048
    assert small < big
    assert L.moe_swiglu_workspace_size(16, 8, 384, 7000, 2048) == 0


def test_noalloc_scratch_limit_at_k2_shapes():
    # the header's limit for moe_grouped_swiglu_noalloc at Kimi-K2 shapes: 2,760 tokens fit its
    # 64 MiB scratch, 2,761 do not
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m, "MOE_NOALLOC_SCRATCH_BYTES not found"
    cap = int(m.group(1)) << int(m.group(2))
    assert cap == 64 << 20
    assert "up to 2,760 tokens" in hdr
    L = _lib.lib()
    assert L.moe_swiglu_workspace_size(2760, 8, 384, 7168, 2048) <= cap
    assert L.moe_swiglu_workspace_size(2761, 8, 384, 7168, 2048) > cap


def test_profile_api_without_gpu():
    L = _lib.lib()
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    assert L.moe_profile_read(99, ctypes.byref(ms), ctypes.byref(n)) == 2
    assert L.moe_profile_read(0, ctypes.byref(ms), ctypes.byref(n)) == 0 and n.value == 0
    assert L.moe_profile_enable_kinds(1 << 5) == 2          # no such kind
    assert L.moe_profile_enable_kinds(1 << 2) == 0
    assert L.moe_profile_enable(0) == 0


def test_fused_neighbour_calls_validate_on_host():
    L = _lib.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.cast(buf, ctypes.c_void_p)
    # RMSNorm + quantisation: cols not a multiple of 128, negative or infinite eps, null, misaligned
    assert L.moe_rmsnorm_quantize_rows(p, p, 1e-6, 4, 100, NULL, p, p, NULL) == 2
    assert L.moe_rmsnorm_quantize_rows(p, p, -1.0, 4, 128, NULL, p, p, NULL) == 2
    assert L.moe_rmsnorm_quantize_rows(p, p, float("inf"), 4, 128, NULL, p, p, NULL) == 2
    assert L.moe_rmsnorm_quantize_rows(p, p, float("nan"), 4, 128, NULL, p, p, NULL) == 2
    assert L.moe_rmsnorm_quantize_rows(p, NULL, 1e-6, 4, 128, NULL, p, p, NULL) == 1
    assert L.moe_rmsnorm_quantize_rows(ctypes.c_void_p(p.value + 2), p, 1e-6, 4, 128, NULL, p, p, NULL) == 3
    assert L.moe_rmsnorm_quantize_rows(NULL, NULL, 1e-6, 0, 128, NULL, NULL, NULL, NULL) == 0
    # experts on quantised activations: null scales, misaligned codes, workspace without x_q/x_s
    args = [p] * 7
    assert L.moe_grouped_swiglu_q(p, NULL, 4, 2, 8, 128, 128, p, p, *args, p, 1 << 16, 0, NULL) == 1
    assert L.moe_grouped_swiglu_q(ctypes.c_void_p(p.value + 4), p, 4, 2, 8, 128, 128, p, p, *args, p, 1 << 16, 0,
                                  NULL) == 3
    q_ws = L.moe_swiglu_q_workspace_size(4, 2, 8, 128, 128)
    assert 0 < q_ws < L.moe_swiglu_workspace_size(4, 2, 8, 128, 128)
    assert L.moe_grouped_swiglu_q(p, p, 4, 2, 8, 128, 128, p, p, *args, p, q_ws - 1, 0, NULL) == 4
    # top-1 experts with the combine in the down epilogue: slot_pos and weights required and 4-B aligned,
    # shapes and workspace checked like moe_grouped_swiglu (the workspace of K = 1)
    wargs = [p] * 6
    assert L.moe_grouped_swiglu_top1(p, 4, 8, 128, 128, p, p, p, NULL, *wargs, p, p, 1 << 16, 0, NULL) == 1
    assert L.moe_grouped_swiglu_top1(p, 4, 8, 128, 128, p, p, NULL, p, *wargs, p, p, 1 << 16, 0, NULL) == 1
    assert L.moe_grouped_swiglu_top1(p, 4, 8, 128, 128, p, p, p, ctypes.c_void_p(p.value + 2), *wargs, p, p,
                                     1 << 16, 0, NULL) == 3
    assert L.moe_grouped_swiglu_top1(p, 4, 8, 128, 128, p, p, ctypes.c_void_p(p.value + 2), p, *wargs, p, p,
                                     1 << 16, 0, NULL) == 3
    assert L.moe_grouped_swiglu_top1(p, 4, 8, 130, 128, p, p, p, p, *wargs, p, p, 1 << 16, 0, NULL) == 2
    assert L.moe_grouped_swiglu_top1(p, -1, 8, 128, 128, p, p, p, p, *wargs, p, p, 1 << 16, 0, NULL) == 2
    t1_ws = L.moe_swiglu_workspace_size(4, 1, 8, 128, 128)
    assert L.moe_grouped_swiglu_top1(p, 4, 8, 128, 128, p, p, p, p, *wargs, p, p, t1_ws - 1, 0, NULL) == 4
    assert L.moe_grouped_swiglu_top1(NULL, 0, 8, 128, 128, NULL, NULL, NULL, NULL, *([NULL] * 6), NULL, NULL, 0,
                                     0, NULL) == 0
    # combine with the residual: the residual is required
    assert L.moe_combine_residual(p, p, p, NULL, NULL, 4, 2, 128, p, NULL) == 1
    assert L.moe_combine_residual(p, p, p, NULL, p, 4, 2, 130, p, NULL) == 2
