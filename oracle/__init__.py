"""Plain CPU oracle of the Kimi-K2 routed-expert MoE layer (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP library
under ``mixture_experts_ffn_ids_amd`` and never imports it.

The arithmetic lives in ``moe_oracle.c`` (plain C, OpenMP over tokens); this
module only builds that file with gcc, loads it with ctypes and marshals numpy
arrays. Every function cites the page passage it follows in the C source.
Parity pins: tests/test_oracle_codec.py, tests/test_oracle_dispatch.py,
tests/test_oracle_layer.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GROUP = 128
ERRORS = {0: "ok", 2: "shape", 5: "bad expert id", 6: "duplicate expert id in a row", 9: "out of memory"}


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc into oracle/liboracle.so (IEEE arithmetic, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        lib.orc_e4m3_decode.restype = ctypes.c_double
        lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_bf16_from_double.restype = ctypes.c_uint16
        lib.orc_bf16_from_double.argtypes = [ctypes.c_double]
        lib.orc_quant_rows_bf16.restype = ctypes.c_int
        lib.orc_quant_rows_bf16.argtypes = [P, i64, i64, P, P]
        lib.orc_quant_rows_f32.restype = ctypes.c_int
        lib.orc_quant_rows_f32.argtypes = [P, i64, i64, P, P]
        lib.orc_dispatch.restype = ctypes.c_int
        lib.orc_dispatch.argtypes = [P, i64, i32, i32, P, P, P, P]
        lib.orc_moe_forward.restype = ctypes.c_int
        lib.orc_moe_forward.argtypes = [P, i64, i32, P, P, i32, i32, i32,
                                        P, P, P, P, P, P,
                                        P, P, P, P, P, P, i32,
                                        P, P, i64, P, P, i32]
        lib.orc_rmsnorm_rows.restype = ctypes.c_int
        lib.orc_rmsnorm_rows.argtypes = [P, P, ctypes.c_float, i64, i64, P]
        lib.orc_expert_rows.restype = ctypes.c_int
        lib.orc_expert_rows.argtypes = [P, i64, i32, i32, i32, P, P, P, P, P, P, P, P, i64, P, P, P, i32]
        lib.orc_threads.restype = ctypes.c_int
        lib.orc_threads.argtypes = [i32]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int):
    if rc != 0:
        raise OracleError(ERRORS.get(rc, f"error {rc}"))


# --------------------------------------------------------------------------- codecs
def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode e4m3 codes (uint8) to float64 (OCP E4M3FN: bias 7, max 448, no inf)."""
    lib = _load()
    table = np.array([lib.orc_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round float32 values to e4m3 codes (nearest, ties to even code, saturating at 448)."""
    lib = _load()
    flat = np.asarray(v, dtype=np.float32).ravel()
    out = np.fromiter((lib.orc_e4m3_encode(float(t)) for t in flat), dtype=np.uint8, count=flat.size)
    return out.reshape(np.shape(v))


def bf16_from_f64(v: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 bit patterns (uint16), nearest-even, one rounding."""
    lib = _load()
    flat = np.asarray(v, dtype=np.float64).ravel()
    out = np.fromiter((lib.orc_bf16_from_double(float(t)) for t in flat), dtype=np.uint16, count=flat.size)
    return out.reshape(np.shape(v))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quant_rows_bf16(x_bits: np.ndarray):
    """Per-row, per-128-group dynamic e4m3 quantisation of bfloat16 rows -> (codes, scales)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // GROUP), np.float32)
    _check(_load().orc_quant_rows_bf16(_ptr(x_bits), rows, cols, _ptr(q), _ptr(s)))
    return q, s


def quant_rows_f32(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // GROUP), np.float32)
    _check(_load().orc_quant_rows_f32(_ptr(x), rows, cols, _ptr(q), _ptr(s)))
    return q, s


# --------------------------------------------------------------------------- dispatch
def dispatch(ids: np.ndarray, E: int):
    """(counts[E], offsets[E+1], sorted_slot[N*K], slot_pos[N*K]) for ids[N, K] (int32)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    N, K = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_slot = np.empty(N * K, np.int32)
    slot_pos = np.empty(N * K, np.int32)
    _check(_load().orc_dispatch(_ptr(ids), N, K, E, _ptr(counts), _ptr(offsets),
                                _ptr(sorted_slot), _ptr(slot_pos)))
    return counts, offsets, sorted_slot, slot_pos


# --------------------------------------------------------------------------- layer
def expert_weight_shapes(d: int, d_ff: int) -> dict:
    """Shapes of the three matrices the oracle reads for one expert, [out, in] as a
    bias-free linear map stores them ("SwiGLU output" page, evidence "mlp")."""
    return {"gate": (d_ff, d), "up": (d_ff, d), "down": (d, d_ff)}


def expert_scale_shapes(d: int, d_ff: int) -> dict:
    """Shapes of the per-128x128-block scales of those matrices (quantisation metadata)."""
    return {k: (o // GROUP, i // GROUP) for k, (o, i) in expert_weight_shapes(d, d_ff).items()}


@dataclass
class ExpertWeightsHost:
    """Stacked FP8 expert weights in host memory.

    w_gate, w_up: uint8 [E, d_ff, d]; s_gate, s_up: float32 [E, d_ff/128, d/128]
    w_down: uint8 [E, d, d_ff];        s_down: float32 [E, d/128, d_ff/128]
    """
    w_gate: np.ndarray
    s_gate: np.ndarray
    w_up: np.ndarray
    s_up: np.ndarray
    w_down: np.ndarray
    s_down: np.ndarray

    @property
    def E(self):
        return self.w_gate.shape[0]

    @property
    def d_ff(self):
        return self.w_gate.shape[1]

    @property
    def d(self):
        return self.w_gate.shape[2]


def moe_forward(x_bits: np.ndarray, ids: np.ndarray, w: np.ndarray, experts: ExpertWeightsHost,
                shared: ExpertWeightsHost | None = None, tokens: np.ndarray | None = None,
                threads: int = 0, residual: np.ndarray | None = None):
    """Layer output for the given tokens (default all): (bf16 bits [n, d], float64 [n, d]).
    residual (bf16 bits [N, d]) is added after the shared expert, before the rounding."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, d = x_bits.shape
    K = ids.shape[1]
    ex = experts
    assert ex.d == d and ids.shape[0] == N and w.shape == ids.shape
    if tokens is not None:
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        n_eval = tokens.size
    else:
        n_eval = N
    out = np.empty((n_eval, d), np.uint16)
    out64 = np.empty((n_eval, d), np.float64)
    sh = shared
    arrs = [np.ascontiguousarray(a) for a in (ex.w_gate, ex.s_gate, ex.w_up, ex.s_up, ex.w_down, ex.s_down)]
    if sh is not None:
        assert sh.E == 1 and sh.d == d
        sharrs = [np.ascontiguousarray(a) for a in (sh.w_gate, sh.s_gate, sh.w_up, sh.s_up, sh.w_down, sh.s_down)]
        sh_dff = sh.d_ff
    else:
        sharrs = [None] * 6
        sh_dff = 0
    if residual is not None:
        residual = np.ascontiguousarray(residual, dtype=np.uint16)
        assert residual.shape == (N, d)
    rc = _load().orc_moe_forward(_ptr(x_bits), N, d, _ptr(ids), _ptr(w), K, ex.E, ex.d_ff,
                                 *[_ptr(a) for a in arrs], *[_ptr(a) for a in sharrs], sh_dff,
                                 _ptr(residual), _ptr(tokens), n_eval, _ptr(out), _ptr(out64),
                                 int(threads))
    _check(rc)
    return out, out64


def rmsnorm_rows(x_bits: np.ndarray, gain_bits: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of bf16 rows [rows, cols] with a bf16 gain [cols]: bf16 bits [rows, cols]."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    gain_bits = np.ascontiguousarray(gain_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    assert gain_bits.shape == (cols,)
    y = np.empty((rows, cols), np.uint16)
    _check(_load().orc_rmsnorm_rows(_ptr(x_bits), _ptr(gain_bits), float(eps), rows, cols, _ptr(y)))
    return y


def expert_rows(x_bits: np.ndarray, experts, tokens: np.ndarray, expert_ids: np.ndarray,
                threads: int = 0):
    """One expert on one token per row: (y float64 [n, d], h codes uint8 [n, d_ff],
    h scales float32 [n, d_ff/128]) for the pairs (tokens[i], expert_ids[i])."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    N, d = x_bits.shape
    ex = experts
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    expert_ids = np.ascontiguousarray(expert_ids, dtype=np.int32)
    n = tokens.size
    y = np.empty((n, d), np.float64)
    hq = np.empty((n, ex.d_ff), np.uint8)
    hs = np.empty((n, ex.d_ff // GROUP), np.float32)
    arrs = [np.ascontiguousarray(a) for a in (ex.w_gate, ex.s_gate, ex.w_up, ex.s_up, ex.w_down, ex.s_down)]
    _check(_load().orc_expert_rows(_ptr(x_bits), N, d, ex.E, ex.d_ff, *[_ptr(a) for a in arrs],
                                   _ptr(tokens), _ptr(expert_ids), n, _ptr(y), _ptr(hq), _ptr(hs), int(threads)))
    return y, hq, hs


def threads_used(threads: int = 0) -> int:
    """Number of OpenMP threads the oracle runs with for the given request (0 = default)."""
    return int(_load().orc_threads(int(threads)))
