"""Python binding of libmoe: the same calls as include/moe.h, taking torch tensors.

Argument marshalling only -- every step of the layer runs in the HIP kernels of
libmoe. PyTorch provides device memory (outputs and workspaces are torch
allocations) and the stream (the current torch stream of the tensors' device).

Layouts (row-major, on one GPU):
    x          [N, d]       torch.bfloat16
    topk_ids   [N, K]       torch.int32
    topk_w     [N, K]       torch.float32
    experts    object with w_gate, w_up [E, d_ff, d] uint8 (e4m3 codes),
               s_gate, s_up [E, d_ff/128, d/128] float32,
               w_down [E, d, d_ff] uint8, s_down [E, d/128, d_ff/128] float32
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from ._lib import (FLAG_CHECKED, FLAG_TILE_16, FLAG_TILE_128, FLAG_TILE_192, FLAG_TILE_224, FLAG_TILE_256,  # noqa: F401
                   KERNEL_COMBINE, KERNEL_DISPATCH, KERNEL_DOWN, KERNEL_GATE_UP, KERNEL_QUANT, check, lib)


def _p(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _want(t: torch.Tensor, dtype, name: str, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


_WS_CACHE: dict = {}
_WS_RETIRED: list = []


def _workspace(nbytes: int, dev: torch.device, tag: str) -> torch.Tensor:
    """A cached uint8 workspace per (device, stream, purpose), grown as needed. Calls on one
    stream run in order, so they can share it; calls on different streams get workspaces of
    their own and may overlap. (A graph capture runs on a stream of its own, so its first call
    allocates inside the capture, from the graph's memory pool.) A workspace that is outgrown
    stays allocated: a captured HIP graph may still address it."""
    key = (str(dev), torch.cuda.current_stream(dev).cuda_stream, tag)
    ws = _WS_CACHE.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _WS_RETIRED.append(ws)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _WS_CACHE[key] = ws
    return ws


@dataclass
class Dispatch:
    counts: torch.Tensor        # [E] int32 (tokens per expert)
    offsets: torch.Tensor       # [E+1] int32
    sorted_slot: torch.Tensor   # [N*K] int32, position -> slot
    slot_pos: torch.Tensor      # [N*K] int32, slot -> position
    N: int
    K: int
    E: int


def quantize_rows(x: torch.Tensor):
    """bf16 rows -> (e4m3 codes uint8 [rows, cols], scales float32 [rows, cols/128])."""
    _want(x, torch.bfloat16, "x", 2)
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, max(cols // 128, 0)), dtype=torch.float32, device=x.device)
    check(lib().moe_quantize_rows(_p(x), rows, cols, _p(q), _p(s), _stream(x.device)), "moe_quantize_rows")
    return q, s


def dispatch(topk_ids: torch.Tensor, E: int, checked: bool = False, _ws_tag: str = "dispatch") -> Dispatch:
    _want(topk_ids, torch.int32, "topk_ids", 2)
    N, K = topk_ids.shape
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_slot = torch.empty(N * K, dtype=torch.int32, device=dev)
    slot_pos = torch.empty(N * K, dtype=torch.int32, device=dev)
    nb = lib().moe_dispatch_workspace_size(N, K, E)
    ws = _workspace(nb, dev, _ws_tag)
    st = lib().moe_dispatch(_p(topk_ids), N, K, E, _p(counts), _p(offsets), _p(sorted_slot), _p(slot_pos),
                            _p(ws), ws.numel(), FLAG_CHECKED if checked else 0, _stream(dev))
    check(st, "moe_dispatch")
    return Dispatch(counts, offsets, sorted_slot, slot_pos, N, K, E)


def identity_dispatch(N: int, device, _ws_tag: str = "dispatch") -> Dispatch:
    """Dispatch of every token to a single expert (E = 1, K = 1): the shared expert's rows."""
    return dispatch(torch.zeros((N, 1), dtype=torch.int32, device=device), 1, _ws_tag=_ws_tag)


_SIDE: dict = {}


def _side_stream(dev: torch.device) -> torch.cuda.Stream:
    """A second stream per device (default priority) for the shared expert."""
    key = str(dev)
    s = _SIDE.get(key)
    if s is None:
        s = torch.cuda.Stream(device=dev)
        _SIDE[key] = s
    return s


def _expert_dims(experts, d: int, N: int, disp: Dispatch):
    ex = experts
    for name in ("w_gate", "w_up", "w_down"):
        _want(getattr(ex, name), torch.uint8, name, 3)
    for name in ("s_gate", "s_up", "s_down"):
        _want(getattr(ex, name), torch.float32, name, 3)
    E, d_ff, d_w = ex.w_gate.shape
    if d_w != d or disp.N != N or disp.E != E:
        raise ValueError("activations, dispatch and expert weights disagree on N, d or E")
    if tuple(ex.w_up.shape) != (E, d_ff, d) or tuple(ex.w_down.shape) != (E, d, d_ff):
        raise ValueError("expert weight shapes disagree")
    if (tuple(ex.s_gate.shape) != (E, d_ff // 128, d // 128) or tuple(ex.s_up.shape) != (E, d_ff // 128, d // 128)
            or tuple(ex.s_down.shape) != (E, d // 128, d_ff // 128)):
        raise ValueError("expert scale shapes disagree")
    return E, d_ff


def _y_out(out, rows: int, d: int, device):
    if out is None:
        return torch.empty((rows, d), dtype=torch.bfloat16, device=device)
    _want(out, torch.bfloat16, "out", 2)
    if tuple(out.shape) != (rows, d):
        raise ValueError(f"out must be [{rows}, {d}]")
    return out


def grouped_swiglu(x: torch.Tensor, disp: Dispatch, experts, flags: int = 0,
                   out: torch.Tensor | None = None, _ws_tag: str = "swiglu") -> torch.Tensor:
    """y_sorted [N*K, d] bf16: each sorted row through its expert's SwiGLU MLP (unweighted)."""
    _want(x, torch.bfloat16, "x", 2)
    N, d = x.shape
    E, d_ff = _expert_dims(experts, d, N, disp)
    ex, K = experts, disp.K
    out = _y_out(out, N * K, d, x.device)
    nb = lib().moe_swiglu_workspace_size(N, K, E, d, d_ff)
    ws = _workspace(nb, x.device, _ws_tag)
    st = lib().moe_grouped_swiglu(_p(x), N, K, E, d, d_ff, _p(disp.offsets), _p(disp.sorted_slot),
                                  _p(ex.w_gate), _p(ex.s_gate), _p(ex.w_up), _p(ex.s_up), _p(ex.w_down),
                                  _p(ex.s_down), _p(out), _p(ws), ws.numel(), int(flags), _stream(x.device))
    check(st, "moe_grouped_swiglu")
    return out


def grouped_swiglu_noalloc(x: torch.Tensor, disp: Dispatch, experts, flags: int = 0,
                           out: torch.Tensor | None = None) -> torch.Tensor:
    """grouped_swiglu without a workspace: the library's fixed per-GPU scratch array holds the
    intermediates, so the call allocates nothing (out, when given, is the only output). Calls
    that may overlap in time on one GPU must not be made; problems whose workspace would exceed
    MOE_NOALLOC_SCRATCH_BYTES raise MOE_ERR_WORKSPACE."""
    _want(x, torch.bfloat16, "x", 2)
    N, d = x.shape
    E, d_ff = _expert_dims(experts, d, N, disp)
    ex, K = experts, disp.K
    out = _y_out(out, N * K, d, x.device)
    st = lib().moe_grouped_swiglu_noalloc(_p(x), N, K, E, d, d_ff, _p(disp.offsets), _p(disp.sorted_slot),
                                          _p(ex.w_gate), _p(ex.s_gate), _p(ex.w_up), _p(ex.s_up), _p(ex.w_down),
                                          _p(ex.s_down), _p(out), int(flags), _stream(x.device))
    check(st, "moe_grouped_swiglu_noalloc")
    return out


def grouped_swiglu_q(xq: torch.Tensor, xs: torch.Tensor, disp: Dispatch, experts, flags: int = 0,
                     out: torch.Tensor | None = None, _ws_tag: str = "swiglu") -> torch.Tensor:
    """grouped_swiglu on activations already quantised: xq [N, d] uint8 e4m3 codes and
    xs [N, d/128] float32 scales, as quantize_rows or rmsnorm_quantize write them."""
    _want(xq, torch.uint8, "xq", 2)
    _want(xs, torch.float32, "xs", 2)
    N, d = xq.shape
    if tuple(xs.shape) != (N, d // 128):
        raise ValueError("xs must be [N, d/128]")
    E, d_ff = _expert_dims(experts, d, N, disp)
    ex, K = experts, disp.K
    out = _y_out(out, N * K, d, xq.device)
    nb = lib().moe_swiglu_q_workspace_size(N, K, E, d, d_ff)
    ws = _workspace(nb, xq.device, _ws_tag)
    st = lib().moe_grouped_swiglu_q(_p(xq), _p(xs), N, K, E, d, d_ff, _p(disp.offsets), _p(disp.sorted_slot),
                                    _p(ex.w_gate), _p(ex.s_gate), _p(ex.w_up), _p(ex.s_up), _p(ex.w_down),
                                    _p(ex.s_down), _p(out), _p(ws), ws.numel(), int(flags), _stream(xq.device))
    check(st, "moe_grouped_swiglu_q")
    return out


def grouped_swiglu_top1(x: torch.Tensor, disp: Dispatch, topk_w: torch.Tensor, experts, flags: int = 0,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """out [N, d] bf16 = topk_w[n] * expert(x[n]) for a top-1 dispatch (K = 1): the grouped
    experts with the combine done by the down projection's epilogue. Bit-identical to
    combine(grouped_swiglu(x, disp, experts), disp, topk_w)."""
    _want(x, torch.bfloat16, "x", 2)
    _want(topk_w, torch.float32, "topk_w", 2)
    N, d = x.shape
    if disp.K != 1 or tuple(topk_w.shape) != (N, 1):
        raise ValueError("grouped_swiglu_top1 needs a K = 1 dispatch and topk_w of shape [N, 1]")
    E, d_ff = _expert_dims(experts, d, N, disp)
    ex = experts
    out = _y_out(out, N, d, x.device)
    if out.data_ptr() == x.data_ptr() and N:
        raise ValueError("out must not overlap x")
    nb = lib().moe_swiglu_workspace_size(N, 1, E, d, d_ff)
    ws = _workspace(nb, x.device, "swiglu")
    st = lib().moe_grouped_swiglu_top1(_p(x), N, E, d, d_ff, _p(disp.offsets), _p(disp.sorted_slot),
                                       _p(disp.slot_pos), _p(topk_w),
                                       _p(ex.w_gate), _p(ex.s_gate), _p(ex.w_up), _p(ex.s_up), _p(ex.w_down),
                                       _p(ex.s_down), _p(out), _p(ws), ws.numel(), int(flags), _stream(x.device))
    check(st, "moe_grouped_swiglu_top1")
    return out


def combine(y_sorted: torch.Tensor, disp: Dispatch, topk_w: torch.Tensor,
            shared: torch.Tensor | None = None, out: torch.Tensor | None = None,
            residual: torch.Tensor | None = None) -> torch.Tensor:
    """out [N, d] bf16 = sum_k w[n,k] * y_sorted[slot_pos[n*K+k]] (+ shared[n]) (+ residual[n]).
    With a residual, out may be the residual tensor itself (updated in place)."""
    _want(y_sorted, torch.bfloat16, "y_sorted", 2)
    _want(topk_w, torch.float32, "topk_w", 2)
    N, K = topk_w.shape
    d = y_sorted.shape[1]
    if disp.N != N or disp.K != K or y_sorted.shape[0] != N * K:
        raise ValueError("combine shapes disagree")
    for name, t in (("shared", shared), ("residual", residual)):
        if t is not None:
            _want(t, torch.bfloat16, name, 2)
            if tuple(t.shape) != (N, d):
                raise ValueError(f"{name} must be [N, d]")
    out = _y_out(out, N, d, y_sorted.device)
    if residual is None:
        st = lib().moe_combine(_p(y_sorted), _p(disp.slot_pos), _p(topk_w), _p(shared), N, K, d, _p(out),
                               _stream(y_sorted.device))
        check(st, "moe_combine")
    else:
        st = lib().moe_combine_residual(_p(y_sorted), _p(disp.slot_pos), _p(topk_w), _p(shared), _p(residual),
                                        N, K, d, _p(out), _stream(y_sorted.device))
        check(st, "moe_combine_residual")
    return out


def rmsnorm_quantize(h: torch.Tensor, gain: torch.Tensor, eps: float, keep_normed: bool = False):
    """The block's RMSNorm of h [rows, cols] bf16 with gain [cols] bf16, fused with its e4m3
    quantisation: (codes uint8 [rows, cols], scales float32 [rows, cols/128], and the
    normalised bf16 rows when keep_normed, else None)."""
    _want(h, torch.bfloat16, "h", 2)
    _want(gain, torch.bfloat16, "gain", 1)
    rows, cols = h.shape
    if gain.shape[0] != cols:
        raise ValueError("gain must have one entry per column")
    q = torch.empty((rows, cols), dtype=torch.uint8, device=h.device)
    s = torch.empty((rows, max(cols // 128, 0)), dtype=torch.float32, device=h.device)
    y = torch.empty_like(h) if keep_normed else None
    check(lib().moe_rmsnorm_quantize_rows(_p(h), _p(gain), float(eps), rows, cols, _p(y), _p(q), _p(s),
                                          _stream(h.device)), "moe_rmsnorm_quantize_rows")
    return q, s, y


def moe_layer(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, experts,
              shared_expert=None, flags: int = 0) -> torch.Tensor:
    """The whole layer: dispatch -> grouped SwiGLU experts -> weighted combine (+ shared expert).

    Enqueues kernels only (no host synchronisation, no allocation inside the library), so a
    call can be captured into a HIP graph (torch.cuda.graph) once it has run eagerly with the
    same shapes, which sizes the cached workspaces."""
    E = experts.w_gate.shape[0]
    disp = dispatch(topk_ids, E)
    if disp.K == 1 and shared_expert is None:
        # one choice per token: the combine is done by the down projection's epilogue
        return grouped_swiglu_top1(x, disp, topk_w, experts, flags)
    shared = None
    if shared_expert is not None:
        # the shared expert is independent of the routed experts until the combine: it runs on
        # a second stream (with workspaces of its own), so that its small launches fill the
        # routed launches' idle CUs instead of queueing behind them
        main = torch.cuda.current_stream(x.device)
        side = _side_stream(x.device)
        side.wait_stream(main)
        x.record_stream(side)
        with torch.cuda.stream(side):
            sdisp = identity_dispatch(x.shape[0], x.device, _ws_tag="dispatch_shared")
            shared = grouped_swiglu(x, sdisp, shared_expert, _ws_tag="swiglu_shared")
        shared.record_stream(main)
    y = grouped_swiglu(x, disp, experts, flags)
    if shared is not None:
        torch.cuda.current_stream(x.device).wait_stream(_side_stream(x.device))
    return combine(y, disp, topk_w, shared)


def moe_block_ffn(hidden: torch.Tensor, gain: torch.Tensor, eps: float, topk_ids: torch.Tensor,
                  topk_w: torch.Tensor, experts, shared_expert=None, flags: int = 0,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """The FFN half of a MoE block around the layer, with its neighbours fused in:
    hidden + layer(RMSNorm(hidden)). The RMSNorm runs in the same pass as the activation
    quantisation and the residual addition in the combine; the routing (ids, weights) is
    given. Returns the new residual stream (out may be hidden itself)."""
    E = experts.w_gate.shape[0]
    xq, xs, _ = rmsnorm_quantize(hidden, gain, eps)
    disp = dispatch(topk_ids, E)
    shared = None
    if shared_expert is not None:
        # on a second stream, as in moe_layer
        main = torch.cuda.current_stream(hidden.device)
        side = _side_stream(hidden.device)
        side.wait_stream(main)
        xq.record_stream(side)
        xs.record_stream(side)
        with torch.cuda.stream(side):
            sdisp = identity_dispatch(hidden.shape[0], hidden.device, _ws_tag="dispatch_shared")
            shared = grouped_swiglu_q(xq, xs, sdisp, shared_expert, _ws_tag="swiglu_shared")
        shared.record_stream(main)
    y = grouped_swiglu_q(xq, xs, disp, experts, flags)
    if shared is not None:
        torch.cuda.current_stream(hidden.device).wait_stream(_side_stream(hidden.device))
    return combine(y, disp, topk_w, shared, out=out, residual=hidden)


# ---------------------------------------------------------------- dense block
_ONES: dict = {}


def _unit_weights(N: int, dev: torch.device) -> torch.Tensor:
    """[N, 1] float32 ones, cached per device (a larger cached column is sliced; an outgrown
    one stays allocated, as a captured graph may address it)."""
    key = str(dev)
    t = _ONES.get(key)
    if t is None or t.shape[0] < N:
        if t is not None:
            _WS_RETIRED.append(t)
        t = torch.ones((max(N, 1), 1), dtype=torch.float32, device=dev)
        _ONES[key] = t
    return t[:N]


def dense_swiglu(x: torch.Tensor, mlp, flags: int = 0, out: torch.Tensor | None = None) -> torch.Tensor:
    """The dense block's SwiGLU MLP, down(silu(gate x) * up x), through the grouped kernels
    as one expert that every token visits (E = 1, K = 1): out [N, d] bf16 in token order.
    mlp holds the three projections like an expert set with E = 1; the intermediate size is
    whatever its weights have (any multiple of 128)."""
    _want(x, torch.bfloat16, "x", 2)
    if mlp.w_gate.shape[0] != 1:
        raise ValueError("a dense MLP is an expert set with E = 1")
    return grouped_swiglu(x, identity_dispatch(x.shape[0], x.device), mlp, flags, out)


def dense_block_ffn(hidden: torch.Tensor, gain: torch.Tensor, eps: float, mlp, flags: int = 0,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """The FFN half of a dense block: hidden + MLP(RMSNorm(hidden)), with the RMSNorm fused
    into the activation quantisation and the residual addition done by the combine (one
    choice of weight 1 per token). out may be hidden itself."""
    _want(hidden, torch.bfloat16, "hidden", 2)
    if mlp.w_gate.shape[0] != 1:
        raise ValueError("a dense MLP is an expert set with E = 1")
    N = hidden.shape[0]
    xq, xs, _ = rmsnorm_quantize(hidden, gain, eps)
    disp = identity_dispatch(N, hidden.device)
    y = grouped_swiglu_q(xq, xs, disp, mlp, flags)
    return combine(y, disp, _unit_weights(N, hidden.device), out=out, residual=hidden)


# ---------------------------------------------------------------- profiling
def profile_enable(on: bool = True, kinds=None):
    """Time every kernel kind (on), none (off), or only the given KERNEL_* kinds."""
    if kinds is None or not on:
        check(lib().moe_profile_enable(1 if on else 0), "moe_profile_enable")
    else:
        mask = 0
        for k in kinds:
            mask |= 1 << int(k)
        check(lib().moe_profile_enable_kinds(mask), "moe_profile_enable_kinds")


def profile_reset():
    check(lib().moe_profile_reset(), "moe_profile_reset")


def profile_read(kind: int):
    """(total milliseconds, launches) of one kernel kind since the last reset."""
    ms = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    check(lib().moe_profile_read(kind, ctypes.byref(ms), ctypes.byref(n)), "moe_profile_read")
    return ms.value, n.value
