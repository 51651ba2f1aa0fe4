"""Helpers shared by the GPU parity tests: moving seeded inputs to the device and the
layer tolerance (per-token relative L2 <= 1e-2 and elementwise |err| <= 2e-2 * max|ref|,
against the oracle's value before its final bfloat16 rounding)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from workloads.gen import DeviceExperts, HostExperts

REL_L2_TOL = 1e-2
ELEM_TOL = 2e-2


def say(msg: str):
    """Name the case before a GPU step, flushed, so a fault leaves a trace."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def experts_dev(h: HostExperts, device="cuda") -> DeviceExperts:
    return DeviceExperts(*(torch.from_numpy(np.ascontiguousarray(a)).to(device)
                           for a in (h.w_gate, h.s_gate, h.w_up, h.s_up, h.w_down, h.s_down)))


def layer_errors(gpu_bits: np.ndarray, ref64: np.ndarray):
    """(max per-token relative L2, max |err| / max |ref|)."""
    g = oracle.bf16_to_f32(gpu_bits).astype(np.float64)
    r = np.asarray(ref64, dtype=np.float64)
    assert g.shape == r.shape
    if r.size == 0:
        return 0.0, 0.0
    diff = g - r
    num = np.sqrt((diff ** 2).sum(axis=1))
    den = np.sqrt((r ** 2).sum(axis=1))
    rel = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    scale = np.abs(r).max()
    elem = np.abs(diff).max() / scale if scale > 0 else np.abs(diff).max()
    return float(rel.max()), float(elem)


def assert_layer_close(gpu_bits: np.ndarray, ref64: np.ndarray, what: str = ""):
    g = oracle.bf16_to_f32(gpu_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    rel, elem = layer_errors(gpu_bits, ref64)
    print(f"[parity] {what}: max per-token rel L2 {rel:.3e}, max elementwise err/max|ref| {elem:.3e}", flush=True)
    assert rel <= REL_L2_TOL, f"{what}: per-token relative L2 {rel} > {REL_L2_TOL}"
    assert elem <= ELEM_TOL, f"{what}: elementwise error {elem} > {ELEM_TOL} * max|ref|"
