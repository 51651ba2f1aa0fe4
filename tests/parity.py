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


class WholeBatch:
    """Whole-batch comparison against the oracle, fed chunk by chunk so that the oracle's
    float64 result never has to be held for the whole batch: per-token relative L2 for every
    token, and the elementwise bar against the largest |ref| over the whole batch."""

    def __init__(self, what: str, n: int):
        self.what = what
        self.rel = np.zeros(n, np.float64)
        self.max_diff = 0.0
        self.max_ref = 0.0
        self.done = 0

    def add(self, rows: np.ndarray, gpu_bits: np.ndarray, ref64: np.ndarray):
        g = oracle.bf16_to_f32(gpu_bits).astype(np.float64)
        assert np.all(np.isfinite(g)), f"{self.what}: non-finite output"
        r = np.asarray(ref64, dtype=np.float64)
        diff = g - r
        num = np.sqrt((diff ** 2).sum(axis=1))
        den = np.sqrt((r ** 2).sum(axis=1))
        self.rel[rows] = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
        self.max_diff = max(self.max_diff, float(np.abs(diff).max()) if diff.size else 0.0)
        self.max_ref = max(self.max_ref, float(np.abs(r).max()) if r.size else 0.0)
        self.done += len(rows)

    def summary(self) -> dict:
        n = self.rel.size
        worst = int(self.rel.argmax()) if n else -1
        elem = self.max_diff / self.max_ref if self.max_ref > 0 else self.max_diff
        return {"tokens": n, "max_rel_l2": float(self.rel.max()) if n else 0.0,
                "p99_9_rel_l2": float(np.quantile(self.rel, 0.999)) if n else 0.0,
                "median_rel_l2": float(np.median(self.rel)) if n else 0.0,
                "worst_token": worst, "elem_err_over_max_ref": float(elem),
                "tokens_above_half_bar": int((self.rel > REL_L2_TOL / 2).sum())}

    def check(self):
        assert self.done == self.rel.size, f"{self.what}: {self.done} of {self.rel.size} tokens compared"
        s = self.summary()
        print(f"[whole-batch] {self.what}: " + " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}"
                                                     for k, v in s.items()), flush=True)
        assert s["max_rel_l2"] <= REL_L2_TOL, f"{self.what}: per-token relative L2 {s['max_rel_l2']} > {REL_L2_TOL}"
        assert s["elem_err_over_max_ref"] <= ELEM_TOL, \
            f"{self.what}: elementwise error {s['elem_err_over_max_ref']} > {ELEM_TOL} * max|ref|"
        return s
