"""Seeded generators for features, routing and FP8 expert weights.

Recipes (all seeded; seed 0 unless a test picks another):
  * features x[N, d]: float32 N(0, 1) rows; for the K2 workloads each row is
    then RMS-normalised in float32 (mean of squares, eps 1e-6, gain 1, the
    normalisation on the "Input features" page, evidence "rmsnorm") and
    rounded to bfloat16;
  * routing ids[N, K]: K distinct experts per token, either uniform (the first
    K of a uniformly random permutation) or Zipf(1.2) without replacement over
    a seeded permutation of the experts (Gumbel top-K on log r^-1.2);
  * routing weights w[N, K]: softmax of N(0,1) logits, U(0,1) normalised to
    sum 1, Dirichlet(1), or all ones (a shard's unweighted rows);
  * expert weights: W ~ 0.02 N(0,1) in float32 per projection, one scale per
    128 x 128 block s = blockmax / 448, codes = e4m3(W / s) through torch's
    float8_e4m3fn cast (a library codec, independent of both the oracle's and
    the kernels' converters).

Host weights use numpy's PCG64; device weights are drawn on the GPU with
torch's generator (the 16.9 GB K2 expert set is too slow to draw on the CPU).
The two draws differ; a test takes all of its inputs from one of them and
copies device weights to the host for the oracle.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from .configs import Config

GROUP = 128
FP8_MAX = 448.0

# stream ids for SeedSequence spawning
_S_X, _S_IDS, _S_W, _S_EXPERTS, _S_SHARED, _S_HIDDEN = 1, 2, 3, 4, 5, 6


def _rng(seed: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, *extra])))


# --------------------------------------------------------------------------- features
def make_x_bits(cfg: Config, seed: int | None = None) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of the layer input x[N, d]."""
    seed = cfg.seed if seed is None else seed
    x = _rng(seed, _S_X).standard_normal((cfg.N, cfg.d), dtype=np.float32)
    t = torch.from_numpy(x)
    if cfg.x_mode == "rmsnorm":
        var = t.pow(2).mean(-1, keepdim=True)
        t = t * torch.rsqrt(var + 1e-6)
    elif cfg.x_mode != "normal":
        raise ValueError(cfg.x_mode)
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def make_block_inputs(cfg: Config, seed: int | None = None):
    """Inputs of the FFN half of a block around the layer: the residual stream h[N, d] as
    bfloat16 bits (float32 N(0,1) rows, not normalised: the block's RMSNorm does that) and
    the RMSNorm gain [d] as bfloat16 bits (1, the gain the recipe above uses)."""
    seed = cfg.seed if seed is None else seed
    h = _rng(seed, _S_HIDDEN).standard_normal((cfg.N, cfg.d), dtype=np.float32)
    h_bits = torch.from_numpy(h).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    gain_bits = np.full(cfg.d, 0x3F80, np.uint16)   # bfloat16 1.0
    return h_bits, gain_bits


# --------------------------------------------------------------------------- routing
def make_routing(cfg: Config, seed: int | None = None):
    """(ids int32 [N, K], weights float32 [N, K]) with K distinct ids per row."""
    seed = cfg.seed if seed is None else seed
    N, E, K = cfg.N, cfg.E, cfg.K
    r = _rng(seed, _S_IDS)
    if cfg.ids_mode == "uniform":
        ids = np.argsort(r.random((N, E)), axis=1, kind="stable")[:, :K]
    elif cfg.ids_mode == "zipf":
        perm = r.permutation(E)                       # rank -> expert
        logp = -1.2 * np.log(np.arange(1, E + 1, dtype=np.float64))
        logp_expert = np.empty(E)
        logp_expert[perm] = logp                       # expert perm[r] has rank r+1
        gumbel = -np.log(-np.log(r.random((N, E))))
        ids = np.argsort(-(logp_expert[None, :] + gumbel), axis=1, kind="stable")[:, :K]
    else:
        raise ValueError(cfg.ids_mode)
    ids = np.ascontiguousarray(ids.astype(np.int32))

    rw = _rng(seed, _S_W)
    if cfg.w_mode == "softmax":
        logits = rw.standard_normal((N, K))
        e = np.exp(logits - logits.max(axis=1, keepdims=True))
        w = e / e.sum(axis=1, keepdims=True)
    elif cfg.w_mode == "uniform":
        u = rw.random((N, K))
        w = u / u.sum(axis=1, keepdims=True)
    elif cfg.w_mode == "dirichlet":
        w = rw.dirichlet(np.ones(K), size=N)
    elif cfg.w_mode == "ones":
        w = np.ones((N, K))
    else:
        raise ValueError(cfg.w_mode)
    return ids, np.ascontiguousarray(w.astype(np.float32))


# --------------------------------------------------------------------------- weights
def _block_quantise(W: torch.Tensor):
    """W[..., out, in] float32 -> (codes uint8 same shape, scales float32 [..., out/128, in/128])."""
    *lead, o, i = W.shape
    blk = W.reshape(*lead, o // GROUP, GROUP, i // GROUP, GROUP)
    amax = blk.abs().amax(dim=(-3, -1))
    s = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (blk / s[..., :, None, :, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(*lead, o, i), s.to(torch.float32)


@dataclass
class HostExperts:
    """Stacked expert weights as numpy arrays (layouts as in the oracle and the ABI)."""
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


@dataclass
class DeviceExperts:
    """Stacked expert weights as torch tensors on one device."""
    w_gate: torch.Tensor
    s_gate: torch.Tensor
    w_up: torch.Tensor
    s_up: torch.Tensor
    w_down: torch.Tensor
    s_down: torch.Tensor

    @property
    def E(self):
        return self.w_gate.shape[0]

    @property
    def d_ff(self):
        return self.w_gate.shape[1]

    @property
    def d(self):
        return self.w_gate.shape[2]


def _host_set(E: int, d: int, d_ff: int, std: float, seed: int, stream: int) -> HostExperts:
    out = {}
    for p, (name, o, i) in enumerate((("gate", d_ff, d), ("up", d_ff, d), ("down", d, d_ff))):
        qs, ss = [], []
        for e in range(E):
            W = _rng(seed, stream, e, p).standard_normal((o, i), dtype=np.float32) * np.float32(std)
            q, s = _block_quantise(torch.from_numpy(W))
            qs.append(q.numpy())
            ss.append(s.numpy())
        out["w_" + name] = np.ascontiguousarray(np.stack(qs))
        out["s_" + name] = np.ascontiguousarray(np.stack(ss))
    return HostExperts(**out)


def make_experts_host(cfg: Config, seed: int | None = None, E: int | None = None) -> HostExperts:
    """Routed expert weights drawn on the CPU (small shapes)."""
    seed = cfg.seed if seed is None else seed
    return _host_set(cfg.E if E is None else E, cfg.d, cfg.d_ff, cfg.weight_std, seed, _S_EXPERTS)


def make_shared_host(cfg: Config, seed: int | None = None) -> HostExperts:
    """The shared expert (E = 1) drawn on the CPU."""
    seed = cfg.seed if seed is None else seed
    return _host_set(1, cfg.d, cfg.d_ff, cfg.weight_std, seed, _S_SHARED)


_DEVICE_CACHE: dict = {}


def _device_set(E: int, d: int, d_ff: int, std: float, seed: int, stream: int, device) -> DeviceExperts:
    device = torch.device(device)
    key = (E, d, d_ff, std, seed, stream, str(device))
    if key in _DEVICE_CACHE:
        return _DEVICE_CACHE[key]
    g = torch.Generator(device=device)
    chunk = 8
    out = {}
    for p, (name, o, i) in enumerate((("gate", d_ff, d), ("up", d_ff, d), ("down", d, d_ff))):
        q_all = torch.empty((E, o, i), dtype=torch.uint8, device=device)
        s_all = torch.empty((E, o // GROUP, i // GROUP), dtype=torch.float32, device=device)
        for e0 in range(0, E, chunk):
            e1 = min(E, e0 + chunk)
            g.manual_seed(((seed * 7 + stream) * 3 + p) * 1_000_003 + e0)
            W = torch.randn((e1 - e0, o, i), generator=g, device=device, dtype=torch.float32) * std
            q, s = _block_quantise(W)
            q_all[e0:e1].copy_(q)
            s_all[e0:e1].copy_(s)
            del W, q, s
        out["w_" + name] = q_all
        out["s_" + name] = s_all
    res = DeviceExperts(**out)
    _DEVICE_CACHE[key] = res
    return res


def make_experts_device(cfg: Config, device="cuda", seed: int | None = None) -> DeviceExperts:
    """Routed expert weights drawn on a GPU (K2 shapes: 16.9 GB of e4m3 codes)."""
    seed = cfg.seed if seed is None else seed
    return _device_set(cfg.E, cfg.d, cfg.d_ff, cfg.weight_std, seed, _S_EXPERTS, device)


def make_shared_device(cfg: Config, device="cuda", seed: int | None = None) -> DeviceExperts:
    seed = cfg.seed if seed is None else seed
    return _device_set(1, cfg.d, cfg.d_ff, cfg.weight_std, seed, _S_SHARED, device)


def experts_to_host(dev: DeviceExperts, experts=None) -> HostExperts:
    """Copy device weights to host memory. With ``experts`` (a list of expert ids),
    only those experts are copied and the rest of the host arrays stay zero, which
    is enough for an oracle that evaluates only tokens routed to those experts."""
    if experts is None:
        return HostExperts(*(t.cpu().numpy() for t in (dev.w_gate, dev.s_gate, dev.w_up, dev.s_up,
                                                         dev.w_down, dev.s_down)))
    out = []
    for t in (dev.w_gate, dev.s_gate, dev.w_up, dev.s_up, dev.w_down, dev.s_down):
        a = np.zeros(tuple(t.shape), dtype=np.uint8 if t.dtype == torch.uint8 else np.float32)
        for e in sorted(set(int(v) for v in experts)):
            a[e] = t[e].cpu().numpy()
        out.append(a)
    return HostExperts(*out)


# --------------------------------------------------------------------------- bundles
@dataclass
class Workload:
    cfg: Config
    x_bits: np.ndarray
    ids: np.ndarray
    w: np.ndarray
    experts_host: HostExperts | None = None
    shared_host: HostExperts | None = None
    experts_dev: DeviceExperts | None = None
    shared_dev: DeviceExperts | None = None
    extra: dict = field(default_factory=dict)


def make_workload(cfg: Config, weights: str = "host", device="cuda", seed: int | None = None) -> Workload:
    """Inputs of one configuration. weights: "host" (numpy draw), "device" (GPU draw) or "none"."""
    x = make_x_bits(cfg, seed)
    ids, w = make_routing(cfg, seed)
    wl = Workload(cfg, x, ids, w)
    if weights == "host":
        wl.experts_host = make_experts_host(cfg, seed)
        if cfg.shared:
            wl.shared_host = make_shared_host(cfg, seed)
    elif weights == "device":
        wl.experts_dev = make_experts_device(cfg, device, seed)
        if cfg.shared:
            wl.shared_dev = make_shared_device(cfg, device, seed)
    elif weights != "none":
        raise ValueError(weights)
    return wl
