"""Seeded synthetic inputs for the channel-wise gated delta rule.

This module is shared by the HIP path's tests/benchmark and the fp64 oracle.
It holds none of the method's arithmetic: it only draws random numbers and
rounds them once to their storage dtype.  Gate values are produced already
activated (alpha as an fp32 log-decay <= 0, b in (0, 2), w in (0, 1)) because
the recurrence takes them that way (Muir reading notes, arXiv:2611.08376,
section 2.1: alpha in (0,1)^dk, b in (0,2)^dk, w in (0,1)^dv).

Every tensor comes from its own numpy PCG64 stream seeded by
``SeedSequence(seed, spawn_key=(crc32(name), step))``, so adding a tensor or a
step never shifts the others.  Values are drawn in fp64 and rounded once with
round-to-nearest-even (``torch.Tensor.to``); the oracle reads the rounded
values upcast to fp64, so input rounding is not counted as error.

Workloads (the five configurations of this project; sizes may be overridden
for small parity cases that keep the same value distributions):

  tiny      B1 H1 T256 d64, fp32; alpha = exp(-0.1 softplus(N)) per channel;
            b = 2 sigmoid(N), w = sigmoid(N) per channel; gamma = 1, z = 0;
            S0 = 0; chunk 64; seed 0.
  kda       B4 H16 T4096 d128, bf16 q/k/v; b = w = beta per token,
            beta = sigmoid(N); alpha per channel as in tiny; no gain; S0 = 0;
            chunk 64; seed 1.
  gdn2      B2 H16 T16384 d128, bf16; per-channel alpha (as tiny), b, w;
            gamma = 1 + 0.1 N static per (head, channel); z ~ N(0,1) per
            token; S0 = 0.02 N in fp32; chunk 64; seed 2.
  stress    B1 H16 T32768 d128, bf16; per head a random half of the key
            channels is slow (1 - alpha ~ U(1e-4, 1e-3)), the other half fast
            (1 - alpha ~ U(0.1, 0.5)); keys k_raw = N(0,1) + 3 * mask with 6
            distinct channels per token; b, w, gamma, z, S0 as gdn2; chunk
            64 and 128; seed 3.
  decode    256 sequences x H16, fp32 state 128 x 128 ~ 0.02 N; per step one
            token of bf16 q, k, v and gates as gdn2; 1024 steps; seed 4.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str            # storage dtype of q, k, v, b, w, z: "bf16" or "f32"
    chunk: int
    seed: int
    gates: str            # "gdn2" (per-channel b, w), "kda" (per-token beta)
    alpha: str            # "softplus", "bimodal" (per channel) or "scalar" (per token)
    sparse_keys: bool
    gain: bool            # gamma and z present
    s0: bool              # nonzero initial state
    steps: int = 0        # decode steps (decode workload only)

    def with_sizes(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 1, 256, 64, 64, "f32", 64, 0, "gdn2", "softplus",
                     False, False, False),
    "kda": Workload("kda", 4, 16, 4096, 128, 128, "bf16", 64, 1, "kda", "softplus",
                    False, False, False),
    "gdn2": Workload("gdn2", 2, 16, 16384, 128, 128, "bf16", 64, 2, "gdn2",
                     "softplus", False, True, True),
    "stress": Workload("stress", 1, 16, 32768, 128, 128, "bf16", 64, 3, "gdn2",
                       "bimodal", True, True, True),
    "decode": Workload("decode", 256, 16, 1, 128, 128, "bf16", 64, 4, "gdn2",
                       "softplus", False, True, True, steps=1024),
    # scalar-gate case (Gated DeltaNet): one decay and one beta per token
    # (b = w = beta), at the long-context shape
    "gdn": Workload("gdn", 1, 16, 32768, 128, 128, "bf16", 128, 5, "kda", "scalar",
                    False, False, True),
}


def _rng(seed: int, name: str, step: int = 0) -> np.random.Generator:
    key = (zlib.crc32(name.encode()) & 0x7FFFFFFF, int(step))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _store(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.to(torch.float32)
    raise ValueError(dtype)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def _log_alpha(wl: Workload, shape, step: int) -> np.ndarray:
    if wl.alpha == "softplus":
        x = _rng(wl.seed, "log_alpha", step).standard_normal(shape)
        return -0.1 * _softplus(x)
    if wl.alpha == "scalar":  # one decay per token: [B,H,T]
        x = _rng(wl.seed, "log_alpha", step).standard_normal(shape[:-1])
        return -0.1 * _softplus(x)
    if wl.alpha == "bimodal":
        B, H, T, dk = shape
        # one fixed slow/fast split of the key channels per head
        split = _rng(wl.seed, "alpha_split").random((H, dk)).argsort(axis=1) < dk // 2
        g = _rng(wl.seed, "log_alpha", step)
        slow = g.uniform(1e-4, 1e-3, shape)
        fast = g.uniform(0.1, 0.5, shape)
        one_minus = np.where(split[None, :, None, :], slow, fast)
        return np.log1p(-one_minus)
    raise ValueError(wl.alpha)


def _keys(wl: Workload, shape, step: int) -> np.ndarray:
    g = _rng(wl.seed, "k", step)
    x = g.standard_normal(shape)
    if wl.sparse_keys:
        B, H, T, dk = shape
        # 6 distinct channels per token carry a +3 offset
        order = _rng(wl.seed, "k_mask", step).random(shape).argsort(axis=-1)
        x = x + 3.0 * (order < 6)
    return x


def make_inputs(wl: Workload, step: int = 0, device: Optional[str] = None) -> dict:
    """Draw one batch of inputs for ``wl``.

    Returns a dict of torch tensors (CPU unless ``device``):
      q, k: [B,H,T,dk]; v: [B,H,T,dv] (storage dtype);
      log_alpha: [B,H,T,dk] fp32 ([B,H,T] for a scalar decay);
      b: [B,H,T,dk] or [B,H,T] (kda: per-token beta); w: [B,H,T,dv] or [B,H,T];
      gamma: [H,dk] fp32 or None; z: [B,H,T,dk] or None; S0: [B,H,dk,dv] fp32
      or None; plus the gate modes "b_mode"/"w_mode" ("channel" or "token").
    For the decode workload T = 1 and ``step`` selects the token.
    """
    B, H, T, dk, dv = wl.B, wl.H, wl.T, wl.dk, wl.dv
    s = step
    out = {}
    out["q"] = _store(_rng(wl.seed, "q", s).standard_normal((B, H, T, dk)), wl.dtype)
    out["k"] = _store(_keys(wl, (B, H, T, dk), s), wl.dtype)
    out["v"] = _store(_rng(wl.seed, "v", s).standard_normal((B, H, T, dv)), wl.dtype)
    out["log_alpha"] = _store(_log_alpha(wl, (B, H, T, dk), s), "f32")
    if wl.gates == "kda":
        beta = _sigmoid(_rng(wl.seed, "beta", s).standard_normal((B, H, T)))
        out["b"] = _store(beta, wl.dtype)
        out["w"] = out["b"]
        out["b_mode"] = out["w_mode"] = "token"
    else:
        out["b"] = _store(2.0 * _sigmoid(_rng(wl.seed, "b", s).standard_normal((B, H, T, dk))),
                          wl.dtype)
        out["w"] = _store(_sigmoid(_rng(wl.seed, "w", s).standard_normal((B, H, T, dv))),
                          wl.dtype)
        out["b_mode"] = out["w_mode"] = "channel"
    if wl.gain:
        out["gamma"] = _store(1.0 + 0.1 * _rng(wl.seed, "gamma").standard_normal((H, dk)), "f32")
        out["z"] = _store(_rng(wl.seed, "z", s).standard_normal((B, H, T, dk)), wl.dtype)
    else:
        out["gamma"] = None
        out["z"] = None
    if wl.s0:
        out["S0"] = _store(0.02 * _rng(wl.seed, "S0").standard_normal((B, H, dk, dv)), "f32")
    else:
        out["S0"] = None
    if device is not None:
        for key, val in list(out.items()):
            if isinstance(val, torch.Tensor):
                out[key] = val.to(device)
    return out


def key_participation_ratio(k_unit: np.ndarray) -> float:
    """Mean of (sum k^2)^2 / sum k^4 over tokens: effective number of key channels."""
    k2 = np.asarray(k_unit, dtype=np.float64) ** 2
    return float(np.mean(k2.sum(-1) ** 2 / np.maximum((k2 ** 2).sum(-1), 1e-300)))


def make_inputs_device(wl: Workload, device: str, seed: int = 0, steps: int = 0) -> dict:
    """The same recipe as ``make_inputs``, drawn with torch's generator on
    ``device`` (fast, for benchmarks; the values differ from ``make_inputs``).

    With ``steps`` > 0 every per-token tensor gets a leading step dimension
    (decode: [steps, B, H, d]); gamma and S0 stay static.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(1000003 * wl.seed + seed)
    B, H, T, dk, dv = wl.B, wl.H, wl.T, wl.dk, wl.dv
    lead = (steps,) if steps else ()
    tok = lead + (B, H) + ((T,) if not steps else ())
    f32 = dict(device=device, dtype=torch.float32)
    sdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    def normal(*shape):
        return torch.randn(shape, generator=gen, **f32)

    def uniform(lo, hi, *shape):
        return lo + (hi - lo) * torch.rand(shape, generator=gen, **f32)

    out = {"q": normal(*tok, dk).to(sdt)}
    kraw = normal(*tok, dk)
    if wl.sparse_keys:
        order = torch.rand(tok + (dk,), generator=gen, **f32).argsort(dim=-1)
        kraw = kraw + 3.0 * (order < 6).float()
    out["k"] = kraw.to(sdt)
    out["v"] = normal(*tok, dv).to(sdt)
    if wl.alpha == "softplus":
        out["log_alpha"] = -0.1 * torch.nn.functional.softplus(normal(*tok, dk))
    elif wl.alpha == "scalar":
        out["log_alpha"] = -0.1 * torch.nn.functional.softplus(normal(*tok))
    else:
        split = torch.rand((H, dk), generator=gen, **f32).argsort(dim=1) < dk // 2
        split = split.view((1,) * len(lead) + (1, H) + ((1,) if not steps else ()) + (dk,))
        om = torch.where(split, uniform(1e-4, 1e-3, *tok, dk), uniform(0.1, 0.5, *tok, dk))
        out["log_alpha"] = torch.log1p(-om)
    if wl.gates == "kda":
        out["b"] = torch.sigmoid(normal(*tok)).to(sdt)
        out["w"] = out["b"]
    else:
        out["b"] = (2.0 * torch.sigmoid(normal(*tok, dk))).to(sdt)
        out["w"] = torch.sigmoid(normal(*tok, dv)).to(sdt)
    out["gamma"] = (1.0 + 0.1 * normal(H, dk)) if wl.gain else None
    out["z"] = normal(*tok, dk).to(sdt) if wl.gain else None
    out["S0"] = (0.02 * normal(B, H, dk, dv)) if wl.s0 else None
    return out
