"""Seeded synthetic inputs shared by the GPU path and the CPU oracle.

This module draws random numbers and rounds them to the storage type; it holds
none of the eviction method's arithmetic.  Both sides of a parity check read
the very same bytes: the GPU gets the bf16 (or fp32) buffers, the oracle gets
those values widened to float64.

Recipe (every array is a pure function of the workload name and the indices):
  * queries of the observation window  Q_win[i] ~ N(0, 1) / tau_i
  * keys and values                    K, V ~ N(0, 1)
  * sink keys (first `sinks` rows of every KV head) point along the mean of the
    group's window queries: K[g, :sinks] = 4 * sqrt(d) * unit(mean_{i in g, r} Q_win[i, r])
  * decode queries q ~ N(0, 1) / tau_i; appended k_new, v_new ~ N(0, 1)
  * output projection (CriticalKV, LaProx): o_proj weight [hidden, Hq*d] ~
    N(0, 1/hidden); LaProx instances are layers, each with its own projection
  * tau: a fixed list for the tiny case, else log-uniform in [0.1, 3] per
    (layer, query head); small tau gives a sharp (sparse) head, large tau a
    dispersed one.
fp32 draws are rounded to bf16 round-to-nearest-even once.
"""
from __future__ import annotations

import math
import zlib
from typing import Dict

import numpy as np

from .configs import Workload

SEED_BASE = 20260000


def _cfg_id(cfg: Workload) -> int:
    return zlib.crc32(cfg.name.encode()) & 0x7FFFFFFF


def _rng(cfg: Workload, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, _cfg_id(cfg), *ids])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (bf16 bits as uint16, or float32) -> float64 values."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def taus(cfg: Workload, layer: int) -> np.ndarray:
    if isinstance(cfg.tau[0], str):
        _, lo, hi = cfg.tau
        r = _rng(cfg, 1, layer)
        return np.exp(r.uniform(math.log(lo), math.log(hi), size=cfg.hq))
    t = np.asarray(cfg.tau, dtype=np.float64)
    assert t.size == cfg.hq
    return t


def make_instance(cfg: Workload, inst: int = 0, n_override: int | None = None) -> Dict[str, np.ndarray]:
    """One (layer, sequence) instance in storage form (uint16 bf16 bits or float32).

    n_override shortens the cache (for parity cases that must run on the CPU).
    """
    n = cfg.n if n_override is None else n_override
    layer = inst // cfg.batch
    tau = taus(cfg, layer)
    r = _rng(cfg, 0, inst)
    hq, hkv, d, w, G = cfg.hq, cfg.hkv, cfg.d, cfg.w, cfg.group
    q = r.standard_normal((hq, w, d), dtype=np.float32) / tau[:, None, None].astype(np.float32)
    k = r.standard_normal((hkv, n, d), dtype=np.float32)
    v = r.standard_normal((hkv, n, d), dtype=np.float32)
    q_st = _store(q, cfg.dtype)
    qv = widen(q_st, cfg.dtype).astype(np.float32)
    for g in range(hkv):
        if cfg.sinks:
            m = qv[g * G:(g + 1) * G].reshape(-1, d).mean(axis=0)
            u = m / max(float(np.linalg.norm(m)), 1e-30)
            k[g, :cfg.sinks] = (4.0 * math.sqrt(d)) * u
    out = {"q_win": q_st, "k": _store(k, cfg.dtype), "v": _store(v, cfg.dtype), "tau": tau}
    steps = cfg.decode_steps
    if steps:
        qd = r.standard_normal((steps, hq, d), dtype=np.float32) / tau[None, :, None].astype(np.float32)
        out["q_dec"] = _store(qd, cfg.dtype)
        if cfg.append:
            out["k_new"] = _store(r.standard_normal((steps, hkv, d), dtype=np.float32), cfg.dtype)
            out["v_new"] = _store(r.standard_normal((steps, hkv, d), dtype=np.float32), cfg.dtype)
    if cfg.scorer in ("criticalkv", "laprox"):
        wo = r.standard_normal((cfg.hidden, hq * d), dtype=np.float32) / np.float32(math.sqrt(cfg.hidden))
        out["w_o"] = _store(wo, cfg.dtype)
    return out


def make_batch_torch(cfg: Workload, device, n_override: int | None = None, chunk: int = 8):
    """All instances of a workload, drawn on the device with torch's generator.

    Same distributions and structure as make_instance (a different random
    stream: used where the oracle reads the device bytes back, e.g. benches
    and full-size sampled parity).  Returns a dict of device tensors with a
    leading instance dimension.
    """
    import torch
    n = cfg.n if n_override is None else n_override
    I, hq, hkv, d, w, G = cfg.instances, cfg.hq, cfg.hkv, cfg.d, cfg.w, cfg.group
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(SEED_BASE + _cfg_id(cfg))
    tau = torch.tensor(np.stack([taus(cfg, i // cfg.batch) for i in range(I)]), dtype=torch.float32, device=device)
    q = (torch.randn((I, hq, w, d), generator=gen, device=device) / tau[:, :, None, None]).to(tdt)
    k = torch.empty((I, hkv, n, d), dtype=tdt, device=device)
    v = torch.empty((I, hkv, n, d), dtype=tdt, device=device)
    for s in range(0, I, chunk):
        e = min(I, s + chunk)
        k[s:e] = torch.randn((e - s, hkv, n, d), generator=gen, device=device).to(tdt)
        v[s:e] = torch.randn((e - s, hkv, n, d), generator=gen, device=device).to(tdt)
    if cfg.sinks:
        m = q.float().reshape(I, hkv, G * w, d).mean(dim=2)
        u = m / m.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        k[:, :, :cfg.sinks, :] = ((4.0 * math.sqrt(d)) * u)[:, :, None, :].to(tdt)
    out = {"q_win": q, "k": k, "v": v, "tau": tau}
    if cfg.decode_steps:
        st = cfg.decode_steps
        out["q_dec"] = (torch.randn((st, I, hq, d), generator=gen, device=device) / tau[None, :, :, None]).to(tdt)
        if cfg.append:
            out["k_new"] = torch.randn((st, I, hkv, d), generator=gen, device=device).to(tdt)
            out["v_new"] = torch.randn((st, I, hkv, d), generator=gen, device=device).to(tdt)
    if cfg.scorer == "criticalkv":
        out["w_o"] = (torch.randn((cfg.hidden, hq * d), generator=gen, device=device) / math.sqrt(cfg.hidden)).to(tdt)
    elif cfg.scorer == "laprox":      # one projection per layer
        out["w_o"] = torch.empty((I, cfg.hidden, hq * d), dtype=tdt, device=device)
        for i in range(I):
            out["w_o"][i] = (torch.randn((cfg.hidden, hq * d), generator=gen, device=device)
                             / math.sqrt(cfg.hidden)).to(tdt)
    return out
