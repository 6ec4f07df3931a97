"""Seeded synthetic inputs for the Muir operator.

This module is shared by the HIP library's tests/benchmark and by the oracle
checks, so it holds no arithmetic of the operator itself: it only draws
random tensors with the shapes and value distributions of the workloads
(arXiv 2611.08376: head size d_k = d_v = 128, 16 heads at d = 2,048, 4K
training length, 32K throughput context, streaming decode) and casts them
once to the working dtype.  The caller passes the drawn values to both
sides; neither side draws anything itself.

Recipe (numpy PCG64, one generator per call, fixed draw order):
  q, k   : x ~ N(0,1)^{d_k}; s = silu(x); q = s / ||s||_2 per (b, t, h)
           (the pages' q/k pathway ends in SiLU then unit normalisation)
  v      : N(0, 1)
  log_a  : "uniform"      -> U[-3, -1e-3] i.i.d. per element
           "channel"      -> per (h, j) rate r = exp(U[ln 1e-4, ln 3]),
                             log_a = -r for every b, t
           "channel_slow" -> as "channel", plus round(0.1 d_k) channels per
                             head (seeded choice) with r ~ U[1e-6, 1e-4]
           "zero"         -> 0 (no decay)
           "steep"        -> U[-12, -1e-3] i.i.d. per element (fast rows whose
                             16-token decay exceeds what a single leaf factor spans)
           "spiky"        -> "channel", plus log_a = -1e4 (state wiped: exp = 0)
                             on a seeded 2% of the elements
  erase, write : sigmoid(N(0,1));  gamma : 2 sigmoid(N(0,1))
  dO     : N(0, 1) (only when asked for)
  S0     : S0_scale * N(0, 1) in fp32 (zeros when S0_scale == 0)
Draw order: q, k, v, log_a, erase, write, gamma, dO, S0.  Values are drawn in
float32, transformed in float32, then rounded once (round-to-nearest-even)
to the requested dtype.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

_DT = {"bf16": torch.bfloat16, "f32": torch.float32, "fp32": torch.float32}


def _silu_unit(x: np.ndarray) -> np.ndarray:
    s = x / (1.0 + np.exp(-x))
    n = np.sqrt(np.sum(s * s, axis=-1, keepdims=True))
    return s / np.maximum(n, np.float32(1e-12))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _decay_rates(rng: np.random.Generator, H: int, dk: int, mode: str) -> np.ndarray:
    """Per-(head, channel) positive rates for the 'channel' modes, shape [H, dk]."""
    lo, hi = math.log(1e-4), math.log(3.0)
    r = np.exp(rng.uniform(lo, hi, size=(H, dk))).astype(np.float32)
    if mode == "channel_slow":
        nslow = int(round(0.1 * dk))
        for h in range(H):
            idx = rng.choice(dk, size=nslow, replace=False)
            r[h, idx] = rng.uniform(1e-6, 1e-4, size=nslow).astype(np.float32)
    return r


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(_DT[dtype])


def seq_inputs(B: int, T: int, H: int, dk: int, dv: int, *, dtype: str = "bf16",
               decay: str = "uniform", seed: int = 0, with_dO: bool = False,
               S0_scale: float = 0.0, with_dST: bool = False) -> Dict[str, torch.Tensor]:
    """Inputs of one chunkwise call, as CPU tensors in ``dtype`` ([B, T, H, D] layout).

    Keys: q, k, v, log_a, erase, write, gamma (dtype); dO (dtype, if asked);
    S0 (fp32 [B, H, dk, dv] or None); dS_T (fp32 or None).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    f32 = np.float32
    q = _silu_unit(rng.standard_normal((B, T, H, dk), dtype=f32))
    k = _silu_unit(rng.standard_normal((B, T, H, dk), dtype=f32))
    v = rng.standard_normal((B, T, H, dv), dtype=f32)
    if decay == "uniform":
        log_a = rng.uniform(-3.0, -1e-3, size=(B, T, H, dk)).astype(f32)
    elif decay in ("channel", "channel_slow"):
        r = _decay_rates(rng, H, dk, decay)
        log_a = np.broadcast_to(-r[None, None, :, :], (B, T, H, dk)).astype(f32)
    elif decay == "zero":
        log_a = np.zeros((B, T, H, dk), dtype=f32)
    elif decay == "steep":
        log_a = rng.uniform(-12.0, -1e-3, size=(B, T, H, dk)).astype(f32)
    elif decay == "spiky":
        r = _decay_rates(rng, H, dk, "channel")
        log_a = np.broadcast_to(-r[None, None, :, :], (B, T, H, dk)).astype(f32).copy()
        log_a[rng.random((B, T, H, dk)) < 0.02] = -1e4
    else:
        raise ValueError(f"unknown decay mode {decay!r}")
    erase = _sigmoid(rng.standard_normal((B, T, H, dk), dtype=f32))
    write = _sigmoid(rng.standard_normal((B, T, H, dv), dtype=f32))
    gamma = 2.0 * _sigmoid(rng.standard_normal((B, T, H, dk), dtype=f32))
    out = {n: _cast(a, dtype) for n, a in
           (("q", q), ("k", k), ("v", v), ("log_a", log_a), ("erase", erase), ("write", write), ("gamma", gamma))}
    out["dO"] = _cast(rng.standard_normal((B, T, H, dv), dtype=f32), dtype) if with_dO else None
    if S0_scale:
        out["S0"] = torch.from_numpy(S0_scale * rng.standard_normal((B, H, dk, dv), dtype=f32))
    else:
        out["S0"] = None
    out["dS_T"] = torch.from_numpy(rng.standard_normal((B, H, dk, dv), dtype=f32)) if with_dST else None
    return out


def varlen_lengths(N: int, max_len: int, chunk: int, seed: int = 0) -> np.ndarray:
    """Lengths of N packed documents, int64: a mix of an empty one, a single
    token, exact chunk multiples, one chunk plus one token and uniform draws
    in [1, max_len] (documents of mixed length, packed end to end)."""
    rng = np.random.Generator(np.random.PCG64([seed, 1 << 21]))
    fixed = [0, 1, chunk, chunk + 1, max_len]
    lens = list(rng.integers(1, max_len + 1, size=N))
    for i, n in enumerate(fixed[:N]):
        lens[i] = min(n, max_len)
    rng.shuffle(lens)
    return np.asarray(lens, dtype=np.int64)


def varlen_inputs(lens, H: int, dk: int, dv: int, *, dtype: str = "bf16", decay: str = "uniform",
                  seed: int = 0, S0_scale: float = 0.0, with_dST: bool = False) -> Dict[str, torch.Tensor]:
    """Inputs of one packed variable-length call: the seq_inputs recipe over
    T_total = sum(lens) tokens in [T_total, H, D] layout (dO included), plus
    cu_seqlens (int32 [N + 1]) and per-sequence S0 / dS_T ([N, H, dk, dv]
    fp32 or None)."""
    lens = np.asarray(lens, dtype=np.int64)
    N, total = len(lens), int(lens.sum())
    flat = seq_inputs(1, total, H, dk, dv, dtype=dtype, decay=decay, seed=seed, with_dO=True)
    out = {n: t[0] for n, t in flat.items() if t is not None}
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    out["cu_seqlens"] = torch.from_numpy(cu)
    rng = np.random.Generator(np.random.PCG64([seed, 1 << 22]))
    f32 = np.float32
    out["S0"] = torch.from_numpy(S0_scale * rng.standard_normal((N, H, dk, dv), dtype=f32)) if S0_scale else None
    out["dS_T"] = torch.from_numpy(rng.standard_normal((N, H, dk, dv), dtype=f32)) if with_dST else None
    return out


GATE_RANKS = (64, 64, 128, 128, 128)


def gate_inputs(M: int, d: int, H: int, dk: int, dv: int, *, dtype: str = "bf16", seed: int = 0,
                with_grads: bool = True) -> Dict[str, torch.Tensor]:
    """Inputs of one gate-prologue call (random weights stand in for trained
    ones): x [M, d] ~ N(0, 1); W_down ~ N(0, 1/d) so z ~ N(0, 1); each up
    matrix ~ N(0, 0.25 / rank); biases ~ N(0, 1) except the decay gate's,
    which put exp(log_a) at exp(-r) for log-uniform rates r in [1e-4, 3]
    per channel (slow and fast rows).  With grads: upstream gradients of the
    five gates ~ N(0, 1).  Returns CPU tensors in dtype; weights in a linear
    layer's [out, in] layout (W_down [512, d], up matrices [width, rank]);
    W_up and bias flat, packed in the gate order (log_a, erase, g, write,
    gamma)."""
    rng = np.random.Generator(np.random.PCG64([seed, 1 << 23]))
    f32 = np.float32
    widths = (H * dk, H * dk, H * dv, H * dv, H * dk)
    x = rng.standard_normal((M, d), dtype=f32)
    Wd = rng.standard_normal((sum(GATE_RANKS), d), dtype=f32) / np.sqrt(d)
    ups = [rng.standard_normal((w, r), dtype=f32) * (0.5 / np.sqrt(r)) for r, w in zip(GATE_RANKS, widths)]
    rates = np.exp(rng.uniform(np.log(1e-4), np.log(3.0), size=widths[0]))
    biases = [(-np.log(np.expm1(rates))).astype(f32)] + [rng.standard_normal(w, dtype=f32) for w in widths[1:]]
    out = {"x": _cast(x, dtype), "W_down": _cast(Wd.astype(f32), dtype),
           "W_up": _cast(np.concatenate([u.reshape(-1) for u in ups]), dtype),
           "bias": _cast(np.concatenate(biases), dtype)}
    if with_grads:
        for n, D in zip(("log_a", "erase", "g", "write", "gamma"), (dk, dk, dv, dv, dk)):
            out["d" + n] = _cast(rng.standard_normal((M, H, D), dtype=f32), dtype)
    return out


def step_rates(H: int, dk: int, seed: int = 0, mode: str = "channel") -> np.ndarray:
    """Per-(head, channel) decay rates for a decode stream, fixed over steps, [H, dk] fp32."""
    rng = np.random.Generator(np.random.PCG64([seed, 1 << 20]))
    return _decay_rates(rng, H, dk, mode)


def step_inputs(N: int, H: int, dk: int, dv: int, step: int, *, rates: np.ndarray,
                dtype: str = "bf16", seed: int = 0) -> Dict[str, torch.Tensor]:
    """Inputs of decode step ``step`` for N streams ([N, H, D] layout, CPU tensors).

    Each step has its own PCG64 stream keyed by (seed, step), so any subset
    of steps can be regenerated independently.  log_a = -rates for every step.
    """
    rng = np.random.Generator(np.random.PCG64([seed, step]))
    f32 = np.float32
    q = _silu_unit(rng.standard_normal((N, H, dk), dtype=f32))
    k = _silu_unit(rng.standard_normal((N, H, dk), dtype=f32))
    v = rng.standard_normal((N, H, dv), dtype=f32)
    log_a = np.broadcast_to(-rates[None, :, :], (N, H, dk)).astype(f32)
    erase = _sigmoid(rng.standard_normal((N, H, dk), dtype=f32))
    write = _sigmoid(rng.standard_normal((N, H, dv), dtype=f32))
    gamma = 2.0 * _sigmoid(rng.standard_normal((N, H, dk), dtype=f32))
    return {n: _cast(a, dtype) for n, a in
            (("q", q), ("k", k), ("v", v), ("log_a", log_a), ("erase", erase), ("write", write), ("gamma", gamma))}


def step_inputs_torch(N: int, H: int, dk: int, dv: int, steps: int, *, device, dtype: str = "bf16",
                      seed: int = 0) -> Dict[str, torch.Tensor]:
    """All `steps` decode inputs at once, drawn on `device` with a seeded torch
    generator (same distributions as `step_inputs`; values differ from the
    numpy stream).  Shapes [steps, N, H, D]; log_a is [N, H, dk], fixed over
    steps (per-channel rates exp(U[ln 1e-4, ln 3]))."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = _DT[dtype]

    def unit(x):
        s = torch.nn.functional.silu(x)
        return s / s.norm(dim=-1, keepdim=True).clamp_min(1e-12)

    shp_k, shp_v = (steps, N, H, dk), (steps, N, H, dv)
    out = {"q": unit(torch.randn(shp_k, generator=g, device=device)).to(dt),
           "k": unit(torch.randn(shp_k, generator=g, device=device)).to(dt),
           "v": torch.randn(shp_v, generator=g, device=device).to(dt)}
    rates = torch.exp(torch.empty((H, dk), device=device).uniform_(math.log(1e-4), math.log(3.0), generator=g))
    out["log_a"] = (-rates).expand(N, H, dk).contiguous().to(dt)
    out["erase"] = torch.sigmoid(torch.randn(shp_k, generator=g, device=device)).to(dt)
    out["write"] = torch.sigmoid(torch.randn(shp_v, generator=g, device=device)).to(dt)
    out["gamma"] = (2 * torch.sigmoid(torch.randn(shp_k, generator=g, device=device))).to(dt)
    return out


def stream_segment_torch(index: int, seg_len: int, H: int, dk: int, dv: int, *, device, dtype: str = "bf16",
                         decay: str = "channel_slow", seed: int = 0) -> Dict[str, torch.Tensor]:
    """Segment `index` (tokens index*seg_len .. +seg_len-1) of one long stream
    (B = 1), drawn on `device`: [1, seg_len, H, D] tensors with the seq_inputs
    distributions.  The per-(head, channel) decay rates belong to the stream
    (drawn once, on the host, from `seed` with the 'channel' or
    'channel_slow' recipe); the other tensors are drawn per segment with a
    torch generator seeded from (seed, index), so any segment can be
    regenerated on its own.  Values differ from the numpy streams."""
    rates = step_rates(H, dk, seed=seed, mode=decay)
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + 7 + index)
    dt = _DT[dtype]

    def unit(x):
        s = torch.nn.functional.silu(x)
        return s / s.norm(dim=-1, keepdim=True).clamp_min(1e-12)

    shp_k, shp_v = (1, seg_len, H, dk), (1, seg_len, H, dv)
    out = {"q": unit(torch.randn(shp_k, generator=g, device=device)).to(dt),
           "k": unit(torch.randn(shp_k, generator=g, device=device)).to(dt),
           "v": torch.randn(shp_v, generator=g, device=device).to(dt)}
    out["log_a"] = torch.from_numpy(-rates).to(device)[None, None].expand(shp_k).to(dt).contiguous()
    out["erase"] = torch.sigmoid(torch.randn(shp_k, generator=g, device=device)).to(dt)
    out["write"] = torch.sigmoid(torch.randn(shp_v, generator=g, device=device)).to(dt)
    out["gamma"] = (2 * torch.sigmoid(torch.randn(shp_k, generator=g, device=device))).to(dt)
    return out


@dataclass(frozen=True)
class Workload:
    """One workload: a name, its sizes and its input recipe."""
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    chunk: int
    dtype: str
    decay: str
    backward: bool = False
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 256, 2, 64, 64, 64, "f32", "uniform"),
    "layer_fwd_4k": Workload("layer_fwd_4k", 8, 4096, 16, 128, 128, 64, "bf16", "channel"),
    "layer_fwdbwd_4k": Workload("layer_fwdbwd_4k", 8, 4096, 16, 128, 128, 64, "bf16", "channel", backward=True),
    "long_32k_c128": Workload("long_32k_c128", 1, 32768, 16, 128, 128, 128, "bf16", "channel_slow", backward=True),
    "long_32k_c256": Workload("long_32k_c256", 1, 32768, 16, 128, 128, 256, "bf16", "channel_slow", backward=True),
    # one 1M-token stream: chunked prefill in 32K-token segments chained through
    # the state, then decode tokens (stream_segment_torch draws the segments)
    "stream_1m": Workload("stream_1m", 1, 1 << 20, 16, 128, 128, 64, "bf16", "channel_slow",
                          extra={"segment": 32768, "decode_steps": 64, "seed": 31}),
    "decode_64x16": Workload("decode_64x16", 64, 4096, 16, 128, 128, 1, "bf16", "channel",
                             extra={"steps": 4096}),
    # packed documents of mixed length at the layer's width: N = 16 documents
    # of up to 4,096 tokens (varlen_lengths), about 32K tokens in all; B = N,
    # T = the longest length
    "varlen_32k": Workload("varlen_32k", 16, 4096, 16, 128, 128, 64, "bf16", "channel", backward=True,
                           extra={"lengths_seed": 41, "seed": 43}),
}
