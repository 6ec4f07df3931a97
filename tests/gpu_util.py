"""Helpers of the GPU parity tests: device inputs, error metric, oracle calls.

Error metric: for an output tensor, max |gpu - oracle| / max |oracle|, over
the whole tensor and, separately, over each (batch, head) slice of it; a
test asserts the larger of the two, so a head whose values are small next
to the others' cannot hide its errors behind their scale.
"""
import numpy as np
import torch

import oracle


def _np64(x) -> np.ndarray:
    return np.asarray(x.detach().cpu().double().numpy() if hasattr(x, "detach") else x, dtype=np.float64)


def rel_err(x, y) -> float:
    """max |x - y| / max |y| over a whole tensor (inf-norm relative error)."""
    x, y = _np64(x), _np64(y)
    den = np.abs(y).max() if y.size else 0.0
    num = np.abs(x - y).max() if y.size else 0.0
    if den == 0:
        return float(num)
    return float(num / den)


def rel_err_heads(x, y, axes) -> float:
    """The worst over the slices that fix the indices on `axes` (the batch and
    head axes of a tensor) of max |x - y| / max |y| within the slice; a slice
    whose reference is all zero contributes max |x - y|."""
    x, y = _np64(x), _np64(y)
    assert x.shape == y.shape, (x.shape, y.shape)
    if y.size == 0:
        return 0.0
    rest = [a for a in range(y.ndim) if a not in axes]
    xs = np.transpose(x, list(axes) + rest).reshape(-1, int(np.prod([y.shape[a] for a in rest])))
    ys = np.transpose(y, list(axes) + rest).reshape(xs.shape)
    num = np.abs(xs - ys).max(axis=1)
    den = np.abs(ys).max(axis=1)
    r = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(r.max())


# batch and head axes of each kind of tensor
SEQ_AXES = (0, 2)      # [B, T, H, D]
STATE_AXES = (0, 1)    # [B, H, dk, dv]
STEP_AXES = (0, 1)     # [N, H, D]


def err2(x, y, axes) -> float:
    """max(whole-tensor error, worst per-(batch, head) error)."""
    return max(rel_err(x, y), rel_err_heads(x, y, axes))


def grad_axes(name: str):
    return STATE_AXES if name == "dS0" else SEQ_AXES


def untile_states(x):
    """Saved chunk states (S_chunks) to plain [..., dk, dv]: the library keeps
    each state as 16 x 16 tiles, element (r, j) at flat position
    ((r // 16) * (dv // 16) + j // 16) * 256 + (r % 16) * 16 + j % 16."""
    *lead, dk, dv = x.shape
    t = x.reshape(*lead, dk // 16, dv // 16, 16, 16)
    return t.transpose(-3, -2).reshape(*lead, dk, dv)


TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("q", "k", "v", "log_a", "erase", "write", "gamma")


def to_dev(inp, dev="cuda"):
    return {n: (None if t is None else t.to(dev).contiguous()) for n, t in inp.items()}


def oracle_fwd(inp):
    return oracle.fwd(*(inp[n] for n in NAMES), S0=inp.get("S0"))


def oracle_bwd(inp):
    return oracle.bwd(*(inp[n] for n in NAMES), inp["dO"], S0=inp.get("S0"), dS_T=inp.get("dS_T"))
