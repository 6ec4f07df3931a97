"""Helpers of the GPU parity tests: device inputs, error metric, oracle calls."""
import numpy as np
import torch

import oracle


def rel_err(x, y) -> float:
    """max |x - y| / max |y| over a whole tensor (inf-norm relative error)."""
    x = np.asarray(x.detach().cpu().double().numpy() if hasattr(x, "detach") else x, dtype=np.float64)
    y = np.asarray(y.detach().cpu().double().numpy() if hasattr(y, "detach") else y, dtype=np.float64)
    den = np.abs(y).max()
    num = np.abs(x - y).max()
    if den == 0:
        return float(num)
    return float(num / den)


TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("q", "k", "v", "log_a", "erase", "write", "gamma")


def to_dev(inp, dev="cuda"):
    return {n: (None if t is None else t.to(dev).contiguous()) for n, t in inp.items()}


def oracle_fwd(inp):
    return oracle.fwd(*(inp[n] for n in NAMES), S0=inp.get("S0"))


def oracle_bwd(inp):
    return oracle.bwd(*(inp[n] for n in NAMES), inp["dO"], S0=inp.get("S0"), dS_T=inp.get("dS_T"))
