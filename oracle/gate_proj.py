"""fp64 CPU oracle of the gate prologue that feeds the Muir operator.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP library and the library never imports it.

What it computes (arXiv 2611.08376; wolonglab summary page, §Methodology
and fig:arch (b), (c)): all five gates of a token come from ONE low-rank
projection -- a shared down-projection of the token's input x to
R_tot = 512 channels, split into five rank slices (r_f, r_b, r_g, r_w, r_q)
= (64, 64, 128, 128, 128), each slice up-projected to its gate's width with
a per-channel bias.  The q / k pathways end in SiLU and a per-head L2
normalisation (fig:arch (b): the linear-Conv-SiLU pathways; the operator
needs unit keys and queries).

Readings where the pages are silent (each one stated where it is used):
  * slice order = the order fig:arch lists the gates: decay f (log alpha),
    erase b, output gate g, write w, readout q (gamma), at column offsets
    0, 64, 128, 256, 384 of the down-projection;
  * widths: f, b, q have H*dk channels (key channels), g, w have H*dv;
  * no bias on the down-projection; the per-channel biases sit on the
    up-projections, so that each low-rank gate keeps an operating point of
    its own;
  * activations: log alpha = log sigmoid (a log-decay, <= 0); erase, write
    and the output gate are sigmoids; gamma = 2 sigmoid (a gain in (0, 2)
    around 1);
  * L2 normalisation of a head's vector u: u / sqrt(sum u^2 + 1e-6).

Parameter layout, that of a linear layer's weight ([out, in]): W_down
[512, d] (z = x W_down^T); W_up holds the five up matrices back to back,
each row-major [width_i, r_i] (pre_i = z_i U_i^T + c_i); bias holds the five
bias vectors back to back.  Every function here is plain numpy in float64;
reverse mode is the adjoint of each step, written out by hand.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np

GATES = ("log_a", "erase", "g", "write", "gamma")  # f, b, g, w, q
RANKS = (64, 64, 128, 128, 128)
R_TOT = 512
L2_EPS = 1e-6


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def widths(H: int, dk: int, dv: int) -> Tuple[int, ...]:
    """Output channels of each gate: key-channel gates H*dk, value-channel gates H*dv."""
    return (H * dk, H * dk, H * dv, H * dv, H * dk)


def slices(H: int, dk: int, dv: int) -> List[Dict[str, Tuple[int, int]]]:
    """Per gate: its column range of the down-projection output, its row
    range of the packed W_up (flattened offset and shape) and of the packed bias."""
    out, z0, w0, b0 = [], 0, 0, 0
    for r, wd in zip(RANKS, widths(H, dk, dv)):
        out.append({"z": (z0, z0 + r), "w": (w0, w0 + r * wd), "b": (b0, b0 + wd), "shape": (wd, r)})
        z0, w0, b0 = z0 + r, w0 + r * wd, b0 + wd
    return out


def up_numel(H: int, dk: int, dv: int) -> Tuple[int, int]:
    """(elements of the packed W_up, elements of the packed bias)."""
    s = slices(H, dk, dv)
    return s[-1]["w"][1], s[-1]["b"][1]


def _sigmoid(x):
    # split by sign so exp never overflows
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def _log_sigmoid(x):
    # log sigmoid(x) = -log(1 + e^-x) = min(x, 0) - log1p(e^-|x|)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def _act(name: str, pre):
    if name == "log_a":
        return _log_sigmoid(pre)
    s = _sigmoid(pre)
    return 2.0 * s if name == "gamma" else s


def _act_grad(name: str, pre):
    """d act / d pre."""
    s = _sigmoid(pre)
    if name == "log_a":
        return 1.0 - s  # d/dx log sigmoid(x) = sigmoid(-x)
    d = s * (1.0 - s)
    return 2.0 * d if name == "gamma" else d


def gate_fwd(x, W_down, W_up, bias, H: int, dk: int, dv: int) -> Dict[str, np.ndarray]:
    """Gates of every token of x [M, d].  Returns {"z": [M, 512],
    "log_a", "erase", "write", "gamma": [M, H, dk or dv], "g": [M, H, dv]}."""
    x, W_down, W_up, bias = (_f64(a) for a in (x, W_down, W_up, bias))
    M = x.shape[0]
    z = x @ W_down.T  # the shared down-projection
    out = {"z": z}
    for name, sl, D in zip(GATES, slices(H, dk, dv), (dk, dk, dv, dv, dk)):
        U = W_up[sl["w"][0]:sl["w"][1]].reshape(sl["shape"])
        c = bias[sl["b"][0]:sl["b"][1]]
        pre = z[:, sl["z"][0]:sl["z"][1]] @ U.T + c  # this gate's rank slice, up-projected, plus channel bias
        out[name] = _act(name, pre).reshape(M, H, D)
    return out


def gate_bwd(x, W_down, W_up, bias, d_gates: Dict[str, object], H: int, dk: int, dv: int
             ) -> Dict[str, np.ndarray]:
    """Reverse mode of gate_fwd: from the gradients of the five gates
    (d_gates[name], shaped like the gate) to dx [M, d], dW_down [512, d],
    dW_up and dbias (packed like W_up and bias)."""
    x, W_down, W_up, bias = (_f64(a) for a in (x, W_down, W_up, bias))
    M = x.shape[0]
    z = x @ W_down.T
    dz = np.zeros_like(z)
    dW_up = np.zeros_like(W_up)
    dbias = np.zeros_like(bias)
    for name, sl in zip(GATES, slices(H, dk, dv)):
        U = W_up[sl["w"][0]:sl["w"][1]].reshape(sl["shape"])
        c = bias[sl["b"][0]:sl["b"][1]]
        zi = z[:, sl["z"][0]:sl["z"][1]]
        pre = zi @ U.T + c
        dpre = _f64(d_gates[name]).reshape(M, -1) * _act_grad(name, pre)
        dbias[sl["b"][0]:sl["b"][1]] = dpre.sum(axis=0)
        dW_up[sl["w"][0]:sl["w"][1]] = (dpre.T @ zi).reshape(-1)
        dz[:, sl["z"][0]:sl["z"][1]] = dpre @ U
    return {"dx": dz @ W_down, "dW_down": dz.T @ x, "dW_up": dW_up, "dbias": dbias}


def qk_norm_fwd(u) -> np.ndarray:
    """SiLU, then L2 normalisation over the last axis (one head's channels)."""
    u = _f64(u)
    s = u * _sigmoid(u)
    return s / np.sqrt((s * s).sum(axis=-1, keepdims=True) + L2_EPS)


def qk_norm_bwd(u, dy) -> np.ndarray:
    """Reverse mode of qk_norm_fwd."""
    u, dy = _f64(u), _f64(dy)
    sg = _sigmoid(u)
    s = u * sg
    n = np.sqrt((s * s).sum(axis=-1, keepdims=True) + L2_EPS)
    y = s / n
    ds = (dy - y * (y * dy).sum(axis=-1, keepdims=True)) / n  # through s / |s|
    return ds * (sg * (1.0 + u * (1.0 - sg)))  # through silu
