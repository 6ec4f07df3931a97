"""fp64 sequential CPU oracle for the Muir gated delta-rule operator.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares
no code with the HIP library (``gated_delta_rule_muir_amd``) and the library
never imports it; the two meet only through the seeded input generators in
``muir_inputs``.

The arithmetic lives in ``muir_oracle.c`` (plain C, fp64, one token at a
time; OpenMP only over independent (batch, head) streams).  This module
compiles it with gcc, loads it with ctypes and converts numpy arrays.

Source of the recurrence: arXiv 2611.08376 ("Muir: Linear Attention with
Sensitivity-Allocated Gating and Matched-Filter Readout"), abstract and the
Methodology section of the wolonglab summary page (row-wise decay, erase of
the key's prediction, gated write, readout gate on the normalised query).
The exact placement of each gate is a reading of that prose; it is written
out in ``muir_oracle.c`` and pinned by ``tests/test_oracle_pins.py``.

``oracle.gate_proj`` is the fp64 numpy oracle of the gate prologue (the fused
low-rank gate projection and the q / k SiLU + L2 normalisation), pinned by
``tests/test_oracle_gate_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "muir_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``muir_oracle.c`` into ``liboracle.so`` with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-fPIC", "-shared", "-fopenmp", "-std=c99",
               "-Wall", "-Wno-unused-variable", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_fwd.argtypes = [I, I, I, I, I] + [P] * 7 + [P, P, P, I]
        lib.oracle_fwd.restype = I
        lib.oracle_step.argtypes = [I, I, I, I] + [P] * 7 + [P, P, I]
        lib.oracle_step.restype = I
        lib.oracle_bwd.argtypes = [I, I, I, I, I] + [P] * 7 + [P, P, P] + [P] * 8 + [I]
        lib.oracle_bwd.restype = I
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Contiguous fp64 copy of a numpy array or torch tensor (values unchanged)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{name} failed with code {rc}")


def fwd(q, k, v, log_a, erase, write, gamma, S0=None, nthreads: int = 0):
    """Sequential recurrence over [B, T, H, D] inputs.  Returns (o, S_T) in fp64."""
    q, k, v, log_a, erase, write, gamma = (_f64(x) for x in (q, k, v, log_a, erase, write, gamma))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    S0 = None if S0 is None else _f64(S0)
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    rc = _load().oracle_fwd(B, T, H, dk, dv, *(_ptr(a) for a in (q, k, v, log_a, erase, write, gamma)),
                            _ptr(S0), _ptr(o), _ptr(S_T), int(nthreads))
    _check(rc, "oracle_fwd")
    return o, S_T


def step(q, k, v, log_a, erase, write, gamma, S, nthreads: int = 0):
    """One decode step for [N, H, D] inputs; returns (o [N,H,dv], S_new [N,H,dk,dv])."""
    q, k, v, log_a, erase, write, gamma = (_f64(x) for x in (q, k, v, log_a, erase, write, gamma))
    N, H, dk = q.shape
    dv = v.shape[2]
    S = _f64(S).copy()
    o = np.zeros((N, H, dv))
    rc = _load().oracle_step(N, H, dk, dv, *(_ptr(a) for a in (q, k, v, log_a, erase, write, gamma)),
                             _ptr(S), _ptr(o), int(nthreads))
    _check(rc, "oracle_step")
    return o, S


def bwd(q, k, v, log_a, erase, write, gamma, dO, S0=None, dS_T=None, nthreads: int = 0):
    """Reverse mode of the recurrence.

    Returns a dict with dq, dk, dv, dlog_a, derase, dwrite, dgamma, dS0 (fp64).
    """
    q, k, v, log_a, erase, write, gamma, dO = (_f64(x) for x in (q, k, v, log_a, erase, write, gamma, dO))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    S0 = None if S0 is None else _f64(S0)
    dS_T = None if dS_T is None else _f64(dS_T)
    out = {n: np.zeros((B, T, H, dk)) for n in ("dq", "dk", "dlog_a", "derase", "dgamma")}
    out.update({n: np.zeros((B, T, H, dv)) for n in ("dv", "dwrite")})
    out["dS0"] = np.zeros((B, H, dk, dv))
    rc = _load().oracle_bwd(B, T, H, dk, dv, *(_ptr(a) for a in (q, k, v, log_a, erase, write, gamma)),
                            _ptr(S0), _ptr(dO), _ptr(dS_T),
                            *(_ptr(out[n]) for n in ("dq", "dk", "dv", "dlog_a", "derase", "dwrite", "dgamma", "dS0")),
                            int(nthreads))
    _check(rc, "oracle_bwd")
    return out
