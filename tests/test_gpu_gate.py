"""GPU parity of the gate prologue (fused low-rank gate projection, q / k
SiLU + L2) against the fp64 oracle in oracle/gate_proj.py.

Metric as elsewhere: max |gpu - oracle| / max |oracle| per tensor, <= 1e-4
for fp32 and 2e-2 for bf16 inputs.  The bf16 path rounds z, the gates'
pre-activation gradients and dz to bf16 between its products (the oracle
keeps fp64 throughout); that rounding is inside the bf16 tolerance."""
import sys

import numpy as np
import pytest
import torch

import muir_inputs
from gpu_util import TOL, rel_err
from oracle import gate_proj as gp

pytestmark = pytest.mark.gpu

GATES = ("log_a", "erase", "g", "write", "gamma")


def _lib():
    import gated_delta_rule_muir_amd as m
    m.lib()
    return m


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    # name, M, d, H, dk, dv, dtype
    ("f32_M300_d256_H2_d64", 300, 256, 2, 64, 64, "f32"),
    ("bf16_M1000_d512_H4_d128", 1000, 512, 4, 128, 128, "bf16"),
    ("bf16_M129_d64_H1_dk64_dv128", 129, 64, 1, 64, 128, "bf16"),
    ("f32_M9000_d128_H1_d64_splits", 9000, 128, 1, 64, 64, "f32"),
    ("bf16_M9000_d256_H2_d128_splits", 9000, 256, 2, 128, 128, "bf16"),
    # key widths of 192 columns (a half group of 128 in the weight-gradient
    # kernel) with the tokens split 3 ways
    ("bf16_M9000_d128_H3_dk64_dv128_splits", 9000, 128, 3, 64, 128, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gate_proj_matches_oracle(case):
    name, M, d, H, dk, dv, dtype = case
    m = _lib()
    _say(f"gate case={name}")
    inp = muir_inputs.gate_inputs(M, d, H, dk, dv, dtype=dtype, seed=31)
    dev = {k: t.to("cuda") for k, t in inp.items()}
    args = (dev["x"], dev["W_down"], dev["W_up"], dev["bias"])
    out = m.muir_gate_proj_fwd(*args, H=H, dk=dk, dv=dv)
    dG = {n: dev["d" + n] for n in GATES}
    g1 = m.muir_gate_proj_bwd(*args, dG, H=H, dk=dk, dv=dv, z=out["z"])
    g2 = m.muir_gate_proj_bwd(*args, dG, H=H, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = gp.gate_fwd(inp["x"], inp["W_down"], inp["W_up"], inp["bias"], H, dk, dv)
    rg = gp.gate_bwd(inp["x"], inp["W_down"], inp["W_up"], inp["bias"], {n: inp["d" + n] for n in GATES}, H, dk, dv)
    errs = {n: rel_err(out[n], ref[n]) for n in ("z",) + GATES}
    errs.update({n: rel_err(g1[n], rg[n]) for n in ("dx", "dW_down", "dW_up", "dbias")})
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)
    # recomputing z inside gives the same gradients bit for bit
    for n in ("dx", "dW_down", "dW_up", "dbias"):
        assert torch.equal(g1[n], g2[n]), n
    assert bool(torch.all(out["log_a"] <= 0))


def test_gate_proj_gradients_are_deterministic():
    m = _lib()
    M, d, H, dk, dv = 5000, 256, 2, 64, 64
    inp = muir_inputs.gate_inputs(M, d, H, dk, dv, dtype="bf16", seed=32)
    dev = {k: t.to("cuda") for k, t in inp.items()}
    args = (dev["x"], dev["W_down"], dev["W_up"], dev["bias"])
    dG = {n: dev["d" + n] for n in GATES}
    a = m.muir_gate_proj_bwd(*args, dG, H=H, dk=dk, dv=dv)
    b = m.muir_gate_proj_bwd(*args, dG, H=H, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_gate_proj_without_tokens():
    m = _lib()
    H, dk, dv, d = 2, 64, 64, 128
    sw, su, sb = m.gate_param_shapes(d, H, dk, dv)
    x = torch.zeros((0, d), dtype=torch.bfloat16, device="cuda")
    W = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in (sw, su, sb)]
    out = m.muir_gate_proj_fwd(x, *W, H=H, dk=dk, dv=dv)
    assert out["log_a"].shape == (0, H, dk) and out["g"].shape == (0, H, dv)
    g = m.muir_gate_proj_bwd(x, *W, {n: out[n] for n in GATES}, H=H, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for n in ("dW_down", "dW_up", "dbias"):
        assert g[n].shape == W[("dW_down", "dW_up", "dbias").index(n)].shape
        assert int(torch.count_nonzero(g[n])) == 0, n


QK_CASES = [("f32", 64, 1000), ("f32", 128, 77), ("bf16", 64, 4097), ("bf16", 128, 3000)]


@pytest.mark.parametrize("dtype,D,rows", QK_CASES)
def test_qk_norm_matches_oracle(dtype, D, rows):
    m = _lib()
    _say(f"qk_norm dtype={dtype} D={D} rows={rows}")
    rng = np.random.Generator(np.random.PCG64(40 + D))
    u = muir_inputs._cast(rng.standard_normal((rows, D), dtype=np.float32) * 2, dtype)
    dy = muir_inputs._cast(rng.standard_normal((rows, D), dtype=np.float32), dtype)
    u[0] = 0  # an all-zero head stays finite (the 1e-6 guard)
    y = m.muir_qk_norm_fwd(u.cuda())
    du = m.muir_qk_norm_bwd(u.cuda(), dy.cuda())
    torch.cuda.synchronize()
    ey = rel_err(y, gp.qk_norm_fwd(u))
    ed = rel_err(du, gp.qk_norm_bwd(u, dy))
    _say(f"  y={ey:.2e} du={ed:.2e}")
    assert ey <= TOL[dtype] and ed <= TOL[dtype]
    assert bool(torch.all(torch.isfinite(y))) and bool(torch.all(y[0] == 0))
