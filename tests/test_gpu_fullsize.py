"""Parity at the workloads' full sizes, in the launch configuration bench.py
times, on outputs the oracle can compute one (batch, head) at a time.

  layer 4K  : B=8, T=4096, H=16, d=128, chunk 64, bf16   (forward and backward)
  long 32K  : B=1, T=32768, H=16, d=128, chunk 128 / 256  (forward and backward)
  decode    : 64 streams x 16 heads x d=128, 4096 steps  (every step's output);
              512 streams x 16 heads, 16 steps (a state beyond the Infinity Cache)

Tolerance: max |gpu - oracle| / max |oracle| per tensor on the sampled slice <= 2e-2.
"""
import sys

import numpy as np
import pytest
import torch

import muir_inputs
import oracle
from gpu_util import NAMES, rel_err

pytestmark = pytest.mark.gpu
TOL = 2e-2
GRADS = ("dq", "dk", "dv", "dlog_a", "derase", "dwrite", "dgamma")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _lib():
    import gated_delta_rule_muir_amd as m
    m.lib()
    return m


def _check_heads(name, inp, o, S_T, g, heads, with_bwd=True):
    for (b, h) in heads:
        sl = {n: inp[n][b:b + 1, :, h:h + 1] for n in NAMES}
        dO = inp["dO"][b:b + 1, :, h:h + 1]
        o_ref, S_ref = oracle.fwd(*(sl[n] for n in NAMES))
        errs = {"o": rel_err(o[b:b + 1, :, h:h + 1], o_ref), "S_T": rel_err(S_T[b:b + 1, h:h + 1], S_ref)}
        if with_bwd:
            gr = oracle.bwd(*(sl[n] for n in NAMES), dO)
            for n in GRADS:
                errs[n] = rel_err(g[n][b:b + 1, :, h:h + 1], gr[n])
            errs["dS0"] = rel_err(g["dS0"][b:b + 1, h:h + 1], gr["dS0"])
        _say(f"  {name} b={b} h={h}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for k_, v_ in errs.items():
            assert v_ <= TOL, (name, b, h, k_, v_)


def _run(m, inp, C):
    dv = {n: (t.to("cuda") if t is not None else None) for n, t in inp.items()}
    # as bench.py runs the step: the backward reuses the forward's chunk states and summaries
    B, T, H, d = dv["q"].shape
    ws = torch.empty(m.muir_chunk_fwd_workspace(B, T, H, d, d, C), dtype=torch.uint8, device="cuda")
    o, S_T, Sc = m.muir_chunk_fwd(*(dv[n] for n in NAMES), chunk=C, save_states=True, workspace=ws)
    g = m.muir_chunk_bwd(*(dv[n] for n in NAMES), dv["dO"], S_chunks=Sc, summaries=ws, chunk=C)
    torch.cuda.synchronize()
    out = (o.cpu(), S_T.cpu(), {n: t.cpu() for n, t in g.items()})
    del dv, o, S_T, Sc, g, ws
    torch.cuda.empty_cache()
    return out


def test_layer_4k_fwd_bwd_sampled_heads():
    m = _lib()
    w = muir_inputs.WORKLOADS["layer_fwdbwd_4k"]
    _say(f"layer_4k: generating B={w.B} T={w.T} H={w.H} d={w.dk}")
    inp = muir_inputs.seq_inputs(w.B, w.T, w.H, w.dk, w.dv, dtype=w.dtype, decay=w.decay, seed=0, with_dO=True)
    o, S_T, g = _run(m, inp, w.chunk)
    _check_heads("layer_4k", inp, o, S_T, g, [(0, 0), (3, 7), (7, 15)])


@pytest.mark.parametrize("name", ["long_32k_c128", "long_32k_c256"])
def test_long_32k_fwd_bwd_sampled_heads(name):
    m = _lib()
    w = muir_inputs.WORKLOADS[name]
    _say(f"{name}: generating B={w.B} T={w.T} H={w.H} d={w.dk} C={w.chunk}")
    inp = muir_inputs.seq_inputs(w.B, w.T, w.H, w.dk, w.dv, dtype=w.dtype, decay=w.decay, seed=0, with_dO=True)
    o, S_T, g = _run(m, inp, w.chunk)
    _check_heads(name, inp, o, S_T, g, [(0, 0), (0, 11)])


def test_decode_4096_steps_sampled_streams():
    """64 streams x 16 heads for 4096 steps; streams 0 and 63 are replayed by the
    oracle (a decode stream is the recurrence over its steps) and compared at
    every step and on the final state."""
    m = _lib()
    N, H, d, steps = 64, 16, 128, 4096
    _say("decode: generating inputs on the device")
    inp = muir_inputs.step_inputs_torch(N, H, d, d, steps, device="cuda", seed=5)
    S = torch.zeros((N, H, d, d), dtype=torch.float32, device="cuda")
    picks = [0, N - 1]
    outs = torch.empty((steps, len(picks), H, d), dtype=torch.bfloat16, device="cuda")
    for t in range(steps):
        o = m.muir_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_a"], inp["erase"][t],
                        inp["write"][t], inp["gamma"][t], S)
        outs[t] = o[picks]
    torch.cuda.synchronize()
    _say("decode: oracle on the sampled streams")
    seq = {n: inp[n][:, picks].transpose(0, 1).cpu() for n in ("q", "k", "v", "erase", "write", "gamma")}
    seq["log_a"] = inp["log_a"][picks].unsqueeze(1).expand(len(picks), steps, H, d).cpu()
    o_ref, S_ref = oracle.fwd(*(seq[n] for n in NAMES))
    e_o = rel_err(outs.transpose(0, 1).cpu(), o_ref)
    e_s = rel_err(S[picks].cpu(), S_ref)
    _say(f"  decode o={e_o:.2e} S={e_s:.2e}")
    assert e_o <= TOL and e_s <= TOL


def test_decode_state_beyond_infinity_cache():
    """512 streams x 16 heads (a 512 MiB state, which the step streams with
    non-temporal loads and stores), 16 steps; streams 0 and 511 replayed by
    the oracle at every step and on the final state."""
    m = _lib()
    N, H, d, steps = 512, 16, 128, 16
    _say("decode 512 MiB state: generating inputs on the device")
    inp = muir_inputs.step_inputs_torch(N, H, d, d, steps, device="cuda", seed=6)
    S = torch.zeros((N, H, d, d), dtype=torch.float32, device="cuda")
    picks = [0, N - 1]
    outs = torch.empty((steps, len(picks), H, d), dtype=torch.bfloat16, device="cuda")
    for t in range(steps):
        o = m.muir_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_a"], inp["erase"][t],
                        inp["write"][t], inp["gamma"][t], S)
        outs[t] = o[picks]
    torch.cuda.synchronize()
    seq = {n: inp[n][:, picks].transpose(0, 1).cpu() for n in ("q", "k", "v", "erase", "write", "gamma")}
    seq["log_a"] = inp["log_a"][picks].unsqueeze(1).expand(len(picks), steps, H, d).cpu()
    o_ref, S_ref = oracle.fwd(*(seq[n] for n in NAMES))
    e_o = rel_err(outs.transpose(0, 1).cpu(), o_ref)
    e_s = rel_err(S[picks].cpu(), S_ref)
    _say(f"  decode 512 MiB o={e_o:.2e} S={e_s:.2e}")
    assert e_o <= TOL and e_s <= TOL
    del S


def test_gate_prologue_full_layer():
    """Gate prologue at the layer's shape (M = 8 x 4096 tokens, d = 2048,
    H = 16, dk = dv = 128, bf16), as bench.py runs it.  Every token's gates
    and dx depend on that token alone: sampled tokens against the oracle run
    on those tokens.  The weight gradients are sums over tokens: the full
    call equals the sum of the calls on four quarters of the tokens (to fp32
    summation order), and the first quarter's match the oracle's."""
    m = _lib()
    M, d, H, dk, dv = 8 * 4096, 2048, 16, 128, 128
    _say(f"gate prologue full layer M={M} d={d}")
    inp = muir_inputs.gate_inputs(M, d, H, dk, dv, dtype="bf16", seed=41)
    dev = {k: t.to("cuda") for k, t in inp.items()}
    names = m.GATE_NAMES
    args = (dev["W_down"], dev["W_up"], dev["bias"])
    out = m.muir_gate_proj_fwd(dev["x"], *args, H=H, dk=dk, dv=dv)
    g = m.muir_gate_proj_bwd(dev["x"], *args, {n: dev["d" + n] for n in names}, H=H, dk=dk, dv=dv, z=out["z"])
    q4 = M // 4
    parts = [m.muir_gate_proj_bwd(dev["x"][i * q4:(i + 1) * q4], *args,
                                  {n: dev["d" + n][i * q4:(i + 1) * q4] for n in names}, H=H, dk=dk, dv=dv)
             for i in range(4)]
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(M, 48, replace=False))
    rows[0], rows[-1] = 0, M - 1
    sub = {k: inp[k][rows] for k in ["x"] + ["d" + n for n in names]}
    ref = gp_fwd(sub["x"], inp, H, dk, dv)
    rg = gp_bwd(sub["x"], inp, {n: sub["d" + n] for n in names}, H, dk, dv)
    errs = {n: rel_err(out[n][rows], ref[n]) for n in names}
    errs["dx"] = rel_err(g["dx"][rows], rg["dx"])
    for n in ("dW_down", "dW_up", "dbias"):
        errs[n + "_additive"] = rel_err(g[n], sum(p[n] for p in parts))
    q = {k: inp[k][:q4] for k in ["x"] + ["d" + n for n in names]}
    r0 = gp_bwd(q["x"], inp, {n: q["d" + n] for n in names}, H, dk, dv)
    for n in ("dW_down", "dW_up", "dbias"):
        errs[n + "_q0"] = rel_err(parts[0][n], r0[n])
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= (1e-5 if n.endswith("_additive") else TOL), (n, e)


def gp_fwd(x, inp, H, dk, dv):
    from oracle import gate_proj
    return gate_proj.gate_fwd(x, inp["W_down"], inp["W_up"], inp["bias"], H, dk, dv)


def gp_bwd(x, inp, dG, H, dk, dv):
    from oracle import gate_proj
    return gate_proj.gate_bwd(x, inp["W_down"], inp["W_up"], inp["bias"], dG, H, dk, dv)
