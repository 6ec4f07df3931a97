"""GPU parity of the chunkwise backward against the fp64 oracle's reverse mode.

Every gradient tensor is compared with max |gpu - oracle| / max |oracle|,
over the whole tensor and over each (batch, head) slice, against 1e-4 (fp32
inputs) or 2e-2 (bf16 inputs).  The per-token gradients are fp32 unless a
case asks for bf16 gradients (bf16 inputs only; then rounded once from the
same fp32 values, which one test checks bit for bit).
"""
import sys

import numpy as np
import pytest
import torch

import muir_inputs
import oracle
from gpu_util import NAMES, SEQ_AXES, STATE_AXES, TOL, err2, grad_axes, oracle_bwd, rel_err, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dlog_a", "derase", "dwrite", "dgamma", "dS0")


def _lib():
    import gated_delta_rule_muir_amd as m
    m.lib()
    return m


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    # name, B, T, H, d, C, dtype, decay, S0 scale, dS_T
    ("tiny_f32_c64", 1, 256, 2, 64, 64, "f32", "uniform", 0.0, False),
    ("f32_d64_c64_S0_dST", 1, 128, 2, 64, 64, "f32", "uniform", 0.1, True),
    ("f32_d128_c64", 1, 128, 1, 128, 64, "f32", "channel", 0.1, True),
    ("bf16_d128_c64", 2, 256, 2, 128, 64, "bf16", "channel", 0.0, False),
    ("bf16_d128_c128_S0", 1, 256, 2, 128, 128, "bf16", "channel_slow", 0.1, True),
    ("bf16_d128_c256", 1, 512, 2, 128, 256, "bf16", "channel_slow", 0.0, False),
    ("bf16_d64_c64_uniform", 1, 192, 3, 64, 64, "bf16", "uniform", 0.1, True),
    ("f32_d64_c64_steep", 1, 128, 2, 64, 64, "f32", "steep", 0.1, True),
    ("bf16_d128_c128_steep", 1, 256, 2, 128, 128, "bf16", "steep", 0.0, False),
    ("f32_d128_c64_spiky", 1, 128, 2, 128, 64, "f32", "spiky", 0.1, True),
    ("bf16_d128_c64_spiky", 1, 256, 2, 128, 64, "bf16", "spiky", 0.0, True),
    # every (dtype, d, chunk) kernel instance over several chunks
    ("f32_d128_c128", 1, 384, 2, 128, 128, "f32", "channel_slow", 0.1, True),
    ("f32_d64_c128", 1, 384, 2, 64, 128, "f32", "uniform", 0.1, True),
    ("f32_d128_c256", 1, 768, 1, 128, 256, "f32", "channel_slow", 0.1, True),
    ("f32_d64_c256", 1, 768, 2, 64, 256, "f32", "channel", 0.1, True),
    ("bf16_d64_c128", 2, 384, 2, 64, 128, "bf16", "channel", 0.1, True),
    ("bf16_d64_c256", 1, 768, 3, 64, 256, "bf16", "channel_slow", 0.1, True),
]


def _check_grads(g, ref, dtype, gdt=torch.float32):
    errs = {n: err2(g[n], ref[n], grad_axes(n)) for n in GRADS}
    _say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n in GRADS:
        want = torch.float32 if n == "dS0" else gdt
        assert g[n].dtype == want, (n, g[n].dtype)
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_chunk_bwd_matches_oracle(case):
    name, B, T, H, d, C, dtype, decay, s0, dst = case
    m = _lib()
    _say(f"chunk_bwd case={name}")
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype=dtype, decay=decay, seed=7, S0_scale=s0,
                                 with_dO=True, with_dST=dst)
    dv = to_dev(inp)
    g = m.muir_chunk_bwd(*(dv[n] for n in NAMES), dv["dO"], S0=dv["S0"], dS_T=dv["dS_T"], chunk=C)
    torch.cuda.synchronize()
    _check_grads(g, oracle_bwd(inp), dtype)


BF16_GRAD_CASES = [
    # name, B, T, H, d, C, decay, S0 scale, dS_T   (bf16 inputs; the direct and two-sweep forms)
    ("d128_c64", 2, 256, 2, 128, 64, "channel", 0.1, True),
    ("d64_c64_steep", 1, 192, 3, 64, 64, "steep", 0.0, False),
    ("d128_c128", 1, 384, 2, 128, 128, "channel_slow", 0.1, True),
    ("d128_c256", 1, 512, 2, 128, 256, "spiky", 0.1, True),
]


@pytest.mark.parametrize("case", BF16_GRAD_CASES, ids=[c[0] for c in BF16_GRAD_CASES])
def test_bf16_gradients(case):
    """bf16 gradients (opt-in for bf16 inputs) against the oracle, and equal
    bit for bit to the fp32 gradients of the same call rounded once to bf16
    (both forms accumulate the same fp32 values; only the store differs)."""
    name, B, T, H, d, C, decay, s0, dst = case
    m = _lib()
    _say(f"bf16 gradients case={name}")
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype="bf16", decay=decay, seed=17, S0_scale=s0,
                                 with_dO=True, with_dST=dst)
    dv = to_dev(inp)
    args = [dv[n] for n in NAMES]
    ws = torch.empty(m.muir_chunk_fwd_workspace(B, T, H, d, d, C), dtype=torch.uint8, device="cuda")
    _, _, Sc = m.muir_chunk_fwd(*args, dv["S0"], chunk=C, save_states=True, workspace=ws)
    kw = dict(S0=dv["S0"], S_chunks=Sc, summaries=ws, dS_T=dv["dS_T"], chunk=C)
    gb = m.muir_chunk_bwd(*args, dv["dO"], grad_dtype=torch.bfloat16, **kw)
    gf = m.muir_chunk_bwd(*args, dv["dO"], **kw)
    torch.cuda.synchronize()
    _check_grads(gb, oracle_bwd(inp), "bf16", torch.bfloat16)
    for n in GRADS:
        if n == "dS0":
            assert torch.equal(gb[n], gf[n])
        else:
            assert gf[n].dtype == torch.float32
            assert torch.equal(gb[n], gf[n].to(torch.bfloat16)), n


def test_bf16_gradients_refused_for_fp32_inputs():
    m = _lib()
    inp = to_dev(muir_inputs.seq_inputs(1, 64, 1, 64, 64, dtype="f32", seed=1, with_dO=True))
    with pytest.raises(TypeError):
        m.muir_chunk_bwd(*(inp[n] for n in NAMES), inp["dO"], chunk=64, grad_dtype=torch.bfloat16)


def test_bwd_with_saved_states_equals_recompute():
    """Passing the forward's chunk-start states gives the same gradients as
    letting the backward recompute them."""
    m = _lib()
    B, T, H, d, C = 1, 256, 2, 128, 64
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype="bf16", decay="channel", seed=8, S0_scale=0.1,
                                 with_dO=True)
    dv = to_dev(inp)
    _, _, Sc = m.muir_chunk_fwd(*(dv[n] for n in NAMES), dv["S0"], chunk=C, save_states=True)
    g1 = m.muir_chunk_bwd(*(dv[n] for n in NAMES), dv["dO"], S0=dv["S0"], S_chunks=Sc, chunk=C)
    g2 = m.muir_chunk_bwd(*(dv[n] for n in NAMES), dv["dO"], S0=dv["S0"], chunk=C)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("C", [64, 128, 256])
def test_bwd_with_saved_summaries_equals_recompute(C):
    """Passing the forward's workspace (its chunk summaries, with the chunk
    deltas a bf16 forward keeps when it saves its chunk states) gives the same
    gradients as letting the backward recompute them, with and without the
    saved chunk states."""
    m = _lib()
    B, T, H, d = 2, 512, 2, 128
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype="bf16", decay="channel", seed=9, S0_scale=0.1,
                                 with_dO=True, with_dST=True)
    dv = to_dev(inp)
    ws = torch.empty(m.muir_chunk_fwd_workspace(B, T, H, d, d, C), dtype=torch.uint8, device="cuda")
    _, _, Sc = m.muir_chunk_fwd(*(dv[n] for n in NAMES), dv["S0"], chunk=C, save_states=True, workspace=ws)
    ref = m.muir_chunk_bwd(*(dv[n] for n in NAMES), dv["dO"], S0=dv["S0"], dS_T=dv["dS_T"], chunk=C)
    g1 = m.muir_chunk_bwd(*(dv[n] for n in NAMES), dv["dO"], S0=dv["S0"], S_chunks=Sc, dS_T=dv["dS_T"],
                          summaries=ws, chunk=C)
    g2 = m.muir_chunk_bwd(*(dv[n] for n in NAMES), dv["dO"], S0=dv["S0"], dS_T=dv["dS_T"], summaries=ws,
                          chunk=C)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(g1[n], ref[n]), n
        assert torch.equal(g2[n], ref[n]), n


@pytest.mark.parametrize("dtype,d", [("f32", 128), ("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_split_scan_matches_oracle(dtype, d):
    """One head over 64 chunks: the state scans split into 8 segments (each
    segment's transition, the segment recurrence, then each segment's scan
    from its start), forward and backward, against the oracle.  The reverse
    scan takes the forward's segment transitions, transposed: from the
    forward's workspace, from the forward scan it reruns, or (fp32, chunk
    states given without summaries) formed on their own; every way gives the
    same gradients, bit for bit."""
    m = _lib()
    B, T, H, C = 1, 4096, 1, 64
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype=dtype, decay="channel", seed=12, S0_scale=0.1,
                                 with_dO=True, with_dST=True)
    dv = to_dev(inp)
    code = m.MUIR_F32 if dtype == "f32" else m.MUIR_BF16
    ws = torch.empty(m.muir_chunk_fwd_workspace(B, T, H, d, d, C, code), dtype=torch.uint8, device="cuda")
    o, S_T, Sc = m.muir_chunk_fwd(*(dv[n] for n in NAMES), dv["S0"], chunk=C, save_states=True, workspace=ws)
    bargs = (*(dv[n] for n in NAMES), dv["dO"])
    g = m.muir_chunk_bwd(*bargs, S0=dv["S0"], S_chunks=Sc, summaries=ws, dS_T=dv["dS_T"], chunk=C)
    others = [m.muir_chunk_bwd(*bargs, S0=dv["S0"], S_chunks=Sc, dS_T=dv["dS_T"], chunk=C),
              m.muir_chunk_bwd(*bargs, S0=dv["S0"], dS_T=dv["dS_T"], chunk=C)]
    torch.cuda.synchronize()
    for g2 in others:
        for n in GRADS:
            assert torch.equal(g[n], g2[n]), n
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    ref = oracle.bwd(*(inp[n] for n in NAMES), inp["dO"], S0=inp["S0"], dS_T=inp["dS_T"])
    errs = {"o": err2(o, o_ref, SEQ_AXES), "S_T": err2(S_T, S_ref, STATE_AXES)}
    errs.update({n: err2(g[n], ref[n], grad_axes(n)) for n in GRADS})
    _say(f"split scan {dtype} d={d}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)


GATE_CASES = [
    # name, B, T, H, d, C, dtype, decay, gate form
    ("bf16_d128_c64_static", 2, 256, 2, 128, 64, "bf16", "channel", "static"),
    ("bf16_d128_c64_none", 2, 256, 2, 128, 64, "bf16", "channel", "none"),
    ("bf16_d128_c128_static", 1, 256, 2, 128, 128, "bf16", "channel_slow", "static"),
    ("f32_d64_c64_static", 1, 128, 2, 64, 64, "f32", "uniform", "static"),
    ("f32_d64_c64_none", 1, 128, 2, 64, 64, "f32", "steep", "none"),
]


@pytest.mark.parametrize("case", GATE_CASES, ids=[c[0] for c in GATE_CASES])
def test_readout_gate_forms(case):
    """Static readout gate ([H, dk], one per head and key channel) and no gate
    (gamma = 1): forward and backward against the oracle run with the gate
    expanded to every token; a static gate's gradient is the oracle's
    per-token gradient summed over batch and tokens (wolonglab summary,
    tab:abl: dynamic vs static vs no readout)."""
    name, B, T, H, d, C, dtype, decay, form = case
    m = _lib()
    _say(f"gate case={name}")
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype=dtype, decay=decay, seed=13, S0_scale=0.1,
                                 with_dO=True, with_dST=True)
    tok = dict(inp)
    if form == "static":
        g_dev_src = inp["gamma"][0, 0].clone()  # one token's gate as the static [H, dk] gate
        tok["gamma"] = g_dev_src[None, None].expand(B, T, H, d).contiguous()
    else:
        g_dev_src = None
        tok["gamma"] = torch.ones_like(inp["gamma"])
    dv = to_dev(inp)
    gam = None if g_dev_src is None else g_dev_src.to("cuda")
    args = [dv["q"], dv["k"], dv["v"], dv["log_a"], dv["erase"], dv["write"], gam]
    o, S_T, Sc = m.muir_chunk_fwd(*args, dv["S0"], chunk=C, save_states=True)
    g = m.muir_chunk_bwd(*args, dv["dO"], S0=dv["S0"], S_chunks=Sc, dS_T=dv["dS_T"], chunk=C)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.fwd(*(tok[n] for n in NAMES), S0=tok["S0"])
    ref = oracle.bwd(*(tok[n] for n in NAMES), tok["dO"], S0=tok["S0"], dS_T=tok["dS_T"])
    errs = {"o": err2(o, o_ref, SEQ_AXES), "S_T": err2(S_T, S_ref, STATE_AXES)}
    errs.update({n: err2(g[n], ref[n], grad_axes(n)) for n in GRADS if n != "dgamma"})
    if form == "static":
        assert tuple(g["dgamma"].shape) == (H, d) and g["dgamma"].dtype == torch.float32
        errs["dgamma"] = err2(g["dgamma"], ref["dgamma"].sum(axis=(0, 1)), (0,))
    else:
        assert g["dgamma"] is None
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)


@pytest.mark.parametrize("form", ["static", "none"])
def test_step_readout_gate_forms(form):
    """Decode steps with a static gate and without a gate, against the oracle's step."""
    m = _lib()
    N, H, dk, steps = 3, 2, 128, 5
    rates = muir_inputs.step_rates(H, dk, seed=3)
    S_gpu = torch.zeros((N, H, dk, dk), dtype=torch.float32, device="cuda")
    S_ref = np.zeros((N, H, dk, dk))
    for s in range(steps):
        inp = muir_inputs.step_inputs(N, H, dk, dk, s, rates=rates, dtype="bf16", seed=3)
        d = to_dev(inp)
        gs = inp["gamma"][0] if form == "static" else None  # [H, dk]
        o = m.muir_step(d["q"], d["k"], d["v"], d["log_a"], d["erase"], d["write"],
                        None if gs is None else gs.to("cuda"), S_gpu)
        tok = dict(inp)
        tok["gamma"] = gs[None].expand(N, H, dk).contiguous() if gs is not None else torch.ones_like(inp["gamma"])
        o_ref, S_ref = oracle.step(*(tok[n] for n in NAMES), S_ref)
        torch.cuda.synchronize()
        assert rel_err(o, o_ref) <= TOL["bf16"], (s, rel_err(o, o_ref))
    assert rel_err(S_gpu, S_ref) <= TOL["bf16"]
