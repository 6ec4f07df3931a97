"""GPU parity of sequences that do not fill whole chunks: a partial last chunk
(T % chunk != 0) and packed variable-length sequences, against the fp64
oracle run on each real sequence on its own.

Tolerances as elsewhere: max |gpu - oracle| / max |oracle|, over each whole
tensor and over each head's slice of it, <= 1e-4 (fp32 inputs) or 2e-2
(bf16 inputs).  The gradients are fp32 unless a case asks for bf16 ones."""
import sys

import numpy as np
import pytest
import torch

import muir_inputs
import oracle
from gpu_util import NAMES, SEQ_AXES, STATE_AXES, TOL, err2, grad_axes, oracle_bwd, oracle_fwd, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dlog_a", "derase", "dwrite", "dgamma", "dS0")
SEQ_GRADS = ("dq", "dk", "dv", "dlog_a", "derase", "dwrite")


def _lib():
    import gated_delta_rule_muir_amd as m
    m.lib()
    return m


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


TAIL_CASES = [
    # name, B, T, H, d, C, dtype, decay, gradient dtype
    ("f32_d64_c64_T100", 1, 100, 2, 64, 64, "f32", "uniform", torch.float32),
    ("f32_d128_c256_T37", 1, 37, 2, 128, 256, "f32", "channel", torch.float32),
    ("bf16_d128_c64_T200", 2, 200, 2, 128, 64, "bf16", "channel", torch.float32),
    ("bf16_d64_c64_T1", 2, 1, 2, 64, 64, "bf16", "uniform", torch.float32),
    ("bf16_d128_c128_T300", 1, 300, 2, 128, 128, "bf16", "channel_slow", torch.float32),
    ("bf16_d128_c64_T255_spiky", 1, 255, 2, 128, 64, "bf16", "spiky", torch.float32),
    ("bf16_d128_c64_T200_bf16grads", 2, 200, 2, 128, 64, "bf16", "channel", torch.bfloat16),
    ("bf16_d64_c256_T300_bf16grads", 1, 300, 2, 64, 256, "bf16", "channel_slow", torch.bfloat16),
]


@pytest.mark.parametrize("case", TAIL_CASES, ids=[c[0] for c in TAIL_CASES])
def test_tail_chunk_matches_oracle(case):
    """A sequence that ends inside a chunk: outputs, final state and every
    gradient against the oracle, which has no chunks at all."""
    name, B, T, H, d, C, dtype, decay, gdt = case
    m = _lib()
    _say(f"tail case={name}")
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype=dtype, decay=decay, seed=21, S0_scale=0.1,
                                 with_dO=True, with_dST=True)
    dv = to_dev(inp)
    args = [dv[n] for n in NAMES]
    o, S_T, Sc = m.muir_chunk_fwd(*args, dv["S0"], chunk=C, save_states=True)
    assert tuple(Sc.shape) == (B, H, (T + C - 1) // C, d, d)
    g = m.muir_chunk_bwd(*args, dv["dO"], S0=dv["S0"], dS_T=dv["dS_T"], chunk=C, grad_dtype=gdt)
    torch.cuda.synchronize()
    for n in GRADS:
        assert g[n].dtype == (torch.float32 if n == "dS0" else gdt), n
    o_ref, S_ref = oracle_fwd(inp)
    ref = oracle_bwd(inp)
    errs = {"o": err2(o, o_ref, SEQ_AXES), "S_T": err2(S_T, S_ref, STATE_AXES)}
    errs.update({n: err2(g[n], ref[n], grad_axes(n)) for n in GRADS})
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)


def test_tail_chunk_saved_forward_results():
    """The backward of a partial-chunk call given the forward's chunk states
    and summaries (its workspace) equals the backward that recomputes them."""
    m = _lib()
    B, T, H, d, C = 2, 190, 2, 128, 64
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype="bf16", decay="channel", seed=22, S0_scale=0.1,
                                 with_dO=True)
    dv = to_dev(inp)
    args = [dv[n] for n in NAMES]
    ws = torch.empty(m.muir_chunk_fwd_workspace(B, T, H, d, d, C), dtype=torch.uint8, device="cuda")
    _, _, Sc = m.muir_chunk_fwd(*args, dv["S0"], chunk=C, save_states=True, workspace=ws)
    g1 = m.muir_chunk_bwd(*args, dv["dO"], S0=dv["S0"], S_chunks=Sc, summaries=ws, chunk=C)
    g2 = m.muir_chunk_bwd(*args, dv["dO"], S0=dv["S0"], chunk=C)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(g1[n], g2[n]), n


def _split_oracle(inp, lens, gamma_form):
    """The oracle on every packed sequence alone; returns packed o and
    per-token gradients, stacked S_T and dS0, and dgamma in the form's shape."""
    cu = np.concatenate([[0], np.cumsum(lens)])
    H, dk = inp["q"].shape[1], inp["q"].shape[2]
    dvv = inp["v"].shape[2]
    o = np.zeros((int(cu[-1]), H, dvv))
    grads = {n: np.zeros(tuple(inp[n[1:]].shape)) for n in SEQ_GRADS}
    dgam_tok = np.zeros((int(cu[-1]), H, dk))
    S_T, dS0 = [], []
    for i, L in enumerate(lens):
        a, b = int(cu[i]), int(cu[i + 1])
        one = {n: inp[n][a:b][None] for n in ("q", "k", "v", "log_a", "erase", "write", "dO")}
        if gamma_form == "token":
            one["gamma"] = inp["gamma"][a:b][None]
        elif gamma_form == "static":
            one["gamma"] = inp["gamma_static"][None, None].expand(1, int(L), H, dk)
        else:
            one["gamma"] = torch.ones((1, int(L), H, dk), dtype=inp["q"].dtype)
        one["S0"] = None if inp["S0"] is None else inp["S0"][i:i + 1]
        one["dS_T"] = None if inp["dS_T"] is None else inp["dS_T"][i:i + 1]
        if L == 0:
            S_T.append(np.zeros((H, dk, dvv)) if one["S0"] is None else one["S0"][0].double().numpy())
            dS0.append(np.zeros((H, dk, dvv)) if one["dS_T"] is None else one["dS_T"][0].double().numpy())
            continue
        o1, s1 = oracle_fwd(one)
        r = oracle_bwd(one)
        o[a:b] = o1[0]
        S_T.append(s1[0])
        for n in SEQ_GRADS:
            grads[n][a:b] = r[n][0]
        dgam_tok[a:b] = r["dgamma"][0]
        dS0.append(r["dS0"][0])
    grads["dS0"] = np.stack(dS0)
    if gamma_form == "token":
        grads["dgamma"] = dgam_tok
    elif gamma_form == "static":
        grads["dgamma"] = dgam_tok.sum(axis=0)
    return o, np.stack(S_T), grads


VARLEN_CASES = [
    # name, N, max_len, H, d, C, dtype, decay, gate form, gradient dtype
    ("f32_d64_c64_token", 6, 200, 2, 64, 64, "f32", "uniform", "token", torch.float32),
    ("bf16_d128_c64_token", 7, 300, 2, 128, 64, "bf16", "channel", "token", torch.float32),
    ("bf16_d128_c64_static", 5, 260, 2, 128, 64, "bf16", "channel", "static", torch.float32),
    ("bf16_d128_c128_none", 6, 400, 2, 128, 128, "bf16", "channel_slow", "none", torch.float32),
    ("f32_d128_c64_static", 5, 150, 1, 128, 64, "f32", "steep", "static", torch.float32),
    ("bf16_d128_c64_token_bf16grads", 7, 300, 2, 128, 64, "bf16", "channel", "token", torch.bfloat16),
]

# packed [T_total, H, D] tensors: the head axis (sequences are compared whole)
PACKED_AXES = (1,)


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[c[0] for c in VARLEN_CASES])
def test_varlen_matches_per_sequence_oracle(case):
    """Packed sequences of mixed length (an empty one, one token, exact chunk
    multiples, one past a chunk, random lengths): each sequence's outputs,
    final state and gradients equal the oracle's on that sequence alone."""
    name, N, max_len, H, d, C, dtype, decay, form, gdt = case
    m = _lib()
    lens = muir_inputs.varlen_lengths(N, max_len, C, seed=5)
    _say(f"varlen case={name} lens={lens.tolist()}")
    inp = muir_inputs.varlen_inputs(lens, H, d, d, dtype=dtype, decay=decay, seed=23, S0_scale=0.1,
                                    with_dST=True)
    inp["gamma_static"] = inp["gamma"][0].clone()
    dv = to_dev(inp)
    gam = {"token": dv["gamma"], "static": dv["gamma_static"], "none": None}[form]
    args = [dv["q"], dv["k"], dv["v"], dv["log_a"], dv["erase"], dv["write"], gam]
    cu = dv["cu_seqlens"]
    o, S_T = m.muir_chunk_varlen_fwd(*args, cu, dv["S0"], chunk=C)
    g = m.muir_chunk_varlen_bwd(*args, dv["dO"], cu, S0=dv["S0"], dS_T=dv["dS_T"], chunk=C, grad_dtype=gdt)
    torch.cuda.synchronize()
    for n in SEQ_GRADS:
        assert g[n].dtype == gdt, n
    o_ref, S_ref, ref = _split_oracle(inp, lens, form)
    errs = {"o": err2(o, o_ref, PACKED_AXES), "S_T": err2(S_T, S_ref, STATE_AXES)}
    errs.update({n: err2(g[n], ref[n], PACKED_AXES) for n in SEQ_GRADS})
    errs["dS0"] = err2(g["dS0"], ref["dS0"], STATE_AXES)
    if form == "none":
        assert g["dgamma"] is None
    else:
        errs["dgamma"] = err2(g["dgamma"], ref["dgamma"], PACKED_AXES if form == "token" else (0,))
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)


@pytest.mark.parametrize("form", ["token", "static"])
def test_varlen_backward_reuses_the_forward(form):
    """A keeping forward leaves its packed inputs, summaries and chunk states
    in its workspace; the backward that takes it gives the recomputing
    backward's results bit for bit (the same kernels on the same data), and
    the keeping forward the plain forward's."""
    m = _lib()
    N, max_len, H, d, C = 6, 300, 2, 128, 64
    lens = muir_inputs.varlen_lengths(N, max_len, C, seed=9)
    _say(f"varlen reuse form={form} lens={lens.tolist()}")
    inp = muir_inputs.varlen_inputs(lens, H, d, d, dtype="bf16", decay="channel", seed=29, S0_scale=0.1,
                                    with_dST=True)
    inp["gamma_static"] = inp["gamma"][0].clone()
    dv = to_dev(inp)
    gam = dv["gamma"] if form == "token" else dv["gamma_static"]
    args = [dv["q"], dv["k"], dv["v"], dv["log_a"], dv["erase"], dv["write"], gam]
    cu = dv["cu_seqlens"]
    gm = m.MUIR_GAMMA_TOKEN if form == "token" else m.MUIR_GAMMA_STATIC
    ws = torch.empty(m.muir_chunk_varlen_fwd_workspace(N, max_len, H, d, d, C, gamma_mode=gm), dtype=torch.uint8,
                     device="cuda")
    o1, S1 = m.muir_chunk_varlen_fwd(*args, cu, dv["S0"], chunk=C, max_len=max_len, keep=True, workspace=ws)
    o2, S2 = m.muir_chunk_varlen_fwd(*args, cu, dv["S0"], chunk=C, max_len=max_len)
    kw = dict(S0=dv["S0"], dS_T=dv["dS_T"], chunk=C, max_len=max_len)
    g1 = m.muir_chunk_varlen_bwd(*args, dv["dO"], cu, fwd_workspace=ws, **kw)
    g2 = m.muir_chunk_varlen_bwd(*args, dv["dO"], cu, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    for n in GRADS:
        assert torch.equal(g1[n], g2[n]), n


def test_varlen_equal_lengths_equal_batched_call():
    """Packed sequences that all have the same whole-chunk length give
    exactly the batched call's results (the same kernels on the same data)."""
    m = _lib()
    N, L, H, d, C = 3, 128, 2, 128, 64
    inp = muir_inputs.varlen_inputs([L] * N, H, d, d, dtype="bf16", decay="channel", seed=24, S0_scale=0.1,
                                    with_dST=True)
    dv = to_dev(inp)
    packed = [dv[n] for n in NAMES]
    batched = [t.view(N, L, *t.shape[1:]) for t in packed]
    o1, S1 = m.muir_chunk_varlen_fwd(*packed, dv["cu_seqlens"], dv["S0"], chunk=C)
    g1 = m.muir_chunk_varlen_bwd(*packed, dv["dO"], dv["cu_seqlens"], S0=dv["S0"], dS_T=dv["dS_T"], chunk=C)
    o2, S2, _ = m.muir_chunk_fwd(*batched, dv["S0"], chunk=C)
    g2 = m.muir_chunk_bwd(*batched, dv["dO"].view(N, L, H, d), S0=dv["S0"], dS_T=dv["dS_T"], chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(N, L, H, d), o2) and torch.equal(S1, S2)
    for n in GRADS:
        assert torch.equal(g1[n].view_as(g2[n]), g2[n]), n


def test_varlen_without_tokens():
    """Only empty sequences: the final states are the initial ones and the
    initial states' gradients are the final states'."""
    m = _lib()
    N, H, d = 3, 2, 64
    z = torch.zeros((0, H, d), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    S0 = torch.randn((N, H, d, d), device="cuda")
    dS_T = torch.randn((N, H, d, d), device="cuda")
    o, S_T = m.muir_chunk_varlen_fwd(z, z, z, z, z, z, z, cu, S0, chunk=64)
    g = m.muir_chunk_varlen_bwd(z, z, z, z, z, z, z, z, cu, S0=S0, dS_T=dS_T, chunk=64)
    torch.cuda.synchronize()
    assert o.shape == (0, H, d)
    assert torch.equal(S_T, S0) and torch.equal(g["dS0"], dS_T)
