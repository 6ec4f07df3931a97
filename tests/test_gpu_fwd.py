"""GPU parity of the chunkwise forward and the decode step against the fp64 oracle.

Tolerances (max |gpu - oracle| / max |oracle| per output tensor): 1e-4 for
fp32 inputs, 2e-2 for bf16 inputs with fp32 state and accumulation.
"""
import sys

import numpy as np
import pytest
import torch

import muir_inputs
import oracle
from gpu_util import NAMES, SEQ_AXES, STATE_AXES, STEP_AXES, TOL, err2, oracle_fwd, rel_err, to_dev, untile_states

pytestmark = pytest.mark.gpu


def _lib():
    import gated_delta_rule_muir_amd as m
    m.lib()
    return m


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype,dk", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_step_matches_oracle(dtype, dk):
    m = _lib()
    N, H, steps = 3, 2, 6
    _say(f"step dtype={dtype} dk={dk}")
    rates = muir_inputs.step_rates(H, dk, seed=1)
    S_gpu = torch.zeros((N, H, dk, dk), dtype=torch.float32, device="cuda")
    S_ref = np.zeros((N, H, dk, dk))
    for s in range(steps):
        inp = muir_inputs.step_inputs(N, H, dk, dk, s, rates=rates, dtype=dtype, seed=1)
        d = to_dev(inp)
        o = m.muir_step(*(d[n] for n in NAMES), S_gpu)
        o_ref, S_ref = oracle.step(*(inp[n] for n in NAMES), S_ref)
        torch.cuda.synchronize()
        assert err2(o, o_ref, STEP_AXES) <= TOL[dtype], (s, err2(o, o_ref, STEP_AXES))
    assert err2(S_gpu, S_ref, STATE_AXES) <= TOL[dtype]


CASES = [
    # name, B, T, H, d, C, dtype, decay, S0 scale
    ("tiny_f32_c64", 1, 256, 2, 64, 64, "f32", "uniform", 0.0),
    ("f32_d128_c64_S0", 1, 128, 2, 128, 64, "f32", "uniform", 0.1),
    ("bf16_d128_c64", 2, 256, 2, 128, 64, "bf16", "channel", 0.0),
    ("bf16_d128_c128_S0", 1, 256, 2, 128, 128, "bf16", "channel_slow", 0.1),
    ("bf16_d128_c256", 1, 512, 2, 128, 256, "bf16", "channel_slow", 0.0),
    ("bf16_d64_c64_uniform", 2, 192, 3, 64, 64, "bf16", "uniform", 0.1),
    # leaves whose decay range needs the per-pair factors
    ("f32_d64_c64_steep", 1, 128, 2, 64, 64, "f32", "steep", 0.1),
    ("bf16_d128_c128_steep", 1, 256, 2, 128, 128, "bf16", "steep", 0.0),
    ("f32_d128_c64_spiky", 1, 128, 2, 128, 64, "f32", "spiky", 0.1),
    ("bf16_d128_c256_spiky", 1, 512, 2, 128, 256, "bf16", "spiky", 0.1),
    # every (dtype, d, chunk) kernel instance over several chunks
    ("f32_d128_c128", 1, 384, 2, 128, 128, "f32", "channel_slow", 0.1),
    ("f32_d64_c128", 1, 384, 2, 64, 128, "f32", "uniform", 0.1),
    ("f32_d128_c256", 1, 768, 1, 128, 256, "f32", "channel_slow", 0.1),
    ("f32_d64_c256", 1, 768, 2, 64, 256, "f32", "channel", 0.1),
    ("bf16_d64_c128", 2, 384, 2, 64, 128, "bf16", "channel", 0.1),
    ("bf16_d64_c256", 1, 768, 3, 64, 256, "bf16", "channel_slow", 0.1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_chunk_fwd_matches_oracle(case):
    name, B, T, H, d, C, dtype, decay, s0 = case
    m = _lib()
    _say(f"chunk_fwd case={name}")
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype=dtype, decay=decay, seed=3, S0_scale=s0)
    dv = to_dev(inp)
    o, S_T, S_chunks = m.muir_chunk_fwd(*(dv[n] for n in NAMES), dv["S0"], chunk=C, save_states=True)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_fwd(inp)
    eo, es = err2(o, o_ref, SEQ_AXES), err2(S_T, S_ref, STATE_AXES)
    _say(f"  err o={eo:.3e} S_T={es:.3e}")
    assert eo <= TOL[dtype]
    assert es <= TOL[dtype]
    # chunk-start states: the state after c*C tokens
    for c in range(T // C):
        if c == 0:
            ref = np.zeros((B, H, d, d)) if inp["S0"] is None else inp["S0"].double().numpy()
        else:
            pre = {n: inp[n][:, : c * C] for n in NAMES}
            pre["S0"] = inp["S0"]
            ref = oracle_fwd(pre)[1]
        assert rel_err(untile_states(S_chunks[:, :, c]), ref) <= TOL[dtype] or np.abs(ref).max() == 0


def test_chunk_sizes_agree():
    """C = 64, 128 and 256 give the same result (same triangular systems, grouped differently)."""
    m = _lib()
    inp = muir_inputs.seq_inputs(1, 512, 2, 128, 128, dtype="bf16", decay="channel", seed=4)
    dv = to_dev(inp)
    outs = [m.muir_chunk_fwd(*(dv[n] for n in NAMES), chunk=C)[0].float() for C in (64, 128, 256)]
    torch.cuda.synchronize()
    assert rel_err(outs[1], outs[0]) <= 1e-2
    assert rel_err(outs[2], outs[0]) <= 1e-2


def test_steps_equal_chunk_fwd():
    """T decode steps reproduce one chunkwise call (the recurrence at chunk size 1)."""
    m = _lib()
    B, T, H, d = 2, 64, 2, 128
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype="f32", decay="channel", seed=5)
    dv = to_dev(inp)
    o, S_T, _ = m.muir_chunk_fwd(*(dv[n] for n in NAMES), chunk=64)
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    outs = []
    for t in range(T):
        outs.append(m.muir_step(*(dv[n][:, t].contiguous() for n in NAMES), S))
    torch.cuda.synchronize()
    assert rel_err(torch.stack(outs, 1), o) <= 1e-4
    assert rel_err(S, S_T) <= 1e-4


def untile(flat, D, C):
    """A transposed summary part, [D][C], from its 16-token tiles [C/16][D][16]."""
    return flat.reshape(C // 16, D, 16).transpose(1, 0, 2).reshape(D, C)


def test_fwd_summary_intermediates():
    """The chunk summary in the workspace equals the plain chunkwise quantities
    (fp32 path, one head): W, U~, Q', O~, Kbar, exp(L_C), and each 16-token
    leaf block's (I + A_II)^-1 and P_II.  The transposed parts are laid out in
    16-token tiles."""
    from chunkwise_model import chunk_summary
    m = _lib()
    B, T, H, d, C = 1, 128, 1, 64, 64
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype="f32", decay="uniform", seed=6)
    dv = to_dev(inp)
    nbytes = m.muir_chunk_fwd_workspace(B, T, H, d, d, C, m.MUIR_F32)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    m.muir_chunk_fwd(*(dv[n] for n in NAMES), chunk=C, workspace=ws)
    torch.cuda.synchronize()
    per = nbytes // (T // C)
    ref = chunk_summary(*(inp[n][0, :, 0].double().numpy() for n in NAMES), C)
    n = C * d
    for c in range(T // C):
        blk = ws[c * per:(c + 1) * per].view(torch.float32).cpu().double().numpy()
        W = blk[:n].reshape(C, d)
        Qp = blk[n: 2 * n].reshape(C, d)
        # the transposed parts are stored as 16-token tiles [C/16][d][16]
        KbT, UtT, OtT = (untile(blk[k * n:(k + 1) * n], d, C) for k in (2, 3, 4))
        gC = blk[5 * n: 5 * n + d]
        TP = blk[5 * n + d: 5 * n + d + (C // 16) * 512].reshape(C // 16, 2, 16, 16)
        r = ref[c]
        # exp(L_C) of fast channels sits in the fp32 denormal range, where the
        # device exponential flushes to zero: compare it with an absolute floor.
        np.testing.assert_allclose(gC, r["gC"], rtol=1e-4, atol=1e-36)
        leaves_T = np.stack([np.linalg.inv(np.eye(16) + r["A"][16 * i:16 * i + 16, 16 * i:16 * i + 16])
                             for i in range(C // 16)])
        leaves_P = np.stack([r["P"][16 * i:16 * i + 16, 16 * i:16 * i + 16] for i in range(C // 16)])
        for nm, got, want in (("W", W, r["W"]), ("Ut", UtT.T, r["Ut"]), ("Qp", Qp, r["Qp"]),
                              ("Ot", OtT.T, r["Ot"]), ("Kb", KbT.T, r["Kb"]),
                              ("T_II", TP[:, 0], leaves_T), ("P_II", TP[:, 1], leaves_P)):
            e = rel_err(got, want)
            _say(f"  chunk {c} {nm}: {e:.3e}")
            assert e <= 1e-4, (c, nm, e)


def test_fwd_saved_deltas():
    """A bf16 forward that saves its chunk states also keeps, in each chunk
    summary, the chunk's deltas U~ - W S_c (S_c: the state at the chunk's
    start), which the 64-token-chunk backward reads instead of recomputing
    them.  Checked against the chunk model's U~, W and the oracle's S_c."""
    from chunkwise_model import chunk_summary
    m = _lib()
    B, T, H, d, C = 1, 256, 1, 128, 64
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype="bf16", decay="channel", seed=8)
    dv = to_dev(inp)
    nbytes = m.muir_chunk_fwd_workspace(B, T, H, d, d, C)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    m.muir_chunk_fwd(*(dv[n] for n in NAMES), chunk=C, save_states=True, workspace=ws)
    torch.cuda.synchronize()
    per = nbytes // (T // C)
    n = C * d
    dl_off = 5 * n * 2 + d * 4 + (C // 16) * 512 * 2  # after the parts, Gamma_C and the leaf blocks
    ref = chunk_summary(*(inp[nm][0, :, 0].double().numpy() for nm in NAMES), C)
    for c in range(T // C):
        blk = ws[c * per + dl_off: c * per + dl_off + n * 2].view(torch.bfloat16).cpu().double().numpy()
        delta = blk.reshape(C, d)
        if c == 0:
            S_c = np.zeros((d, d))
        else:
            _, S_c = oracle.fwd(*(inp[nm][:, :c * C] for nm in NAMES))
            S_c = S_c[0, 0]
        want = ref[c]["Ut"] - ref[c]["W"] @ S_c
        e = rel_err(delta, want)
        _say(f"  chunk {c} deltas: {e:.3e}")
        assert e <= TOL["bf16"], (c, e)
