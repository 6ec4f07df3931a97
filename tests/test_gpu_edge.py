"""Edge and degenerate cases of the GPU path against the oracle."""
import numpy as np
import pytest
import torch

import muir_inputs
import oracle
from gpu_util import NAMES, TOL, oracle_bwd, oracle_fwd, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _lib():
    import gated_delta_rule_muir_amd as m
    m.lib()
    return m


def test_empty_sequence_passes_state_through():
    m = _lib()
    q = torch.zeros((2, 0, 3, 64), dtype=torch.float32, device="cuda")
    S0 = torch.randn((2, 3, 64, 64), device="cuda")
    o, S_T, _ = m.muir_chunk_fwd(q, q, q, q, q, q, q, S0, chunk=64)
    dS_T = torch.randn((2, 3, 64, 64), device="cuda")
    g = m.muir_chunk_bwd(q, q, q, q, q, q, q, q, S0=S0, dS_T=dS_T, chunk=64)
    o2, S_T2, _ = m.muir_chunk_fwd(q, q, q, q, q, q, q, None, chunk=64)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 64)
    assert torch.equal(S_T, S0) and torch.equal(g["dS0"], dS_T)
    assert torch.count_nonzero(S_T2) == 0


@pytest.mark.parametrize("case", ["no_decay", "full_erase_recall", "zero_gamma", "zero_inputs"])
def test_degenerate_cases(case):
    m = _lib()
    B, T, H, d, C = 1, 128, 2, 64, 64
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype="f32", decay="uniform", seed=9, with_dO=True)
    if case == "no_decay":
        inp["log_a"] = torch.zeros_like(inp["log_a"])
    elif case == "full_erase_recall":
        inp["erase"] = torch.ones_like(inp["erase"])
        inp["gamma"] = torch.ones_like(inp["gamma"])
        inp["q"] = inp["k"].clone()
    elif case == "zero_gamma":
        inp["gamma"] = torch.zeros_like(inp["gamma"])
    elif case == "zero_inputs":
        for n in ("v", "write"):
            inp[n] = torch.zeros_like(inp[n])
    dv = to_dev(inp)
    o, S_T, _ = m.muir_chunk_fwd(*(dv[n] for n in NAMES), chunk=C)
    g = m.muir_chunk_bwd(*(dv[n] for n in NAMES), dv["dO"], chunk=C)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_fwd(inp)
    gr = oracle_bwd(inp)
    if case == "zero_gamma":
        assert torch.count_nonzero(o) == 0
    if case == "zero_inputs":
        assert torch.count_nonzero(o) == 0 and torch.count_nonzero(S_T) == 0
    if case == "full_erase_recall":
        # delta rule: o_t = write_t * v_t exactly (up to fp32 rounding)
        assert rel_err(o, (inp["write"] * inp["v"]).double().numpy()) <= 1e-4
    # A tensor that is zero in exact arithmetic (e.g. d log_a under exact recall,
    # where o does not depend on the decay) holds only rounding noise: compare it
    # against the scale of the other gradients instead of its own.
    scale = max(float(np.abs(gr[n]).max()) for n in gr)
    for name, got, want in [("o", o, o_ref), ("S_T", S_T, S_ref)] + [(n, g[n], gr[n]) for n in gr]:
        if np.abs(want).max() <= 1e-8 * max(scale, 1.0):
            assert float(got.abs().max()) <= 1e-5 * max(scale, 1.0), (case, name)
        else:
            assert rel_err(got, want) <= TOL["f32"], (case, name, rel_err(got, want))


def test_repeated_runs_are_bitwise_identical():
    """No atomics on the path: repeated calls give identical bits (race canary)."""
    m = _lib()
    inp = muir_inputs.seq_inputs(2, 256, 4, 128, 128, dtype="bf16", decay="channel", seed=10, with_dO=True)
    dv = to_dev(inp)
    o1, S1, Sc1 = m.muir_chunk_fwd(*(dv[n] for n in NAMES), chunk=64, save_states=True)
    g1 = m.muir_chunk_bwd(*(dv[n] for n in NAMES), dv["dO"], S_chunks=Sc1, chunk=64)
    for _ in range(3):
        o2, S2, Sc2 = m.muir_chunk_fwd(*(dv[n] for n in NAMES), chunk=64, save_states=True)
        g2 = m.muir_chunk_bwd(*(dv[n] for n in NAMES), dv["dO"], S_chunks=Sc2, chunk=64)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(S1, S2)
        for n in g1:
            assert torch.equal(g1[n], g2[n]), n


def test_split_sequence_chains_state():
    """Two calls chained through S_T -> S0 equal one call (forward and backward)."""
    m = _lib()
    inp = muir_inputs.seq_inputs(1, 256, 2, 128, 128, dtype="f32", decay="channel", seed=12, with_dO=True)
    dv = to_dev(inp)
    o, S_T, _ = m.muir_chunk_fwd(*(dv[n] for n in NAMES), chunk=64)
    a = {n: dv[n][:, :128].contiguous() for n in NAMES}
    b = {n: dv[n][:, 128:].contiguous() for n in NAMES}
    oa, Sa, _ = m.muir_chunk_fwd(*(a[n] for n in NAMES), chunk=64)
    ob, Sb, _ = m.muir_chunk_fwd(*(b[n] for n in NAMES), Sa, chunk=64)
    gb = m.muir_chunk_bwd(*(b[n] for n in NAMES), dv["dO"][:, 128:].contiguous(), S0=Sa, chunk=64)
    ga = m.muir_chunk_bwd(*(a[n] for n in NAMES), dv["dO"][:, :128].contiguous(), dS_T=gb["dS0"], chunk=64)
    g = m.muir_chunk_bwd(*(dv[n] for n in NAMES), dv["dO"], chunk=64)
    torch.cuda.synchronize()
    assert rel_err(torch.cat([oa, ob], 1), o) <= 1e-5
    assert rel_err(Sb, S_T) <= 1e-5
    for n in ("dq", "dk", "dv", "dlog_a", "derase", "dwrite", "dgamma"):
        assert rel_err(torch.cat([ga[n], gb[n]], 1), g[n]) <= 1e-5, n
    assert rel_err(ga["dS0"], g["dS0"]) <= 1e-5


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_input_check_counts_what_breaks_the_preconditions(dtype):
    """muir_check_values counts NaN and infinite values (any input) and
    log-decays above 0, exactly, over odd lengths and offset views; +0 and -0
    are fine log-decays.  The compute calls' check_inputs option raises
    MUIR_ERR_NONFINITE naming the tensor."""
    import gated_delta_rule_muir_amd as m
    m.lib()
    gen = torch.Generator().manual_seed(3)
    x = torch.randn(10007, generator=gen).to(dtype)
    la = -torch.rand(10007, generator=gen).to(dtype)
    x[[5, 700, 10006]] = float("nan")
    x[[1, 9000]] = float("inf")
    x[4444] = -float("inf")
    la[[0, 17, 5000, 10005]] = torch.tensor([0.5, 1e-3, 7.0, 1e-30]).to(dtype)
    la[[20, 21]] = torch.tensor([0.0, -0.0]).to(dtype)
    la[30] = float("nan")
    xd, lad = x.cuda(), la.cuda()
    got = m.muir_check_inputs({"v": xd, "log_a": lad}, raise_on_error=False)
    # 1e-30 is tiny but above 0, and counts; the NaN log-decay counts once, as non-finite
    assert got["v"] == (6, 0), got
    assert got["log_a"] == (1, 4), got
    # a view that starts one element in, and an odd length
    got = m.muir_check_inputs({"v": xd[1:9001], "log_a": lad[18:10005]}, raise_on_error=False)
    assert got["v"] == (5, 0) and got["log_a"] == (1, 1), got
    with pytest.raises(m.MuirError) as e:
        m.muir_check_inputs({"v": xd})
    assert e.value.code == 9 and "v:" in str(e.value)
    clean = {"q": torch.randn(64, device="cuda").to(dtype), "log_a": -torch.rand(64, device="cuda").to(dtype)}
    assert m.muir_check_inputs(clean) == {"q": (0, 0), "log_a": (0, 0)}

    inp = to_dev(muir_inputs.seq_inputs(1, 64, 2, 64, 64, dtype="bf16" if dtype == torch.bfloat16 else "f32",
                                        seed=2, with_dO=True))
    args = [inp[n] for n in NAMES]
    m.muir_chunk_fwd(*args, chunk=64, check_inputs=True)  # clean: no error
    bad = dict(inp)
    bad["log_a"] = inp["log_a"].clone()
    bad["log_a"][0, 3, 1, 7] = 0.25
    with pytest.raises(m.MuirError) as e:
        m.muir_chunk_fwd(*(bad[n] for n in NAMES), chunk=64, check_inputs=True)
    assert e.value.code == 9 and "log_a" in str(e.value)
    bad = dict(inp)
    bad["dO"] = inp["dO"].clone()
    bad["dO"][0, 0, 0, 0] = float("nan")
    with pytest.raises(m.MuirError):
        m.muir_chunk_bwd(*args, bad["dO"], chunk=64, check_inputs=True)
