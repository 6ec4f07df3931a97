"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Page citations refer to arXiv 2611.08376 ("Muir: Linear Attention with
Sensitivity-Allocated Gating and Matched-Filter Readout"): its abstract and
the Methodology section of the wolonglab summary page.  None of these tests
re-types the oracle's loop: each compares it with a closed form, an
invariant, an independent algorithm or brute-force differences.
"""
import json
import os

import numpy as np
import pytest

import oracle
from chunkwise_model import chunkwise_fwd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_inputs(rng, B=1, T=12, H=2, dk=6, dv=5, decay=(-1.5, -0.01)):
    silu = lambda x: x / (1 + np.exp(-x))
    q = _unit(silu(rng.standard_normal((B, T, H, dk))))
    k = _unit(silu(rng.standard_normal((B, T, H, dk))))
    v = rng.standard_normal((B, T, H, dv))
    la = rng.uniform(decay[0], decay[1], size=(B, T, H, dk))
    er = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, dk))))
    wr = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, dv))))
    ga = 2 / (1 + np.exp(-rng.standard_normal((B, T, H, dk))))
    return dict(q=q, k=k, v=v, log_a=la, erase=er, write=wr, gamma=ga)


def call_fwd(x, S0=None):
    return oracle.fwd(x["q"], x["k"], x["v"], x["log_a"], x["erase"], x["write"], x["gamma"], S0=S0)


# --- closed forms --------------------------------------------------------------

def test_no_decay_no_erase_is_causal_linear_attention():
    """a = 1 (log_a = 0) and zero erase: the state only accumulates k u^T, so the
    output is plain causal linear attention O = (Qt K^T masked) U + Qt S0
    (abstract: linear attention compresses context into a key-value state)."""
    rng = np.random.default_rng(1)
    x = rand_inputs(rng, B=2, T=17, H=3, dk=7, dv=4)
    x["log_a"][:] = 0.0
    x["erase"][:] = 0.0
    S0 = rng.standard_normal((2, 3, 7, 4))
    o, S_T = call_fwd(x, S0)
    for b in range(2):
        for h in range(3):
            qt = x["gamma"][b, :, h] * x["q"][b, :, h]
            K = x["k"][b, :, h]
            U = x["write"][b, :, h] * x["v"][b, :, h]
            ref = np.tril(qt @ K.T) @ U + qt @ S0[b, h]
            np.testing.assert_allclose(o[b, :, h], ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(S_T[b, h], S0[b, h] + K.T @ U, rtol=0, atol=1e-12)


def test_no_erase_is_gated_linear_attention_with_row_decay():
    """Zero erase leaves the channel-wise decayed sum S_t = diag(a_t) S_{t-1} + k_t u_t^T.
    Its closed form uses the 3D decay tensor exp(L_t - L_s) on KEY channels (the
    Methodology's row-wise decay); a column-wise decay would fail this."""
    rng = np.random.default_rng(2)
    x = rand_inputs(rng, B=1, T=13, H=2, dk=5, dv=3)
    x["erase"][:] = 0.0
    S0 = rng.standard_normal((1, 2, 5, 3))
    o, S_T = call_fwd(x, S0)
    for h in range(2):
        L = np.cumsum(x["log_a"][0, :, h], axis=0)
        qt = x["gamma"][0, :, h] * x["q"][0, :, h]
        K = x["k"][0, :, h]
        U = x["write"][0, :, h] * x["v"][0, :, h]
        T = L.shape[0]
        ref = np.zeros((T, 3))
        for t in range(T):
            ref[t] = (qt[t] * np.exp(L[t])) @ S0[0, h]
            for s in range(t + 1):
                ref[t] += np.sum(qt[t] * K[s] * np.exp(L[t] - L[s])) * U[s]
        np.testing.assert_allclose(o[0, :, h], ref, rtol=0, atol=1e-12)


def test_zero_decay_leaves_only_current_token():
    """alpha = 0 (log_a = -inf): the state is wiped each step, nothing is left to
    erase, and o_t = (qt_t . k_t) u_t, S_T = k_T u_T^T."""
    rng = np.random.default_rng(3)
    x = rand_inputs(rng, B=2, T=9, H=2, dk=6, dv=4)
    x["log_a"][:] = -np.inf
    S0 = rng.standard_normal((2, 2, 6, 4))
    o, S_T = call_fwd(x, S0)
    qt = x["gamma"] * x["q"]
    U = x["write"] * x["v"]
    ref = np.sum(qt * x["k"], axis=-1, keepdims=True) * U
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)
    ref_S = np.einsum("bhj,bhm->bhjm", x["k"][:, -1], U[:, -1])
    np.testing.assert_allclose(S_T, ref_S, rtol=0, atol=1e-13)


def test_full_erase_recalls_last_write_exactly():
    """Delta rule (abstract: erase the prediction for the incoming key before
    writing): with erase = 1 and ||k|| = 1 the state maps k_t to exactly u_t
    after step t, so reading with q = k and gamma = 1 returns u_t."""
    rng = np.random.default_rng(4)
    x = rand_inputs(rng, B=1, T=20, H=2, dk=8, dv=5)
    x["erase"][:] = 1.0
    x["gamma"][:] = 1.0
    x["q"] = x["k"].copy()
    S0 = rng.standard_normal((1, 2, 8, 5))
    o, _ = call_fwd(x, S0)
    np.testing.assert_allclose(o, x["write"] * x["v"], rtol=0, atol=1e-12)


def test_overwrite_same_key_keeps_last_value():
    """Writing the same unit key twice with full erase and no decay leaves only
    the second value for that key, whatever else was stored along other keys."""
    dk, dv = 4, 3
    k1 = np.array([1.0, 0, 0, 0])
    k2 = np.array([0, 1.0, 0, 0])
    ks = np.stack([k1, k2, k1])[None, :, None, :]
    vs = np.array([[1.0, 2, 3], [4.0, 5, 6], [7.0, 8, 9]])[None, :, None, :]
    T = 3
    ones_k = np.ones((1, T, 1, dk))
    o, S_T = oracle.fwd(ks, ks, vs, 0 * ones_k, ones_k, np.ones((1, T, 1, dv)), ones_k)
    np.testing.assert_allclose(S_T[0, 0].T @ k1, [7, 8, 9], atol=1e-15)
    np.testing.assert_allclose(S_T[0, 0].T @ k2, [4, 5, 6], atol=1e-15)


# --- sensitivity structure (pins the erase placement) ---------------------------

def _one_step_state(S, q, k, v, la, er, wr, ga):
    _, Sn = oracle.step(q[None, None], k[None, None], v[None, None], la[None, None], er[None, None],
                        wr[None, None], ga[None, None], S[None, None])
    return Sn[0, 0]


def test_erase_sensitivity_is_key_energy_times_row_energy():
    """Methodology: how much a change in the erase gate of channel j moves the
    state scales with k_{t,j}^2 times the energy already in row j, while a
    change in the write gate moves the written value v_t itself.  Measured by central
    differences of one oracle step:  ||dS_t/d erase_j|| = |k_j| ||S'_j||  and
    ||dS_t/d write_m|| = |v_m|.  Reading the prediction through k and erasing
    along erase*k instead would give |k_j| ||k^T S'|| and fail here."""
    rng = np.random.default_rng(5)
    dk, dv = 7, 5
    S = rng.standard_normal((dk, dv)) * rng.uniform(0.1, 3.0, size=(dk, 1))
    q = _unit(rng.standard_normal(dk))
    k = _unit(rng.standard_normal(dk))
    v = rng.standard_normal(dv)
    la = rng.uniform(-1, -0.01, dk)
    er = rng.uniform(0.2, 0.8, dk)
    wr = rng.uniform(0.2, 0.8, dv)
    ga = rng.uniform(0.5, 1.5, dk)
    Sp = np.exp(la)[:, None] * S
    eps = 1e-6
    alt = np.linalg.norm(k @ Sp)
    for j in range(dk):
        e = np.zeros(dk)
        e[j] = eps
        g = (_one_step_state(S, q, k, v, la, er + e, wr, ga) - _one_step_state(S, q, k, v, la, er - e, wr, ga)) / (2 * eps)
        want = abs(k[j]) * np.linalg.norm(Sp[j])
        assert abs(np.linalg.norm(g) - want) <= 1e-7 * max(1.0, want)
        if abs(k[j]) > 1e-3 and abs(np.linalg.norm(Sp[j]) - alt) > 1e-3:
            assert abs(np.linalg.norm(g) - abs(k[j]) * alt) > 1e-4
    for m in range(dv):
        e = np.zeros(dv)
        e[m] = eps
        g = (_one_step_state(S, q, k, v, la, er, wr + e, ga) - _one_step_state(S, q, k, v, la, er, wr - e, ga)) / (2 * eps)
        assert abs(np.linalg.norm(g) - abs(v[m])) <= 1e-7 * max(1.0, abs(v[m]))


# --- invariants -----------------------------------------------------------------

def test_linear_in_state_and_values():
    """For fixed gates, keys and queries, (S0, write*v) -> (o, S_T) is linear."""
    rng = np.random.default_rng(6)
    x = rand_inputs(rng, B=1, T=11, H=2, dk=5, dv=4)
    S0 = rng.standard_normal((1, 2, 5, 4))
    v2 = rng.standard_normal(x["v"].shape)
    o1, s1 = call_fwd(x, S0)
    y = dict(x)
    y["v"] = v2
    o2, s2 = call_fwd(y, None)
    z = dict(x)
    z["v"] = x["v"] + v2
    o3, s3 = call_fwd(z, S0)
    np.testing.assert_allclose(o3, o1 + o2, atol=1e-12)
    np.testing.assert_allclose(s3, s1 + s2, atol=1e-12)


def test_value_columns_are_independent():
    """Permuting the value channels (v, write, S0 columns) permutes o and S_T."""
    rng = np.random.default_rng(7)
    x = rand_inputs(rng, B=1, T=10, H=1, dk=4, dv=6)
    S0 = rng.standard_normal((1, 1, 4, 6))
    perm = rng.permutation(6)
    o, S_T = call_fwd(x, S0)
    y = dict(x)
    y["v"] = x["v"][..., perm]
    y["write"] = x["write"][..., perm]
    o2, S_T2 = call_fwd(y, S0[..., perm])
    np.testing.assert_allclose(o2, o[..., perm], atol=1e-13)
    np.testing.assert_allclose(S_T2, S_T[..., perm], atol=1e-13)


def test_readout_gate_touches_only_the_output():
    """gamma scales the query only at readout (Methodology): scaling gamma by c
    scales o by c and leaves the state unchanged; gamma = 1 is the GDN-2 readout."""
    rng = np.random.default_rng(8)
    x = rand_inputs(rng, B=1, T=9, H=2, dk=5, dv=3)
    o, S_T = call_fwd(x)
    y = dict(x)
    y["gamma"] = 2.5 * x["gamma"]
    o2, S_T2 = call_fwd(y)
    np.testing.assert_allclose(o2, 2.5 * o, atol=1e-13)
    np.testing.assert_array_equal(S_T2, S_T)


def test_steps_equal_sequence_and_split_sequence():
    """T decode steps reproduce one T-token call, and splitting a sequence into
    two calls chained through the state reproduces one call."""
    rng = np.random.default_rng(9)
    x = rand_inputs(rng, B=2, T=8, H=2, dk=4, dv=3)
    S0 = rng.standard_normal((2, 2, 4, 3))
    o, S_T = call_fwd(x, S0)
    S = S0.copy()
    for t in range(8):
        ot, S = oracle.step(*(x[n][:, t] for n in ("q", "k", "v", "log_a", "erase", "write", "gamma")), S)
        np.testing.assert_allclose(ot, o[:, t], atol=1e-13)
    np.testing.assert_allclose(S, S_T, atol=1e-13)
    a = {n: x[n][:, :5] for n in x}
    b = {n: x[n][:, 5:] for n in x}
    oa, Sa = call_fwd(a, S0)
    ob, Sb = call_fwd(b, Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, atol=1e-13)
    np.testing.assert_allclose(Sb, S_T, atol=1e-13)


# --- independent algorithm: the chunkwise triangular system ---------------------

@pytest.mark.parametrize("C", [1, 2, 4, 8, 16, 48])
def test_chunkwise_triangular_system_matches_recurrence(C):
    """Methodology: training expresses each chunk as a triangular system.  An
    independent fp64 chunkwise model (dense decay tensor + library triangular
    solve) equals the token-by-token oracle for every chunk size."""
    rng = np.random.default_rng(10 + C)
    x = rand_inputs(rng, B=2, T=48, H=2, dk=6, dv=5, decay=(-3.0, -1e-3))
    S0 = rng.standard_normal((2, 2, 6, 5))
    o, S_T = call_fwd(x, S0)
    o2, S_T2 = chunkwise_fwd(x["q"], x["k"], x["v"], x["log_a"], x["erase"], x["write"], x["gamma"], S0, C)
    scale = max(1.0, np.abs(o).max())
    assert np.abs(o - o2).max() <= 1e-12 * scale
    assert np.abs(S_T - S_T2).max() <= 1e-12 * max(1.0, np.abs(S_T).max())


# --- brute force: gradients by central differences ------------------------------

@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_central_differences(seed):
    """Reverse mode of the oracle against fp64 central differences of its forward,
    for every input and the initial state, with random upstream dO and dS_T."""
    rng = np.random.default_rng(100 + seed)
    B, T, H, dk, dv = 1, 6, 2, 4, 3
    x = rand_inputs(rng, B=B, T=T, H=H, dk=dk, dv=dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    dO = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    g = oracle.bwd(x["q"], x["k"], x["v"], x["log_a"], x["erase"], x["write"], x["gamma"], dO, S0=S0, dS_T=dST)

    def loss(xx, s0):
        o, S_T = call_fwd(xx, s0)
        return float(np.sum(o * dO) + np.sum(S_T * dST))

    eps = 1e-6
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_a", "dlog_a"), ("erase", "derase"),
             ("write", "dwrite"), ("gamma", "dgamma")]
    for name, gname in names:
        fd = np.zeros_like(x[name])
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd[idx] = (loss(xp, S0) - loss(xm, S0)) / (2 * eps)
        err = np.abs(fd - g[gname]).max() / max(1.0, np.abs(fd).max())
        assert err <= 1e-6, (name, err)
    fd = np.zeros_like(S0)
    it = np.nditer(S0, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        sp, sm = S0.copy(), S0.copy()
        sp[idx] += eps
        sm[idx] -= eps
        fd[idx] = (loss(x, sp) - loss(x, sm)) / (2 * eps)
    assert np.abs(fd - g["dS0"]).max() / max(1.0, np.abs(fd).max()) <= 1e-6


def test_backward_with_zero_decay_is_finite():
    """log_a = -inf (zero decay) gives finite gradients (d log_a = 0 there)."""
    rng = np.random.default_rng(11)
    x = rand_inputs(rng, B=1, T=5, H=1, dk=3, dv=2)
    x["log_a"][:, 2] = -np.inf
    dO = rng.standard_normal((1, 5, 1, 2))
    g = oracle.bwd(x["q"], x["k"], x["v"], x["log_a"], x["erase"], x["write"], x["gamma"], dO)
    for n, a in g.items():
        assert np.all(np.isfinite(a)), n
    assert np.all(g["dlog_a"][:, 2] == 0.0)


def test_backward_checkpoint_segments():
    """The oracle replays its forward from checkpoints every 64 tokens; a
    sequence crossing several segments equals the sum over two chained calls."""
    rng = np.random.default_rng(12)
    x = rand_inputs(rng, B=1, T=150, H=1, dk=3, dv=2)
    dO = rng.standard_normal((1, 150, 1, 2))
    g = oracle.bwd(x["q"], x["k"], x["v"], x["log_a"], x["erase"], x["write"], x["gamma"], dO)
    # split at 70: the second half's dS0 is the first half's dS_T
    a = {n: x[n][:, :70] for n in x}
    b = {n: x[n][:, 70:] for n in x}
    _, Sa = call_fwd(a)
    gb = oracle.bwd(*(b[n] for n in ("q", "k", "v", "log_a", "erase", "write", "gamma")), dO[:, 70:], S0=Sa)
    ga = oracle.bwd(*(a[n] for n in ("q", "k", "v", "log_a", "erase", "write", "gamma")), dO[:, :70], dS_T=gb["dS0"])
    for n in ("dq", "dk", "dv", "dlog_a", "derase", "dwrite", "dgamma"):
        np.testing.assert_allclose(np.concatenate([ga[n], gb[n]], axis=1), g[n], atol=1e-11)


# --- hand-worked golden examples --------------------------------------------------

def _golden_cases():
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    """Small exact examples worked by hand from the stated mechanism (decay rows,
    erase the prediction for k, write w*v, read S_t through gamma*q)."""
    arr = {n: np.array(case["inputs"][n], dtype=np.float64)[None, :, None, :]
           for n in ("q", "k", "v", "log_a", "erase", "write", "gamma")}
    o, S_T = oracle.fwd(*(arr[n] for n in ("q", "k", "v", "log_a", "erase", "write", "gamma")))
    np.testing.assert_allclose(o[0, :, 0], np.array(case["o"], dtype=np.float64), atol=1e-14)
    np.testing.assert_allclose(S_T[0, 0], np.array(case["S_T"], dtype=np.float64), atol=1e-14)
