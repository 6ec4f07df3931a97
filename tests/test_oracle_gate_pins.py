"""Pins of the gate-prologue oracle (oracle/gate_proj.py) against closed
forms, the packed layout fixed by the gate ranks, linearity of the
projections and central differences.

Source: arXiv 2611.08376, wolonglab summary page, §Methodology (one
down-projection shared by the five gates, five up-projections with channel
biases) and fig:arch (b), (c) (gate order f, b, g, w, q with ranks 64, 64,
128, 128, 128 summing to 512).  None of these tests re-types the oracle.
"""
import math

import numpy as np
import pytest

from oracle import gate_proj as gp

H, DK, DV = 1, 2, 3  # small widths: key gates 2 channels, value gates 3


def _params(rng, d, scale=0.2):
    nw, nb = gp.up_numel(H, DK, DV)
    return (rng.standard_normal((512, d)) * scale, rng.standard_normal(nw) * scale,
            rng.standard_normal(nb) * scale)


def test_packed_sizes_follow_the_ranks():
    """W_up holds 2*64 + 2*64 + 3*128 + 3*128 + 2*128 values for widths
    (H*dk, H*dk, H*dv, H*dv, H*dk) = (2, 2, 3, 3, 2); the biases 2+2+3+3+2."""
    assert gp.up_numel(H, DK, DV) == (128 + 128 + 384 + 384 + 256, 12)
    assert sum(gp.RANKS) == 512


def test_zero_up_weights_give_the_bias_activations():
    rng = np.random.default_rng(0)
    Wd, _, _ = _params(rng, 4)
    nw, nb = gp.up_numel(H, DK, DV)
    x = rng.standard_normal((3, 4))
    out = gp.gate_fwd(x, Wd, np.zeros(nw), np.zeros(nb), H, DK, DV)
    assert np.allclose(out["log_a"], -math.log(2.0), rtol=0, atol=1e-15)
    for n in ("erase", "g", "write"):
        assert np.allclose(out[n], 0.5, rtol=0, atol=1e-15)
    assert np.allclose(out["gamma"], 1.0, rtol=0, atol=1e-15)
    b = np.linspace(-3, 3, nb)
    out = gp.gate_fwd(x, Wd, np.zeros(nw), b, H, DK, DV)
    sig = [1 / (1 + math.exp(-t)) for t in b]
    # bias slices in gate order: f [0:2], b [2:4], g [4:7], w [7:10], q [10:12]
    assert np.allclose(out["log_a"][0, 0], [math.log(s) for s in sig[0:2]], rtol=1e-14)
    assert np.allclose(out["erase"][1, 0], sig[2:4], rtol=1e-14)
    assert np.allclose(out["g"][2, 0], sig[4:7], rtol=1e-14)
    assert np.allclose(out["write"][0, 0], sig[7:10], rtol=1e-14)
    assert np.allclose(out["gamma"][1, 0], [2 * s for s in sig[10:12]], rtol=1e-14)


def _logit(y):
    return np.log(y) - np.log1p(-y)


def _pre(out):
    """Pre-activations recovered by inverting each activation."""
    return {"log_a": _logit(np.exp(out["log_a"])), "erase": _logit(out["erase"]), "g": _logit(out["g"]),
            "write": _logit(out["write"]), "gamma": _logit(out["gamma"] / 2)}


# (z column, gate it belongs to, column of that gate's up matrix [width, rank])
ROUTES = [(0, "log_a", 0), (63, "log_a", 63), (64, "erase", 0), (127, "erase", 63), (128, "g", 0),
          (255, "g", 127), (256, "write", 0), (383, "write", 127), (384, "gamma", 0), (511, "gamma", 127)]
# flat offset of each gate's up matrix in W_up, and its width
UP_AT = {"log_a": (0, 2), "erase": (128, 2), "g": (256, 3), "write": (640, 3), "gamma": (1024, 2)}


@pytest.mark.parametrize("col,gate,row", ROUTES)
def test_each_gate_reads_only_its_rank_slice(col, gate, row):
    """A down-projection that maps the token to one channel of z moves only
    the gate whose rank slice holds that channel, by that column of its up
    matrix (stored [width, rank], a linear layer's [out, in])."""
    rng = np.random.default_rng(col)
    Wd = np.zeros((512, 1))
    Wd[col, 0] = 1.0
    nw, nb = gp.up_numel(H, DK, DV)
    Wu = rng.uniform(-1, 1, nw)
    out = gp.gate_fwd(np.ones((1, 1)), Wd, Wu, np.zeros(nb), H, DK, DV)
    pre = _pre(out)
    for name in gp.GATES:
        got = pre[name].reshape(-1)
        if name == gate:
            off, w = UP_AT[name]
            rank = 64 if name in ("log_a", "erase") else 128
            assert np.allclose(got, Wu[off + row: off + w * rank: rank], rtol=1e-9, atol=1e-12)
        else:
            assert np.allclose(got, 0.0, atol=1e-12), name


def test_pre_activations_are_linear_in_the_input():
    """Every gate is an activation of (x W_down)_slice U + c: after inverting
    the activation and removing the bias, the response to x1 + x2 is the sum
    of the responses to x1 and x2, and scales with x."""
    rng = np.random.default_rng(3)
    Wd, Wu, b = _params(rng, 5)
    x1, x2 = rng.standard_normal((2, 5)), rng.standard_normal((2, 5))
    nb = b.size
    p0 = _pre(gp.gate_fwd(np.zeros((2, 5)), Wd, Wu, b, H, DK, DV))
    p1 = _pre(gp.gate_fwd(x1, Wd, Wu, b, H, DK, DV))
    p2 = _pre(gp.gate_fwd(x2, Wd, Wu, b, H, DK, DV))
    p12 = _pre(gp.gate_fwd(x1 + x2, Wd, Wu, b, H, DK, DV))
    p3 = _pre(gp.gate_fwd(-2.5 * x1, Wd, Wu, b, H, DK, DV))
    for n in gp.GATES:
        assert np.allclose(p12[n] - p0[n], (p1[n] - p0[n]) + (p2[n] - p0[n]), rtol=1e-9, atol=1e-10)
        assert np.allclose(p3[n] - p0[n], -2.5 * (p1[n] - p0[n]), rtol=1e-9, atol=1e-10)
    assert nb == 12


def test_log_decay_is_a_nonpositive_log_sigmoid():
    """log alpha = log sigmoid(pre): <= 0 everywhere, ~ pre far below 0 and
    ~ -e^-pre far above it (closed forms, no overflow)."""
    nw, nb = gp.up_numel(H, DK, DV)
    Wd = np.zeros((512, 1))
    for pre, expect in ((-40.0, -40.0 - math.log1p(math.exp(-40.0))), (40.0, -math.log1p(math.exp(-40.0))),
                        (-800.0, -800.0), (0.0, -math.log(2.0))):
        b = np.full(nb, pre)
        out = gp.gate_fwd(np.zeros((1, 1)), Wd, np.zeros(nw), b, H, DK, DV)
        assert np.all(out["log_a"] <= 0)
        assert np.allclose(out["log_a"], expect, rtol=1e-15, atol=0), pre
        assert np.all(np.isfinite(out["gamma"])) and np.all((out["gamma"] >= 0) & (out["gamma"] <= 2))


def test_gate_backward_matches_central_differences():
    rng = np.random.default_rng(11)
    M, d = 3, 4
    Wd, Wu, b = _params(rng, d, scale=0.5)
    x = rng.standard_normal((M, d))
    fwd = gp.gate_fwd(x, Wd, Wu, b, H, DK, DV)
    dG = {n: rng.standard_normal(fwd[n].shape) for n in gp.GATES}
    g = gp.gate_bwd(x, Wd, Wu, b, dG, H, DK, DV)

    def loss(x_, Wd_, Wu_, b_):
        o = gp.gate_fwd(x_, Wd_, Wu_, b_, H, DK, DV)
        return sum(float(np.sum(o[n] * dG[n])) for n in gp.GATES)

    eps = 1e-6
    args = {"x": x, "Wd": Wd, "Wu": Wu, "b": b}
    names = {"x": "dx", "Wd": "dW_down", "Wu": "dW_up", "b": "dbias"}
    for a, gname in names.items():
        flat = args[a].reshape(-1)
        # every element of the small tensors, a spread sample of the large ones
        idx = range(flat.size) if flat.size <= 64 else rng.choice(flat.size, 64, replace=False)
        for i in idx:
            p = {k: v.copy() for k, v in args.items()}
            m = {k: v.copy() for k, v in args.items()}
            p[a].reshape(-1)[i] += eps
            m[a].reshape(-1)[i] -= eps
            fd = (loss(p["x"], p["Wd"], p["Wu"], p["b"]) - loss(m["x"], m["Wd"], m["Wu"], m["b"])) / (2 * eps)
            got = g[gname].reshape(-1)[i]
            assert abs(fd - got) <= 1e-6 * max(1.0, abs(fd)), (a, i, fd, got)


def test_qk_norm_closed_forms():
    """SiLU then L2 over a head: silu(1) = 1/(1+e^-1); equal channels give
    1/sqrt(dk) each; a negative-only vector keeps its signs; norm is 1 up to the
    1e-6 guard."""
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    y = gp.qk_norm_fwd(np.array([[1.0, 0.0, 0.0, 0.0]]))
    assert np.allclose(y, [[s1 / math.sqrt(s1 * s1 + 1e-6), 0, 0, 0]], rtol=1e-15)
    y = gp.qk_norm_fwd(np.full((2, 16), 2.0))
    s2 = 2.0 / (1.0 + math.exp(-2.0))
    assert np.allclose(y, s2 / math.sqrt(16 * s2 * s2 + 1e-6), rtol=1e-15)
    rng = np.random.default_rng(5)
    u = rng.standard_normal((7, 3, 32)) * 3
    y = gp.qk_norm_fwd(u)
    s = u / (1 + np.exp(-u))
    n2 = (s * s).sum(-1)
    assert np.allclose((y * y).sum(-1), n2 / (n2 + 1e-6), rtol=1e-14)
    assert np.all(np.sign(y) == np.sign(s))
    assert np.all(gp.qk_norm_fwd(np.zeros((1, 8))) == 0)


def test_qk_norm_backward():
    """Central differences; and a radial upstream gradient dy = y changes only
    the norm, so its gradient vanishes up to the 1e-6 guard."""
    rng = np.random.default_rng(6)
    u = rng.standard_normal((3, 8))
    dy = rng.standard_normal((3, 8))
    g = gp.qk_norm_bwd(u, dy)
    eps = 1e-6
    for i in range(u.size):
        p, m = u.copy(), u.copy()
        p.reshape(-1)[i] += eps
        m.reshape(-1)[i] -= eps
        fd = (np.sum(gp.qk_norm_fwd(p) * dy) - np.sum(gp.qk_norm_fwd(m) * dy)) / (2 * eps)
        assert abs(fd - g.reshape(-1)[i]) <= 1e-7 * max(1.0, abs(fd))
    y = gp.qk_norm_fwd(u)
    assert np.abs(gp.qk_norm_bwd(u, y)).max() <= 1e-5
