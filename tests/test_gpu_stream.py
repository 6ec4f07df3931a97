"""Long streams through the state contract: chunked prefill, then decode.

test_stream_1m_prefill_then_decode: the `stream_1m` workload (bench.py's
stream line, same inputs): one stream of 1,048,576 tokens with 16 heads
(d=128, bf16, chunk 64) prefilled in 32K-token segments chained through the
fp32 state, then 64 decode tokens.  Heads 0 and 15 are followed by the fp64
oracle segment by segment (its own state chained the same way, which is the
plain recurrence over the whole stream): o of every token, the state after
the prefill, every decode output and the final state, each within 2e-2.

test_chunked_prefill_then_decode_256k:

A 256K-token sequence (B=1, H=2, d=128, bf16, chunk 64) is run through
muir_chunk_fwd in 32K-token segments, each segment starting from the
previous segment's final state (S_T -> S0).  The stream then continues with
64 muir_step decode tokens from that state (abstract: constant-memory
inference; the fp32 state is the whole context).

Checks:
  * every chained segment matches the same tokens of one call over the whole
    sequence (o and the final state) within the bf16 tolerance: with two heads
    both calls split their state scan into segments, at different places, so
    the rounding differs;
  * head 0 against the fp64 oracle, sequentially over all 256K + 64 tokens:
    o of every prefill token, the state after the prefill, every decode
    output and the final state, each within 2e-2 (max |gpu - oracle| / max |oracle|).
"""
import sys

import numpy as np
import pytest
import torch

import muir_inputs
import oracle
from gpu_util import NAMES, SEQ_AXES, STATE_AXES, STEP_AXES, err2, rel_err

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_chunked_prefill_then_decode_256k():
    import gated_delta_rule_muir_amd as m
    m.lib()
    B, T, H, d, C, SEG = 1, 262144, 2, 128, 64, 32768
    STEPS = 64
    _say(f"[stream] inputs B={B} T={T} H={H} d={d}")
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype="bf16", decay="channel_slow", seed=21)
    dv = {n: inp[n].to("cuda") for n in NAMES}

    o_full, S_full, _ = m.muir_chunk_fwd(*(dv[n] for n in NAMES), chunk=C)
    S = None
    ws = torch.empty(m.muir_chunk_fwd_workspace(B, SEG, H, d, d, C), dtype=torch.uint8, device="cuda")
    for s0 in range(0, T, SEG):
        seg = {n: dv[n][:, s0:s0 + SEG].contiguous() for n in NAMES}
        o_seg, S, _ = m.muir_chunk_fwd(*(seg[n] for n in NAMES), S, chunk=C, workspace=ws)
        e = rel_err(o_seg, o_full[:, s0:s0 + SEG])
        assert e <= TOL, (s0, e)
    e = rel_err(S, S_full)
    assert e <= TOL, e
    _say("[stream] chained segments match the single call")

    rates = muir_inputs.step_rates(H, d, seed=21)
    steps = [muir_inputs.step_inputs(B, H, d, d, t, rates=rates, dtype="bf16", seed=21) for t in range(STEPS)]
    Sg = S.clone()
    o_dec = []
    for t in range(STEPS):
        si = {n: steps[t][n].to("cuda") for n in NAMES}
        o_dec.append(m.muir_step(*(si[n] for n in NAMES), Sg).cpu())
    torch.cuda.synchronize()

    # oracle, head 0, the whole stream
    h = 0
    sl = {n: inp[n][:, :, h:h + 1] for n in NAMES}
    _say("[stream] oracle prefill (head 0) ...")
    o_ref, S_ref = oracle.fwd(*(sl[n] for n in NAMES))
    errs = {"o_prefill": rel_err(o_full[:, :, h:h + 1], o_ref), "S_prefill": rel_err(S[:, h:h + 1], S_ref)}
    Sr = S_ref
    worst = 0.0
    for t in range(STEPS):
        st = {n: steps[t][n][:, h:h + 1] for n in NAMES}
        o_r, Sr = oracle.step(*(st[n] for n in NAMES), Sr)
        worst = max(worst, rel_err(o_dec[t][:, h:h + 1], o_r))
    errs["o_decode"] = worst
    errs["S_final"] = rel_err(Sg[:, h:h + 1], Sr)
    _say("[stream] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= TOL, (k_, v_)


def test_stream_1m_prefill_then_decode():
    import gated_delta_rule_muir_amd as m
    m.lib()
    w = muir_inputs.WORKLOADS["stream_1m"]
    H, d, C, seg = w.H, w.dk, w.chunk, w.extra["segment"]
    seed, steps = w.extra["seed"], w.extra["decode_steps"]
    nseg = w.T // seg
    heads = [0, H - 1]
    _say(f"[stream_1m] T={w.T} H={H} d={d} chunk={C}: {nseg} segments of {seg}, then {steps} decode tokens")
    ws = torch.empty(m.muir_chunk_fwd_workspace(1, seg, H, d, d, C), dtype=torch.uint8, device="cuda")
    S = None
    S_ref = None
    worst = 0.0
    for i in range(nseg):
        x = muir_inputs.stream_segment_torch(i, seg, H, d, d, device="cuda", decay=w.decay, seed=seed)
        o, S, _ = m.muir_chunk_fwd(*(x[n] for n in NAMES), S, chunk=C, workspace=ws)
        sl = {n: x[n][:, :, heads].cpu() for n in NAMES}
        o_h = o[:, :, heads].cpu()
        o_ref, S_ref = oracle.fwd(*(sl[n] for n in NAMES), S0=S_ref)
        e = err2(o_h, o_ref, SEQ_AXES)
        worst = max(worst, e)
        if i % 8 == 7 or i == nseg - 1:
            _say(f"[stream_1m] {(i + 1) * seg} tokens: o worst so far {worst:.2e}")
        assert e <= TOL, (i, e)
    e_s = err2(S[:, heads].cpu(), S_ref, STATE_AXES)
    _say(f"[stream_1m] state after the prefill: {e_s:.2e}")
    assert e_s <= TOL
    x = muir_inputs.stream_segment_torch(nseg, steps, H, d, d, device="cuda", decay=w.decay, seed=seed)
    worst_d = 0.0
    for t in range(steps):
        xt = {n: x[n][:, t].contiguous() for n in NAMES}  # [1, H, D]
        od = m.muir_step(*(xt[n] for n in NAMES), S)
        o_r, S_ref = oracle.step(*(xt[n][:, heads].cpu() for n in NAMES), S_ref)
        worst_d = max(worst_d, err2(od[:, heads].cpu(), o_r, STEP_AXES))
    torch.cuda.synchronize()
    e_f = err2(S[:, heads].cpu(), S_ref, STATE_AXES)
    _say(f"[stream_1m] decode o worst {worst_d:.2e}, final state {e_f:.2e}")
    assert worst_d <= TOL and e_f <= TOL
