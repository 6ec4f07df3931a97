#!/usr/bin/env python3
"""Benchmark of the Muir gated delta-rule operator on one MI355X.

One timed step = one chunkwise forward (saving chunk states) plus one
chunkwise backward over the headline workload: B=8, T=4096, H=16,
dk=dv=128, chunk 64, bf16 inputs, fp32 gradients, fp32 running state,
synthetic seeded inputs already resident in HBM.  `value` is tokens/s (B*T
per step time).

Beside it the line carries:
  roofline      the dominant kernel's algorithmic bytes per launch over its
                average duration (HIP events recorded by the library between
                its own launches, on the launch stream, inside the timed loop);
                algorithmic bytes are the operator's own inputs and outputs
                (inputs, o / dO, saved chunk states and gradients, at the
                dtypes written), never the kernels' intermediates, which show
                up only in the measured `traffic`
  kernels       the same for every kernel of the step
  step_model    the whole step's algorithmic bytes and flops over its time
  cpu_baseline  the fp64 sequential oracle on the host cores, on a bounded
                sample of the same workload (4 batch rows: 64 heads x 4096)
  secondary     the same step with bf16 gradients, the forward alone on the
                same inputs (without and with saved chunk states), the step with a
                static readout gate and with none, long-context fwd+bwd
                (T=32768, chunk 128 and 256), packed documents of mixed length
                (about 32K tokens, fwd+bwd), one 1M-token stream (chunked
                prefill chained through the state, then decode), the gate
                prologue at the layer's shape (fused low-rank gate projection
                and q / k SiLU + L2, fwd + bwd), and the streaming decode step
                (64 streams x 16 heads, 4096 steps; and a 512 MiB state)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]

`roofline.traffic` is the dominant kernel's measured HBM bytes per launch,
read from profiles/traffic_<kernel>_<workload>.json (FETCH_SIZE and WRITE_SIZE
counter runs, each scaled by the same counter over a copy of known size, see
--calib-copy); it is null when the library sources have changed since those
counters were taken (the record holds their SHA-256).
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

METRIC = "fwd+bwd tokens/s & MFMA util, H=16 d=128 T=4K/32K; decode tok/s & HBM GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Algorithmic bytes per token-head (d = head size, C = chunk; e, es, eg: bytes
# of an input, of a saved chunk-state element and of a gradient element): the
# operator's own inputs and outputs only -- the seven inputs, o, dO, the
# chunk-start states the forward saves for the backward, and the seven
# gradients, each at the dtype written.  The kernels' intermediates (chunk
# summaries, deltas, state gradients) are not counted: they appear only in
# the measured traffic, whose ratio to these bytes shows what the
# decomposition into kernels costs.
def step_bytes(d: int, C: int, e: int = 2, es: int = 2, eg: int = 4, ni: int = 7):
    """(forward, backward) algorithmic bytes per token-head: inputs ni d e, o
    d e and the saved states d^2 es / C; inputs, dO, saved states and the
    gradients ni d eg.  ni = 7 per-token inputs, or 6 when the readout gate is
    static or absent (it is then not a per-token input, nor its gradient a
    per-token output)."""
    fwd = ni * d * e + d * e + d * d * es / C
    bwd = ni * d * e + d * e + d * d * es / C + ni * d * eg
    return fwd, bwd


def kernel_bytes(d: int, C: int, e: int = 2, es: int = 2, eg: int = 4, ni: int = 7):
    """Algorithmic bytes per token-head that each kernel of the step itself
    moves: the prep kernel reads the inputs, the forward scan writes o and
    the chunk-start states, the reverse scan reads dO, and the chunk
    gradient kernel reads the inputs, dO and the states and writes the seven
    gradients (dO is counted by both backward kernels, which both read it)."""
    st = d * d * es / C
    return {"fwd_prep": ni * d * e, "fwd_scan": d * e + st, "bwd_scan": d * e,
            "bwd_chunk": ni * d * e + d * e + st + ni * d * eg}


def step_flops(d: int, C: int):
    """Algorithmic flops per token-head: forward and backward (incl. recompute)."""
    fwd = 5 * C * d + C * C / 3 + 6 * d * d
    bwd = 12 * C * d + C * C / 3 + 14 * d * d
    return fwd, bwd


HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "gated_delta_rule_muir_amd", "csrc")


# the source file that defines each measured kernel
KERNEL_SOURCE = {"fwd_prep": "fwd.hip", "fwd_scan": "scan.hip", "bwd_scan": "scan.hip",
                 "bwd_chunk": "bwd_chunk.hip", "step": "step.hip"}


def kernel_sources_sha256(kernel: str) -> str:
    """SHA-256 over the source of `kernel` and the library headers it includes,
    transitively (file names and contents, sorted by name)."""
    seen, todo = set(), [KERNEL_SOURCE[kernel]]
    while todo:
        fn = todo.pop()
        if fn in seen:
            continue
        seen.add(fn)
        with open(os.path.join(CSRC, fn)) as f:
            for inc in re.findall(r'^\s*#include\s+"([^"]+)"', f.read(), flags=re.M):
                if os.path.exists(os.path.join(CSRC, inc)):
                    todo.append(inc)
    h = hashlib.sha256()
    for fn in sorted(seen):
        h.update(fn.encode())
        with open(os.path.join(CSRC, fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """Counter-measured HBM bytes per launch of `kernel`, or None if there is
    no record or the kernel's sources changed since it was taken."""
    path = os.path.join(HERE, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_sha256") != kernel_sources_sha256(kernel):
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def calib_copy(torch, mib: int = 1024, reps: int = 3):
    """A plain elementwise copy of known size (reads and writes `mib` MiB per
    launch) whose counter readings calibrate FETCH_SIZE / WRITE_SIZE."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def gen_seq(B, T, H, d, dtype, decay, seed, torch, muir_inputs):
    inp = muir_inputs.seq_inputs(B, T, H, d, d, dtype=dtype, decay=decay, seed=seed, with_dO=True)
    return {n: (t.to("cuda") if t is not None else None) for n, t in inp.items()}, inp


def time_fwdbwd(m, dv, C, steps, warmup, torch, hiprt, names, profile=True, grad_dtype=None):
    """Run warmup + timed fwd+bwd steps; returns (ms_per_step, per-kernel avg ms).
    grad_dtype: the gradients' dtype (None: fp32)."""
    B, T, H, d = dv["q"].shape
    dev = dv["q"].device
    gcode = m.MUIR_BF16 if grad_dtype == torch.bfloat16 else m.MUIR_F32
    gam = dv["gamma"]
    gm = m.MUIR_GAMMA_NONE if gam is None else m.MUIR_GAMMA_STATIC if gam.dim() == 2 else m.MUIR_GAMMA_TOKEN
    fws = torch.empty(m.muir_chunk_fwd_workspace(B, T, H, d, d, C, gamma_mode=gm), dtype=torch.uint8, device=dev)
    bws = torch.empty(m.muir_chunk_bwd_workspace(B, T, H, d, d, C, gamma_mode=gm, grad_dtype=gcode),
                      dtype=torch.uint8, device=dev)
    args = [dv[n] for n in names]

    def step():
        o, S_T, Sc = m.muir_chunk_fwd(*args, chunk=C, save_states=True, workspace=fws)
        g = m.muir_chunk_bwd(*args, dv["dO"], S_chunks=Sc, summaries=fws, chunk=C, workspace=bws,
                             grad_dtype=grad_dtype)
        return o, g

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    per_step = 3 + 3  # events: fwd (before, prep, scan), bwd (before, bscan, bchunk)
    pool = hiprt.EventPool(per_step * steps) if profile else None
    if pool is not None:
        m.muir_set_profile_events(pool.arr, pool.n)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = None
    if pool is not None:
        rec = m.muir_profile_events_recorded()
        m.muir_set_profile_events(None)
        if rec != per_step * steps:
            raise RuntimeError(f"expected {per_step * steps} profile events, got {rec}")
        names_k = ["fwd_prep", "fwd_scan", None, "bwd_scan", "bwd_chunk"]
        acc = {k: 0.0 for k in names_k if k}
        for s in range(steps):
            base = s * per_step
            for i, kn in enumerate(names_k):
                if kn is None:
                    continue
                acc[kn] += pool.elapsed_ms(base + i, base + i + 1)
        kern = {k: v / steps for k, v in acc.items()}
        pool.close()
    return (t1 - t0) * 1e3 / steps, kern


def time_fwd(m, dv, C, steps, warmup, torch, hiprt, names, save_states):
    """Warmup + timed forward calls alone (with or without saving the chunk
    states); returns (ms_per_call, per-kernel avg ms)."""
    B, T, H, d = dv["q"].shape
    fws = torch.empty(m.muir_chunk_fwd_workspace(B, T, H, d, d, C), dtype=torch.uint8, device=dv["q"].device)
    args = [dv[n] for n in names]
    o = torch.empty_like(dv["q"])

    def call():
        m.muir_chunk_fwd(*args, chunk=C, save_states=save_states, workspace=fws, out=o)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    per = 3  # events: before, prep, scan
    pool = hiprt.EventPool(per * steps)
    m.muir_set_profile_events(pool.arr, pool.n)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rec = m.muir_profile_events_recorded()
    m.muir_set_profile_events(None)
    if rec != per * steps:
        raise RuntimeError(f"expected {per * steps} profile events, got {rec}")
    acc = {"fwd_prep": 0.0, "fwd_scan": 0.0}
    for s_ in range(steps):
        acc["fwd_prep"] += pool.elapsed_ms(s_ * per, s_ * per + 1)
        acc["fwd_scan"] += pool.elapsed_ms(s_ * per + 1, s_ * per + 2)
    pool.close()
    return (t1 - t0) * 1e3 / steps, {k: v / steps for k, v in acc.items()}


def fwd_report(kern, ms, d, C, nth, save_states, e=2, es=2):
    """The forward alone: per-kernel algorithmic bytes (kernel_bytes; the
    scan's saved states only when it saves them), the dominant kernel's
    roofline, and the forward's bytes and flops (step_bytes, step_flops)
    over its time."""
    st = d * d * es / C if save_states else 0.0
    kb = {"fwd_prep": 7 * d * e, "fwd_scan": d * e + st}
    kernels = {}
    for kn, t in kern.items():
        byt = kb[kn] * nth
        kernels[kn] = {"avg_us": t * 1e3, "alg_bytes": byt, "GBs": byt / (t * 1e-3) / 1e9,
                       "hbm_frac": byt / (t * 1e-3) / 1e9 / HBM_PEAK_GBS}
    dom = max(kern, key=lambda k: kern[k])
    roof = {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["GBs"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": kernels[dom]["GBs"] / HBM_PEAK_GBS,
            "alg_bytes_per_launch": kb[dom] * nth, "avg_launch_us": kernels[dom]["avg_us"]}
    fb = (8 * d * e + st) * nth
    ff = step_flops(d, C)[0] * nth
    t = ms * 1e-3
    model = {"alg_bytes": fb, "alg_GBs": fb / t / 1e9, "alg_flops": ff,
             "hbm_floor_us": fb / (HBM_PEAK_GBS * 1e9) * 1e6,
             "mfma_floor_us": ff / (BF16_PEAK_TFLOPS * 1e12) * 1e6,
             "frac": max(fb / (HBM_PEAK_GBS * 1e9), ff / (BF16_PEAK_TFLOPS * 1e12)) / t,
             "mfma_util_alg": ff / t / (BF16_PEAK_TFLOPS * 1e12)}
    return kernels, roof, model


def roofline_report(kern, ms, d, C, nth, workload, eg, ni=7):
    """Per-kernel and whole-step figures from the algorithmic bytes (step_bytes,
    kernel_bytes; gradients of eg bytes) of nth token-heads.  `roofline` is
    the dominant (longest) kernel's: its algorithmic bytes per launch over its
    average launch time, against the HBM peak (every kernel and the step are
    below the bf16 MFMA ridge, see step_model), plus its measured HBM traffic
    per launch when the counter record matches its sources."""
    kb = kernel_bytes(d, C, eg=eg, ni=ni)
    kernels = {}
    for kn, t in kern.items():
        byt = kb[kn] * nth
        kernels[kn] = {"avg_us": t * 1e3, "alg_bytes": byt, "GBs": byt / (t * 1e-3) / 1e9,
                       "hbm_frac": byt / (t * 1e-3) / 1e9 / HBM_PEAK_GBS}
    dom = max(kern, key=lambda k: kern[k])
    traffic = measured_traffic(dom, workload) if eg == 4 and ni == 7 else None
    roof = {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["GBs"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": kernels[dom]["GBs"] / HBM_PEAK_GBS, "traffic": traffic,
            "traffic_over_alg": None if traffic is None else traffic / (kb[dom] * nth),
            "alg_bytes_per_launch": kb[dom] * nth, "avg_launch_us": kernels[dom]["avg_us"]}
    fb, bb = step_bytes(d, C, eg=eg, ni=ni)
    fwd_f, bwd_f = step_flops(d, C)
    sb, sf = (fb + bb) * nth, (fwd_f + bwd_f) * nth
    t = ms * 1e-3
    step_model = {"alg_bytes": sb, "alg_GBs": sb / t / 1e9, "alg_flops": sf,
                  "hbm_floor_us": sb / (HBM_PEAK_GBS * 1e9) * 1e6,
                  "mfma_floor_us": sf / (BF16_PEAK_TFLOPS * 1e12) * 1e6,
                  "frac": max(sb / (HBM_PEAK_GBS * 1e9), sf / (BF16_PEAK_TFLOPS * 1e12)) / t,
                  "mfma_util_alg": sf / t / (BF16_PEAK_TFLOPS * 1e12)}
    return kernels, roof, step_model


def cpu_baseline(inp_cpu, names, torch):
    """The oracle (fwd + bwd) on a bounded sample of the workload (the first
    `rows` batch rows, all heads, full length), all host cores."""
    import oracle
    rows = 4
    sl = {n: (inp_cpu[n][:rows] if inp_cpu[n] is not None else None) for n in list(names) + ["dO"]}
    B, T, H, d = sl["q"].shape
    nproc = os.cpu_count() or 1
    try:
        nproc = len(os.sched_getaffinity(0))
    except Exception:
        pass
    threads = min(nproc, B * H)
    args = [sl[n].float().numpy() for n in names]
    dO = sl["dO"].float().numpy()
    t0 = time.perf_counter()
    oracle.fwd(*args, nthreads=threads)
    oracle.bwd(*args, dO, nthreads=threads)
    t = time.perf_counter() - t0
    return {"value": B * T / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fwd+bwd of batch rows 0..{B - 1} of the workload (B={B}, T={T}, H={H}, d={d}), fp64, "
                      f"{t:.2f} s wall on {threads} threads"}


def decode_bench(m, torch, hiprt, N=64, H=16, d=128, steps=4096, seed=0):
    """Streaming decode: `steps` consecutive muir_step calls on an fp32 state."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dev = "cuda"

    def unit(x):
        s = torch.nn.functional.silu(x)
        return s / s.norm(dim=-1, keepdim=True).clamp_min(1e-12)

    bf = torch.bfloat16
    shp = (steps, N, H, d)
    q = unit(torch.randn(shp, generator=g, device=dev)).to(bf)
    k = unit(torch.randn(shp, generator=g, device=dev)).to(bf)
    v = torch.randn(shp, generator=g, device=dev).to(bf)
    rates = torch.exp(torch.empty((H, d), device=dev).uniform_(-9.2103, 1.0986, generator=g))
    log_a = (-rates).to(bf).expand(N, H, d).contiguous()
    erase = torch.sigmoid(torch.randn(shp, generator=g, device=dev)).to(bf)
    write = torch.sigmoid(torch.randn(shp, generator=g, device=dev)).to(bf)
    gamma = (2 * torch.sigmoid(torch.randn(shp, generator=g, device=dev))).to(bf)
    S = torch.zeros((N, H, d, d), dtype=torch.float32, device=dev)
    o = torch.empty((N, H, d), dtype=bf, device=dev)
    for t in range(8):  # warmup
        m.muir_step(q[t], k[t], v[t], log_a, erase[t], write[t], gamma[t], S, out=o)
    S.zero_()
    torch.cuda.synchronize()
    pool = hiprt.EventPool(2 * steps)
    m.muir_set_profile_events(pool.arr, pool.n)
    t0 = time.perf_counter()
    for t in range(steps):
        m.muir_step(q[t], k[t], v[t], log_a, erase[t], write[t], gamma[t], S, out=o)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    m.muir_set_profile_events(None)
    kt = sum(pool.elapsed_ms(2 * i, 2 * i + 1) for i in range(steps)) / steps
    pool.close()
    wall = (t1 - t0) * 1e3 / steps
    # the same steps replayed from one captured HIP graph (as a serving loop
    # would issue them), from the same initial state: its final state must
    # equal the eager run's bit for bit
    S_eager = S.clone()
    graph = torch.cuda.CUDAGraph()
    S.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for t in range(steps):
            m.muir_step(q[t], k[t], v[t], log_a, erase[t], write[t], gamma[t], S, out=o)
    S.zero_()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    graph_ok = bool(torch.equal(S, S_eager))
    del graph, S_eager
    gwall = (t3 - t2) * 1e3 / steps
    state_bytes = 2 * N * H * d * d * 4
    in_bytes = N * H * d * 2 * 7 + N * H * d * 2
    del q, k, v, erase, write, gamma
    torch.cuda.empty_cache()
    return {"workload": f"decode N={N} H={H} d={d} fp32 state, {steps} steps",
            "tokens_per_s": N / (wall * 1e-3), "wall_us_per_step": wall * 1e3,
            "kernel_us_per_step": kt * 1e3,
            "graph_tokens_per_s": N / (gwall * 1e-3), "graph_wall_us_per_step": gwall * 1e3,
            "graph_matches_eager": graph_ok,
            "hbm_GBs_at_kernel_time": (state_bytes + in_bytes) / (kt * 1e-3) / 1e9,
            "bytes_per_step": state_bytes + in_bytes,
            "graph_hbm_GBs": (state_bytes + in_bytes) / (gwall * 1e-3) / 1e9,
            "note": ("state (%d MiB) may be served partly from the 256 MB Infinity Cache" if N * H * d * d * 4 < (256 << 20)
                     else "state (%d MiB) larger than the 256 MB Infinity Cache") % (N * H * d * d * 4 >> 20)}


def stream_bench(m, torch, muir_inputs):
    """The stream_1m workload: one stream (B=1) prefilled in segments chained
    through the state (S_T -> S0), then decode tokens from that state.  The
    segments are muir_inputs.stream_segment_torch draws, the same inputs on
    which tests/test_gpu_stream.py checks heads 0 and H-1 against the oracle;
    they are drawn on the GPU before the timed region."""
    w = muir_inputs.WORKLOADS["stream_1m"]
    H, d, chunk, seg = w.H, w.dk, w.chunk, w.extra["segment"]
    seed, steps = w.extra["seed"], w.extra["decode_steps"]
    names = ("q", "k", "v", "log_a", "erase", "write", "gamma")
    segs = []
    for i in range(w.T // seg):
        x = muir_inputs.stream_segment_torch(i, seg, H, d, d, device="cuda", decay=w.decay, seed=seed)
        segs.append([x[n] for n in names])
    x = muir_inputs.stream_segment_torch(w.T // seg, steps, H, d, d, device="cuda", decay=w.decay, seed=seed)
    dec = [[x[n][:, t].contiguous() for n in names] for t in range(steps)]
    ws = torch.empty(m.muir_chunk_fwd_workspace(1, seg, H, d, d, chunk), dtype=torch.uint8, device="cuda")
    o = torch.empty((1, seg, H, d), dtype=torch.bfloat16, device="cuda")
    m.muir_chunk_fwd(*segs[0], chunk=chunk, workspace=ws, out=o)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    S = None
    for xs in segs:
        _, S, _ = m.muir_chunk_fwd(*xs, S, chunk=chunk, workspace=ws, out=o)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    od = torch.empty((1, H, d), dtype=torch.bfloat16, device="cuda")
    for xt in dec:
        m.muir_step(*xt, S, out=od)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    del segs, dec
    torch.cuda.empty_cache()
    return {"workload": f"stream_1m: one stream, H={H} d={d}: prefill {w.T} tokens in {seg}-token segments "
                        f"(chunk {chunk}, state chained), then {steps} decode tokens",
            "prefill_tokens_per_s": w.T / (t1 - t0), "decode_us_per_token": (t2 - t1) * 1e6 / steps,
            "parity": "same inputs as tests/test_gpu_stream.py::test_stream_1m_prefill_then_decode, which checks "
                      f"heads 0 and {H - 1} against the fp64 oracle over every token"}


def varlen_bench(m, torch, muir_inputs, steps=10, warmup=3):
    """The varlen_32k workload: packed documents of mixed length (an empty
    one, one token, exact chunk multiples, one past a chunk, uniform draws up
    to 4,096 tokens), forward (keeping its chunk states) then backward
    (reusing them; fp32 gradients), timed around whole steps.  The inputs are the
    ones tests/test_gpu_fullsize.py::test_varlen_full_layer checks against the
    oracle on every document and head."""
    w = muir_inputs.WORKLOADS["varlen_32k"]
    lens = muir_inputs.varlen_lengths(w.B, w.T, w.chunk, seed=w.extra["lengths_seed"])
    inp = muir_inputs.varlen_inputs(lens, w.H, w.dk, w.dv, dtype=w.dtype, decay=w.decay, seed=w.extra["seed"])
    dv = {n: (t.to("cuda") if t is not None else None) for n, t in inp.items()}
    names = ("q", "k", "v", "log_a", "erase", "write", "gamma")
    args = [dv[n] for n in names]
    cu, L = dv["cu_seqlens"], int(lens.max())
    fws = torch.empty(m.muir_chunk_varlen_fwd_workspace(w.B, L, w.H, w.dk, w.dv, w.chunk), dtype=torch.uint8,
                      device="cuda")
    bws = torch.empty(m.muir_chunk_varlen_bwd_workspace(w.B, L, w.H, w.dk, w.dv, w.chunk), dtype=torch.uint8,
                      device="cuda")
    o = torch.empty_like(dv["v"])

    def step():
        # as the fixed-length step: the forward keeps its chunk states, the
        # backward reuses them
        m.muir_chunk_varlen_fwd(*args, cu, chunk=w.chunk, max_len=L, workspace=fws, out=o, final_state=False,
                                keep=True)
        m.muir_chunk_varlen_bwd(*args, dv["dO"], cu, chunk=w.chunk, max_len=L, workspace=bws, want_dS0=False,
                                fwd_workspace=fws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    total = int(lens.sum())
    nth = total * w.H
    fb, bb = step_bytes(w.dk, w.chunk)
    fwd_f, bwd_f = step_flops(w.dk, w.chunk)
    sb = (fb + bb) * nth
    t = ms * 1e-3
    return {"workload": f"varlen_32k: {w.B} packed documents of lengths {lens.tolist()} ({total} tokens), "
                        f"H={w.H} d={w.dk} chunk {w.chunk}, bf16 inputs, fp32 gradients; the forward keeps its chunk states "
                        f"for the backward",
            "tokens_per_s": total / t, "ms_per_step": ms,
            "step_model": {"alg_bytes": sb, "alg_GBs": sb / t / 1e9, "hbm_floor_us": sb / (HBM_PEAK_GBS * 1e9) * 1e6,
                           "frac": sb / (HBM_PEAK_GBS * 1e9) / t,
                           "mfma_util_alg": (fwd_f + bwd_f) * nth / t / (BF16_PEAK_TFLOPS * 1e12)},
            "parity": "same inputs as tests/test_gpu_fullsize.py::test_varlen_full_layer (every document and "
                      "head against the fp64 oracle)"}


def gate_bench(m, torch, hiprt, M=32768, d=2048, H=16, dk=128, dv=128, steps=10, warmup=2, seed=0):
    """The gate prologue at the layer's shape (M = B*T tokens of width d):
    fused gate projection forward + backward and the q / k SiLU + L2
    normalisation forward + backward.  bf16, random weights, inputs drawn on
    the GPU with the muir_inputs.gate_inputs recipe."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    bf = torch.bfloat16
    sw, su, sb = m.gate_param_shapes(d, H, dk, dv)
    x = torch.randn((M, d), generator=g, device="cuda").to(bf)
    W_down = (torch.randn(sw, generator=g, device="cuda") / d ** 0.5).to(bf)
    W_up = (torch.randn(su, generator=g, device="cuda") * (0.5 / 128 ** 0.5)).to(bf)
    bias = torch.randn(sb, generator=g, device="cuda").to(bf)
    dG = {n: torch.randn((M, H, D), generator=g, device="cuda").to(bf)
          for n, D in zip(m.GATE_NAMES, (dk, dk, dv, dv, dk))}
    qk = torch.randn((2, M, H, dk), generator=g, device="cuda").to(bf)
    dqk = torch.randn((2, M, H, dk), generator=g, device="cuda").to(bf)
    ws = torch.empty(m.muir_gate_proj_bwd_workspace(M, d, H, dk, dv), dtype=torch.uint8, device="cuda")

    def step():
        out = m.muir_gate_proj_fwd(x, W_down, W_up, bias, H=H, dk=dk, dv=dv)
        gr = m.muir_gate_proj_bwd(x, W_down, W_up, bias, dG, H=H, dk=dk, dv=dv, z=out["z"], workspace=ws)
        y = m.muir_qk_norm_fwd(qk)
        du = m.muir_qk_norm_bwd(qk, dqk)
        return out, gr, y, du

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    per = 8  # events: before/after each of the four calls
    pool = hiprt.EventPool(per * steps)
    m.muir_set_profile_events(pool.arr, pool.n)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rec = m.muir_profile_events_recorded()
    m.muir_set_profile_events(None)
    if rec != per * steps:
        raise RuntimeError(f"expected {per * steps} profile events, got {rec}")
    us = {k: 0.0 for k in ("proj_fwd", "proj_bwd", "qk_norm_fwd", "qk_norm_bwd")}
    for s_ in range(steps):
        for i, k in enumerate(us):
            us[k] += pool.elapsed_ms(s_ * per + 2 * i, s_ * per + 2 * i + 1) * 1e3 / steps
    pool.close()
    e = 2
    rw = 64 * H * dk * 2 + 128 * (H * dv * 2 + H * dk)  # sum over the gates of rank x width
    fwd_flops = 2 * M * d * 512 + 2 * M * rw
    bwd_flops = 3 * 2 * M * rw + 2 * 2 * M * d * 512  # pre, dz, dW_up; dx, dW_down
    gw = M * H * (3 * dk + 2 * dv) * e
    fwd_bytes = M * d * e + M * 512 * e + gw
    bwd_bytes = M * d * e + M * 512 * e + gw + M * d * e  # x, z, dG in; dx out (weight grads are small)
    qk_bytes = 5 * (2 * M * H * dk * e)  # q and k; fwd: u in, y out; bwd: u, dy in, du out
    peak_f, peak_b = BF16_PEAK_TFLOPS * 1e12, HBM_PEAK_GBS * 1e9

    def roof(fl, by, t_us):
        t = t_us * 1e-6
        floor = max(fl / peak_f, by / peak_b)
        return {"tflops": fl / t / 1e12, "alg_GBs": by / t / 1e9, "alg_flops": fl, "alg_bytes": by,
                "bound": "mfma" if fl / peak_f >= by / peak_b else "hbm", "frac": floor / t}
    res = {"workload": f"gate prologue, M={M} tokens (8 x 4096) d={d} H={H} dk={dk} dv={dv} bf16",
           "avg_us": us, "ms_per_step": (t1 - t0) * 1e3 / steps,
           "proj_fwd": roof(fwd_flops, fwd_bytes, us["proj_fwd"]),
           "proj_bwd": roof(bwd_flops, bwd_bytes, us["proj_bwd"]),
           "qk_norm": {"alg_GBs": qk_bytes / ((us["qk_norm_fwd"] + us["qk_norm_bwd"]) * 1e-6) / 1e9}}
    del x, W_down, W_up, bias, dG, qk, dqk, ws
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary", default="",
                    help="comma-separated secondary lines to run (default: all), e.g. gate_prologue_4k")
    ap.add_argument("--decode-steps", type=int, default=4096)
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run a 1 GiB elementwise copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the operator runs on one MI355X); --gpus {args.gpus} "
              "is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import muir_inputs
    import gated_delta_rule_muir_amd as m
    from gated_delta_rule_muir_amd import hiprt
    m.lib()  # fails loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    names = ("q", "k", "v", "log_a", "erase", "write", "gamma")
    if args.calib_copy:
        log("[bench] calibration copy: 3 x 1 GiB read + 1 GiB write")
        calib_copy(torch)

    wl = muir_inputs.WORKLOADS["layer_fwdbwd_4k"]
    B, T, H, d, C = wl.B, wl.T, wl.H, wl.dk, wl.chunk
    log(f"[bench] generating {wl.name} inputs B={B} T={T} H={H} d={d} C={C} {wl.dtype}")
    dv, inp_cpu = gen_seq(B, T, H, d, wl.dtype, wl.decay, 0, torch, muir_inputs)
    log(f"[bench] timing fwd+bwd: warmup={args.warmup} steps={args.steps}")
    ms, kern = time_fwdbwd(m, dv, C, args.steps, args.warmup, torch, hiprt, names)
    ntok = B * T
    nth = B * T * H
    log(f"[bench] {ms:.3f} ms/step -> {ntok / (ms * 1e-3):.4g} tokens/s")

    kernels, roof, step_model = roofline_report(kern, ms, d, C, nth, wl.name, eg=4)
    result = {
        "metric": METRIC, "value": ntok / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "dk": d, "dv": d, "chunk": C,
                   "inputs": "bf16, seeded (muir_inputs), per-channel decay rates 1e-4..3",
                   "gradients": "fp32", "saved_chunk_states": "bf16", "running_state": "fp32",
                   "step": "muir_chunk_fwd (saving chunk states; its workspace keeps the chunk "
                           "summaries) + muir_chunk_bwd (reusing both), fp32 gradients"},
        "roofline": roof,
        "kernels": kernels,
        "step_model": step_model,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) on one batch row ...")
        result["cpu_baseline"] = cpu_baseline(inp_cpu, names, torch)
        log(f"[bench] cpu baseline {result['cpu_baseline']['value']:.4g} tokens/s")
    del inp_cpu
    if not args.no_secondary:
        sec = {}
        chosen = set(filter(None, args.secondary.split(",")))
        want = lambda name: not chosen or name in chosen  # noqa: E731
        if want("layer_fwdbwd_4k_bf16grads"):
            log("[bench] secondary: the same step with bf16 gradients")
            ms2, k2 = time_fwdbwd(m, dv, C, max(5, args.steps // 2), 2, torch, hiprt, names,
                                  grad_dtype=torch.bfloat16)
            kern2, roof2, sm2 = roofline_report(k2, ms2, d, C, nth, wl.name, eg=2)
            sec["layer_fwdbwd_4k_bf16grads"] = {"tokens_per_s": ntok / (ms2 * 1e-3), "ms_per_step": ms2,
                                                 "gradients": "bf16", "kernels": kern2, "roofline": roof2,
                                                 "step_model": sm2}
            log(f"[bench]   {ntok / (ms2 * 1e-3):.4g} tokens/s")
        if want("layer_fwd_4k"):
            # the forward alone at the same shape and inputs: as a prefill or
            # inference pass (no chunk states kept), and as a training forward
            log("[bench] secondary: the forward alone (without and with saved chunk states)")
            line = {"workload": "layer_fwd_4k: B=8 T=4096 H=16 d=128 chunk 64, bf16 inputs, fp32 state; "
                                "muir_chunk_fwd alone on the step's inputs"}
            # one untimed round of both forms first: the first timed round after
            # the step measured up to 10% slower, in both orders
            for save in (False, True):
                time_fwd(m, dv, C, 10, 3, torch, hiprt, names, save)
            for key, save in (("no_saved_states", False), ("saved_states", True)):
                ms3, k3 = time_fwd(m, dv, C, max(10, args.steps), 3, torch, hiprt, names, save)
                kern3, roof3, fm3 = fwd_report(k3, ms3, d, C, nth, save)
                line[key] = {"tokens_per_s": ntok / (ms3 * 1e-3), "ms_per_call": ms3, "kernels": kern3,
                             "roofline": roof3, "fwd_model": fm3}
                log(f"[bench]   {key}: {ntok / (ms3 * 1e-3):.4g} tokens/s ({ms3:.3f} ms)")
            sec["layer_fwd_4k"] = line
        if want("gamma_forms_4k"):
            # the step with a static readout gate (one [H, dk] vector) and with
            # none, on the same inputs otherwise
            log("[bench] secondary: the step with a static readout gate and with none")
            line = {"workload": "gamma_forms_4k: the layer_fwdbwd_4k step with the readout gate static "
                                "(gamma of token 0 of batch row 0, [H, dk]) or absent; fp32 gradients"}
            for key, gam in (("static", dv["gamma"][0, 0].contiguous()), ("none", None)):
                dvg = dict(dv)
                dvg["gamma"] = gam
                ms4, k4 = time_fwdbwd(m, dvg, C, max(10, args.steps // 2), 3, torch, hiprt, names)
                kern4, roof4, sm4 = roofline_report(k4, ms4, d, C, nth, f"gamma_{key}_4k", eg=4, ni=6)
                line[key] = {"tokens_per_s": ntok / (ms4 * 1e-3), "ms_per_step": ms4, "kernels": kern4,
                             "roofline": roof4, "step_model": sm4}
                log(f"[bench]   {key}: {ntok / (ms4 * 1e-3):.4g} tokens/s ({ms4:.3f} ms)")
            sec["gamma_forms_4k"] = line
        del dv
        torch.cuda.empty_cache()
        for name in ("long_32k_c128", "long_32k_c256"):
            if not want(name):
                continue
            w = muir_inputs.WORKLOADS[name]
            log(f"[bench] secondary {name}")
            dv2, _ = gen_seq(w.B, w.T, w.H, w.dk, w.dtype, w.decay, 0, torch, muir_inputs)
            ms2, k2 = time_fwdbwd(m, dv2, w.chunk, 5, 2, torch, hiprt, names)
            kern2, roof2, sm2 = roofline_report(k2, ms2, w.dk, w.chunk, w.B * w.T * w.H, w.name, eg=4)
            sec[name] = {"tokens_per_s": w.B * w.T / (ms2 * 1e-3), "ms_per_step": ms2, "gradients": "fp32",
                         "kernels": kern2, "roofline": roof2, "step_model": sm2}
            log(f"[bench]   {sec[name]['tokens_per_s']:.4g} tokens/s")
            del dv2
            torch.cuda.empty_cache()
        if want("varlen_32k"):
            log("[bench] secondary varlen_32k (packed documents of mixed length, fwd+bwd)")
            sec["varlen_32k"] = varlen_bench(m, torch, muir_inputs)
            log(f"[bench]   {sec['varlen_32k']['tokens_per_s']:.4g} tokens/s ({sec['varlen_32k']['ms_per_step']:.3f} ms)")
            torch.cuda.empty_cache()
        if want("stream_1m"):
            log("[bench] secondary stream (1M-token prefill, then decode)")
            sec["stream_1m"] = stream_bench(m, torch, muir_inputs)
            log(f"[bench]   prefill {sec['stream_1m']['prefill_tokens_per_s']:.4g} tokens/s, "
                f"decode {sec['stream_1m']['decode_us_per_token']:.1f} us/token")
        if want("gate_prologue_4k"):
            log("[bench] secondary gate prologue (fused gate projection + q/k SiLU-L2, fwd+bwd)")
            sec["gate_prologue_4k"] = gate_bench(m, torch, hiprt)
            gpb = sec["gate_prologue_4k"]
            log(f"[bench]   proj fwd {gpb['avg_us']['proj_fwd']:.1f} us ({gpb['proj_fwd']['tflops']:.0f} TFLOP/s), "
                f"bwd {gpb['avg_us']['proj_bwd']:.1f} us ({gpb['proj_bwd']['tflops']:.0f} TFLOP/s)")
        if want("decode_64x16"):
            log(f"[bench] secondary decode ({args.decode_steps} steps)")
            sec["decode_64x16"] = decode_bench(m, torch, hiprt, steps=args.decode_steps)
            log(f"[bench]   {sec['decode_64x16']['kernel_us_per_step']:.2f} us/step kernel")
        if want("decode_512x16"):
            # the same step on a 512 MiB state, which the 256 MB Infinity Cache cannot hold
            log("[bench] secondary decode, 512 streams (512 MiB state), 256 steps")
            sec["decode_512x16"] = decode_bench(m, torch, hiprt, N=512, steps=256)
            log(f"[bench]   {sec['decode_512x16']['kernel_us_per_step']:.2f} us/step kernel, "
                f"{sec['decode_512x16']['graph_wall_us_per_step']:.2f} us/step graph")
        result["secondary"] = sec
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
