"""The no-allocation forward (muir_chunk_fwd_noalloc): called through the C
ABI, its results equal muir_chunk_fwd's bit for bit (the same kernels on the
same inputs; only the workspace differs), on calls in a row that reuse the
one scratch array -- each smaller than the one before, the last with a
partial chunk (staged in the scratch) -- and it refuses work beyond its fixed
scratch with MUIR_ERR_SCRATCH."""
import sys

import pytest
import torch

import muir_inputs
from gpu_util import NAMES, to_dev

pytestmark = pytest.mark.gpu

CALLS = [
    # B, T, H, d, C, dtype, decay, S0 scale, gate form
    (2, 1024, 16, 128, 64, "bf16", "channel", 0.1, "token"),    # 76 MiB of the 128 MiB scratch
    (1, 300, 4, 128, 128, "bf16", "channel_slow", 0.1, "token"),  # partial last chunk: staged
    (1, 130, 2, 64, 64, "f32", "uniform", 0.0, "static"),
]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_noalloc_forward_equals_the_workspace_forward():
    import gated_delta_rule_muir_amd as m
    m.lib()
    for i, (B, T, H, d, C, dtype, decay, s0, form) in enumerate(CALLS):
        _say(f"noalloc call {i}: B={B} T={T} H={H} d={d} C={C} {dtype} gate={form}")
        need = m.muir_chunk_fwd_workspace(B, T, H, d, d, C, m.MUIR_BF16 if dtype == "bf16" else m.MUIR_F32,
                                          m.MUIR_GAMMA_STATIC if form == "static" else m.MUIR_GAMMA_TOKEN)
        assert 0 < need <= m.NOALLOC_SCRATCH_BYTES
        inp = to_dev(muir_inputs.seq_inputs(B, T, H, d, d, dtype=dtype, decay=decay, seed=40 + i, S0_scale=s0))
        if form == "static":
            inp["gamma"] = inp["gamma"][0, 0].contiguous()
        args = [inp[n] for n in NAMES]
        ref = m.muir_chunk_fwd(*args, inp["S0"], chunk=C, save_states=True)
        got = m.muir_chunk_fwd_noalloc(*args, inp["S0"], chunk=C, save_states=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "S_T", "S_chunks"), got, ref):
            assert torch.equal(a, b), (i, name)


def test_noalloc_forward_refuses_work_beyond_the_scratch():
    import gated_delta_rule_muir_amd as m
    m.lib()
    B, T, H, d = 1, 8192, 16, 128
    assert m.muir_chunk_fwd_workspace(B, T, H, d, d, 64) > m.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((B, T, H, d), dtype=torch.bfloat16, device="cuda")
    o = torch.full((B, T, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MuirError) as e:
        m.muir_chunk_fwd_noalloc(x, x, x, x, x, x, x, chunk=64, out=o)
    assert e.value.code == 8  # MUIR_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())  # nothing was launched
