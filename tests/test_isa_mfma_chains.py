"""Static check of the compiled kernels (gfx950 ISA, no GPU needed): no MFMA
takes as its accumulator input the result of a recent MFMA of the other
shape (a 16x16x32 bf16 result read by a 16x16x16 product, or the reverse)
at a shifted register range -- the accumulator only partly the producer's
result, or the consumer's own destination partly on the accumulator.  Such a pair -- emitted by
the register allocator when chains of the two shapes interleave -- gave
wrong results on hardware with no wait inserted between them; pairs of one
shape are handled and pass every parity test."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_muir_amd", "csrc")
SOURCES = ["fwd.hip", "scan.hip", "bwd_chunk.hip", "gate_proj.hip", "step.hip"]
WINDOW = 24  # instructions (s_nop counts its wait states)
WRITERS = ("v_", "ds_read", "global_load", "buffer_load", "flat_load", "scratch_load", "ds_bpermute")
NON_WRITERS = ("v_cmp", "v_readfirstlane", "v_readlane", "v_writelane")


def _range(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok) or re.match(r"([va])(\d+)()$", tok)
    if not m:
        return None
    lo = int(m.group(2))
    return m.group(1), lo, int(m.group(3)) if m.group(3) else lo


def _mixed_pairs(asm: str):
    found, last, n = [], {}, 0
    for line in asm.splitlines():
        if re.match(r"^\S+:", line):
            if line.startswith("_Z"):
                last, n = {}, 0
            continue
        s = line.strip()
        if not s or s.startswith((".", ";")):
            continue
        op, _, rest = s.partition(" ")
        ops = [o.strip() for o in rest.split(",")] if rest else []
        n += 1 + (int(ops[0]) if op == "s_nop" and ops else 0)
        if op.startswith("v_mfma") and len(ops) > 3:
            c, d = _range(ops[3]), _range(ops[0])
            # the product's own destination shifted against its accumulator
            shifted = bool(c and d and c[0] == d[0] and c != d and not (d[2] < c[1] or c[2] < d[1]))
            for r in range(c[1], c[2] + 1) if c else ():
                w = last.get((c[0], r))
                if w and n - w[0] <= WINDOW and w[2] != op and (w[1] != c or shifted):
                    found.append(f"{s}  <- {w[2]} {w[1]} {n - w[0]} instructions back")
                    break
        if op.startswith(WRITERS) and not op.startswith(NON_WRITERS) and ops:
            d = _range(ops[0])
            for r in range(d[1], d[2] + 1) if d else ():
                last[(d[0], r)] = (n, d, op) if op.startswith("v_mfma") else None
    return found


def _asm(src: str) -> str:
    cmd = ["hipcc", "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-munsafe-fp-atomics", os.path.join(CSRC, src), "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not installed")
def test_no_mixed_shape_accumulator_pairs():
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        asms = dict(zip(SOURCES, ex.map(_asm, SOURCES)))
    bad = {src: _mixed_pairs(a) for src, a in asms.items()}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, bad


def test_checker_flags_a_mixed_pair():
    """The checker itself, on a hand-written sequence of the failing form."""
    asm = "\n".join([
        "_Zkernel:",
        "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[38:41], v[42:45], 0",
        "\tv_mov_b32_e32 v40, v50",
        "\tv_mfma_f32_16x16x16_bf16 v[2:5], v[50:51], v[42:43], v[0:3]",
        "\tv_mfma_f32_16x16x32_bf16 v[8:11], v[38:41], v[42:45], v[8:11]",
        "\tv_mfma_f32_16x16x32_bf16 v[10:13], v[38:41], v[42:45], v[8:11]",  # one shape: allowed
    ])
    found = _mixed_pairs(asm)
    assert len(found) == 1 and "v[2:5]" in found[0]
