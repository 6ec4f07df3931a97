"""C ABI checks that run without a GPU: the library loads, exports every
function include/muir.h declares, and rejects bad arguments with the
documented status before launching anything (only invalid calls are made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muir.h")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_WORKSPACE, ERR_ALIGN, ERR_HIP, ERR_MODE, ERR_SCRATCH, ERR_NONFINITE = range(10)


def _lib():
    import gated_delta_rule_muir_amd as m
    if not os.path.exists(m.library_path()):
        pytest.skip("libmuir.so not built")
    return m, m.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muir_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("muir_chunk_fwd", "muir_chunk_bwd", "muir_step", "muir_chunk_fwd_workspace",
              "muir_chunk_bwd_workspace", "muir_chunk_varlen_fwd", "muir_chunk_varlen_bwd",
              "muir_chunk_varlen_fwd_workspace", "muir_chunk_varlen_bwd_workspace",
              "muir_status_string", "muir_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    _, L = _lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings_cover_every_code():
    _, L = _lib()
    seen = set()
    for code in range(10):
        s = L.muir_status_string(code).decode()
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 10
    assert L.muir_status_string(99).decode() == "unknown status"
    assert L.muir_abi_version() == 10


def _dims(m, B=1, T=128, H=2, dk=64, dv=64, chunk=64, dtype=1, gamma_mode=0, grad_dtype=0):
    return m._Dims(B, T, H, dk, dv, chunk, dtype, gamma_mode, grad_dtype)


FAKE = [ctypes.c_void_p(0x10000 + 0x1000 * i) for i in range(16)]  # aligned, never dereferenced


def _fwd(m, L, d, ptrs=None, ws=FAKE[12], ws_bytes=1 << 40):
    p = list(FAKE[:7]) if ptrs is None else ptrs
    return L.muir_chunk_fwd(ctypes.byref(d) if d is not None else None, *p, None, FAKE[7], None, None,
                            ws, ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), ERR_DTYPE),
    (dict(dk=64, dv=128), ERR_SHAPE),  # dk != dv
    (dict(dk=96, dv=96), ERR_SHAPE),
    (dict(chunk=32), ERR_SHAPE),
    (dict(B=-1), ERR_SHAPE),
    (dict(gamma_mode=3), ERR_MODE),
    (dict(gamma_mode=-1), ERR_MODE),
])
def test_fwd_rejects_bad_sizes(kw, code):
    m, L = _lib()
    assert _fwd(m, L, _dims(m, **kw)) == code
    assert L.muir_chunk_fwd_workspace(ctypes.byref(_dims(m, **kw))) == 0


def test_fwd_rejects_null_misaligned_and_small_workspace():
    m, L = _lib()
    d = _dims(m)
    assert _fwd(m, L, None) == ERR_NULL
    p = list(FAKE[:7])
    p[3] = None
    assert _fwd(m, L, d, ptrs=p) == ERR_NULL
    p = list(FAKE[:7])
    p[2] = ctypes.c_void_p(0x10008)
    assert _fwd(m, L, d, ptrs=p) == ERR_ALIGN
    need = L.muir_chunk_fwd_workspace(ctypes.byref(d))
    assert need > 0
    assert _fwd(m, L, d, ws_bytes=need - 1) == ERR_WORKSPACE
    assert _fwd(m, L, d, ws=None) == ERR_WORKSPACE
    # the readout gate is required unless the gate is absent
    p = list(FAKE[:7])
    p[6] = None
    assert _fwd(m, L, d, ptrs=p) == ERR_NULL
    assert _fwd(m, L, _dims(m, gamma_mode=1), ptrs=p) == ERR_NULL
    dn = _dims(m, gamma_mode=2)
    assert _fwd(m, L, dn, ptrs=p, ws_bytes=L.muir_chunk_fwd_workspace(ctypes.byref(dn)) - 1) == ERR_WORKSPACE


def test_bwd_rejects_bad_arguments():
    m, L = _lib()
    d = _dims(m)
    need = L.muir_chunk_bwd_workspace(ctypes.byref(d))
    assert need > L.muir_chunk_fwd_workspace(ctypes.byref(d))

    def call(dd, grads=None, ws_bytes=1 << 40, summaries=None):
        g = list(FAKE[:7]) if grads is None else grads
        return L.muir_chunk_bwd(ctypes.byref(dd), *FAKE[:7], None, None, summaries, FAKE[8], None, *g,
                                None, FAKE[12], ctypes.c_size_t(ws_bytes), None)
    assert call(_dims(m, chunk=48)) == ERR_SHAPE
    g = list(FAKE[:7])
    g[5] = None
    assert call(d, grads=g) == ERR_NULL
    assert call(d, ws_bytes=need - 1) == ERR_WORKSPACE
    assert call(d, summaries=ctypes.c_void_p(FAKE[8].value + 8)) == ERR_ALIGN
    # dgamma (the seventh gradient) is required unless the gate is absent
    g = list(FAKE[:7])
    g[6] = None
    assert call(d, grads=g) == ERR_NULL
    assert call(_dims(m, gamma_mode=1), grads=g) == ERR_NULL
    dn = _dims(m, gamma_mode=2)
    assert call(dn, grads=g, ws_bytes=L.muir_chunk_bwd_workspace(ctypes.byref(dn)) - 1) == ERR_WORKSPACE


def test_gradient_dtype_is_checked_and_sized():
    """Per-token gradients are fp32 (grad_dtype 0, the zero-initialised
    default) or, for bf16 inputs only, bf16; anything else is a dtype error.
    A staged (partial-chunk) backward sizes its gradient copies by that type."""
    m, L = _lib()
    for kw in (dict(dtype=0, grad_dtype=1), dict(grad_dtype=2), dict(grad_dtype=-1)):
        assert L.muir_chunk_bwd_workspace(ctypes.byref(_dims(m, **kw))) == 0, kw
        assert L.muir_chunk_varlen_bwd_workspace(ctypes.byref(_dims(m, **kw))) == 0, kw
        dd = _dims(m, **kw)
        assert L.muir_chunk_bwd(ctypes.byref(dd), *FAKE[:7], None, None, None, FAKE[8], None, *FAKE[:7],
                                None, FAKE[12], ctypes.c_size_t(1 << 40), None) == ERR_DTYPE
    assert m._Dims().grad_dtype == 0
    for T in (128, 100):
        f32 = L.muir_chunk_bwd_workspace(ctypes.byref(_dims(m, T=T, grad_dtype=0)))
        b16 = L.muir_chunk_bwd_workspace(ctypes.byref(_dims(m, T=T, grad_dtype=1)))
        assert f32 > 0 and b16 > 0
        # whole chunks: no staging, same workspace; a tail stages the gradients
        assert (f32 == b16) if T == 128 else (f32 > b16)
    # the forward ignores it (fp32 inputs with a bf16 gradient code are fine there)
    assert L.muir_chunk_fwd_workspace(ctypes.byref(_dims(m, dtype=0, grad_dtype=1))) > 0
    assert (L.muir_chunk_fwd_workspace(ctypes.byref(_dims(m, T=100, grad_dtype=0))) ==
            L.muir_chunk_fwd_workspace(ctypes.byref(_dims(m, T=100, grad_dtype=1))))


def test_noalloc_fwd_checks_before_touching_the_gpu():
    """The no-allocation forward rejects work beyond its fixed scratch
    (MUIR_NOALLOC_SCRATCH_BYTES) and bad arguments before any HIP call."""
    m, L = _lib()
    text = open(HEADER).read()
    assert re.search(r"#define MUIR_NOALLOC_SCRATCH_BYTES \(\(size_t\)128 << 20\)", text)
    assert m.NOALLOC_SCRATCH_BYTES == 128 << 20

    def call(dd, ptrs=None):
        p = list(FAKE[:7]) if ptrs is None else ptrs
        return L.muir_chunk_fwd_noalloc(ctypes.byref(dd) if dd is not None else None, *p, None, FAKE[7], None,
                                        None, None)
    big = _dims(m, B=1, T=65536, H=16, dk=128, dv=128)
    assert L.muir_chunk_fwd_workspace(ctypes.byref(big)) > m.NOALLOC_SCRATCH_BYTES
    assert call(big) == ERR_SCRATCH
    fits = _dims(m, B=1, T=2048, H=16, dk=128, dv=128)
    assert 0 < L.muir_chunk_fwd_workspace(ctypes.byref(fits)) <= m.NOALLOC_SCRATCH_BYTES
    assert call(None) == ERR_NULL
    assert call(_dims(m, dtype=4)) == ERR_DTYPE
    assert call(_dims(m, chunk=32)) == ERR_SHAPE
    p = list(FAKE[:7])
    p[1] = None
    assert call(fits, ptrs=p) == ERR_NULL
    p[1] = ctypes.c_void_p(0x10008)
    assert call(fits, ptrs=p) == ERR_ALIGN


def test_check_values_rejects_bad_arguments():
    m, L = _lib()
    chk = L.muir_check_values
    assert chk(10, 3, FAKE[0], 0, FAKE[1], None) == ERR_DTYPE
    assert chk(-1, 1, FAKE[0], 0, FAKE[1], None) == ERR_SHAPE
    assert chk(0, 1, None, 0, None, None) == OK  # nothing to check, nothing launched
    assert chk(10, 1, None, 0, FAKE[1], None) == ERR_NULL
    assert chk(10, 1, FAKE[0], 1, None, None) == ERR_NULL
    assert chk(10, 0, ctypes.c_void_p(0x10002), 0, FAKE[1], None) == ERR_ALIGN  # fp32 needs 4-byte alignment
    assert chk(10, 1, FAKE[0], 0, ctypes.c_void_p(0x10002), None) == ERR_ALIGN


def test_step_rejects_bad_arguments():
    m, L = _lib()
    step = L.muir_step
    args = list(FAKE[:7]) + [FAKE[7], FAKE[8], None]
    assert step(2, 2, 96, 128, 1, 0, *args) == ERR_SHAPE
    assert step(2, 2, 128, 100, 1, 0, *args) == ERR_SHAPE
    assert step(2, 2, 128, 128, 3, 0, *args) == ERR_DTYPE
    assert step(2, 2, 128, 128, 1, 5, *args) == ERR_MODE
    assert step(0, 2, 128, 128, 1, 0, *args) == OK  # nothing to do, nothing launched
    bad = list(args)
    bad[7] = None
    assert step(2, 2, 128, 128, 1, 0, *bad) == ERR_NULL
    bad = list(args)
    bad[0] = ctypes.c_void_p(0x10004)
    assert step(2, 2, 128, 128, 1, 0, *bad) == ERR_ALIGN
    bad = list(args)
    bad[6] = None  # gamma
    assert step(2, 2, 128, 128, 1, 0, *bad) == ERR_NULL
    assert step(2, 2, 128, 128, 1, 1, *bad) == ERR_NULL


def test_profile_event_registration():
    m, L = _lib()
    assert L.muir_set_profile_events(None, 4) == ERR_NULL
    assert L.muir_set_profile_events(None, 0) == OK
    assert L.muir_profile_events_recorded() == 0


def test_workspace_sizes_scale_with_work():
    m, L = _lib()
    a = L.muir_chunk_fwd_workspace(ctypes.byref(_dims(m, B=1, T=256)))
    b = L.muir_chunk_fwd_workspace(ctypes.byref(_dims(m, B=2, T=256)))
    assert b == 2 * a and a % 256 == 0
    assert L.muir_chunk_fwd_workspace(ctypes.byref(_dims(m, T=0))) == 0 or True


def test_partial_chunk_needs_a_staging_area():
    """A T that ends inside a chunk is accepted; its workspace holds the
    padded shape's workspace plus zero-padded copies of the sequences."""
    m, L = _lib()
    for fn in (L.muir_chunk_fwd_workspace, L.muir_chunk_bwd_workspace):
        whole = fn(ctypes.byref(_dims(m, T=128)))
        tail = fn(ctypes.byref(_dims(m, T=100)))
        assert whole > 0 and tail > whole
    d = _dims(m, T=100)
    need = L.muir_chunk_fwd_workspace(ctypes.byref(d))
    assert _fwd(m, L, d, ws_bytes=need - 1) == ERR_WORKSPACE
    # the packed entry points size for B documents of at most dims.T tokens
    # each, as one packed sequence of B ceil(T / C) chunks with a staging copy
    # of every sequence tensor: the size depends on T only through ceil(T / C),
    # holds a staging area even for whole chunks, and grows with B
    for fv, fd in ((L.muir_chunk_varlen_fwd_workspace, L.muir_chunk_fwd_workspace),
                   (L.muir_chunk_varlen_bwd_workspace, L.muir_chunk_bwd_workspace)):
        assert fv(ctypes.byref(_dims(m, B=3, T=100))) == fv(ctypes.byref(_dims(m, B=3, T=128)))
        assert fv(ctypes.byref(_dims(m, B=3, T=128))) > fd(ctypes.byref(_dims(m, B=3, T=128)))
        assert fv(ctypes.byref(_dims(m, B=4, T=128))) > fv(ctypes.byref(_dims(m, B=3, T=128)))
        assert fv(ctypes.byref(_dims(m, chunk=48))) == 0


def test_varlen_rejects_bad_arguments():
    m, L = _lib()
    d = _dims(m, B=3, T=100)
    fneed = L.muir_chunk_varlen_fwd_workspace(ctypes.byref(d))
    bneed = L.muir_chunk_varlen_bwd_workspace(ctypes.byref(d))

    def fwd(dd, cu=FAKE[13], ptrs=None, ws_bytes=1 << 40):
        p = list(FAKE[:7]) if ptrs is None else ptrs
        return L.muir_chunk_varlen_fwd(ctypes.byref(dd) if dd is not None else None, cu, *p, None, FAKE[7],
                                       None, 0, FAKE[12], ctypes.c_size_t(ws_bytes), None)

    def bwd(dd, cu=FAKE[13], grads=None, ws_bytes=1 << 40, fws=None):
        g = list(FAKE[:7]) if grads is None else grads
        return L.muir_chunk_varlen_bwd(ctypes.byref(dd), cu, *FAKE[:7], None, FAKE[8], None, *g, None, fws,
                                       FAKE[12], ctypes.c_size_t(ws_bytes), None)
    assert fwd(None) == ERR_NULL
    assert fwd(d, cu=None) == ERR_NULL
    assert bwd(d, cu=None) == ERR_NULL
    assert fwd(_dims(m, B=3, T=100, dtype=7)) == ERR_DTYPE
    assert fwd(_dims(m, B=3, T=100, gamma_mode=4)) == ERR_MODE
    assert bwd(_dims(m, B=3, T=100, chunk=32)) == ERR_SHAPE
    assert fwd(d, ws_bytes=fneed - 1) == ERR_WORKSPACE
    assert bwd(d, ws_bytes=bneed - 1) == ERR_WORKSPACE
    p = list(FAKE[:7])
    p[4] = ctypes.c_void_p(0x10004)
    assert fwd(d, ptrs=p) == ERR_ALIGN
    g = list(FAKE[:7])
    g[0] = None
    assert bwd(d, grads=g) == ERR_NULL
    # a forward workspace to reuse must be 16-byte aligned like the others
    assert bwd(d, fws=ctypes.c_void_p(0x10004)) == ERR_ALIGN


def _gdims(m, M=256, d=128, H=2, dk=64, dv=64, dtype=1):
    return m._GateDims(M, d, H, dk, dv, dtype)


def test_gate_proj_rejects_bad_arguments():
    m, L = _lib()
    fwd = lambda dd, p: L.muir_gate_proj_fwd(ctypes.byref(dd) if dd is not None else None, *p, None)
    p = list(FAKE[:10])
    assert fwd(None, p) == ERR_NULL
    assert fwd(_gdims(m, dtype=4), p) == ERR_DTYPE
    for kw in (dict(d=100), dict(d=0), dict(M=-1), dict(dk=96), dict(dv=32), dict(H=0)):
        assert fwd(_gdims(m, **kw), p) == ERR_SHAPE, kw
        assert L.muir_gate_proj_bwd_workspace(ctypes.byref(_gdims(m, **kw))) == 0
    assert fwd(_gdims(m, M=0), [None] * 10) == OK  # no tokens: nothing launched
    assert L.muir_gate_proj_bwd(ctypes.byref(_gdims(m, M=0)), *([None] * 11), None, None, None, None, 0, None) == ERR_NULL
    for i in range(10):
        q = list(p)
        q[i] = None
        assert fwd(_gdims(m), q) == ERR_NULL, i
        q[i] = ctypes.c_void_p(FAKE[i].value + 4)
        assert fwd(_gdims(m), q) == ERR_ALIGN, i
    d = _gdims(m)
    need = L.muir_gate_proj_bwd_workspace(ctypes.byref(d))
    assert need > 0

    def bwd(dd, ptrs=None, z=None, ws=FAKE[15], ws_bytes=1 << 40):
        q = list(FAKE[:13]) if ptrs is None else ptrs
        return L.muir_gate_proj_bwd(ctypes.byref(dd), *q[:4], z, *q[4:], ws, ctypes.c_size_t(ws_bytes), None)
    assert bwd(d, ws_bytes=need - 1) == ERR_WORKSPACE
    assert bwd(d, ws=None) == ERR_WORKSPACE
    assert bwd(d, z=ctypes.c_void_p(0x10002)) == ERR_ALIGN
    q = list(FAKE[:13])
    q[8] = None  # dgamma
    assert bwd(d, ptrs=q) == ERR_NULL
    # the workspace grows with the tokens
    assert L.muir_gate_proj_bwd_workspace(ctypes.byref(_gdims(m, M=4096))) > need


def test_qk_norm_rejects_bad_arguments():
    m, L = _lib()
    assert L.muir_qk_norm_fwd(10, 96, 1, FAKE[0], FAKE[1], None) == ERR_SHAPE
    assert L.muir_qk_norm_fwd(-1, 64, 1, FAKE[0], FAKE[1], None) == ERR_SHAPE
    assert L.muir_qk_norm_fwd(10, 64, 2, FAKE[0], FAKE[1], None) == ERR_DTYPE
    assert L.muir_qk_norm_fwd(10, 64, 1, None, FAKE[1], None) == ERR_NULL
    assert L.muir_qk_norm_fwd(10, 64, 1, FAKE[0], ctypes.c_void_p(0x10002), None) == ERR_ALIGN
    assert L.muir_qk_norm_bwd(10, 64, 1, FAKE[0], None, FAKE[1], None) == ERR_NULL
    assert L.muir_qk_norm_fwd(0, 64, 1, None, None, None) == OK


def test_binding_refuses_cpu_tensors():
    """The Python binding never computes on the CPU: CPU tensors are rejected."""
    import torch
    m, _ = _lib()
    q = torch.zeros(1, 64, 1, 64)
    with pytest.raises((ValueError, RuntimeError, AssertionError)):
        m.muir_chunk_fwd(q, q, q, q, q, q, q, chunk=64)
