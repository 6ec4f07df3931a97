"""Muir gated delta-rule operator on AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libmuir.so`` (declared in ``include/muir.h``).
Every step of the operator runs in the library's HIP kernels; this module
only checks tensor arguments, allocates outputs and workspaces with torch
(device memory plumbing) and passes raw pointers plus the current HIP stream.
If the library has not been built, importing works but every call raises.

Operator (arXiv 2611.08376, abstract and Methodology): per head, a state
S (dk x dv) is decayed row-wise by exp(log_a_t), the prediction of the
erase-gated key is erased, the gated value write_t*v_t is written along k_t,
and the output reads S_t through gamma_t*q_t.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["muir_check_inputs", "muir_chunk_fwd", "muir_chunk_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "muir_chunk_bwd", "muir_step",
           "muir_chunk_fwd_workspace",
           "muir_chunk_bwd_workspace", "muir_chunk_varlen_fwd", "muir_chunk_varlen_bwd",
           "muir_chunk_varlen_fwd_workspace", "muir_chunk_varlen_bwd_workspace",
           "muir_gate_proj_fwd", "muir_gate_proj_bwd", "muir_gate_proj_bwd_workspace",
           "muir_qk_norm_fwd", "muir_qk_norm_bwd",
           "gate_param_shapes", "GATE_NAMES", "GATE_RANKS",
           "muir_set_profile_events", "muir_profile_events_recorded",
           "lib", "library_path", "MuirError", "STATUS"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmuir.so")

MUIR_F32, MUIR_BF16 = 0, 1
MUIR_GAMMA_TOKEN, MUIR_GAMMA_STATIC, MUIR_GAMMA_NONE = 0, 1, 2
STATUS = {0: "MUIR_OK", 1: "MUIR_ERR_NULL", 2: "MUIR_ERR_SHAPE", 3: "MUIR_ERR_DTYPE",
          4: "MUIR_ERR_WORKSPACE", 5: "MUIR_ERR_ALIGN", 6: "MUIR_ERR_HIP", 7: "MUIR_ERR_MODE",
          8: "MUIR_ERR_SCRATCH", 9: "MUIR_ERR_NONFINITE"}
# size of the fixed scratch array of muir_chunk_fwd_noalloc (MUIR_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 128 << 20


class MuirError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)} ({_status_text(code)})")


class _GateDims(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int32), ("d", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class _Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("gamma_mode", ctypes.c_int32), ("grad_dtype", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded ``libmuir.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run __graft_entry__.build() "
                               "(or python -m gated_delta_rule_muir_amd._build) first")
        L = ctypes.CDLL(_LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(_Dims)
        L.muir_abi_version.restype = I32
        L.muir_status_string.argtypes = [ctypes.c_int]
        L.muir_status_string.restype = ctypes.c_char_p
        L.muir_chunk_fwd_workspace.argtypes = [D]
        L.muir_chunk_fwd_workspace.restype = SZ
        L.muir_chunk_bwd_workspace.argtypes = [D]
        L.muir_chunk_bwd_workspace.restype = SZ
        L.muir_chunk_fwd.argtypes = [D] + [P] * 7 + [P, P, P, P] + [P, SZ, P]
        L.muir_chunk_fwd.restype = ctypes.c_int
        L.muir_chunk_fwd_noalloc.argtypes = [D] + [P] * 7 + [P, P, P, P] + [P]
        L.muir_chunk_fwd_noalloc.restype = ctypes.c_int
        L.muir_chunk_bwd.argtypes = [D] + [P] * 7 + [P, P, P, P, P] + [P] * 8 + [P, SZ, P]
        L.muir_chunk_bwd.restype = ctypes.c_int
        L.muir_chunk_varlen_fwd_workspace.argtypes = [D]
        L.muir_chunk_varlen_fwd_workspace.restype = SZ
        L.muir_chunk_varlen_bwd_workspace.argtypes = [D]
        L.muir_chunk_varlen_bwd_workspace.restype = SZ
        L.muir_chunk_varlen_fwd.argtypes = [D, P] + [P] * 7 + [P, P, P] + [I32] + [P, SZ, P]
        L.muir_chunk_varlen_fwd.restype = ctypes.c_int
        L.muir_chunk_varlen_bwd.argtypes = [D, P] + [P] * 7 + [P, P, P] + [P] * 8 + [P] + [P, SZ, P]
        L.muir_chunk_varlen_bwd.restype = ctypes.c_int
        GD = ctypes.POINTER(_GateDims)
        L.muir_gate_proj_bwd_workspace.argtypes = [GD]
        L.muir_gate_proj_bwd_workspace.restype = SZ
        L.muir_gate_proj_fwd.argtypes = [GD] + [P] * 10 + [P]
        L.muir_gate_proj_fwd.restype = ctypes.c_int
        L.muir_gate_proj_bwd.argtypes = [GD] + [P] * 5 + [P] * 5 + [P] * 4 + [P, SZ, P]
        L.muir_gate_proj_bwd.restype = ctypes.c_int
        L.muir_qk_norm_fwd.argtypes = [ctypes.c_int64, I32, I32, P, P, P]
        L.muir_qk_norm_fwd.restype = ctypes.c_int
        L.muir_qk_norm_bwd.argtypes = [ctypes.c_int64, I32, I32, P, P, P, P]
        L.muir_qk_norm_bwd.restype = ctypes.c_int
        L.muir_check_values.argtypes = [ctypes.c_int64, I32, P, I32, P, P]
        L.muir_check_values.restype = ctypes.c_int
        L.muir_step.argtypes = [I32] * 6 + [P] * 7 + [P, P, P]
        L.muir_step.restype = ctypes.c_int
        L.muir_set_profile_events.argtypes = [P, I32]
        L.muir_set_profile_events.restype = I32
        L.muir_profile_events_recorded.restype = I32
        _lib = L
    return _lib


def _status_text(code: int) -> str:
    try:
        return lib().muir_status_string(code).decode()
    except Exception:  # library missing while formatting an error
        return STATUS.get(code, str(code))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MUIR_BF16
    if t.dtype == torch.float32:
        return MUIR_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_io(name: str, t: torch.Tensor, shape, dtype, device) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor (the operator runs only in the HIP library)")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dims(B, T, H, dk, dv, chunk, dtype, gamma_mode=MUIR_GAMMA_TOKEN, grad_dtype=MUIR_F32) -> _Dims:
    return _Dims(B, T, H, dk, dv, chunk, dtype, gamma_mode, grad_dtype)


def _grad_code(grad_dtype, dt) -> int:
    """Code of the per-token gradients' element type: fp32 (the default) or,
    for bf16 inputs, bf16."""
    if grad_dtype is None or grad_dtype == torch.float32:
        return MUIR_F32
    if grad_dtype == torch.bfloat16 and dt == torch.bfloat16:
        return MUIR_BF16
    raise TypeError(f"grad_dtype {grad_dtype}: fp32, or bf16 for bf16 inputs")


def _gamma_mode(gamma, lead, H, dk, dt, dev) -> int:
    """The readout gate's form from its shape: None (no gate), [H, dk] (static
    per head and key channel) or lead + [H, dk] (per token)."""
    if gamma is None:
        return MUIR_GAMMA_NONE
    if gamma.dim() == 2:
        _check_io("gamma", gamma, (H, dk), dt, dev)
        return MUIR_GAMMA_STATIC
    _check_io("gamma", gamma, tuple(lead) + (H, dk), dt, dev)
    return MUIR_GAMMA_TOKEN


def muir_check_inputs(tensors, *, log_decay=("log_a",), raise_on_error: bool = True):
    """Debug check of input tensors against the operator's preconditions:
    every value finite, and the log-decay tensors (names in `log_decay`) at
    most 0.  `tensors` maps names to GPU tensors (None entries are skipped).
    Counts on the device with muir_check_values, then reads the counts back
    (this synchronises with the current stream).  Returns {name: (non-finite
    count, positive log-decay count)}; with raise_on_error, raises MuirError
    (MUIR_ERR_NONFINITE) naming the tensors at fault."""
    items = [(n, t) for n, t in tensors.items() if t is not None]
    if not items:
        return {}
    dev = items[0][1].device
    counts = torch.zeros((len(items), 2), dtype=torch.int32, device=dev)
    for i, (n, t) in enumerate(items):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n}: must be a contiguous GPU tensor")
        rc = lib().muir_check_values(t.numel(), _dtype_code(t), _ptr(t), 1 if n in log_decay else 0,
                                     ctypes.c_void_p(counts.data_ptr() + 8 * i), _stream(t.device))
        if rc != 0:
            raise MuirError(rc, f"muir_check_values({n})")
    c = counts.cpu().tolist()
    out = {n: (int(c[i][0]), int(c[i][1])) for i, (n, _) in enumerate(items)}
    bad = {n: v for n, v in out.items() if v[0] or v[1]}
    if bad and raise_on_error:
        detail = ", ".join(f"{n}: {a} non-finite, {b} log-decays above 0" for n, (a, b) in bad.items())
        raise MuirError(9, f"input check ({detail})")
    return out


def muir_chunk_fwd_workspace(B, T, H, dk, dv, chunk, dtype=MUIR_BF16, gamma_mode=MUIR_GAMMA_TOKEN) -> int:
    d = _dims(B, T, H, dk, dv, chunk, dtype, gamma_mode)
    return int(lib().muir_chunk_fwd_workspace(ctypes.byref(d)))


def muir_chunk_bwd_workspace(B, T, H, dk, dv, chunk, dtype=MUIR_BF16, gamma_mode=MUIR_GAMMA_TOKEN,
                             grad_dtype=MUIR_F32) -> int:
    d = _dims(B, T, H, dk, dv, chunk, dtype, gamma_mode, grad_dtype)
    return int(lib().muir_chunk_bwd_workspace(ctypes.byref(d)))


def _nchunks(T: int, chunk: int) -> int:
    return (T + chunk - 1) // chunk if chunk > 0 else 0


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def muir_chunk_fwd(q, k, v, log_a, erase, write, gamma, S0=None, *, chunk: int = 64,
                   save_states: bool = False, final_state: bool = True,
                   workspace: Optional[torch.Tensor] = None, out=None, check_inputs: bool = False
                   ) -> Tuple[torch.Tensor, Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Chunkwise forward.  Inputs [B, T, H, D] (bf16 or fp32, on one GPU);
    gamma [B, T, H, dk], or [H, dk] (a static gate), or None (no gate).
    check_inputs: first run muir_check_inputs on them (debugging; synchronises).

    Any T: a partial last chunk runs on zero-padded copies in the workspace.
    Returns (o [B,T,H,dv] in the input dtype, S_T [B,H,dk,dv] fp32 or None,
    S_chunks [B,H,ceil(T/chunk),dk,dv] in the input dtype (the chunk-start
    states kept for muir_chunk_bwd, each stored as 16 x 16 tiles, see
    include/muir.h) or None).
    """
    B, T, H, dk = q.shape
    dv = v.shape[3]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for n, t in (("q", q), ("k", k), ("log_a", log_a), ("erase", erase)):
        _check_io(n, t, (B, T, H, dk), dt, dev)
    gm = _gamma_mode(gamma, (B, T), H, dk, dt, dev)
    for n, t in (("v", v), ("write", write)):
        _check_io(n, t, (B, T, H, dv), dt, dev)
    if S0 is not None:
        _check_io("S0", S0, (B, H, dk, dv), torch.float32, dev)
    if check_inputs:
        muir_check_inputs(dict(q=q, k=k, v=v, log_a=log_a, erase=erase, write=write, gamma=gamma, S0=S0))
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=dt, device=dev)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if final_state else None
    S_chunks = (torch.empty((B, H, _nchunks(T, chunk), dk, dv), dtype=dt, device=dev)
                if save_states else None)
    d = _dims(B, T, H, dk, dv, chunk, code, gm)
    nbytes = int(lib().muir_chunk_fwd_workspace(ctypes.byref(d)))
    ws = _workspace(nbytes, dev, workspace)
    rc = lib().muir_chunk_fwd(ctypes.byref(d), *(_ptr(t) for t in (q, k, v, log_a, erase, write, gamma)),
                              _ptr(S0), _ptr(o), _ptr(S_T), _ptr(S_chunks),
                              _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    if rc != 0:
        raise MuirError(rc, "muir_chunk_fwd")
    return o, S_T, S_chunks


def muir_chunk_fwd_noalloc(q, k, v, log_a, erase, write, gamma, S0=None, *, chunk: int = 64,
                           save_states: bool = False, final_state: bool = True, out=None, S_T_out=None,
                           S_chunks_out=None):
    """muir_chunk_fwd without a workspace: the library takes it from its fixed
    per-GPU scratch array (NOALLOC_SCRATCH_BYTES), so the C call allocates
    nothing; calls that need more raise MuirError (MUIR_ERR_SCRATCH).  Calls
    that overlap in time on one GPU race on that array.  Outputs may be passed
    in (out, S_T_out, S_chunks_out); those not passed are allocated here,
    before the call.  Returns (o, S_T or None, S_chunks or None)."""
    B, T, H, dk = q.shape
    dv = v.shape[3]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for n, t in (("q", q), ("k", k), ("log_a", log_a), ("erase", erase)):
        _check_io(n, t, (B, T, H, dk), dt, dev)
    gm = _gamma_mode(gamma, (B, T), H, dk, dt, dev)
    for n, t in (("v", v), ("write", write)):
        _check_io(n, t, (B, T, H, dv), dt, dev)
    if S0 is not None:
        _check_io("S0", S0, (B, H, dk, dv), torch.float32, dev)
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check_io("out", o, (B, T, H, dv), dt, dev)
    S_T = None
    if final_state:
        S_T = S_T_out if S_T_out is not None else torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        _check_io("S_T_out", S_T, (B, H, dk, dv), torch.float32, dev)
    S_chunks = None
    if save_states:
        shp = (B, H, _nchunks(T, chunk), dk, dv)
        S_chunks = S_chunks_out if S_chunks_out is not None else torch.empty(shp, dtype=dt, device=dev)
        _check_io("S_chunks_out", S_chunks, shp, dt, dev)
    d = _dims(B, T, H, dk, dv, chunk, code, gm)
    rc = lib().muir_chunk_fwd_noalloc(ctypes.byref(d), *(_ptr(t) for t in (q, k, v, log_a, erase, write, gamma)),
                                      _ptr(S0), _ptr(o), _ptr(S_T), _ptr(S_chunks), _stream(dev))
    if rc != 0:
        raise MuirError(rc, "muir_chunk_fwd_noalloc")
    return o, S_T, S_chunks


def muir_chunk_bwd(q, k, v, log_a, erase, write, gamma, dO, S0=None, S_chunks=None, dS_T=None, *,
                   chunk: int = 64, summaries: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, want_dS0: bool = True,
                   grad_dtype: Optional[torch.dtype] = None, check_inputs: bool = False):
    """Chunkwise backward (check_inputs: as muir_chunk_fwd's, over the inputs, dO, S0 and dS_T).  Returns a dict of gradients (dq, dk, dv, dlog_a,
    derase, dwrite in `grad_dtype`: fp32 by default, or bf16 for bf16 inputs,
    accumulated in fp32 and rounded once; dgamma in `grad_dtype` for a
    per-token gate, [H, dk] fp32 (summed over batch and tokens) for a static
    one, None without a gate; dS0 in fp32).

    `S_chunks` (from muir_chunk_fwd(save_states=True)) and `summaries` (the
    `workspace` tensor of that forward call, left unchanged) are saved forward
    results; each one that is None is recomputed inside.  For bf16 with
    chunk 64 they are used only as a pair (the summaries then also hold the
    chunk deltas that the saving forward kept): both are recomputed when
    either is None."""
    B, T, H, dk = q.shape
    dv = v.shape[3]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for n, t in (("q", q), ("k", k), ("log_a", log_a), ("erase", erase)):
        _check_io(n, t, (B, T, H, dk), dt, dev)
    gm = _gamma_mode(gamma, (B, T), H, dk, dt, dev)
    for n, t in (("v", v), ("write", write), ("dO", dO)):
        _check_io(n, t, (B, T, H, dv), dt, dev)
    if S0 is not None:
        _check_io("S0", S0, (B, H, dk, dv), torch.float32, dev)
    if dS_T is not None:
        _check_io("dS_T", dS_T, (B, H, dk, dv), torch.float32, dev)
    if S_chunks is not None:
        _check_io("S_chunks", S_chunks, (B, H, _nchunks(T, chunk), dk, dv), dt, dev)
    if summaries is not None:
        need = muir_chunk_fwd_workspace(B, T, H, dk, dv, chunk, code, gm)
        if (not summaries.is_cuda or summaries.device != dev or not summaries.is_contiguous()
                or summaries.numel() * summaries.element_size() < need):
            raise ValueError(f"summaries: expected the forward workspace ({need} bytes on {dev})")
    gcode = _grad_code(grad_dtype, dt)
    if check_inputs:
        muir_check_inputs(dict(q=q, k=k, v=v, log_a=log_a, erase=erase, write=write, gamma=gamma, dO=dO,
                               S0=S0, dS_T=dS_T))
    gd = dict(dtype=torch.bfloat16 if gcode == MUIR_BF16 else torch.float32, device=dev)
    g = {n: torch.empty((B, T, H, dk), **gd) for n in ("dq", "dk", "dlog_a", "derase")}
    g.update({n: torch.empty((B, T, H, dv), **gd) for n in ("dv", "dwrite")})
    g["dgamma"] = (torch.empty((B, T, H, dk), **gd) if gm == MUIR_GAMMA_TOKEN else
                   torch.empty((H, dk), dtype=torch.float32, device=dev) if gm == MUIR_GAMMA_STATIC else None)
    g["dS0"] = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None
    d = _dims(B, T, H, dk, dv, chunk, code, gm, gcode)
    nbytes = int(lib().muir_chunk_bwd_workspace(ctypes.byref(d)))
    ws = _workspace(nbytes, dev, workspace)
    rc = lib().muir_chunk_bwd(ctypes.byref(d), *(_ptr(t) for t in (q, k, v, log_a, erase, write, gamma)),
                              _ptr(S0), _ptr(S_chunks), _ptr(summaries), _ptr(dO), _ptr(dS_T),
                              *(_ptr(g[n]) for n in ("dq", "dk", "dv", "dlog_a", "derase", "dwrite",
                                                     "dgamma", "dS0")),
                              _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    if rc != 0:
        raise MuirError(rc, "muir_chunk_bwd")
    return g


def muir_chunk_varlen_fwd_workspace(N, max_len, H, dk, dv, chunk, dtype=MUIR_BF16,
                                    gamma_mode=MUIR_GAMMA_TOKEN) -> int:
    d = _dims(N, max_len, H, dk, dv, chunk, dtype, gamma_mode)
    return int(lib().muir_chunk_varlen_fwd_workspace(ctypes.byref(d)))


def muir_chunk_varlen_bwd_workspace(N, max_len, H, dk, dv, chunk, dtype=MUIR_BF16,
                                    gamma_mode=MUIR_GAMMA_TOKEN, grad_dtype=MUIR_F32) -> int:
    d = _dims(N, max_len, H, dk, dv, chunk, dtype, gamma_mode, grad_dtype)
    return int(lib().muir_chunk_varlen_bwd_workspace(ctypes.byref(d)))


def _check_cu(cu_seqlens, dev, total: int, max_len: Optional[int]) -> Tuple[int, int]:
    """Validates the [N + 1] int32 offsets of packed sequences; returns
    (N, max_len).  Reading them back costs one device-to-host copy: callers
    that know the longest length pass max_len (then only the shape is
    checked, and max_len must bound every length)."""
    if not cu_seqlens.is_cuda or cu_seqlens.device != dev:
        raise ValueError(f"cu_seqlens: must be an int32 tensor on {dev}")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens: expected a 1-D int32 tensor [N + 1]")
    if not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens: must be contiguous")
    N = cu_seqlens.numel() - 1
    if max_len is None:
        c = cu_seqlens.cpu()
        lens = c[1:] - c[:-1]
        if int(c[0]) != 0 or int(c[-1]) != total or (N > 0 and int(lens.min()) < 0):
            raise ValueError(f"cu_seqlens: must start at 0, not decrease and end at {total}")
        max_len = int(lens.max()) if N > 0 else 0
    return N, int(max_len)


def muir_chunk_varlen_fwd(q, k, v, log_a, erase, write, gamma, cu_seqlens, S0=None, *, chunk: int = 64,
                          max_len: Optional[int] = None, final_state: bool = True, keep: bool = False,
                          workspace: Optional[torch.Tensor] = None, out=None
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Forward of packed variable-length sequences: inputs [T_total, H, D]
    with sequence n in rows cu_seqlens[n] .. cu_seqlens[n+1]-1 (cu_seqlens an
    int32 GPU tensor [N + 1]); gamma [T_total, H, dk], [H, dk] or None; S0
    [N, H, dk, dv] fp32 or None.  Returns (o [T_total, H, dv], S_T [N, H, dk,
    dv] fp32 or None).  keep: leave the chunk states, summaries and packed
    inputs in `workspace` (which must then be given) for
    muir_chunk_varlen_bwd(fwd_workspace=workspace)."""
    if keep and workspace is None:
        raise ValueError("keep: pass the workspace that the backward will take")
    Tt, H, dk = q.shape
    dv = v.shape[2]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for n, t in (("q", q), ("k", k), ("log_a", log_a), ("erase", erase)):
        _check_io(n, t, (Tt, H, dk), dt, dev)
    gm = _gamma_mode(gamma, (Tt,), H, dk, dt, dev)
    for n, t in (("v", v), ("write", write)):
        _check_io(n, t, (Tt, H, dv), dt, dev)
    N, L = _check_cu(cu_seqlens, dev, Tt, max_len)
    if S0 is not None:
        _check_io("S0", S0, (N, H, dk, dv), torch.float32, dev)
    o = out if out is not None else torch.empty((Tt, H, dv), dtype=dt, device=dev)
    S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if final_state else None
    d = _dims(N, L, H, dk, dv, chunk, code, gm)
    ws = _workspace(int(lib().muir_chunk_varlen_fwd_workspace(ctypes.byref(d))), dev, workspace)
    rc = lib().muir_chunk_varlen_fwd(ctypes.byref(d), _ptr(cu_seqlens),
                                     *(_ptr(t) for t in (q, k, v, log_a, erase, write, gamma)),
                                     _ptr(S0), _ptr(o), _ptr(S_T), 1 if keep else 0, _ptr(ws),
                                     ctypes.c_size_t(ws.numel()), _stream(dev))
    if rc != 0:
        raise MuirError(rc, "muir_chunk_varlen_fwd")
    return o, S_T


def muir_chunk_varlen_bwd(q, k, v, log_a, erase, write, gamma, dO, cu_seqlens, S0=None, dS_T=None, *,
                          chunk: int = 64, max_len: Optional[int] = None,
                          workspace: Optional[torch.Tensor] = None, want_dS0: bool = True,
                          grad_dtype: Optional[torch.dtype] = None, fwd_workspace: Optional[torch.Tensor] = None):
    """Backward of muir_chunk_varlen_fwd.  Returns the gradients as
    muir_chunk_bwd does (per-token ones [T_total, H, D] in `grad_dtype`, fp32
    by default) and dS0 [N, H, dk, dv].  fwd_workspace: the workspace of a
    keep=True forward on the same sequences, reused instead of recomputing."""
    Tt, H, dk = q.shape
    dv = v.shape[2]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for n, t in (("q", q), ("k", k), ("log_a", log_a), ("erase", erase)):
        _check_io(n, t, (Tt, H, dk), dt, dev)
    gm = _gamma_mode(gamma, (Tt,), H, dk, dt, dev)
    for n, t in (("v", v), ("write", write), ("dO", dO)):
        _check_io(n, t, (Tt, H, dv), dt, dev)
    N, L = _check_cu(cu_seqlens, dev, Tt, max_len)
    if S0 is not None:
        _check_io("S0", S0, (N, H, dk, dv), torch.float32, dev)
    if dS_T is not None:
        _check_io("dS_T", dS_T, (N, H, dk, dv), torch.float32, dev)
    gcode = _grad_code(grad_dtype, dt)
    gd = dict(dtype=torch.bfloat16 if gcode == MUIR_BF16 else torch.float32, device=dev)
    g = {n: torch.empty((Tt, H, dk), **gd) for n in ("dq", "dk", "dlog_a", "derase")}
    g.update({n: torch.empty((Tt, H, dv), **gd) for n in ("dv", "dwrite")})
    g["dgamma"] = (torch.empty((Tt, H, dk), **gd) if gm == MUIR_GAMMA_TOKEN else
                   torch.empty((H, dk), dtype=torch.float32, device=dev) if gm == MUIR_GAMMA_STATIC else None)
    g["dS0"] = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None
    d = _dims(N, L, H, dk, dv, chunk, code, gm, gcode)
    ws = _workspace(int(lib().muir_chunk_varlen_bwd_workspace(ctypes.byref(d))), dev, workspace)
    rc = lib().muir_chunk_varlen_bwd(ctypes.byref(d), _ptr(cu_seqlens),
                                     *(_ptr(t) for t in (q, k, v, log_a, erase, write, gamma)),
                                     _ptr(S0), _ptr(dO), _ptr(dS_T),
                                     *(_ptr(g[n]) for n in ("dq", "dk", "dv", "dlog_a", "derase", "dwrite",
                                                            "dgamma", "dS0")),
                                     _ptr(fwd_workspace), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    if rc != 0:
        raise MuirError(rc, "muir_chunk_varlen_bwd")
    return g


def muir_step(q, k, v, log_a, erase, write, gamma, S, *, out=None, check_inputs: bool = False) -> torch.Tensor:
    """One decode step for [N, H, D] inputs (gamma [N, H, dk], or [H, dk] for a
    static gate, or None); S [N, H, dk, dv] fp32 is updated in place.
    Returns o [N, H, dv] in the input dtype.  check_inputs: as muir_chunk_fwd's
    (the state included)."""
    N, H, dk = q.shape
    dv = v.shape[2]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for n, t in (("q", q), ("k", k), ("log_a", log_a), ("erase", erase)):
        _check_io(n, t, (N, H, dk), dt, dev)
    gm = _gamma_mode(gamma, (N,), H, dk, dt, dev)
    for n, t in (("v", v), ("write", write)):
        _check_io(n, t, (N, H, dv), dt, dev)
    _check_io("S", S, (N, H, dk, dv), torch.float32, dev)
    if check_inputs:
        muir_check_inputs(dict(q=q, k=k, v=v, log_a=log_a, erase=erase, write=write, gamma=gamma, S=S))
    o = out if out is not None else torch.empty((N, H, dv), dtype=dt, device=dev)
    rc = lib().muir_step(N, H, dk, dv, code, gm, *(_ptr(t) for t in (q, k, v, log_a, erase, write, gamma)),
                         _ptr(S), _ptr(o), _stream(dev))
    if rc != 0:
        raise MuirError(rc, "muir_step")
    return o


# The fused gate projection: gate order and ranks of the shared down-projection.
GATE_NAMES = ("log_a", "erase", "g", "write", "gamma")
GATE_RANKS = (64, 64, 128, 128, 128)


def gate_param_shapes(d: int, H: int, dk: int, dv: int):
    """Shapes of (W_down, W_up, bias) of the gate projection, in a linear
    layer's [out, in] layout: W_down [512, d]; W_up the five up matrices
    [width_i, rank_i] back to back (flat); bias the five bias vectors back to
    back (flat)."""
    widths = (H * dk, H * dk, H * dv, H * dv, H * dk)
    return (sum(GATE_RANKS), d), (sum(r * w for r, w in zip(GATE_RANKS, widths)),), (sum(widths),)


def muir_gate_proj_bwd_workspace(M, d, H, dk, dv, dtype=MUIR_BF16) -> int:
    gd = _GateDims(M, d, H, dk, dv, dtype)
    return int(lib().muir_gate_proj_bwd_workspace(ctypes.byref(gd)))


def _gate_args(x, W_down, W_up, bias, H, dk, dv):
    lead = tuple(x.shape[:-1])
    d = x.shape[-1]
    M = 1
    for n in lead:
        M *= n
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    _check_io("x", x, tuple(x.shape), dt, dev)
    sw, su, sb = gate_param_shapes(d, H, dk, dv)
    _check_io("W_down", W_down, sw, dt, dev)
    _check_io("W_up", W_up, su, dt, dev)
    _check_io("bias", bias, sb, dt, dev)
    return lead, M, d, dev, dt, _GateDims(M, d, H, dk, dv, code)


def muir_gate_proj_fwd(x, W_down, W_up, bias, *, H: int, dk: int, dv: int):
    """The five gates of every token of x [..., d] from the fused low-rank
    projection.  Returns {"z": [..., 512], "log_a", "erase", "gamma": [..., H, dk],
    "g", "write": [..., H, dv]} in x's dtype."""
    lead, M, d, dev, dt, gd = _gate_args(x, W_down, W_up, bias, H, dk, dv)
    out = {"z": torch.empty(lead + (512,), dtype=dt, device=dev)}
    for n, D in zip(GATE_NAMES, (dk, dk, dv, dv, dk)):
        out[n] = torch.empty(lead + (H, D), dtype=dt, device=dev)
    rc = lib().muir_gate_proj_fwd(ctypes.byref(gd), _ptr(x), _ptr(W_down), _ptr(W_up), _ptr(bias),
                                  _ptr(out["z"]), *(_ptr(out[n]) for n in GATE_NAMES), _stream(dev))
    if rc != 0:
        raise MuirError(rc, "muir_gate_proj_fwd")
    return out


def muir_gate_proj_bwd(x, W_down, W_up, bias, d_gates, *, H: int, dk: int, dv: int, z=None,
                       workspace: Optional[torch.Tensor] = None):
    """Reverse mode of muir_gate_proj_fwd from the gates' gradients
    (d_gates[name], shaped like the gates).  Returns {"dx" (x's dtype),
    "dW_down", "dW_up", "dbias" (fp32)}.  z: the forward's z, or None."""
    lead, M, d, dev, dt, gd = _gate_args(x, W_down, W_up, bias, H, dk, dv)
    for n, D in zip(GATE_NAMES, (dk, dk, dv, dv, dk)):
        _check_io("d" + n, d_gates[n], lead + (H, D), dt, dev)
    if z is not None:
        _check_io("z", z, lead + (512,), dt, dev)
    sw, su, sb = gate_param_shapes(d, H, dk, dv)
    g = {"dx": torch.empty(tuple(x.shape), dtype=dt, device=dev),
         "dW_down": torch.empty(sw, dtype=torch.float32, device=dev),
         "dW_up": torch.empty(su, dtype=torch.float32, device=dev),
         "dbias": torch.empty(sb, dtype=torch.float32, device=dev)}
    ws = _workspace(int(lib().muir_gate_proj_bwd_workspace(ctypes.byref(gd))), dev, workspace)
    rc = lib().muir_gate_proj_bwd(ctypes.byref(gd), _ptr(x), _ptr(W_down), _ptr(W_up), _ptr(bias), _ptr(z),
                                  *(_ptr(d_gates[n]) for n in GATE_NAMES),
                                  *(_ptr(g[n]) for n in ("dx", "dW_down", "dW_up", "dbias")),
                                  _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    if rc != 0:
        raise MuirError(rc, "muir_gate_proj_bwd")
    return g


def muir_qk_norm_fwd(u, *, out=None):
    """SiLU then L2 normalisation over the last axis (64 or 128 channels: one head)."""
    D = u.shape[-1]
    _check_io("u", u, tuple(u.shape), u.dtype, u.device)
    y = out if out is not None else torch.empty_like(u)
    rc = lib().muir_qk_norm_fwd(u.numel() // max(D, 1), D, _dtype_code(u), _ptr(u), _ptr(y), _stream(u.device))
    if rc != 0:
        raise MuirError(rc, "muir_qk_norm_fwd")
    return y


def muir_qk_norm_bwd(u, dy):
    """Gradient of sum(dy * muir_qk_norm_fwd(u)) with respect to u."""
    D = u.shape[-1]
    _check_io("u", u, tuple(u.shape), u.dtype, u.device)
    _check_io("dy", dy, tuple(u.shape), u.dtype, u.device)
    du = torch.empty_like(u)
    rc = lib().muir_qk_norm_bwd(u.numel() // max(D, 1), D, _dtype_code(u), _ptr(u), _ptr(dy), _ptr(du),
                                _stream(u.device))
    if rc != 0:
        raise MuirError(rc, "muir_qk_norm_bwd")
    return du


def muir_set_profile_events(events=None, count: int = 0) -> None:
    """Register a ctypes array of hipEvent_t handles for per-kernel timing
    (see include/muir.h); ``None`` turns it off."""
    rc = lib().muir_set_profile_events(events, int(count) if events is not None else 0)
    if rc != 0:
        raise MuirError(rc, "muir_set_profile_events")


def muir_profile_events_recorded() -> int:
    return int(lib().muir_profile_events_recorded())
