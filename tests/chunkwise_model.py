"""Test-only fp64 NumPy model of the chunkwise (parallel) form.

The Methodology section of the wolonglab summary page of arXiv 2611.08376
says training expresses each chunk as a triangular system.  This model
writes that form out plainly -- a dense C x C x d_k decay tensor and a
library triangular solve -- so that the sequential oracle can be checked
against an independent derivation: the two must agree to rounding for every
chunk size.  It shares no code with the oracle (C) or with the HIP library.

Per chunk of C tokens with chunk-initial state S (d_k x d_v):
  L_r   = sum_{i<=r} log_a_i                        (chunk-local, per channel)
  A_ri  = sum_j erase_rj k_rj k_ij exp(L_rj - L_ij)    for i < r
  P_ri  = sum_j gamma_rj q_rj k_ij exp(L_rj - L_ij)    for i <= r
  (I + A) D = W*V - (exp(L) * erase * k) S              D: per-token deltas
  O     = (exp(L) * gamma * q) S + P D
  S_new = diag(exp(L_C)) S + (exp(L_C - L) * k)^T D
"""
from __future__ import annotations

import numpy as np


def chunkwise_fwd(q, k, v, log_a, erase, write, gamma, S0, C):
    q, k, v, la, er, wr, ga = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_a, erase, write, gamma))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for c0 in range(0, T, C):
                c1 = min(c0 + C, T)
                n = c1 - c0
                kk, qq, vv = k[b, c0:c1, h], q[b, c0:c1, h], v[b, c0:c1, h]
                L = np.cumsum(la[b, c0:c1, h], axis=0)
                dec = np.exp(L[:, None, :] - L[None, :, :])  # [r, i, j]
                ek = er[b, c0:c1, h] * kk
                qt = ga[b, c0:c1, h] * qq
                A = np.einsum("rj,ij,rij->ri", ek, kk, dec) * np.tril(np.ones((n, n)), -1)
                P = np.einsum("rj,ij,rij->ri", qt, kk, dec) * np.tril(np.ones((n, n)), 0)
                U = wr[b, c0:c1, h] * vv
                rhs = U - (np.exp(L) * ek) @ S
                D = np.linalg.solve(np.eye(n) + A, rhs)
                o[b, c0:c1, h] = (np.exp(L) * qt) @ S + P @ D
                S = np.exp(L[-1])[:, None] * S + (np.exp(L[-1][None, :] - L) * kk).T @ D
            S_T[b, h] = S
    return o, S_T


def chunk_summary(q, k, v, log_a, erase, write, gamma, C):
    """Per-chunk quantities of the chunkwise form, for one (b, h) sequence
    given as [T, D] arrays: returns a list of dicts with
      W = (I+A)^-1 (exp(L) * ek), U~ = (I+A)^-1 (write*v), Q' = exp(L)*qt - P W,
      O~ = P U~, Kbar = exp(L_C - L) * k, gC = exp(L_C), and A, P
    (test-only; used to inspect the GPU path's intermediate workspace)."""
    q, k, v, la, er, wr, ga = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_a, erase, write, gamma))
    T = q.shape[0]
    out = []
    for c0 in range(0, T, C):
        kk, qq, vv = k[c0:c0 + C], q[c0:c0 + C], v[c0:c0 + C]
        n = kk.shape[0]
        L = np.cumsum(la[c0:c0 + C], axis=0)
        dec = np.exp(L[:, None, :] - L[None, :, :])
        ek = er[c0:c0 + C] * kk
        qt = ga[c0:c0 + C] * qq
        A = np.einsum("rj,ij,rij->ri", ek, kk, dec) * np.tril(np.ones((n, n)), -1)
        P = np.einsum("rj,ij,rij->ri", qt, kk, dec) * np.tril(np.ones((n, n)), 0)
        Tm = np.linalg.inv(np.eye(n) + A)
        W = Tm @ (np.exp(L) * ek)
        Ut = Tm @ (wr[c0:c0 + C] * vv)
        out.append(dict(W=W, Ut=Ut, Qp=np.exp(L) * qt - P @ W, Ot=P @ Ut,
                        Kb=np.exp(L[-1][None, :] - L) * kk, gC=np.exp(L[-1]), A=A, P=P))
    return out
