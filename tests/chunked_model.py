"""Chunked form of the gated delta rule in numpy (test-only model, fp64 by default).

The GPU path evaluates the recurrence S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T
chunk by chunk (chunk size C).  Within a chunk with incoming state S, rows i = 0..n-1:

  H_i   = cumulative sum of g since the last alpha = 0 token (reset) at or before i
  e_i   = exp(H_i) if no reset in [0, i], else 0          (decay from chunk start)
  G_ij  = exp(H_i - H_j) if j >= last reset at/before i    (decay from j to i), j <= i
  A     = strict_lower( diag(b) (K K^T * G) ),   T = (I + A)^{-1}
  X     = K S,   Y = diag(b) (V - diag(e) X),   U = T Y         (pseudo-values)
  O     = scale (diag(e) Q S + lower(Q K^T * G) U)
  S    <- e_{n-1} S + K^T diag(G_{n-1, .}) U

which follows from S_i = e_i S + sum_{j<=i} G_ij k_j u_j^T with
u_i = b_i (v_i - a_i S_{i-1}^T k_i).  This module exists to pin that algebra against
the token-by-token oracle, and to simulate the rounding of the bf16 path (``rnd``
hooks), so that precision choices are checked on the CPU before any kernel runs.
It shares no code with the oracle or with the HIP library.
"""
from __future__ import annotations

import numpy as np


def bf16(x):
    """Round to bfloat16 (round to nearest even) via fp32, returned as float64."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    out = b.astype(np.uint32).view(np.float32).astype(np.float64)
    # keep non-finite values as they are
    return np.where(np.isfinite(f), out, f.astype(np.float64))


def split(x):
    hi = bf16(x)
    return hi, bf16(np.asarray(x, np.float64) - hi)


def f16(x):
    """Round to IEEE binary16 (round to nearest even), returned as float64."""
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def gates(g):
    """Reset-aware in-chunk gate scan. Returns H, e, Gam (lower incl. diagonal)."""
    n = len(g)
    H = np.zeros(n)
    last = -1
    acc = 0.0
    rho = np.zeros(n, dtype=np.int64)
    for i in range(n):
        if np.isneginf(g[i]):
            last = i
            acc = 0.0
        else:
            acc += g[i]
        H[i] = acc
        rho[i] = last
    e = np.where(rho < 0, np.exp(H), 0.0)
    ii, jj = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    Gam = np.where((jj <= ii) & (rho[ii] <= jj), np.exp(np.minimum(H[ii] - H[jj], 0.0)), 0.0)
    return H, e, Gam


class Policy:
    """Which operands are rounded to bf16 (hi), split into hi + lo bf16 pairs (split) or
    rounded to fp16 (f16); ``qk`` rounds q and k themselves ("f16": the matrix operands are
    fp16 copies of the bf16 inputs), ``p_diag`` puts P's diagonal into the rounded P."""

    def __init__(self, exact=True, S_in_X="hi", S_in_O="split", Y_in_U="hi", T="hi",
                 P="hi", U_in_O="split", U_in_S="split", o_round=True, qk="exact", p_diag=False):
        self.exact = exact
        self.S_in_X, self.S_in_O, self.Y_in_U, self.T = S_in_X, S_in_O, Y_in_U, T
        self.P, self.U_in_O, self.U_in_S, self.o_round = P, U_in_O, U_in_S, o_round
        self.qk, self.p_diag = qk, p_diag

    @staticmethod
    def apply(x, mode):
        if mode == "exact":
            return [np.asarray(x, np.float64)]
        if mode == "hi":
            return [bf16(x)]
        if mode == "split":
            return list(split(x))
        if mode == "f16":
            return [f16(x)]
        raise ValueError(mode)


EXACT = Policy(exact=True)
# the bf16-input path of the kernel: every matrix operand an fp16 rounding of its fp32 value
# (q, k exactly, being bf16 values within the fp16 range); o rounded to bf16 on output
F16_OPERANDS = Policy(exact=False, S_in_X="f16", S_in_O="f16", Y_in_U="f16", T="f16", P="f16",
                      U_in_O="f16", U_in_S="f16", qk="f16", p_diag=True)


def _prod(Aparts, Bparts, max_terms=3):
    # hi*hi + hi*lo + lo*hi (lo*lo dropped)
    out = 0.0
    for i, a in enumerate(Aparts):
        for j, b in enumerate(Bparts):
            if i + j <= 1:
                out = out + a @ b
    return out


def chunk_chain(q, k, v, g, beta, S0=None, C=64, scale=1.0, pol: Policy = EXACT):
    """Run one (sequence, head) chain in chunks. q, k: [T, dk]; v: [T, dv]; g, beta: [T]."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    ex = pol.exact
    for t0 in range(0, T, C):
        n = min(C, T - t0)
        K, Q, V = k[t0:t0 + n], q[t0:t0 + n], v[t0:t0 + n]
        b = beta[t0:t0 + n]
        _, e, Gam = gates(g[t0:t0 + n])
        A = np.tril(b[:, None] * (K @ K.T) * Gam, -1)
        Tm = np.linalg.inv(np.eye(n) + A)
        P = np.tril((Q @ K.T) * Gam, -1)
        Pd = np.einsum("ij,ij->i", Q, K)
        if ex:
            X = K @ S
            Y = b[:, None] * (V - e[:, None] * X)
            U = Tm @ Y
            Ob = e[:, None] * (Q @ S) + Pd[:, None] * U + P @ U
            S = e[-1] * S + K.T @ (Gam[-1][:, None] * U)
        else:
            Kr, Qr = (f16(K), f16(Q)) if pol.qk == "f16" else (K, Q)
            X = _prod([Kr], Policy.apply(S, pol.S_in_X))
            Y = b[:, None] * (V - e[:, None] * X)
            Toff = Tm - np.eye(n)
            U = Y + _prod(Policy.apply(Toff, pol.T), Policy.apply(Y, pol.Y_in_U))
            QS = _prod([Qr], Policy.apply(S, pol.S_in_O))
            if pol.p_diag:
                Ob = e[:, None] * QS + _prod(Policy.apply(P + np.diag(Pd), pol.P),
                                             Policy.apply(U, pol.U_in_O))
            else:
                Ob = e[:, None] * QS + Pd[:, None] * U + _prod(Policy.apply(P, pol.P),
                                                               Policy.apply(U, pol.U_in_O))
            Ud = Gam[-1][:, None] * U
            S = e[-1] * S + _prod([Kr.T], Policy.apply(Ud, pol.U_in_S))
        O[t0:t0 + n] = scale * Ob
    if not ex and pol.o_round:
        O = bf16(O)
    return S, O
