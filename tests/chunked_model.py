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


# ---------------------------------------------------------------------------------------
# Model of the chunk kernel's own arithmetic (test-only).  ``chunk_chain`` above rounds
# whole operands of the 64-row chunk form; ``kernel_chain`` below follows the kernel step
# by step instead, so that its numerical choices are pinned on the CPU:
#   * the gate wave's scan of a 64-row chunk in fp32 (a Hillis-Steele scan over the 64
#     lanes), Gamma_ij = 2^(H_i log2e - H_j log2e) and e, G_last from __expf, as the
#     kernel computes them -- or the compensated variant (hi + lo scan, differences
#     taken before scaling);
#   * the 16-row block substitution (I + A) U = Y with -A_bj and U_j rounded to the
#     operand type, U_b = z + (T_bb - I) z;
#   * the 16x16 diagonal-block inverse T_bb by the algorithm named in ``inv``, with the
#     operand roundings of the matrix cores;
#   * fp16 operands (bf16 inputs) or fp32 operands (fp32 inputs); fp32 accumulation is
#     modelled as exact (its rounding is ~2^-24 relative, below every effect studied here).
# Rows past the window are zero rows (g = beta = 0, inert), as in the kernel.

L2E32 = np.float32(1.4426950408889634)


def f32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def _expf(x):
    """__expf: the hardware exp2 of fp32(x * log2 e) (modelled as correctly rounded)."""
    y = (np.asarray(x, np.float32) * L2E32).astype(np.float32)
    with np.errstate(over="ignore"):
        return np.exp2(y.astype(np.float64)).astype(np.float32).astype(np.float64)


def _shift_up(a, off, fill):
    out = np.empty_like(a)
    out[:off] = fill
    out[off:] = a[:-off]
    return out


def gate_scan_f32(g64, compensated=False):
    """The gate wave's reset-aware scan of one 64-row chunk, in fp32 arithmetic.

    Returns (h, l, rho): H = h + l (l = 0 unless compensated) and the last reset row.
    Lane i adds lane i - off's partial sum in steps off = 1, 2, 4, ..., 32 unless a reset
    already lies in its segment; the compensated scan carries the rounding error of each
    addition in l (Knuth's two-sum), so that H is kept to about 2^-48 relative."""
    lanes = np.arange(64)
    g64 = np.asarray(g64, np.float32)
    reset = np.isneginf(g64)
    h = np.where(reset, np.float32(0), g64).astype(np.float32)
    lo = np.zeros(64, np.float32)
    seg = reset.astype(np.int64)
    rho = np.where(reset, lanes, -1)
    for off in (1, 2, 4, 8, 16, 32):
        ho = _shift_up(h, off, np.float32(0))
        loo = _shift_up(lo, off, np.float32(0))
        so = _shift_up(seg, off, 0)
        ro = _shift_up(rho, off, -1)
        act = lanes >= off
        add = act & (seg == 0)
        s = (h + ho).astype(np.float32)
        if compensated:
            bp = (s - h).astype(np.float32)
            err = ((h - (s - bp)) + (ho - bp)).astype(np.float32)
            lo = np.where(add, (lo + loo + err).astype(np.float32), lo)
        h = np.where(add, s, h)
        seg = np.where(act, seg | so, seg)
        rho = np.where(act, np.maximum(rho, ro), rho)
    return h.astype(np.float32), lo, rho


def kernel_gates(g64, mode):
    """Gamma (64x64, lower with the reset mask), e and G_last of one chunk.

    mode "exact": fp64 definition; "f32": a plain fp32 scan, H scaled by log2 e before the
    differences are taken (the kernel's first form); "f32c": compensated scan, the
    differences of the (hi, lo) pairs taken first, then scaled (fp32 inputs); "f32cb":
    compensated scan, Gamma from the hi part scaled by log2 e (bf16 inputs), G_last
    from the compensated difference."""
    ii, jj = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    if mode == "exact":
        H, e, Gam = gates(np.asarray(g64, np.float64))
        rho = np.full(64, -1)
        last = -1
        for i in range(64):
            if np.isneginf(g64[i]):
                last = i
            rho[i] = last
        lst = np.where(rho[63] <= np.arange(64), np.exp(np.minimum(H[63] - H, 0.0)), 0.0)
        return Gam, e, lst
    h, lo, rho = gate_scan_f32(g64, compensated=(mode == "f32c"))
    e = np.where(rho < 0, _expf(h), 0.0)
    if mode in ("f32", "f32cb"):
        gH = (h * L2E32).astype(np.float32)
        d2 = (gH[ii] - gH[jj]).astype(np.float32)
        if mode == "f32":
            dl = (h[63] - h).astype(np.float32)
        else:
            dl = ((h[63] - h).astype(np.float32) + (lo[63] - lo).astype(np.float32)).astype(np.float32)
    else:
        d = ((h[ii] - h[jj]).astype(np.float32) + (lo[ii] - lo[jj]).astype(np.float32)).astype(np.float32)
        d2 = (d * L2E32).astype(np.float32)
        dl = ((h[63] - h).astype(np.float32) + (lo[63] - lo).astype(np.float32)).astype(np.float32)
    with np.errstate(over="ignore"):
        ex = np.exp2(d2.astype(np.float64)).astype(np.float32).astype(np.float64)
    Gam = np.where((jj <= ii) & (rho[ii] <= jj), ex, 0.0)
    lst = np.where(rho[63] <= np.arange(64), _expf(dl), 0.0)
    return Gam, e, lst


def diag_inverse_model(N, inv, rnd):
    """T - I for T = (I - N)^{-1}, N strictly lower 16x16 (= -A_bb, fp32 values).

    inv "exact": the exact inverse; "prod": the product (I+N)(I+N^2)(I+N^4)(I+N^8) with
    each matrix-core operand rounded by ``rnd``, in the kernel's order; "blk4": two-level
    Neumann over 4x4 blocks, T = (I - F)^{-1} (I - D)^{-1} with D the 4x4 diagonal blocks
    of N, F = (I - D)^{-1} E the rest, each series three terms long."""
    I = np.eye(16)
    if inv == "exact":
        return np.linalg.inv(I - N) - I
    if inv == "prod":
        N2 = rnd(N) @ rnd(N)
        N3 = rnd(N) @ rnd(N2)
        N4 = rnd(N2) @ rnd(N2)
        N8 = rnd(N4) @ rnd(N4)
        P1 = I + N + N2 + N3
        P2 = P1 + rnd(P1) @ rnd(N4)
        Tr = P2 + rnd(P2) @ rnd(N8)
        return Tr - I
    if inv == "blk4":
        blk = (np.arange(16)[:, None] // 4) == (np.arange(16)[None, :] // 4)
        D = np.where(blk, N, 0.0)
        E = np.where(blk, 0.0, N)
        D2 = rnd(D) @ rnd(D)
        D3 = rnd(D) @ rnd(D2)
        Dinv = I + D + D2 + D3                      # (I - D)^{-1}, D^4 = 0
        F = rnd(Dinv) @ rnd(E)                      # (I - D)^{-1} E, strictly block-lower
        F2 = rnd(F) @ rnd(F)
        F3 = rnd(F) @ rnd(F2)
        Finv = I + F + F2 + F3                      # (I - F)^{-1}, F^4 = 0
        return (Dinv - I) + rnd(Finv - I) @ rnd(Dinv)   # T - I = (Finv - I) Dinv + (Dinv - I)
    if inv in ("blk4g", "blk4g9"):
        # the matrix-core sequence of the kernel: T = (I - D)^{-1} (I - G)^{-1}, G = E (I - D)^{-1};
        # "c"/"r" name the two register layouts; a layout change is a product with I (so it
        # rounds its operand)
        blk = (np.arange(16)[:, None] // 4) == (np.arange(16)[None, :] // 4)
        Dr = np.where(blk, N, 0.0)
        Er = np.where(blk, 0.0, N)
        Dc = rnd(Dr)
        D2c = rnd(Dr) @ rnd(Dc)
        D3c = rnd(Dr) @ rnd(D2c)
        Dinvc = I + Dc + D2c + D3c
        Gc = rnd(Er) @ rnd(Dinvc)
        Gr = rnd(Er) @ rnd(Dinvc)
        G2c = rnd(Gr) @ rnd(Gc)
        G3c = rnd(Gr) @ rnd(G2c)
        Ginv1c = Gc + G2c + G3c                     # (I - G)^{-1} - I, G^4 = 0
        if inv == "blk4g9":   # the A-layout (I - D)^{-1} from the accumulator one (one product)
            Dinvr = rnd(Dinvc)
        else:
            D2r = rnd(Dr) @ rnd(Dc)
            D3r = rnd(Dr) @ rnd(D2c)
            Dinvr = I + Dr + D2r + D3r
        return (Dinvr - I) + rnd(Dinvr) @ rnd(Ginv1c)
    raise ValueError(inv)


def kernel_chain(q, k, v, g, beta, S0=None, scale=1.0, path="bf16", gate_mode=None, inv="blk4g9"):
    """One (sequence, head) chain through the kernel's chunk arithmetic (see above).

    path "bf16": fp16 matrix operands (q, k, v bf16 values), o rounded to bf16;
    path "f32": fp32 operands and outputs; path "f64": no rounding at all (pins the
    algebra of the block substitution and of the inverse).  gate_mode defaults to the
    kernel's own ("f32" for bf16 inputs, "f32c" for fp32 inputs, "exact" for f64),
    inv to the kernel's diagonal-block inverse ("blk4g9")."""
    T, dk = k.shape
    dv = v.shape[1]
    rnd = {"bf16": f16, "f32": f32, "f64": lambda x: np.asarray(x, np.float64)}[path]
    gate_mode = gate_mode or {"bf16": "f32", "f32": "f32c", "f64": "exact"}[path]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    for t0 in range(0, T, 64):
        n = min(64, T - t0)
        K = np.zeros((64, dk)); Q = np.zeros((64, dk)); V = np.zeros((64, dv))
        g64 = np.zeros(64, np.float32); b = np.zeros(64)
        K[:n], Q[:n], V[:n] = k[t0:t0 + n], q[t0:t0 + n], v[t0:t0 + n]
        g64[:n] = np.asarray(g[t0:t0 + n], np.float32)
        b[:n] = beta[t0:t0 + n] if path == "f64" else f32(beta[t0:t0 + n])
        Gam, e, lst = kernel_gates(g64, gate_mode)
        Kr, Qr = rnd(K), rnd(Q)
        KK, QK = Kr @ Kr.T, Qr @ Kr.T
        low = np.tril(np.ones((64, 64)), -1) > 0
        r32 = f32 if path != "f64" else rnd
        negA = r32(np.where(low, -(b[:, None] * KK * Gam), 0.0))
        P = rnd(r32(scale * Gam * QK))
        Tm = [rnd(diag_inverse_model(negA[16 * i:16 * i + 16, 16 * i:16 * i + 16], inv, rnd))
              for i in range(4)]
        negA = rnd(negA)
        Sr = rnd(S)
        X = Kr @ Sr
        QS = Qr @ Sr
        Y = b[:, None] * (V - e[:, None] * X)
        U = np.zeros((64, dv))
        for bb in range(4):
            rb = slice(16 * bb, 16 * bb + 16)
            z = Y[rb].copy()
            for j in range(bb):
                z = z + negA[rb, 16 * j:16 * j + 16] @ rnd(U[16 * j:16 * j + 16])
            U[rb] = z + Tm[bb] @ rnd(z)
        Ob = scale * e[:, None] * QS + P @ rnd(U)
        S = e[63] * S + Kr.T @ rnd(lst[:, None] * U)
        O[t0:t0 + n] = Ob[:n]
    if path == "bf16":
        O = bf16(O)
    return S, O
