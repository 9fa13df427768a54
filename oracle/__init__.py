"""fp64 CPU oracle for the Gated DeltaNet replay / prefill path (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  It shares no code with the HIP library and never imports
it; the product path must never reach it.

The arithmetic lives in ``gdn_oracle.c`` (plain C, double precision, token by
token).  This wrapper only widens inputs exactly to float64 and passes pointers.

``adaptive_replay_len`` is plain Python on exact integers (the definition written out:
walk back from the last token, sum the rounded log-gates, stop at the first window
whose sum is at or below the threshold).

Pins (see ``tests/test_oracle_pins.py`` and ``tests/test_oracle_golden.py``): a worked
example derived by hand (``tests/golden/``), explicit-matrix brute force, exact
rational arithmetic, closed forms (alpha=1/beta=0, single token, orthonormal keys
with beta=1, repeated key overwrite), and invariants (alpha=0 makes replay equal
prefill, the attenuation bound, split-prefill composition, r=L and r=0, GVA as
duplicated heads, packing order).  No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import math
import os
import re
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
# GDN_ORACLE_SANITIZE (e.g. "address,undefined" or "thread") selects a separately
# built, instrumented copy; the process must then preload gcc's matching runtime.
_SANITIZE = os.environ.get("GDN_ORACLE_SANITIZE", "").strip()
_LIB_PATH = os.path.join(_HERE, "liboracle.so" if not _SANITIZE else
                         "liboracle_%s.so" % re.sub(r"[^a-z]+", "_", _SANITIZE))
_lib = None
_lock = threading.Lock()


def build(force: bool = False) -> str:
    """Compile the oracle with the host C compiler (gcc -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        extra = [] if not _SANITIZE else ["-fsanitize=" + _SANITIZE, "-fno-sanitize-recover=all",
                                          "-fno-omit-frame-pointer", "-g"]
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math"] + extra + ["-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            dp = ctypes.POINTER(ctypes.c_double)
            ip = ctypes.POINTER(ctypes.c_int64)
            i32, i64 = ctypes.c_int32, ctypes.c_int64
            lib.gdn_oracle_prefill.argtypes = [i64, i32, i32, i32, i32, dp, dp, dp, dp, dp, ip,
                                               dp, ctypes.c_double, dp, dp, i32]
            lib.gdn_oracle_prefill.restype = ctypes.c_int
            lib.gdn_oracle_replay.argtypes = [i64, i32, i32, i32, i32, dp, dp, dp, dp, dp, ip,
                                              ip, ctypes.c_double, dp, dp, i32]
            lib.gdn_oracle_replay.restype = ctypes.c_int
            lib.gdn_oracle_state_relerr.argtypes = [dp, dp, i64, i64, dp]
            lib.gdn_oracle_state_relerr.restype = ctypes.c_int64
            _lib = lib
    return _lib


def widen(x) -> np.ndarray:
    """Exact widening of a bf16 / fp32 / fp64 tensor or array to contiguous float64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu")
            if x.dtype == torch.bfloat16:
                x = x.to(torch.float32)  # exact: every bf16 value is an fp32 value
            return np.ascontiguousarray(x.numpy().astype(np.float64))
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _threads(n):
    if n is not None:
        return int(n)
    return int(os.environ.get("GDN_ORACLE_THREADS", os.cpu_count() or 1))


def _common(q, k, v, g, beta, cu):
    q, k, v, g, beta = (widen(a) for a in (q, k, v, g, beta))
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    assert k.shape == q.shape and v.shape[0] == T and g.shape == (T, h_v) == beta.shape
    assert cu[0] == 0 and cu[-1] == T
    return q, k, v, g, beta, cu, h_qk, h_v, d_k, d_v


def prefill(q, k, v, g, beta, cu_seqlens, S0=None, scale=1.0, want_o=True, threads=None):
    """Full prefill from S0 (None = zero). Returns (S [N,h_v,d_k,d_v], o [T,h_v,d_v] or None)."""
    q, k, v, g, beta, cu, h_qk, h_v, d_k, d_v = _common(q, k, v, g, beta, cu_seqlens)
    N = len(cu) - 1
    S = np.zeros((N, h_v, d_k, d_v), dtype=np.float64)
    o = np.zeros((q.shape[0], h_v, d_v), dtype=np.float64) if want_o else None
    s0 = widen(S0) if S0 is not None else None
    if s0 is not None:
        assert s0.shape == S.shape
    rc = _load().gdn_oracle_prefill(N, h_qk, h_v, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), _iptr(cu), _ptr(s0), float(scale), _ptr(S),
                                    _ptr(o), _threads(threads))
    if rc != 0:
        raise ValueError("oracle prefill rejected its arguments")
    return S, o


def replay(q, k, v, g, beta, cu_seqlens, r, scale=1.0, want_o=True, threads=None):
    """Tail replay from zero over the last r[n] tokens. Returns (S, o [sum r, h_v, d_v] or None)."""
    q, k, v, g, beta, cu, h_qk, h_v, d_k, d_v = _common(q, k, v, g, beta, cu_seqlens)
    N = len(cu) - 1
    rr = np.ascontiguousarray(np.asarray(r, dtype=np.int64))
    assert rr.shape == (N,)
    S = np.zeros((N, h_v, d_k, d_v), dtype=np.float64)
    o = np.zeros((int(rr.sum()), h_v, d_v), dtype=np.float64) if want_o else None
    rc = _load().gdn_oracle_replay(N, h_qk, h_v, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _iptr(cu), _iptr(rr), float(scale), _ptr(S),
                                   _ptr(o), _threads(threads))
    if rc != 0:
        raise ValueError("oracle replay rejected its arguments")
    return S, o


def state_relerr(A, B):
    """Per-state ||A-B||_F/||B||_F (||A||_F if ||B||_F = 0) over the last two axes."""
    A = widen(A); B = widen(B)
    assert A.shape == B.shape and A.ndim >= 2
    n_states = int(np.prod(A.shape[:-2])) if A.ndim > 2 else 1
    elems = A.shape[-1] * A.shape[-2]
    out = np.zeros(n_states, dtype=np.float64)
    nf = _load().gdn_oracle_state_relerr(_ptr(A), _ptr(B), n_states, elems, _ptr(out))
    return out.reshape(A.shape[:-2]) if A.ndim > 2 else out[0], int(nf)


def chain_inputs(inp: dict, seq: int, head: int, window: str = "replay"):
    """Slice one (sequence, v-head) chain's window out of packed inputs.

    Returns (q, k, v, g, beta) with one sequence and one head each, as float64 arrays,
    so the oracle can be run on a sample of a large workload.
    """
    w = inp["workload"]
    cu = inp["cu_host"]; r = inp["r_host"]
    hk = head * w.h_qk // w.h_v
    end = int(cu[seq + 1])
    start = end - int(r[seq]) if window == "replay" else int(cu[seq])
    sl = slice(start, end)
    return (widen(inp["q"][sl, hk:hk + 1]), widen(inp["k"][sl, hk:hk + 1]),
            widen(inp["v"][sl, head:head + 1]), widen(inp["g"][sl, head:head + 1]),
            widen(inp["beta"][sl, head:head + 1]))


GATE_UNIT = 2 ** 32          # log-gates are counted in units of 2^-32 nats
GATE_FLOOR = -(2 ** 52)      # a gate at or below -2^20 nats (alpha ~ 0) counts as -2^20


def quantized_log_gates(g) -> list:
    """Each g (fp32) rounded once, half to even, to an integer number of 2^-32 nats.

    g >= 0 or NaN counts as 0 (no attenuation); g <= -2^20 nats, -inf included, as
    -2^20 nats.  Returns nested Python lists of exact integers, shape of ``g``.
    """
    x = widen(g)
    out = np.where(~(x < 0.0), 0.0, np.where(x <= -2.0 ** 20, float(GATE_FLOOR), np.rint(x * GATE_UNIT)))
    return out.astype(np.int64).tolist()


def adaptive_replay_len(g, cu_seqlens, eps, r_min=0, r_max=2 ** 31 - 1):
    """Per-sequence replay length chosen from the gates.

    The replayed state misses the older state carried through the window, whose
    propagation has norm at most prod alpha_t over the window for unit keys and beta in
    [0, 1] (Tail-Replay, abstract: gated updates attenuate distant tokens).  For every
    sequence n and v-head h, r_h is the smallest r in [0, min(L_n, r_max)] whose last-r
    log-gate sum (in 2^-32 nat units, ``quantized_log_gates``) is at most
    floor(ln(eps) * 2^32), else min(L_n, r_max); the result is max_h r_h clamped to
    [min(r_min, L_n), min(r_max, L_n)].  eps >= 1 makes the empty window qualify.
    """
    if not (eps > 0.0):
        raise ValueError("eps must be positive")
    thr = math.floor(math.log(eps) * GATE_UNIT) if eps < 1.0 else 0
    qg = quantized_log_gates(g)
    cu = [int(c) for c in cu_seqlens]
    H = len(qg[0]) if qg else 0
    out = []
    for n in range(len(cu) - 1):
        b, e = cu[n], cu[n + 1]
        L = e - b
        lim = min(L, r_max)
        best = 0
        for h in range(H):
            r_h = lim
            acc = 0
            for r in range(0, lim + 1):
                if r > 0:
                    acc += qg[e - r][h]
                if acc <= thr:
                    r_h = r
                    break
            best = max(best, r_h)
        out.append(max(min(r_min, L), min(best, min(r_max, L))))
    return np.asarray(out, dtype=np.int64)
