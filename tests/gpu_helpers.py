"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle, compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-5, "bf16": 3e-3}   # max relative Frobenius error of S and of o


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(inp: dict, device="cuda") -> dict:
    out = dict(inp)
    for k in ("q", "k", "v", "g", "beta", "cu_seqlens", "r"):
        out[k] = inp[k].to(device)
    return out


def gpu_run(inp: dict, mode: str, with_o=True, S0=None, o_dtype=None):
    import gated_deltanet_state_gdn_amd as gdn
    w = inp["workload"]
    if mode == "replay":
        tot = int(inp["r_host"].sum())
        cu_out = torch.full((len(inp["r_host"]) + 1,), -1, dtype=torch.int32, device=inp["q"].device)
        S, o, cu_out = gdn.gdn_replay(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                      inp["cu_seqlens"], inp["r"], total_out_tokens=tot,
                                      o_out=True if with_o else None, cu_out=cu_out,
                                      scale=w.scale, o_dtype=o_dtype)
        return S, o, cu_out
    S, o = gdn.gdn_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                           S0=S0, o_out=True if with_o else None, scale=w.scale, o_dtype=o_dtype)
    return S, o, None


def oracle_run(inp: dict, mode: str, with_o=True, S0=None):
    w = inp["workload"]
    if mode == "replay":
        return oracle.replay(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_host"],
                             inp["r_host"], scale=w.scale, want_o=with_o)
    return oracle.prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_host"],
                          S0=S0, scale=w.scale, want_o=with_o)


def _rel(a, b):
    nb = np.linalg.norm(b)
    d = np.linalg.norm(a - b)
    return d / nb if nb > 0 else d


def compare(inp: dict, mode: str, S_gpu, o_gpu, S_ref, o_ref):
    """Max over (sequence, v-head) of the relative Frobenius errors of S and of o."""
    S_g = oracle.widen(S_gpu)
    eS = 0.0
    N, H = S_ref.shape[:2]
    for n in range(N):
        for h in range(H):
            eS = max(eS, _rel(S_g[n, h], S_ref[n, h]))
    eo = 0.0
    if o_ref is not None and o_gpu is not None:
        o_g = oracle.widen(o_gpu)
        cu, r = inp["cu_host"], inp["r_host"]
        row = 0
        for n in range(N):
            cnt = int(r[n]) if mode == "replay" else int(cu[n + 1] - cu[n])
            start = row if mode == "replay" else int(cu[n])
            for h in range(H):
                eo = max(eo, _rel(o_g[start:start + cnt, h], o_ref[start:start + cnt, h]))
            row += cnt
    return eS, eo


def rel(a, b):
    return _rel(np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64))


def sampled_refs(inp: dict, pairs, mode: str, with_o=True):
    """Oracle states (and outputs) of sampled (sequence, v-head) chains of a large
    workload, computed in one threaded oracle call with the chains packed as
    one-head sequences.  Replay of a window from zero = prefill of that window."""
    parts = [oracle.chain_inputs(inp, n, h, mode) for (n, h) in pairs]
    lens = [p[0].shape[0] for p in parts]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    cat = [np.concatenate([p[i] for p in parts]) for i in range(5)]
    S, o = oracle.prefill(*cat, cu, scale=inp["workload"].scale, want_o=with_o)
    outs = []
    for j in range(len(pairs)):
        outs.append((S[j, 0], o[cu[j]:cu[j + 1], 0] if o is not None else None))
    return outs


def sampled_compare(inp: dict, mode: str, S_gpu, o_gpu, cu_out, pairs):
    """Max relative errors of S and o over sampled (sequence, head) chains."""
    refs = sampled_refs(inp, pairs, mode, with_o=o_gpu is not None)
    eS, eo = 0.0, 0.0
    for (n, h), (Sr, orf) in zip(pairs, refs):
        eS = max(eS, rel(oracle.widen(S_gpu[n, h]), Sr))
        if o_gpu is not None:
            if mode == "replay":
                r0 = int(cu_out[n]); cnt = int(inp["r_host"][n])
            else:
                r0 = int(inp["cu_host"][n]); cnt = int(inp["cu_host"][n + 1] - inp["cu_host"][n])
            eo = max(eo, rel(oracle.widen(o_gpu[r0:r0 + cnt, h]), orf))
    return eS, eo
