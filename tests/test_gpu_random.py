"""Seeded random small cases of every call against the fp64 oracle.

Each case draws its own shape and statistics: storage dtype (bf16 / fp32), d_k and d_v in
{64, 128} independently, 1, 2 or 4 q/k heads with 1, 2 or 3 v-heads each, 1-6 packed
sequences of 1-499 tokens with replay lengths from 0 to the whole sequence, the decay
regime (gate mean -2, 0 or +3 before the softplus), key correlation (0, 0.5 or 0.9), resets
(none, one per head anywhere, or inside the window) and the output scale (1 or 0.5); then
one call: replay with outputs, replay of the state only, prefill from a zero or a random
state, or the segmented replay with 1-10 segments (square states).  Every case is checked
at the tolerance of its dtype (relative Frobenius error per sequence and head, as all
parity tests).  The draws are seeded, so the cases are the same on every run.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import TOL, compare, oracle_run, say

pytestmark = pytest.mark.gpu

N_CASES = 150


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_deltanet_state_gdn_amd as gdn
    gdn.load()
    yield


def _cases(seed=2026, n=N_CASES):
    rs = np.random.default_rng(seed)
    out = []
    for ci in range(n):
        dtype = ["bf16", "f32"][rs.integers(0, 2)]
        dk = int(rs.choice([64, 128]))
        dv = int(rs.choice([64, 128]))
        h_qk = int(rs.choice([1, 2, 4]))
        h_v = h_qk * int(rs.choice([1, 2, 3]))
        ns = int(rs.integers(1, 7))
        L = [int(x) for x in rs.integers(1, 500, size=ns)]
        r = [int(rs.integers(0, x + 1)) for x in L]
        mu = float(rs.choice([-2.0, 0.0, 3.0]))
        kc = float(rs.choice([0.0, 0.0, 0.5, 0.9]))
        resets = bool(rs.integers(0, 2))
        scale = float(rs.choice([1.0, 1.0, 0.5]))
        base = W.config(1) if dtype == "bf16" else W.config(0)
        w = W.small(base, L, r, h_qk=h_qk, h_v=h_v, d_k=dk, d_v=dv, dtype=dtype,
                    seed=int(rs.integers(1, 1 << 30)), g_mu=mu, key_corr=kc, reset_heads=resets,
                    reset_in_window=resets and bool(rs.integers(0, 2)), scale=scale)
        modes = ["replay", "replay_S", "prefill"] + (["segmented"] if dk == dv else [])
        mode = modes[rs.integers(0, len(modes))]
        P = int(rs.integers(1, 11))
        s0 = bool(rs.integers(0, 2)) if mode == "prefill" else False
        out.append((ci, w, mode, P, s0))
    return out


def test_random_cases_against_the_oracle():
    import gated_deltanet_state_gdn_amd as gdn
    worst = {}
    for ci, w, mode, P, s0 in _cases():
        say("case %d: %s d_k %d d_v %d h_qk %d h_v %d, %d seqs, mu %g, key corr %g, resets %s, scale %g, %s%s"
            % (ci, w.dtype, w.d_k, w.d_v, w.h_qk, w.h_v, len(w.lengths), w.g_mu, w.key_corr, w.reset_heads,
               w.scale, mode, " P %d" % P if mode == "segmented" else ""))
        inp = W.make_inputs(w, device="cuda")
        host = dict(inp)
        for key in ("q", "k", "v", "g", "beta"):
            host[key] = inp[key].cpu()
        tot = int(inp["r_host"].sum())
        args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"])
        if mode in ("replay", "replay_S"):
            want_o = mode == "replay"
            S, o, _ = gdn.gdn_replay(*args, inp["r"], total_out_tokens=tot, o_out=True if want_o else None,
                                     scale=w.scale)
            S_ref, o_ref = oracle_run(host, "replay", with_o=want_o)
            kind = "replay"
        elif mode == "prefill":
            S0 = None
            if s0:
                S0 = torch.randn((len(w.lengths), w.h_v, w.d_k, w.d_v), dtype=torch.float32,
                                 generator=torch.Generator().manual_seed(ci)) * 0.1
            S, o = gdn.gdn_prefill(*args, S0=None if S0 is None else S0.cuda(), scale=w.scale)
            S_ref, o_ref = oracle_run(host, "prefill", S0=None if S0 is None else S0.double().numpy())
            kind = "prefill"
        else:
            S, o, _ = gdn.gdn_replay_segmented(*args, inp["r"], total_out_tokens=tot, n_segments=P, scale=w.scale)
            S_ref, o_ref = oracle_run(host, "replay")
            kind = "replay"
        torch.cuda.synchronize()
        eS, eo = compare(host, kind, S.cpu(), None if o is None else o.cpu(), S_ref, o_ref)
        say("  relerr S %.3e  o %.3e" % (eS, eo))
        tol = TOL[w.dtype]
        assert np.isfinite(eS) and np.isfinite(eo) and eS <= tol and eo <= tol, (ci, mode, eS, eo)
        key = (w.dtype, mode)
        worst[key] = max(worst.get(key, 0.0), eS, eo)
    for key in sorted(worst):
        say("worst %s %s: %.3e" % (key[0], key[1], worst[key]))
