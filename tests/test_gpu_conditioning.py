"""GPU parity with correlated and repeated keys, against the fp64 oracle.

i.i.d. random unit keys (pairwise cosines ~0.09 at d = 128) are the best-conditioned input
the chunk's UT transform (I + strict_lower(diag(b) K K^T o Gamma))^{-1} can see.  The
keys of a real Gated DeltaNet layer are correlated (a short convolution and a SiLU
precede their L2 norm), so these cases draw keys with mean pairwise cosine 0.5-0.95 and,
at the extreme, one key repeated for every token of a head.  A repeated key with
beta = 1 has a closed form: each token overwrites the state along the key, so
S^T k = v of the last token (up to the key's rounding to bf16: |k|^2 = 1 + O(2^-9)).

Tolerances: relative Frobenius error of S and of o <= 3e-3 (bf16 inputs), <= 1e-5 (fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, compare, gpu_run, oracle_run, rel, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_deltanet_state_gdn_amd as gdn
    gdn.load()
    yield


def _run(w, mode):
    inp = W.make_inputs(w)
    say("case", w.name, mode, "key_corr", w.key_corr, "beta", w.beta_value, "L", list(w.lengths),
        "r", list(w.replay), "mu", w.g_mu)
    S, o, _ = gpu_run(to_dev(inp), mode)
    torch.cuda.synchronize()
    S_ref, o_ref = oracle_run(inp, mode)
    eS, eo = compare(inp, mode, S, o, S_ref, o_ref)
    say("  relerr S %.3e  o %.3e" % (eS, eo))
    return inp, S, o, eS, eo


@pytest.mark.parametrize("corr", [0.5, 0.8, 0.9, 0.95])
@pytest.mark.parametrize("g_mu,g_sigma", [(-5.0, 1.0), (-8.0, 0.5)])
def test_bf16_correlated_keys(corr, g_mu, g_sigma):
    w = W.small(W.config(1), L=[1500, 700], r=[1200, 700], h_qk=2, h_v=4, g_mu=g_mu,
                g_sigma=g_sigma, key_corr=corr)
    for mode in ("replay", "prefill"):
        _, _, _, eS, eo = _run(w, mode)
        assert eS <= TOL["bf16"] and eo <= TOL["bf16"], (mode, eS, eo)


def test_bf16_repeated_key_beta_one_overwrites():
    # One key per head for every token, beta = 1, alpha ~ 0.95 (g = -softplus(N(-3, 1))).
    # A repeated key never contracts errors orthogonal to itself (only the gate does), and
    # each chunk's state update is then a telescoping sum sum_j G k (v_j - a v_{j-1}) whose
    # fp16-rounded terms cancel down to one v: the CPU model of the kernel's arithmetic
    # puts this case at S 1.6e-3 / o 2.1e-3 here, and at 2.9e-3 under the stack's slower
    # gates (alpha ~ 0.993), the edge of the bf16 tolerance, which is why it runs here.
    w = W.small(W.config(2), L=[1000, 333], r=[1000, 333], h_qk=2, h_v=4, key_corr=1.0,
                beta_value=1.0, g_mu=-3.0)
    inp, S, o, eS, eo = _run(w, "prefill")
    assert eS <= TOL["bf16"] and eo <= TOL["bf16"], (eS, eo)
    cu = inp["cu_host"]
    for n in range(2):
        last = int(cu[n + 1]) - 1
        for h in range(4):
            k = oracle.widen(inp["k"][last, h // 2])
            v = oracle.widen(inp["v"][last, h])
            e = rel(oracle.widen(S[n, h]).T @ k, v)
            assert e <= TOL["bf16"], (n, h, e)
    say("  S^T k = v_last within 3e-3 for every (sequence, head)")


def test_bf16_repeated_key_random_beta():
    w = W.small(W.config(1), L=[1200], r=[900], h_qk=2, h_v=2, key_corr=1.0)
    for mode in ("replay", "prefill"):
        _, _, _, eS, eo = _run(w, mode)
        assert eS <= TOL["bf16"] and eo <= TOL["bf16"], (mode, eS, eo)


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("corr", [0.9, 1.0])
def test_fp32_correlated_and_repeated_keys(dk, corr):
    w = W.small(W.config(0), L=[700, 200], r=[600, 77], h_qk=2, h_v=4, d_k=dk, d_v=dk,
                key_corr=corr, beta_value=1.0 if corr == 1.0 else None)
    for mode in ("replay", "prefill"):
        _, _, _, eS, eo = _run(w, mode)
        assert eS <= TOL["f32"] and eo <= TOL["f32"], (mode, eS, eo)
