"""GPU: adaptive replay length (gdn_adaptive_replay_len) against the oracle's rule.

The result is an integer decided by exact integer sums on both sides, so the
comparison is bit-exact.  Gates follow the workloads' recipe g = -softplus(mu + sigma x)
with the (mu, sigma) pairs of the fast- and slow-decay workloads, optionally with one
alpha = 0 token per head.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_deltanet_state_gdn_amd as gdn
    gdn.load()
    yield


def _gates(lens, h_v, mu, sigma, seed, resets=False):
    gen = torch.Generator().manual_seed(seed)
    T = int(sum(lens))
    g = -torch.nn.functional.softplus(mu + sigma * torch.randn((T, h_v), generator=gen))
    if resets:
        rs = np.random.default_rng(seed)
        cu = np.concatenate([[0], np.cumsum(lens)])
        for n, L in enumerate(lens):
            if L > 0:
                for h in range(h_v):
                    g[int(cu[n]) + int(rs.integers(0, L)), h] = float("-inf")
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return g.contiguous(), cu


def _run(g, cu, eps, r_min=0, r_max=2 ** 31 - 1):
    import gated_deltanet_state_gdn_amd as gdn
    gd = g.cuda()
    cud = torch.as_tensor(cu.astype(np.int32)).cuda()
    n = len(cu) - 1
    d = gdn.GdnDesc()
    d.n_seqs, d.h_v, d.total_tokens = n, int(g.shape[1]), int(g.shape[0])
    ws = gdn.workspace(d, gd.device)
    r = gdn.gdn_adaptive_replay_len(gd, cud, eps=eps, r_min=r_min, r_max=r_max, ws=ws)
    st = gdn.gdn_device_status(ws)
    return r.cpu().numpy().astype(np.int64), st


@pytest.mark.parametrize("mu,sigma,resets", [(-5.0, 1.0, False), (-5.0, 1.0, True),
                                             (-3.0, 2.0, False)])
def test_varlen_matches_oracle(mu, sigma, resets):
    rs = np.random.default_rng(7)
    lens = [int(x) for x in rs.integers(0, 3000, size=64)]
    lens[3] = 0
    lens[10] = 1
    g, cu = _gates(lens, 16, mu, sigma, seed=11, resets=resets)
    for eps in (0.5, 1e-3, 1e-8):
        say("case varlen64 mu", mu, "sigma", sigma, "resets", resets, "eps", eps)
        r, st = _run(g, cu, eps)
        want = oracle.adaptive_replay_len(g, cu, eps)
        assert st == 0
        assert np.array_equal(r, want), np.nonzero(r != want)


@pytest.mark.parametrize("resets", [False, True])
def test_slow_decay_full_size(resets):
    w = W.config(4)
    L = int(w.lengths[0])
    g, cu = _gates([L], w.h_v, w.g_mu, w.g_sigma, seed=w.seed, resets=resets)
    for eps, r_max in ((1e-3, 2 ** 31 - 1), (1e-3, 3277), (0.1, 2 ** 31 - 1)):
        say("case slow-decay L", L, "resets", resets, "eps", eps, "r_max", r_max)
        r, st = _run(g, cu, eps, r_max=r_max)
        want = oracle.adaptive_replay_len(g, cu, eps, r_max=r_max)
        say("  r", int(r[0]), "oracle", int(want[0]))
        assert st == 0 and np.array_equal(r, want)


def test_edges():
    lens = [0, 1, 5, 64, 65, 511, 512, 513, 1000]
    for h_v in (1, 3, 48):
        g, cu = _gates(lens, h_v, -2.0, 1.0, seed=h_v)
        g[int(cu[2]) + 4, :] = float("-inf")        # last token of the 5-token sequence
        g[int(cu[3]) + 10, :] = float("nan")        # NaN counts as no attenuation
        g[int(cu[4]) + 3, 0] = 0.25                 # positive counts as 0
        for eps, r_min, r_max in ((1.0, 0, 2 ** 31 - 1), (3.0, 7, 2 ** 31 - 1), (0.2, 0, 0),
                                  (0.01, 600, 2 ** 31 - 1), (1e-4, 3, 100), (1e-300, 0, 2 ** 31 - 1)):
            say("case edges h_v", h_v, "eps", eps, "r_min", r_min, "r_max", r_max)
            r, st = _run(g, cu, eps, r_min=r_min, r_max=r_max)
            want = oracle.adaptive_replay_len(g, cu, eps, r_min=r_min, r_max=r_max)
            assert st == 0 and np.array_equal(r, want), (r, want)
        assert _run(g, cu, 0.5)[0][2] == 1          # alpha = 0 on the last token


def test_bad_cu_sets_status():
    lens = [100, 200, 300]
    g, cu = _gates(lens, 4, -4.0, 1.0, seed=5)
    bad = cu.copy()
    bad[2] = bad[1] - 1                            # sequence 1 ends before it starts
    say("case bad cu")
    r, st = _run(g, bad, 1e-2)
    assert st == 8
    assert r[1] == 0
    want = oracle.adaptive_replay_len(g, cu, 1e-2)
    assert r[0] == want[0]


def test_replay_with_chosen_length_meets_bound():
    # fp32 inputs (error floor ~1e-6): the replayed state is within eps * ||S_before||
    import gated_deltanet_state_gdn_amd as gdn
    w = W.small(W.config(0), L=[4096], r=[1])
    inp = W.make_inputs(w, device="cuda")
    L = 4096
    for eps in (1e-1, 1e-3):
        say("case bound eps", eps)
        r = gdn.gdn_adaptive_replay_len(inp["g"], inp["cu_seqlens"], eps=eps)
        rn = int(r.cpu()[0])
        want = oracle.adaptive_replay_len(inp["g"].cpu(), inp["cu_host"], eps)
        assert rn == int(want[0]) and 0 < rn < L
        S_rep, _, _ = gdn.gdn_replay(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     inp["cu_seqlens"], r, total_out_tokens=rn, o_out=None)
        S_full, _ = gdn.gdn_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                    inp["cu_seqlens"], o_out=None)
        sl = slice(0, L - rn)
        cub = torch.tensor([0, L - rn], dtype=torch.int32, device="cuda")
        S_bef, _ = gdn.gdn_prefill(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["g"][sl],
                                   inp["beta"][sl], cub, o_out=None)
        torch.cuda.synchronize()
        for h in range(w.h_v):
            err = float((S_full[0, h].double() - S_rep[0, h].double()).norm())
            bound = eps * float(S_bef[0, h].double().norm())
            slack = 1e-5 * float(S_full[0, h].double().norm())
            say("  head", h, "r", rn, "err %.3e bound %.3e" % (err, bound))
            assert err <= bound + slack
