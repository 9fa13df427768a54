"""Pins for the oracle's adaptive replay length (``oracle.adaptive_replay_len``).

The rule: the shortest tail whose gates multiply to at most eps in every v-head
(Tail-Replay, arXiv 2608.30310, abstract: gated updates attenuate distant tokens, so
the older state reaches the boundary scaled by at most prod alpha for unit keys and
beta in [0, 1]).  Checked here against closed forms (constant gates, a reset token),
against the products of alpha computed directly in floating point, and against the
recurrence itself: replaying the chosen window is within eps * ||S_before|| of full
prefill.
"""
import math

import numpy as np
import pytest

import oracle


def test_constant_gate_closed_form():
    # g = -2^-7 is exact in fp32 and in 2^-32 units: r = ceil(-ln(eps) / 2^-7)
    c = 2.0 ** -7
    g = np.full((5000, 3), -c, dtype=np.float32)
    for eps in (0.5, 0.1, 1e-3, 1e-6, 1e-12):
        want = math.ceil(-math.log(eps) / c)
        assert want < 5000
        assert oracle.adaptive_replay_len(g, [0, 5000], eps)[0] == want, eps
    # too short to reach eps: the whole sequence; a cap wins over the rule
    assert oracle.adaptive_replay_len(g[:100], [0, 100], 1e-3)[0] == 100
    assert oracle.adaptive_replay_len(g, [0, 5000], 1e-3, r_max=300)[0] == 300
    assert oracle.adaptive_replay_len(g, [0, 5000], 1e-3, r_min=2000)[0] == 2000


def test_reset_token_stops_the_window():
    # alpha = 0 at position p: the window must reach back exactly to it
    # in every head; the sequence's length is the longest head's
    L, p0, p1 = 700, 123, 400
    g = np.full((L, 2), -1e-6, dtype=np.float32)
    g[p0, 0] = -np.inf
    g[p1, 1] = -np.inf
    assert oracle.adaptive_replay_len(g, [0, L], 1e-2)[0] == L - p0
    g[p0, 0] = -5e6         # below -2^20 nats: also alpha ~ 0
    assert oracle.adaptive_replay_len(g, [0, L], 1e-2)[0] == L - p0
    g[p0, 0] = -1e-6        # head 0 never reaches eps: the whole sequence
    assert oracle.adaptive_replay_len(g, [0, L], 1e-2)[0] == L


def test_eps_at_least_one_and_empty_sequences():
    g = np.full((10, 2), -0.5, dtype=np.float32)
    assert list(oracle.adaptive_replay_len(g, [0, 0, 10, 10], 1.0)) == [0, 0, 0]
    assert list(oracle.adaptive_replay_len(g, [0, 0, 10, 10], 2.0, r_min=4)) == [0, 4, 0]
    # positive / NaN gates count as no attenuation
    g2 = np.array([[0.3], [np.nan], [-1.0]], dtype=np.float32)
    assert oracle.adaptive_replay_len(g2, [0, 3], math.exp(-0.5))[0] == 1
    assert oracle.adaptive_replay_len(g2, [0, 3], math.exp(-1.5))[0] == 3


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_minimal_window_against_float_products(seed):
    rs = np.random.default_rng(seed)
    H = 4
    lens = [int(x) for x in rs.integers(0, 400, size=5)]
    cu = np.concatenate([[0], np.cumsum(lens)])
    g = (-np.log1p(np.exp(rs.normal(-3.0, 1.0, size=(int(cu[-1]), H))))).astype(np.float32)
    for eps in (0.3, 1e-2, 1e-4):
        r = oracle.adaptive_replay_len(g, cu, eps)
        for n in range(len(lens)):
            b, e = int(cu[n]), int(cu[n + 1])
            prod = lambda m, h: math.prod(math.exp(float(g[t, h])) for t in range(e - m, e))
            rn = int(r[n])
            assert 0 <= rn <= e - b
            if rn < e - b:   # the window reaches eps in every head ...
                assert all(prod(rn, h) <= eps * (1 + 1e-7) for h in range(H))
            if rn > 0:       # ... and one token fewer does not
                assert any(prod(rn - 1, h) > eps * (1 - 1e-7) for h in range(H))


@pytest.mark.parametrize("seed", [0, 1])
def test_replay_error_within_eps_of_older_state(seed):
    rs = np.random.default_rng(seed)
    T, h_qk, h_v, dk, dv = 260, 1, 2, 8, 6
    q = rs.standard_normal((T, h_qk, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rs.standard_normal((T, h_qk, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rs.standard_normal((T, h_v, dv))
    g = (-0.06 * rs.random((T, h_v))).astype(np.float32).astype(np.float64)
    beta = rs.random((T, h_v))
    for eps in (0.5, 0.1, 0.02):
        r = int(oracle.adaptive_replay_len(g, [0, T], eps)[0])
        assert 0 < r < T
        S_full, _ = oracle.prefill(q, k, v, g, beta, [0, T], want_o=False)
        S_rep, _ = oracle.replay(q, k, v, g, beta, [0, T], [r], want_o=False)
        S_bef, _ = oracle.prefill(q[:T - r], k[:T - r], v[:T - r], g[:T - r], beta[:T - r],
                                  [0, T - r], want_o=False)
        for h in range(h_v):
            err = np.linalg.norm(S_full[0, h] - S_rep[0, h])
            assert err <= eps * np.linalg.norm(S_bef[0, h]) * (1 + 1e-9) + 1e-12
