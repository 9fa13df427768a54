"""Pins for the fp64 oracle, independent of the oracle's own code path.

The oracle evaluates the gated delta rule in its rank-1 form
(p = S^T k; S = a S - a b k p^T + b k v^T).  Every check here reaches the same
quantity another way: explicit (I - b k k^T) matrices, exact rational arithmetic,
closed forms of special cases, or invariants the recurrence must satisfy
(Tail-Replay, arXiv 2608.30310: gated updates attenuate older inputs, so a short
recent suffix approximates the state; gist.science technical summary,
"Metodologia" and "Mecanismos Principais").
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import replay_len


def _rand_case(rs, T, h_qk, h_v, dk, dv, unit_keys=True, beta_max=1.0, g_scale=0.3):
    q = rs.standard_normal((T, h_qk, dk))
    k = rs.standard_normal((T, h_qk, dk))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rs.standard_normal((T, h_v, dv))
    g = -g_scale * rs.random((T, h_v))
    beta = beta_max * rs.random((T, h_v))
    return q, k, v, g, beta


def _brute_force_chain(q, k, v, g, beta, S0):
    """S_T = sum_j (A_T...A_{j+1}) beta_j k_j v_j^T + (A_T...A_1) S0 with explicit A_t."""
    T, dk = k.shape
    A = [math.exp(g[t]) * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    outs = []
    for tend in range(1, T + 1):
        S = np.zeros_like(S0)
        for j in range(tend):
            M = np.eye(dk)
            for m in range(j + 1, tend):
                M = A[m] @ M
            S = S + M @ (beta[j] * np.outer(k[j], v[j]))
        M = np.eye(dk)
        for m in range(tend):
            M = A[m] @ M
        S = S + M @ S0
        outs.append(S)
    o = np.stack([outs[t].T @ q[t] for t in range(T)])
    return outs[-1], o


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_explicit_matrices(seed):
    rs = np.random.default_rng(seed)
    T, h_qk, h_v, dk, dv = 7, 1, 2, 3, 4
    q, k, v, g, beta = _rand_case(rs, T, h_qk, h_v, dk, dv, unit_keys=False, beta_max=1.5)
    S0 = rs.standard_normal((1, h_v, dk, dv))
    S, o = oracle.prefill(q, k, v, g, beta, [0, T], S0=S0, scale=1.0)
    for h in range(h_v):
        Sb, ob = _brute_force_chain(q[:, 0], k[:, 0], v[:, h], g[:, h], beta[:, h], S0[0, h])
        assert np.max(np.abs(S[0, h] - Sb)) <= 1e-13 * max(1.0, np.max(np.abs(Sb)))
        assert np.max(np.abs(o[:, h] - ob)) <= 1e-13 * max(1.0, np.max(np.abs(ob)))


def _exact_chain(q, k, v, alpha, beta, S0):
    """Exact rational recurrence S = alpha (I - beta k k^T) S + beta k v^T."""
    dk, dv = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(len(k)):
        kk, vv, a, b = k[t], v[t], alpha[t], beta[t]
        kS = [sum(kk[i] * S[i][j] for i in range(dk)) for j in range(dv)]
        S = [[a * (S[i][j] - b * kk[i] * kS[j]) + b * kk[i] * vv[j] for j in range(dv)]
             for i in range(dk)]
        outs.append([sum(q[t][i] * S[i][j] for i in range(dk)) for j in range(dv)])
    return S, outs


def test_exact_rational_dyadic_inputs_bit_exact():
    # alpha in {0, 1} and small dyadic inputs keep every intermediate exactly
    # representable in binary64, so the oracle must equal exact arithmetic bit for bit.
    rs = np.random.default_rng(5)
    T, dk, dv = 6, 3, 2
    q = rs.integers(-4, 5, (T, dk)) / 4.0
    k = rs.integers(-4, 5, (T, dk)) / 4.0
    v = rs.integers(-8, 9, (T, dv)) / 8.0
    beta = np.array([0.5, 0.25, 1.0, 0.75, 0.5, 0.125])
    g = np.array([0.0, 0.0, -np.inf, 0.0, 0.0, -np.inf])
    S0 = rs.integers(-4, 5, (dk, dv)) / 2.0
    F = Fraction
    Se, oe = _exact_chain([[F(x) for x in r] for r in q], [[F(x) for x in r] for r in k],
                          [[F(x) for x in r] for r in v], [F(0) if x == -np.inf else F(1) for x in g],
                          [F(x) for x in beta], [[F(x) for x in r] for r in S0])
    S, o = oracle.prefill(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None], [0, T],
                          S0=S0[None, None])
    assert all(S[0, 0, i, j] == float(Se[i][j]) for i in range(dk) for j in range(dv))
    assert all(o[t, 0, j] == float(oe[t][j]) for t in range(T) for j in range(dv))


def test_exact_rational_general_alpha():
    # alpha = the binary64 value exp(g) the oracle uses, carried exactly as a Fraction.
    rs = np.random.default_rng(6)
    T, dk, dv = 8, 3, 3
    q, k, v, g, beta = _rand_case(rs, T, 1, 1, dk, dv, unit_keys=True)
    F = Fraction
    Se, oe = _exact_chain([[F(x) for x in r] for r in q[:, 0]], [[F(x) for x in r] for r in k[:, 0]],
                          [[F(x) for x in r] for r in v[:, 0]], [F(math.exp(x)) for x in g[:, 0]],
                          [F(x) for x in beta[:, 0]], [[F(0)] * dv for _ in range(dk)])
    S, o = oracle.prefill(q, k, v, g, beta, [0, T])
    Se = np.array([[float(x) for x in r] for r in Se])
    oe = np.array([[float(x) for x in r] for r in oe])
    assert np.max(np.abs(S[0, 0] - Se)) <= 1e-15 * np.max(np.abs(Se)) * 10
    assert np.max(np.abs(o[:, 0] - oe)) <= 1e-15 * np.max(np.abs(oe)) * 10


def test_closed_form_identity_update_keeps_state():
    # alpha = 1, beta = 0: S_t = S_{t-1}, so S_T = S0 bit for bit and o_t = S0^T q_t.
    rs = np.random.default_rng(7)
    T, dk, dv = 9, 4, 5
    q, k, v, _, _ = _rand_case(rs, T, 2, 2, dk, dv)
    g = np.zeros((T, 2)); beta = np.zeros((T, 2))
    S0 = rs.standard_normal((1, 2, dk, dv))
    S, o = oracle.prefill(q, k, v, g, beta, [0, T], S0=S0, scale=0.5)
    assert np.array_equal(S, S0)
    for h in range(2):
        np.testing.assert_allclose(o[:, h], 0.5 * q[:, h] @ S0[0, h], rtol=1e-14, atol=1e-15)


def test_closed_form_pure_decay():
    # beta = 0: S_T = (prod alpha) S0.
    rs = np.random.default_rng(8)
    T, dk, dv = 11, 3, 3
    q, k, v, g, _ = _rand_case(rs, T, 1, 1, dk, dv, g_scale=0.5)
    beta = np.zeros((T, 1))
    S0 = rs.standard_normal((1, 1, dk, dv))
    S, _ = oracle.prefill(q, k, v, g, beta, [0, T], S0=S0)
    np.testing.assert_allclose(S[0, 0], math.exp(g.sum()) * S0[0, 0], rtol=1e-14)


def test_closed_form_single_token():
    # One token from a zero state writes beta k v^T; o = scale (beta k v^T)^T q.
    rs = np.random.default_rng(9)
    dk, dv = 5, 4
    q, k, v, g, beta = _rand_case(rs, 1, 1, 1, dk, dv)
    S, o = oracle.replay(q, k, v, g, beta, [0, 1], [1], scale=2.0)
    np.testing.assert_allclose(S[0, 0], beta[0, 0] * np.outer(k[0, 0], v[0, 0]), rtol=1e-15)
    np.testing.assert_allclose(o[0, 0], 2.0 * beta[0, 0] * (k[0, 0] @ q[0, 0]) * v[0, 0], rtol=1e-14)


def test_closed_form_orthonormal_keys_beta_one():
    # beta = 1 with orthonormal keys: S_T = sum_j (prod_{m>j} alpha_m) k_j v_j^T and
    # the read-back S_T^T k_T returns v_T exactly (up to rounding).
    rs = np.random.default_rng(10)
    dk, dv, T = 8, 6, 6
    Qm, _ = np.linalg.qr(rs.standard_normal((dk, dk)))
    k = Qm[:, :T].T.copy()[:, None, :]
    q = rs.standard_normal((T, 1, dk))
    v = rs.standard_normal((T, 1, dv))
    g = -0.2 * rs.random((T, 1))
    beta = np.ones((T, 1))
    S, _ = oracle.prefill(q, k, v, g, beta, [0, T])
    ref = sum(math.exp(g[j + 1:, 0].sum()) * np.outer(k[j, 0], v[j, 0]) for j in range(T))
    np.testing.assert_allclose(S[0, 0], ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S[0, 0].T @ k[-1, 0], v[-1, 0], rtol=1e-13, atol=1e-14)


def test_closed_form_repeated_key_overwrites():
    # With alpha = 1 and beta = 1, writing the same unit key twice leaves S^T k = v_last.
    rs = np.random.default_rng(11)
    dk, dv = 6, 5
    kk = rs.standard_normal(dk); kk /= np.linalg.norm(kk)
    k = np.stack([kk, kk])[:, None]
    q = rs.standard_normal((2, 1, dk))
    v = rs.standard_normal((2, 1, dv))
    g = np.zeros((2, 1)); beta = np.ones((2, 1))
    S, _ = oracle.replay(q, k, v, g, beta, [0, 2], [2])
    np.testing.assert_allclose(S[0, 0].T @ kk, v[1, 0], rtol=1e-14, atol=1e-14)


def _rand_packed(rs, lengths, h_qk, h_v, dk, dv, g_scale=0.1):
    T = int(sum(lengths))
    q, k, v, g, beta = _rand_case(rs, T, h_qk, h_v, dk, dv, g_scale=g_scale)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    return q, k, v, g, beta, cu


def test_invariant_alpha_zero_makes_replay_exact():
    # An alpha = 0 token at p inside the replay window erases all history before p,
    # so replay from zero equals full prefill exactly.
    rs = np.random.default_rng(12)
    L, r = 40, 15
    q, k, v, g, beta, cu = _rand_packed(rs, [L], 1, 3, 4, 5)
    g[L - 10, 0] = -np.inf          # inside the window, head 0
    g[L - r, 1] = -np.inf           # at the first window token, head 1
    g[L - r - 1, 2] = -np.inf       # just before the window, head 2: not exact
    Sf, of = oracle.prefill(q, k, v, g, beta, cu)
    Sr, orr = oracle.replay(q, k, v, g, beta, cu, [r])
    assert np.array_equal(Sf[0, 0], Sr[0, 0]) and np.array_equal(Sf[0, 1], Sr[0, 1])
    # o rows from the reset on agree too (replay rows start at L - r)
    assert np.array_equal(of[L - 10:, 0], orr[r - 10:, 0])
    assert not np.array_equal(Sf[0, 2], Sr[0, 2])


@pytest.mark.parametrize("r", [1, 5, 20, 60])
def test_invariant_attenuation_bound(r):
    # ||S_full - S_replay||_F <= prod_{window} alpha * ||S_before||_F for unit keys and
    # beta in [0, 1]: (I - beta k k^T) is a contraction, so the difference of two runs
    # started from S_before and from 0 shrinks at least by alpha per step.
    rs = np.random.default_rng(100 + r)
    L = 80
    q, k, v, g, beta, cu = _rand_packed(rs, [L], 2, 2, 6, 5, g_scale=0.05)
    Sf, _ = oracle.prefill(q, k, v, g, beta, cu)
    Sr, _ = oracle.replay(q, k, v, g, beta, cu, [r])
    Sb, _ = oracle.prefill(q[:L - r], k[:L - r], v[:L - r], g[:L - r], beta[:L - r], [0, L - r])
    for h in range(2):
        bound = math.exp(g[L - r:, h].sum()) * np.linalg.norm(Sb[0, h])
        assert np.linalg.norm(Sf[0, h] - Sr[0, h]) <= bound * (1 + 1e-12)


def test_invariant_composition_split_prefill():
    # prefill(0..m) then prefill(m..L, S0 = S_m) equals prefill(0..L) exactly.
    rs = np.random.default_rng(13)
    L, m = 33, 14
    q, k, v, g, beta, cu = _rand_packed(rs, [L], 2, 4, 4, 3)
    Sf, of = oracle.prefill(q, k, v, g, beta, cu)
    S1, o1 = oracle.prefill(q[:m], k[:m], v[:m], g[:m], beta[:m], [0, m])
    S2, o2 = oracle.prefill(q[m:], k[m:], v[m:], g[m:], beta[m:], [0, L - m], S0=S1)
    assert np.array_equal(S2, Sf)
    assert np.array_equal(np.concatenate([o1, o2]), of)


def test_invariant_full_and_empty_replay():
    rs = np.random.default_rng(14)
    lengths = [7, 0, 12, 3]
    q, k, v, g, beta, cu = _rand_packed(rs, lengths, 1, 2, 4, 4)
    Sf, of = oracle.prefill(q, k, v, g, beta, cu)
    Sr, orr = oracle.replay(q, k, v, g, beta, cu, lengths)
    assert np.array_equal(Sf, Sr) and np.array_equal(of, orr)
    S0, o0 = oracle.replay(q, k, v, g, beta, cu, [0, 0, 0, 0])
    assert not S0.any() and o0.shape[0] == 0


def test_invariant_packing_order_and_gva():
    rs = np.random.default_rng(15)
    lengths = [9, 4, 13]
    q, k, v, g, beta, cu = _rand_packed(rs, lengths, 2, 4, 4, 3)
    r = [5, 4, 2]
    S, o = oracle.replay(q, k, v, g, beta, cu, r)
    # reverse the packing order
    segs = [slice(cu[i], cu[i + 1]) for i in range(3)][::-1]
    cat = lambda a: np.concatenate([a[s] for s in segs])
    cu2 = np.concatenate([[0], np.cumsum(lengths[::-1])])
    S2, _ = oracle.replay(cat(q), cat(k), cat(v), cat(g), cat(beta), cu2, r[::-1])
    assert np.array_equal(S2[::-1], S)
    # GVA (2 q/k heads shared by 4 v heads) equals MHA with duplicated q/k heads
    qd = np.repeat(q, 2, axis=1); kd = np.repeat(k, 2, axis=1)
    S3, o3 = oracle.replay(qd, kd, v, g, beta, cu, r)
    assert np.array_equal(S3, S) and np.array_equal(o3, o)


def test_thread_count_does_not_change_results():
    rs = np.random.default_rng(16)
    q, k, v, g, beta, cu = _rand_packed(rs, [30, 17], 2, 4, 8, 8)
    S1, o1 = oracle.prefill(q, k, v, g, beta, cu, threads=1)
    S8, o8 = oracle.prefill(q, k, v, g, beta, cu, threads=8)
    assert np.array_equal(S1, S8) and np.array_equal(o1, o8)


def test_relerr_definition():
    rs = np.random.default_rng(17)
    A = rs.standard_normal((3, 4, 5)); B = rs.standard_normal((3, 4, 5))
    e, nf = oracle.state_relerr(A, B)
    for i in range(3):
        assert abs(e[i] - np.linalg.norm(A[i] - B[i]) / np.linalg.norm(B[i])) < 1e-15
    e0, _ = oracle.state_relerr(np.zeros((2, 2)), np.zeros((2, 2)))
    assert e0 == 0.0
    A[1, 2, 3] = np.nan
    assert oracle.state_relerr(A, B)[1] == 1


def test_replay_length_rule():
    # r = ceil(rho * L): 10% of 2048 -> 205, 5% of 8192 -> 410, 10% of 32768 -> 3277,
    # and the slow-decay sweep 1/2/5/10/20% of 32768.
    assert replay_len(2048, 0.10) == 205
    assert replay_len(8192, 0.05) == 410
    assert replay_len(32768, 0.10) == 3277
    assert [replay_len(32768, x) for x in (0.01, 0.02, 0.05, 0.10, 0.20)] == \
        [328, 656, 1639, 3277, 6554]
    assert replay_len(100, 0.0) == 0 and replay_len(100, 1.0) == 100 and replay_len(0, 0.1) == 0


def test_oracle_rejects_bad_windows():
    rs = np.random.default_rng(18)
    q, k, v, g, beta, cu = _rand_packed(rs, [5, 6], 1, 1, 2, 2)
    with pytest.raises(ValueError):
        oracle.replay(q, k, v, g, beta, cu, [6, 1])
    with pytest.raises(ValueError):
        oracle.replay(q, k, v, g, beta, cu, [-1, 1])
