"""The chunked (UT/WY) form the GPU evaluates equals the token-by-token oracle.

Pins the algebra of the chunk decomposition -- reset-aware in-chunk gates, the
(I + A)^{-1} triangular solve, the inter-chunk state pass and the output split
-- before any kernel exists.  Also runs the bf16 precision model at reduced size.
"""
import numpy as np
import pytest

import oracle
from chunked_model import F16_OPERANDS, Policy, bf16, chunk_chain, f16, gates, split


def _case(rs, T, dk, dv, g_mu=-4.0, g_sigma=1.0):
    q = rs.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rs.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rs.standard_normal((T, dv))
    g = -np.log1p(np.exp(g_mu + g_sigma * rs.standard_normal(T)))
    beta = 1.0 / (1.0 + np.exp(-rs.standard_normal(T)))
    return q, k, v, g, beta


def _oracle_chain(q, k, v, g, beta, S0=None, scale=1.0):
    T = len(k)
    S, o = oracle.prefill(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None], [0, T],
                          S0=None if S0 is None else S0[None, None], scale=scale)
    return S[0, 0], o[:, 0]


@pytest.mark.parametrize("T,C", [(300, 64), (64, 64), (63, 64), (1, 64), (129, 16), (77, 8)])
def test_chunked_equals_token_recurrence(T, C):
    rs = np.random.default_rng(T * 31 + C)
    dk, dv = 16, 24
    q, k, v, g, beta = _case(rs, T, dk, dv)
    S0 = rs.standard_normal((dk, dv))
    S, o = _oracle_chain(q, k, v, g, beta, S0, scale=0.7)
    Sc, oc = chunk_chain(q, k, v, g, beta, S0, C=C, scale=0.7)
    assert np.linalg.norm(Sc - S) <= 1e-12 * np.linalg.norm(S)
    assert np.linalg.norm(oc - o) <= 1e-12 * np.linalg.norm(o)


def test_chunked_with_resets():
    # alpha = 0 tokens at a chunk start, mid-chunk, chunk end and twice in one chunk.
    rs = np.random.default_rng(3)
    T, dk, dv, C = 256, 8, 8, 64
    q, k, v, g, beta = _case(rs, T, dk, dv)
    for p in (0, 64, 100, 127, 130, 131, 255):
        g[p] = -np.inf
    S, o = _oracle_chain(q, k, v, g, beta)
    Sc, oc = chunk_chain(q, k, v, g, beta, C=C)
    assert np.isfinite(Sc).all() and np.isfinite(oc).all()
    assert np.linalg.norm(Sc - S) <= 1e-12 * np.linalg.norm(S)
    assert np.linalg.norm(oc - o) <= 1e-12 * np.linalg.norm(o)


def test_gate_scan_definition():
    g = np.array([-0.1, -0.2, -np.inf, -0.3, -0.4])
    H, e, G = gates(g)
    assert np.allclose(H, [-0.1, -0.3, 0.0, -0.3, -0.7])
    assert np.allclose(e, [np.exp(-0.1), np.exp(-0.3), 0, 0, 0])
    # G_ij = prod_{m=j+1..i} alpha_m
    alpha = np.exp(g)
    for i in range(5):
        for j in range(5):
            ref = np.prod(alpha[j + 1:i + 1]) if j <= i else 0.0
            assert abs(G[i, j] - ref) < 1e-15


def test_bf16_rounding_helper():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-30])
    r = bf16(x)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 4 * 2 ** -8 and r[3] == -2.5
    hi, lo = split(np.pi)
    assert abs(hi + lo - np.pi) < 2 ** -16 * np.pi
    # binary16: 11 significant bits, ties to even, 2^-24 the smallest subnormal
    h = f16(np.array([1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 65504.0, 2 ** -24, -0.1]))
    assert h[0] == 1.0 and h[1] == 1.0 + 2 ** -9 and h[2] == 65504.0 and h[3] == 2 ** -24
    assert abs(h[4] + 0.1) <= 2 ** -15


@pytest.mark.slow
@pytest.mark.parametrize("g_mu,g_sigma", [(-5.0, 1.0), (-8.0, 0.5), (-2.0, 1.0)])
def test_precision_layout_meets_bf16_tolerance(g_mu, g_sigma):
    """The fp16-operand layout of the bf16 path stays well within 3e-3 on S and on o.

    Reduced size (d = 128, T = 1024; the stack's, the slow-decay and a fast-decay gate
    distribution); the full-size checks run on the GPU against the oracle.  The margin
    asked for here (S < 1e-3, o < 2.2e-3 with bf16-rounded o, whose own rounding floor is
    ~1.7e-3) leaves the GPU's summation order room.
    """
    rs = np.random.default_rng(21)
    T, d = 1024, 128
    q, k, v, g, beta = _case(rs, T, d, d, g_mu=g_mu, g_sigma=g_sigma)
    q, k, v = bf16(q), bf16(k), bf16(v)
    S, o = _oracle_chain(q, k, v, g, beta)
    Sc, oc = chunk_chain(q, k, v, g, beta, pol=F16_OPERANDS)
    eS = np.linalg.norm(Sc - S) / np.linalg.norm(S)
    eo = np.linalg.norm(oc - o) / np.linalg.norm(o)
    assert eS < 1e-3 and eo < 2.2e-3, (eS, eo)
