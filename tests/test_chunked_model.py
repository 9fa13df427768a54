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


# ---------------------------------------------------------------------------------------
# The model of the kernel's own arithmetic (kernel_chain): its algebra, then the two
# numerical choices it pins -- the gate scan of fp32 inputs and the diagonal-block inverse.

from chunked_model import diag_inverse_model, f32, gate_scan_f32, kernel_chain, kernel_gates


def _keys(rs, T, d, corr):
    """Unit keys with mean pairwise cosine ~corr: normalise(a u + z), a^2 = corr d / (1 - corr),
    u a fixed unit direction, z ~ N(0, I); corr = 1 repeats one key."""
    z = rs.standard_normal((T, d))
    u = rs.standard_normal(d)
    u /= np.linalg.norm(u)
    if corr >= 1.0:
        z[:] = z[0]
    elif corr > 0.0:
        z = z + np.sqrt(corr * d / (1.0 - corr)) * u
    return z / np.linalg.norm(z, axis=1, keepdims=True)


def _corr_case(seed, T, d, corr, g_mu=-5.0, g_sigma=1.0, store=bf16):
    rs = np.random.default_rng(seed)
    q = rs.standard_normal((T, d)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = _keys(rs, T, d, corr)
    v = rs.standard_normal((T, d))
    g = f32(-np.log1p(np.exp(g_mu + g_sigma * rs.standard_normal(T))))
    beta = f32(1.0 / (1.0 + np.exp(-rs.standard_normal(T))))
    return store(q), store(k), store(v), g, beta


def _rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


@pytest.mark.parametrize("T", [1, 63, 64, 200])
def test_kernel_model_algebra_equals_token_recurrence(T):
    # no rounding anywhere: the 16-row block substitution with the two-level inverse of
    # the diagonal blocks is the chunk form, i.e. the token recurrence, to fp64 precision
    q, k, v, g, beta = _corr_case(T, T, 32, 0.6, g_mu=-3.0, store=lambda x: x)
    g[T // 3] = -np.inf
    S, o = _oracle_chain(q, k, v, g, beta, scale=0.5)
    Sc, oc = kernel_chain(q, k, v, g, beta, scale=0.5, path="f64")
    assert _rel(Sc, S) <= 1e-12 and _rel(oc, o) <= 1e-12


@pytest.mark.parametrize("corr", [0.0, 0.9, 1.0])
def test_diag_inverse_two_level_neumann_is_exact(corr):
    # T = (I - D)^{-1} (I - G)^{-1} with D the 4x4 diagonal blocks of N: exact in exact
    # arithmetic (both series terminate), for any strictly lower N
    rs = np.random.default_rng(4)
    K = _keys(rs, 16, 64, corr)
    b = rs.random(16)
    N = -np.tril(b[:, None] * (K @ K.T), -1)
    ex = diag_inverse_model(N, "exact", lambda x: x)
    assert np.max(np.abs(ex + np.eye(16) - np.linalg.inv(np.eye(16) - N))) < 1e-12
    for inv in ("prod", "blk4", "blk4g", "blk4g9"):
        assert np.max(np.abs(diag_inverse_model(N, inv, lambda x: x) - ex)) <= 1e-11 * max(1, np.abs(ex).max())


def test_diag_inverse_fp16_operands_by_key_correlation():
    # With fp16 operands the single-level product (I+N)(I+N^2)(I+N^4)(I+N^8) loses T to
    # cancellation once keys are correlated (its terms grow like binomial coefficients),
    # while the two-level form the kernel uses keeps every intermediate O(1).
    rs = np.random.default_rng(9)
    worst = {}
    for corr in (0.0, 0.9, 1.0):
        K = bf16(_keys(rs, 16, 128, corr))
        b = f32(rs.uniform(0.5, 1.0, 16))
        N = f32(-np.tril(b[:, None] * (K @ K.T), -1))
        ex = diag_inverse_model(N, "exact", lambda x: x)
        scale = max(1.0, np.abs(ex).max())
        worst[corr] = {inv: np.abs(diag_inverse_model(N, inv, f16) - ex).max() / scale
                       for inv in ("prod", "blk4g9")}
    assert worst[0.0]["prod"] < 2e-3 and worst[0.0]["blk4g9"] < 2e-3
    for corr in (0.9, 1.0):
        assert worst[corr]["prod"] > 1e-2
        assert worst[corr]["blk4g9"] < 3e-3 and worst[corr]["blk4g9"] < worst[corr]["prod"] / 10


def test_fp32_gate_scan_partial_chunk():
    # The fp32 workload at alpha ~ 0.05 (g = -softplus(3 + N(0,1))) with a 700-token
    # prefill: in the last, 60-row chunk a plain fp32 scan sums H_63 (rows 60-63 add
    # zeros) in another order than H_59, so the newest token's weight in the state
    # update, exp(H_63 - H_59) = 1, comes out 1 +- ulp(190): the GPU measured 1.52e-5 on
    # S, the model 1.53e-5.  The compensated scan the kernel now uses keeps it ~2e-8.
    import workloads as W
    w = W.small(W.config(0), L=[700, 513], r=[650, 200], h_qk=2, h_v=4, g_mu=3.0, g_sigma=1.0)
    inp = W.make_inputs(w)
    sl = slice(0, 700)
    q, k = (oracle.widen(inp[x][sl, 0]) for x in ("q", "k"))
    v, beta = oracle.widen(inp["v"][sl, 0]), oracle.widen(inp["beta"][sl, 0])
    g = inp["g"][sl, 0].numpy().astype(np.float64)
    S, o = _oracle_chain(q, k, v, g, beta)
    S_old, _ = kernel_chain(q, k, v, g, beta, path="f32", gate_mode="f32")
    S_new, o_new = kernel_chain(q, k, v, g, beta, path="f32")
    assert _rel(S_old, S) > 1e-5
    assert _rel(S_new, S) < 1e-6 and _rel(o_new, o) < 1e-6
    # the compensated scan carries H to ~2^-48 relative: padding rows leave it unchanged
    g64 = np.zeros(64, np.float32)
    g64[:60] = g[640:700]
    h, lo, _ = gate_scan_f32(g64, compensated=True)
    ref = np.cumsum(g64.astype(np.float64))
    assert np.max(np.abs((h.astype(np.float64) + lo) - ref)) < 1e-10
    Gam, e, lst = kernel_gates(g64, "f32c")
    assert lst[59] == 1.0 and lst[63] == 1.0


@pytest.mark.slow
@pytest.mark.parametrize("corr", [0.5, 0.8, 0.9, 0.95, 1.0])
@pytest.mark.parametrize("g_mu,g_sigma", [(-5.0, 1.0), (-8.0, 0.5)])
def test_kernel_model_correlated_keys_within_bf16_tolerance(corr, g_mu, g_sigma):
    """bf16 path with correlated keys (mean key cosine 0.5-0.95, and one repeated key) stays
    within 3e-3 on S and o, close to what an exact diagonal inverse gives; the
    single-level product form it replaced exceeds 3e-3 from cosine 0.9 on."""
    if corr == 1.0 and g_mu == -8.0:
        pytest.skip("a repeated key under slow decay: errors orthogonal to the key are never "
                    "contracted, so the model's own error approaches 3e-3 with any inverse")
    T, d = 1024, 128
    q, k, v, g, beta = _corr_case(int(corr * 100) + 7, T, d, corr, g_mu, g_sigma)
    S, o = _oracle_chain(q, k, v, g, beta)
    Sk, ok = kernel_chain(q, k, v, g, beta, path="bf16")
    Se, oe = kernel_chain(q, k, v, g, beta, path="bf16", inv="exact")
    eS, eo = _rel(Sk, S), _rel(ok, o)
    assert eS < 2.5e-3 and eo < 2.5e-3, (eS, eo)
    assert eS < 1.2 * _rel(Se, S) + 1e-4 and eo < 1.1 * _rel(oe, o) + 1e-4
    if corr >= 0.9:
        Sp, op = kernel_chain(q, k, v, g, beta, path="bf16", inv="prod")
        assert max(_rel(Sp, S), _rel(op, o)) > 3e-3
