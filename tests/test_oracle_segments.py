"""The affine decomposition behind the segment-parallel replay, pinned on the oracle.

Over any stretch of tokens the gated delta rule maps the state affinely:
    S_end = M S_start + S_local,
with S_local the state the stretch builds from zero and M the product of its per-token
maps alpha_t (I - beta_t k_t k_t^T), i.e. the same recurrence run from S_start = I with
v = 0 (d_k = d_v).  These checks use only the fp64 oracle: prefill from an arbitrary
start equals M S_start + S_local; chaining the segments of a window reproduces one
replay of the whole window; a reset inside a segment makes M vanish from that point.
"""
import numpy as np

import oracle


def _inputs(rng, T, h_qk, h_v, d, reset_at=None):
    q = rng.standard_normal((T, h_qk, d))
    k = rng.standard_normal((T, h_qk, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, h_v, d))
    g = -np.log1p(np.exp(rng.normal(-3.0, 1.0, (T, h_v))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, h_v))))
    if reset_at is not None:
        g[reset_at, :] = -np.inf
    return q, k, v, g, beta


def _maps(q, k, v, g, beta, lo, hi, d, h_v):
    """S_local and M of tokens [lo, hi) for every head (oracle prefill of one sequence)."""
    cu = [0, hi - lo]
    sl = slice(lo, hi)
    S_loc, _ = oracle.prefill(q[sl], k[sl], v[sl], g[sl], beta[sl], cu, want_o=False)
    eye = np.broadcast_to(np.eye(d), (1, h_v, d, d)).copy()
    M, _ = oracle.prefill(q[sl], k[sl], np.zeros_like(v[sl]), g[sl], beta[sl], cu, S0=eye, want_o=False)
    return S_loc[0], M[0]


def test_prefill_from_a_start_is_affine_in_the_start():
    rng = np.random.default_rng(11)
    T, h_qk, h_v, d = 150, 1, 2, 16
    q, k, v, g, beta = _inputs(rng, T, h_qk, h_v, d)
    S_loc, M = _maps(q, k, v, g, beta, 0, T, d, h_v)
    S0 = rng.standard_normal((1, h_v, d, d))
    S_end, _ = oracle.prefill(q, k, v, g, beta, [0, T], S0=S0, want_o=False)
    for h in range(h_v):
        np.testing.assert_allclose(S_end[0, h], M[h] @ S0[0, h] + S_loc[h], rtol=0, atol=1e-12)


def test_chained_segments_equal_one_replay():
    rng = np.random.default_rng(12)
    T, h_qk, h_v, d, r = 700, 1, 2, 16, 523
    q, k, v, g, beta = _inputs(rng, T, h_qk, h_v, d)
    S_ref, o_ref = oracle.replay(q, k, v, g, beta, [0, T], [r])
    wbeg = T - r
    chunks = -(-r // 64)
    for P in (1, 2, 3, 5, 9, 12):   # 12 > 9 chunks: trailing segments are empty
        q_ = -(-chunks // P)
        S = np.zeros((h_v, d, d))
        o_parts = []
        for p in range(P):
            lo = min(wbeg + 64 * q_ * p, T)
            hi = min(wbeg + 64 * q_ * (p + 1), T)
            if hi > lo:
                _, o_p = oracle.prefill(q[lo:hi], k[lo:hi], v[lo:hi], g[lo:hi], beta[lo:hi], [0, hi - lo],
                                        S0=S[None].copy())
                o_parts.append(o_p)
            S_loc, M = _maps(q, k, v, g, beta, lo, hi, d, h_v) if hi > lo else \
                (np.zeros((h_v, d, d)), np.broadcast_to(np.eye(d), (h_v, d, d)))
            S = np.einsum("hij,hjk->hik", M, S) + S_loc
        np.testing.assert_allclose(S, S_ref[0], rtol=0, atol=1e-11)
        np.testing.assert_allclose(np.concatenate(o_parts), o_ref, rtol=0, atol=1e-11)


def test_a_reset_inside_a_segment_cuts_its_map():
    rng = np.random.default_rng(13)
    T, h_qk, h_v, d = 200, 1, 1, 16
    q, k, v, g, beta = _inputs(rng, T, h_qk, h_v, d, reset_at=120)
    S_loc, M = _maps(q, k, v, g, beta, 0, T, d, h_v)
    # alpha = 0 at token 120 zeroes everything carried into it: the map from the start is
    # the product of the maps after the reset times zero
    assert np.abs(M).max() == 0.0
    S_tail, _ = oracle.replay(q, k, v, g, beta, [0, T], [T - 120])
    np.testing.assert_allclose(S_loc, S_tail[0], rtol=0, atol=1e-12)
