"""CPU model of the segmented replay's combine step for bf16 inputs (no GPU).

The combine forms S_next = M S + L from fp32 M (a segment's transition map) and fp32 S with
each operand split into fp16 halves, hi = fp16(x) and lo = fp16(x - hi), and the product
taken as hi.hi + hi.lo + lo.hi over 32-wide k-blocks with fp32 accumulation, as the
kernel does on its 16x16x32 fp16 matrix products.  This model checks that arithmetic
against the exact fp64 result for maps of the two gate regimes of the workloads: the
8K/32K gates (alpha ~ 0.993, a 416-token segment leaves |M| ~ 1e-3, so the lo halves of
most entries are fp16 subnormals) and the slow-decay gates (alpha ~ 0.9997, |M| ~ 0.2).
The error is measured against the step's result M S + L, the quantity the combine
produces; it must stay at the level of an fp32 product (<= 1e-6), far inside the bf16
inputs' 3e-3.
"""
import numpy as np
import pytest

D = 128
SEG = 416   # tokens of one segment: 52 chunks cut into 8 segments of 6.5 chunks


def _map(rng, g_mu, g_sigma):
    """prod_t alpha_t (I - beta_t k_t k_t^T) over one segment, fp64 (unit keys)."""
    M = np.eye(D)
    for _ in range(SEG):
        k = rng.standard_normal(D)
        k /= np.linalg.norm(k)
        beta = 1.0 / (1.0 + np.exp(-rng.standard_normal()))
        alpha = np.exp(-np.log1p(np.exp(rng.normal(g_mu, g_sigma))))
        M = alpha * (M - beta * np.outer(k, k @ M))
    return M


def _split(x32):
    hi = x32.astype(np.float16)
    lo = (x32 - hi.astype(np.float32)).astype(np.float16)
    return hi.astype(np.float32), lo.astype(np.float32)


def _combine_split(M32, S32, L32):
    Mh, Ml = _split(M32)
    Sh, Sl = _split(S32)
    acc = np.zeros((D, D), np.float32)
    for kb in range(0, D, 32):
        sl = slice(kb, kb + 32)
        # each fp16 x fp16 product is exact in fp32 (11 + 11 significant bits)
        for A, B in ((Mh, Sh), (Mh, Sl), (Ml, Sh)):
            acc = (acc + (A[:, sl].astype(np.float64) @ B[sl].astype(np.float64)).astype(np.float32)).astype(np.float32)
    return (acc + L32).astype(np.float32)


@pytest.mark.parametrize("g_mu,g_sigma", [(-5.0, 1.0), (-8.0, 0.5)])
def test_split_products_match_fp32_against_the_step_result(g_mu, g_sigma):
    rng = np.random.default_rng(31 + int(-g_mu))
    M = _map(rng, g_mu, g_sigma)
    S = rng.standard_normal((D, D)) * 0.3
    L = rng.standard_normal((D, D)) * 0.3
    M32, S32, L32 = M.astype(np.float32), S.astype(np.float32), L.astype(np.float32)
    exact = M32.astype(np.float64) @ S32.astype(np.float64) + L32.astype(np.float64)
    got = _combine_split(M32, S32, L32).astype(np.float64)
    err = np.linalg.norm(got - exact) / np.linalg.norm(exact)
    assert err <= 1e-6, err
    # (an fp32 product of the same operands, for scale)
    f32 = (M32 @ S32 + L32).astype(np.float64)
    assert np.linalg.norm(f32 - exact) / np.linalg.norm(exact) <= 1e-6


def test_lo_halves_are_what_keeps_the_split_accurate():
    # the pin must fail for a plausible mistake: dropping the lo halves (one fp16
    # product) loses about three decimal digits on the same step
    rng = np.random.default_rng(7)
    M32 = _map(rng, -8.0, 0.5).astype(np.float32)
    S32 = (rng.standard_normal((D, D)) * 0.3).astype(np.float32)
    L32 = (rng.standard_normal((D, D)) * 0.3).astype(np.float32)
    exact = M32.astype(np.float64) @ S32.astype(np.float64) + L32.astype(np.float64)
    Mh, _ = _split(M32)
    Sh, _ = _split(S32)
    hi_only = (Mh.astype(np.float64) @ Sh.astype(np.float64) + L32).astype(np.float64)
    assert np.linalg.norm(hi_only - exact) / np.linalg.norm(exact) > 1e-5
