"""The oracle against a worked example derived by hand (tests/golden/worked_example_d2.json).

The fixture's values come from the recurrence as the Tail-Replay pages state it
(gist.science technical summary, "Mecanismos Principais"; replay from a zero state over
the last r tokens, "Reconstrucao de Estado Independente"), worked out by hand, not by
any code here.  Its inputs are dyadic, so the oracle must reproduce them bit for bit.
"""
import json
import os

import numpy as np
import pytest

import oracle

_FIX = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_example_d2.json")


def load_worked_example():
    """(q, k, v, g, beta) as [T, 1, d] / [T, 1] float64 arrays, and the fixture dict."""
    ex = json.load(open(_FIX))
    q = np.array(ex["q"], dtype=np.float64)[:, None, :]
    k = np.array(ex["k"], dtype=np.float64)[:, None, :]
    v = np.array(ex["v"], dtype=np.float64)[:, None, :]
    g = np.array([float(x) for x in ex["g"]], dtype=np.float64)[:, None]
    beta = np.array(ex["beta"], dtype=np.float64)[:, None]
    return (q, k, v, g, beta), ex


def test_prefill_state_after_every_token():
    (q, k, v, g, beta), ex = load_worked_example()
    for t, S_t in enumerate(ex["prefill"]["S_after_each_token"], start=1):
        S, _ = oracle.prefill(q[:t], k[:t], v[:t], g[:t], beta[:t], [0, t], want_o=False)
        assert np.array_equal(S[0, 0], np.array(S_t, dtype=np.float64)), t


@pytest.mark.parametrize("scale", [1.0, 0.5])
def test_prefill_outputs(scale):
    (q, k, v, g, beta), ex = load_worked_example()
    T = q.shape[0]
    _, o = oracle.prefill(q, k, v, g, beta, [0, T], scale=scale)
    assert np.array_equal(o[:, 0], scale * np.array(ex["prefill"]["o"], dtype=np.float64))


@pytest.mark.parametrize("r", ["0", "1", "2", "3", "5"])
def test_replay_windows(r):
    (q, k, v, g, beta), ex = load_worked_example()
    T = q.shape[0]
    S, o = oracle.replay(q, k, v, g, beta, [0, T], [int(r)])
    want = ex["replay"][r]
    assert np.array_equal(S[0, 0], np.array(want["S"], dtype=np.float64))
    assert np.array_equal(o[:, 0].reshape(-1, 2), np.array(want["o"], dtype=np.float64).reshape(-1, 2))
