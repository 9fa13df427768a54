"""Longest-window-first block order for packed sequences of different lengths.

Every workgroup of a launch with 2 to 256 packed sequences ranks them by chunk count and
maps its position through that order; each (sequence, v-head) unit's arithmetic is
unchanged, so the results must be the same bits as with the plain order (a launch with
257 sequences keeps the plain order), and match the oracle.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import TOL, compare, oracle_run, say, to_dev, gpu_run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_deltanet_state_gdn_amd as gdn
    gdn.load()
    yield


@pytest.mark.parametrize("mode", ["replay", "prefill"])
def test_longest_first_order_is_bit_identical_and_matches_oracle(mode):
    rs = np.random.default_rng(77)
    L = [int(x) for x in rs.integers(0, 400, size=256)]
    L[3], L[100], L[255] = 0, 1, 1100                      # empty, one token, one long window
    r = [int(rs.integers(0, l + 1)) if l else 0 for l in L]
    r[255] = 1100
    w = W.small(W.config(1), L=L, r=r, h_qk=1, h_v=2, d_k=64, d_v=64)
    say("order case", mode, "256 sequences, sum L", sum(L), "sum r", sum(r))
    inp = W.make_inputs(w)
    S, o, _ = gpu_run(to_dev(inp), mode)
    torch.cuda.synchronize()
    S_ref, o_ref = oracle_run(inp, mode)
    eS, eo = compare(inp, mode, S, o, S_ref, o_ref)
    say("  relerr S %.3e  o %.3e" % (eS, eo))
    assert eS <= TOL["bf16"] and eo <= TOL["bf16"], (eS, eo)
    # the same sequences plus one empty one: 257 > 256, so the plain order
    w2 = W.small(W.config(1), L=L + [0], r=r + [0], h_qk=1, h_v=2, d_k=64, d_v=64)
    inp2 = W.make_inputs(w2)
    for x in ("q", "k", "v", "g", "beta"):
        assert torch.equal(inp2[x], inp[x])             # same seeded draws, same tokens
    S2, o2, _ = gpu_run(to_dev(inp2), mode)
    torch.cuda.synchronize()
    assert torch.equal(S2[:256], S)
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16))
