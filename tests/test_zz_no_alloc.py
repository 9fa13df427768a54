"""GPU: the allocation-free adaptive replay length (static device scratch, no workspace)
gives bit for bit the result of gdn_adaptive_replay_len with a caller workspace, on two
calls in a row, the second smaller than the first (the scratch keeps the first call's
per-head lengths, which the second must not read).  The first call fills the scratch to
its limit: n_seqs * h_v = 65536."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_deltanet_state_gdn_amd as gdn
    gdn.load()
    yield


def _gates(n_seqs, h_v, seed, mu):
    rs = np.random.default_rng(seed)
    L = rs.integers(0, 400, size=n_seqs)
    L[::7] = 0                                      # some empty sequences
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    T = int(cu[-1])
    g = -np.log1p(np.exp(mu + rs.standard_normal((T, h_v))))
    if T:
        rows = rs.integers(0, T, size=max(1, T // 500))
        g[rows, rs.integers(0, h_v, size=len(rows))] = -np.inf   # a few alpha = 0 tokens
    return (torch.as_tensor(g.astype(np.float32), device="cuda"),
            torch.as_tensor(cu, device="cuda"))


def test_static_scratch_matches_workspace_variant_twice():
    import gated_deltanet_state_gdn_amd as gdn
    cases = [(2048, 32, 11, -3.0, 1e-3, 8, 300),    # 65536 heads: the scratch's limit
             (37, 16, 12, -5.0, 1e-2, 0, 10**6)]    # then a smaller call
    for n_seqs, h_v, seed, mu, eps, r_min, r_max in cases:
        g, cu = _gates(n_seqs, h_v, seed, mu)
        say("case static adaptive: n_seqs %d h_v %d eps %g" % (n_seqs, h_v, eps))
        r_ws = gdn.gdn_adaptive_replay_len(g, cu, eps=eps, r_min=r_min, r_max=r_max)
        r_st = torch.full((n_seqs,), -7, dtype=torch.int32, device="cuda")
        gdn.gdn_adaptive_replay_len_static(g, cu, eps=eps, r_min=r_min, r_max=r_max, r_out=r_st)
        torch.cuda.synchronize()
        a, b = r_ws.cpu().numpy(), r_st.cpu().numpy()
        say("  r mean %.1f, max %d; equal: %s" % (a.mean(), a.max(), np.array_equal(a, b)))
        assert np.array_equal(a, b)
