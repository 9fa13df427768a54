"""The HIP path against the hand-derived worked example (tests/golden/worked_example_d2.json).

The two-dimensional example is embedded in the first coordinates of d = 64 (fp32 inputs)
and d = 128 (bf16 inputs; every input is exact in bf16).  Padding coordinates carry
zeros, so the state and the outputs outside the 2 x 2 corner must stay exactly zero, and
the corner must equal the hand-derived values (dyadic, so the chunked evaluation has no
rounding to do beyond what the tolerance allows).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import say
from test_oracle_golden import load_worked_example

pytestmark = pytest.mark.gpu

ATOL = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_deltanet_state_gdn_amd as gdn
    gdn.load()   # fails loudly when the library is not built
    yield


def _embed(d, dtype):
    (q, k, v, g, beta), ex = load_worked_example()
    T = q.shape[0]

    def pad(x):
        out = np.zeros((T, 1, d), dtype=np.float32)
        out[:, :, :x.shape[2]] = x
        return torch.from_numpy(out).to(dtype).cuda()

    inp = dict(q=pad(q), k=pad(k), v=pad(v),
               g=torch.from_numpy(g.astype(np.float32)).cuda(),
               beta=torch.from_numpy(beta.astype(np.float32)).cuda(),
               cu=torch.tensor([0, T], dtype=torch.int32, device="cuda"))
    return inp, ex


def _check(S, o, S_want, o_want):
    S = S.double().cpu().numpy()
    corner = S[:2, :2]
    assert np.max(np.abs(corner - np.array(S_want, dtype=np.float64))) <= ATOL
    rest = S.copy()
    rest[:2, :2] = 0
    assert np.count_nonzero(rest) == 0
    if o is not None:
        o = o.double().cpu().numpy()
        want = np.array(o_want, dtype=np.float64).reshape(-1, 2)
        assert o.shape[0] == want.shape[0]
        if want.size:
            assert np.max(np.abs(o[:, :2] - want)) <= ATOL
        assert np.count_nonzero(o[:, 2:]) == 0


@pytest.mark.parametrize("d,dtype", [(64, torch.float32), (128, torch.bfloat16)])
def test_worked_example_prefill(d, dtype):
    import gated_deltanet_state_gdn_amd as gdn
    inp, ex = _embed(d, dtype)
    say("worked example prefill", d, dtype)
    S, o = gdn.gdn_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu"])
    torch.cuda.synchronize()
    _check(S[0, 0], o[:, 0], ex["prefill"]["S_after_each_token"][-1], ex["prefill"]["o"])


@pytest.mark.parametrize("d,dtype", [(64, torch.float32), (128, torch.bfloat16)])
@pytest.mark.parametrize("r", ["0", "1", "2", "3", "5"])
def test_worked_example_replay(d, dtype, r):
    import gated_deltanet_state_gdn_amd as gdn
    inp, ex = _embed(d, dtype)
    say("worked example replay", d, dtype, "r", r)
    rr = torch.tensor([int(r)], dtype=torch.int32, device="cuda")
    S, o, _ = gdn.gdn_replay(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu"], rr,
                             total_out_tokens=int(r))
    torch.cuda.synchronize()
    want = ex["replay"][r]
    _check(S[0, 0], o[:, 0] if int(r) > 0 else None, want["S"], want["o"])
