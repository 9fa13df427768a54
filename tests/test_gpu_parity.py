"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerance (max over (sequence, v-head) of the relative Frobenius error of S and of
o): 1e-5 for fp32 inputs, 3e-3 for bf16 inputs with fp32 state.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, compare, gpu_run, oracle_run, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_deltanet_state_gdn_amd as gdn
    gdn.load()   # fails loudly when the library is not built
    yield


def _check(inp, mode, with_o=True, o_dtype=None):
    w = inp["workload"]
    say("case", w.name, mode, "lengths", list(w.lengths)[:8], "r", list(w.replay)[:8])
    dinp = to_dev(inp)
    S, o, cu_out = gpu_run(dinp, mode, with_o=with_o, o_dtype=o_dtype)
    torch.cuda.synchronize()
    S_ref, o_ref = oracle_run(inp, mode, with_o=with_o)
    eS, eo = compare(inp, mode, S, o, S_ref, o_ref)
    tol = TOL[w.dtype]
    say("  relerr S %.3e  o %.3e  (tol %.0e)" % (eS, eo, tol))
    assert np.isfinite(eS) and np.isfinite(eo)
    assert eS <= tol and eo <= tol, (eS, eo)
    if cu_out is not None:
        cu = np.concatenate([[0], np.cumsum(inp["r_host"])])
        assert np.array_equal(cu_out.cpu().numpy(), cu)
    return S, o


def test_small_fp32_d64():
    w = W.small(W.config(0), L=[300], r=[150])
    inp = W.make_inputs(w)
    _check(inp, "replay")
    _check(inp, "prefill")


def test_small_bf16_d128_gva():
    w = W.small(W.config(2), L=[300], r=[170], h_qk=2, h_v=4)
    inp = W.make_inputs(w)
    _check(inp, "replay")
    _check(inp, "prefill")


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128)])
def test_small_bf16_other_dims(dk, dv):
    w = W.small(W.config(1), L=[200], r=[129], h_qk=2, h_v=2, d_k=dk, d_v=dv)
    inp = W.make_inputs(w)
    _check(inp, "replay")


def test_config0_fp32():
    inp = W.make_inputs(W.config(0))
    _check(inp, "replay")
    _check(inp, "prefill")


def test_config1_bf16():
    inp = W.make_inputs(W.config(1))
    _check(inp, "replay")
    _check(inp, "prefill")
