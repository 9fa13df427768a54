"""Segment-parallel replay (gdn_replay_segmented) on the GPU against the fp64 oracle.

The window of every (sequence, v-head) chain is cut into P chunk-aligned segments whose
local states and transition maps come from one launch, are chained in fp32 and re-run
for the outputs.  The reference is always the oracle's plain token-by-token replay of
the whole window, so the tests see the decomposition and its arithmetic together:

  * the slow-decay layer (16 heads, d = 128, bf16, L = 32768, r = 3277), every head, with
    and without an alpha = 0 token per head inside the window, at P = 8;
  * ragged windows (0, 1, 63, 64, 65, 200, 700 tokens) with grouped value heads, P larger
    than the chunk count of most windows (empty trailing segments), bf16 and fp32,
    d = 64 and 128, with outputs, state only, and the packed output offsets;
  * P = 64 (the largest accepted; most segments empty), and 40 short sequences at P = 4;
  * one stack layer (32 v heads over 16 q/k heads, r = 3277) at 4 segments, every head;
  * bf16 inputs with fp32 outputs and a non-unit output scale;
  * P = 1 gives exactly gdn_replay (bit for bit): one segment's local state is the
    replayed state, its map multiplies a zero start;
  * an invalid device r is reported through the status word.
Tolerances: 3e-3 (bf16 inputs) and 1e-5 (fp32 inputs), relative Frobenius error of S
and o per (sequence, head).
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import TOL, compare, oracle_run, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_deltanet_state_gdn_amd as gdn
    gdn.load()
    yield


def seg_run(inp, P, with_o=True, ws=None, o_dtype=None):
    import gated_deltanet_state_gdn_amd as gdn
    w = inp["workload"]
    tot = int(inp["r_host"].sum())
    cu_out = torch.full((len(inp["r_host"]) + 1,), -1, dtype=torch.int32, device=inp["q"].device)
    S, o, cu_out = gdn.gdn_replay_segmented(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                            inp["cu_seqlens"], inp["r"], total_out_tokens=tot,
                                            n_segments=P, o_out=True if with_o else None, cu_out=cu_out,
                                            scale=w.scale, ws=ws, o_dtype=o_dtype)
    return S, o, cu_out


@pytest.mark.parametrize("resets", [False, True])
def test_slow_decay_layer_all_heads(resets):
    w = W.config(4)
    if resets:
        w = w.with_(reset_heads=True, reset_in_window=True)
    inp = W.make_inputs(w, device="cuda")
    say("case", w.name, "segmented replay P=8, resets in window:", resets)
    S, o, cu_out = seg_run(inp, 8)
    torch.cuda.synchronize()
    assert np.array_equal(cu_out.cpu().numpy(), [0, int(inp["r_host"][0])])
    host = dict(inp)
    for key in ("q", "k", "v", "g", "beta"):
        host[key] = inp[key].cpu()
    S_ref, o_ref = oracle_run(host, "replay")
    eS, eo = compare(host, "replay", S.cpu(), o.cpu(), S_ref, o_ref)
    say("  relerr S %.3e  o %.3e" % (eS, eo))
    assert eS <= TOL["bf16"] and eo <= TOL["bf16"]


RAGGED_L = [700, 65, 300, 1000, 64, 130, 90]
RAGGED_R = [700, 65, 200, 0, 64, 1, 63]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("P", [3, 8])
def test_ragged_windows(dtype, d, P):
    base = W.config(1) if dtype == "bf16" else W.config(0)
    w = W.small(base, RAGGED_L, RAGGED_R, h_qk=2, h_v=4, d_k=d, d_v=d, dtype=dtype, seed=4242 + d + P)
    inp = W.make_inputs(w, device="cuda")
    say("case", dtype, "d", d, "P", P, "windows", RAGGED_R)
    S, o, cu_out = seg_run(inp, P)
    S2, o2, _ = seg_run(inp, P, with_o=False)
    torch.cuda.synchronize()
    assert np.array_equal(cu_out.cpu().numpy(), np.concatenate([[0], np.cumsum(inp["r_host"])]))
    host = dict(inp)
    for key in ("q", "k", "v", "g", "beta"):
        host[key] = inp[key].cpu()
    S_ref, o_ref = oracle_run(host, "replay")
    eS, eo = compare(host, "replay", S.cpu(), o.cpu(), S_ref, o_ref)
    say("  relerr S %.3e  o %.3e" % (eS, eo))
    tol = TOL[dtype]
    assert eS <= tol and eo <= tol
    # the state does not depend on whether outputs were asked for
    assert torch.equal(S, S2)
    # an empty window's state is exactly zero
    assert float(S[3].abs().max()) == 0.0


def test_most_segments_and_many_sequences():
    # P = 64, the largest accepted: most segments of these windows are empty, and the 448
    # virtual sequences are more than the chunk kernel orders by length; then 40 sequences
    # of mixed lengths at P = 4 (160 virtual sequences, ordered longest first)
    rng = __import__("numpy").random.default_rng(99)
    cases = [(W.small(W.config(1), RAGGED_L, RAGGED_R, h_qk=2, h_v=4, seed=6464), 64)]
    Ls = [int(x) for x in rng.integers(1, 400, size=40)]
    Rs = [int(rng.integers(0, L + 1)) for L in Ls]
    cases.append((W.small(W.config(1), Ls, Rs, h_qk=1, h_v=2, seed=4040), 4))
    for w, P in cases:
        inp = W.make_inputs(w, device="cuda")
        say("case", len(inp["r_host"]), "sequences, P", P)
        S, o, cu_out = seg_run(inp, P)
        torch.cuda.synchronize()
        assert np.array_equal(cu_out.cpu().numpy(), np.concatenate([[0], np.cumsum(inp["r_host"])]))
        host = dict(inp)
        for key in ("q", "k", "v", "g", "beta"):
            host[key] = inp[key].cpu()
        S_ref, o_ref = oracle_run(host, "replay")
        eS, eo = compare(host, "replay", S.cpu(), o.cpu(), S_ref, o_ref)
        say("  relerr S %.3e  o %.3e" % (eS, eo))
        assert eS <= TOL["bf16"] and eo <= TOL["bf16"]


def test_stack_layer_shape_all_heads():
    # one layer of the 36-layer stack (16 q/k heads shared by 32 v heads, L = 32768,
    # r = 3277) at 4 segments, the call and segment count the benchmark times; every head
    w = W.config(2).with_(layers=1)
    inp = W.make_inputs(w, device="cuda")
    say("case", w.name, "one layer, segmented replay P=4")
    S, o, cu_out = seg_run(inp, 4)
    torch.cuda.synchronize()
    host = dict(inp)
    for key in ("q", "k", "v", "g", "beta"):
        host[key] = inp[key].cpu()
    S_ref, o_ref = oracle_run(host, "replay")
    eS, eo = compare(host, "replay", S.cpu(), o.cpu(), S_ref, o_ref)
    say("  relerr S %.3e  o %.3e" % (eS, eo))
    assert eS <= TOL["bf16"] and eo <= TOL["bf16"]


def test_fp32_outputs_and_scale():
    # bf16 inputs with fp32 outputs, and a non-unit output scale, through the output pass
    w = W.small(W.config(1), [700, 90, 300], [650, 90, 129], h_qk=2, h_v=4, scale=0.125, seed=1250)
    inp = W.make_inputs(w, device="cuda")
    say("case bf16 inputs, fp32 outputs, scale 0.125, P 4")
    S, o, cu_out = seg_run(inp, 4, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert o.dtype == torch.float32
    host = dict(inp)
    for key in ("q", "k", "v", "g", "beta"):
        host[key] = inp[key].cpu()
    S_ref, o_ref = oracle_run(host, "replay")
    eS, eo = compare(host, "replay", S.cpu(), o.cpu(), S_ref, o_ref)
    say("  relerr S %.3e  o %.3e" % (eS, eo))
    assert eS <= TOL["bf16"] and eo <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_segment_is_gdn_replay_bit_for_bit(dtype):
    from gpu_helpers import gpu_run
    base = W.config(1) if dtype == "bf16" else W.config(0)
    d = 128 if dtype == "bf16" else 64
    w = W.small(base, [900, 200, 64], [777, 130, 64], h_qk=2, h_v=4, d_k=d, d_v=d, dtype=dtype, seed=515)
    inp = W.make_inputs(w, device="cuda")
    S1, o1, c1 = seg_run(inp, 1)
    S0, o0, c0 = gpu_run(inp, "replay")
    torch.cuda.synchronize()
    assert torch.equal(S1, S0) and torch.equal(o1, o0) and torch.equal(c1, c0)


def test_bad_device_r_is_reported():
    import gated_deltanet_state_gdn_amd as gdn
    w = W.small(W.config(1), [300, 200], [100, 50], seed=77)
    inp = W.make_inputs(w, device="cuda")
    inp["r"] = torch.tensor([100, 201], dtype=torch.int32, device="cuda")   # 201 > L = 200
    desc = gdn.make_desc(inp["q"], inp["v"], 2, 150, w.scale)
    ws = torch.zeros(gdn.gdn_segmented_workspace_bytes(desc, 4), dtype=torch.uint8, device="cuda")
    seg_run(inp, 4, ws=ws)
    assert gdn.gdn_device_status(ws) == gdn._lib.GDN_ERR_DEVICE_INPUT
    # a clean call on the same workspace reads OK again
    inp["r"] = torch.tensor([100, 50], dtype=torch.int32, device="cuda")
    seg_run(inp, 4, ws=ws)
    assert gdn.gdn_device_status(ws) == gdn.GDN_OK
