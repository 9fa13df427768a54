"""Full-size workloads on the GPU against the fp64 oracle (sampled where the oracle
cannot cover every chain in seconds), in the launch configuration bench.py times.

  * 36-layer stack, 16 q/k heads shared by 32 v heads, d = 128, L = 32768, r = 3277:
    replay of all layers in one call, every v-head of two layers plus 27 sampled
    (layer, v-head) chains; full prefill of one layer, 8 heads (both v-heads of four
    q/k heads).
  * 64 packed cache hits (varlen), L ~ U{1024..32768}, r = 5-10 % of L: replay of
    every sequence, two heads each; full prefill of the 8 shortest sequences (two heads
    each) and the longest (one head).
  * slow decay (alpha ~ 0.9997), L = 32768: replay budgets 1/2/5/10/20 % and full
    prefill, all heads; the attenuation bound on the GPU's replay error; the alpha = 0
    variant.
Tolerance: 3e-3 relative Frobenius error of S and of o (bf16 inputs, fp32 state).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import gpu_run, rel, sampled_compare, sampled_refs, say

pytestmark = pytest.mark.gpu
TOL = 3e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_deltanet_state_gdn_amd as gdn
    gdn.load()
    yield


def test_stack36_replay_sampled():
    w = W.config(2)
    inp = W.make_inputs(w, device="cuda")
    say("case", w.name, "replay, 36 layers in one call")
    S, o, cu_out = gpu_run(inp, "replay")
    torch.cuda.synchronize()
    assert np.array_equal(cu_out.cpu().numpy(), np.concatenate([[0], np.cumsum(inp["r_host"])]))
    rs = np.random.default_rng(7)
    pairs = [(int(l), int(h)) for l, h in zip(rs.integers(0, 36, 24), rs.integers(0, 32, 24))]
    pairs += [(0, 0), (35, 31), (17, 16)]
    pairs += [(l, h) for l in (5, 30) for h in range(32)]          # two whole layers
    eS, eo = sampled_compare(inp, "replay", S, o, cu_out.cpu(), pairs)
    say("  sampled %d chains: relerr S %.3e  o %.3e" % (len(pairs), eS, eo))
    assert eS <= TOL and eo <= TOL
    # the same launch again, bit for bit: every chain's arithmetic is fixed by the kernel
    # (no atomics, no order that depends on timing), at the size the benchmark times
    for _ in range(2):
        S2, o2, _ = gpu_run(inp, "replay")
        torch.cuda.synchronize()
        assert torch.equal(S, S2) and torch.equal(o, o2)
    del inp, S, o, S2, o2


def test_stack_layer_prefill_sampled():
    w = W.config(2, layers=1)
    inp = W.make_inputs(w, device="cuda")
    say("case", w.name, "full prefill of one layer")
    S, o, _ = gpu_run(inp, "prefill")
    torch.cuda.synchronize()
    pairs = [(0, h) for h in (0, 1, 10, 11, 20, 21, 30, 31)]
    eS, eo = sampled_compare(inp, "prefill", S, o, None, pairs)
    say("  sampled %d chains: relerr S %.3e  o %.3e" % (len(pairs), eS, eo))
    assert eS <= TOL and eo <= TOL


def test_varlen64_replay():
    w = W.config(3)
    inp = W.make_inputs(w, device="cuda")
    say("case", w.name, "replay; sum r =", int(inp["r_host"].sum()))
    S, o, cu_out = gpu_run(inp, "replay")
    torch.cuda.synchronize()
    pairs = [(n, h) for n in range(64) for h in (n % 16, (n + 7) % 16)]
    eS, eo = sampled_compare(inp, "replay", S, o, cu_out.cpu(), pairs)
    say("  %d chains: relerr S %.3e  o %.3e" % (len(pairs), eS, eo))
    assert eS <= TOL and eo <= TOL


def test_varlen64_prefill():
    w = W.config(3)
    inp = W.make_inputs(w, device="cuda")
    say("case", w.name, "full prefill; sum L =", int(inp["cu_host"][-1]))
    S, o, _ = gpu_run(inp, "prefill")
    torch.cuda.synchronize()
    L = np.diff(inp["cu_host"])
    order = np.argsort(L, kind="stable")
    pairs = [(int(n), h) for n in order[:8] for h in (int(n) % 16, (int(n) + 5) % 16)]
    pairs.append((int(order[-1]), 3))
    say("  sampled sequences L =", [int(L[n]) for n, _ in pairs[::2]])
    eS, eo = sampled_compare(inp, "prefill", S, o, None, pairs)
    say("  %d chains: relerr S %.3e  o %.3e" % (len(pairs), eS, eo))
    assert eS <= TOL and eo <= TOL


def test_slow_decay_budget_sweep_and_bound():
    import gated_deltanet_state_gdn_amd as gdn
    w = W.config(4)
    L = w.lengths[0]
    host = W.make_inputs(w)                       # drawn on the CPU (32K tokens)
    dev = {k: host[k].cuda() for k in ("q", "k", "v", "g", "beta", "cu_seqlens")}
    S_full, o_full = gdn.gdn_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["cu_seqlens"])
    torch.cuda.synchronize()
    heads = list(range(16))
    refs_full = sampled_refs(host, [(0, h) for h in heads], "prefill")
    eS = max(rel(oracle.widen(S_full[0, h]), refs_full[h][0]) for h in heads)
    eo = max(rel(oracle.widen(o_full[:, h]), refs_full[h][1]) for h in heads)
    say("  full prefill L=%d: relerr S %.3e  o %.3e" % (L, eS, eo))
    assert eS <= TOL and eo <= TOL
    for rho in W.GATE_SWEEP:
        r = W.replay_len(L, rho)
        rr = torch.tensor([r], dtype=torch.int32, device="cuda")
        S_rep, o_rep, _ = gdn.gdn_replay(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                                         dev["cu_seqlens"], rr, total_out_tokens=r)
        # state at the window start (the history the replay drops)
        cub = torch.tensor([0, L - r], dtype=torch.int32, device="cuda")
        sl = slice(0, L - r)
        S_before, _ = gdn.gdn_prefill(dev["q"][sl], dev["k"][sl], dev["v"][sl], dev["g"][sl],
                                      dev["beta"][sl], cub, o_out=None)
        rel_rf, _ = gdn.gdn_state_relerr(S_rep, S_full)
        torch.cuda.synchronize()
        hinp = dict(host); hinp["r_host"] = np.array([r])
        refs = sampled_refs(hinp, [(0, h) for h in heads], "replay")
        eS = max(rel(oracle.widen(S_rep[0, h]), refs[h][0]) for h in heads)
        eo = max(rel(oracle.widen(o_rep[:, h]), refs[h][1]) for h in heads)
        g = host["g"].numpy()[L - r:]
        worst = 0.0
        for h in heads:
            bound = math.exp(float(g[:, h].sum())) * float(torch.linalg.norm(S_before[0, h]))
            diff = float(torch.linalg.norm(S_full[0, h] - S_rep[0, h]))
            # GPU rounding of both states is allowed on top of the exact bound
            slack = 2 * TOL * float(torch.linalg.norm(S_full[0, h]))
            assert diff <= bound + slack, (rho, h, diff, bound)
            worst = max(worst, diff / (bound + 1e-30))
        say("  r=%5d (%.0f%%): relerr vs oracle S %.3e o %.3e; relerr(S_rep,S_full) median %.3e; "
            "diff/bound max %.3f" % (r, 100 * rho, eS, eo, float(rel_rf.median()), worst))
        assert eS <= TOL and eo <= TOL


def test_slow_decay_reset_variant():
    w = W.config(4).with_(reset_heads=True, reset_in_window=True)
    L = w.lengths[0]
    host = W.make_inputs(w)
    S_rep, S_full = None, None
    dev = {k: host[k].cuda() for k in ("q", "k", "v", "g", "beta", "cu_seqlens", "r")}
    S_rep, _, _ = gpu_run(dev | {"workload": w, "r_host": host["r_host"], "cu_host": host["cu_host"]}, "replay")
    torch.cuda.synchronize()
    heads = list(range(16))
    refs = sampled_refs(host, [(0, h) for h in heads], "prefill", with_o=False)
    e = max(rel(oracle.widen(S_rep[0, h]), refs[h][0]) for h in heads)
    say("  alpha=0 inside the %d-token window: relerr(GPU replay, oracle full) max %.3e" % (host["r_host"][0], e))
    assert e <= TOL
