"""GPU: the step after the rebuild -- suffix prefill from the replayed state.

A cache hit matches a prefix of L tokens; the prompt continues with s new tokens.
Tail-Replay rebuilds each linear-attention state from the last r prefix tokens and
the prompt's remainder is then prefilled from that state (arXiv 2608.30310,
abstract; gist.science technical summary, "Reconstrucao de Estado Independente").
gdn_replay over the prefix followed by gdn_prefill(S0 = rebuilt state) over the
suffix must equal one recurrence from zero over (replay window + suffix): the oracle
computes that directly.  Tolerances as for replay: 1e-5 (fp32), 3e-3 (bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_deltanet_state_gdn_amd as gdn
    gdn.load()
    yield


def _split(inp, prefix, suffix):
    """Packed prefix-only and suffix-only inputs, gathered with torch."""
    cu = inp["cu_host"]
    keys = ("q", "k", "v", "g", "beta")
    pre, suf = {k: [] for k in keys}, {k: [] for k in keys}
    for n, (L, s) in enumerate(zip(prefix, suffix)):
        b = int(cu[n])
        for k in keys:
            x = inp[k]
            pre[k].append(x[b:b + L])
            suf[k].append(x[b + L:b + L + s])
    return ({k: torch.cat(v).contiguous() for k, v in pre.items()},
            {k: torch.cat(v).contiguous() for k, v in suf.items()})


def _compose(w, prefix, suffix, replay, heads=None):
    import gated_deltanet_state_gdn_amd as gdn
    wl = W.small(w, L=[a + b for a, b in zip(prefix, suffix)], r=[1] * len(prefix))
    inp = W.make_inputs(wl)
    say("case", w.name, "prefix", prefix, "suffix", suffix, "r", replay)
    pre, suf = _split(inp, prefix, suffix)
    dev = {k: v.cuda() for k, v in pre.items()}
    dsu = {k: v.cuda() for k, v in suf.items()}
    cu_p = torch.tensor(np.concatenate([[0], np.cumsum(prefix)]), dtype=torch.int32, device="cuda")
    cu_s = torch.tensor(np.concatenate([[0], np.cumsum(suffix)]), dtype=torch.int32, device="cuda")
    r = torch.tensor(replay, dtype=torch.int32, device="cuda")
    S_r, _, _ = gdn.gdn_replay(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], cu_p, r,
                               total_out_tokens=int(sum(replay)), o_out=None, scale=w.scale)
    S_f, o_f = gdn.gdn_prefill(dsu["q"], dsu["k"], dsu["v"], dsu["g"], dsu["beta"], cu_s,
                               S0=S_r, scale=w.scale)
    torch.cuda.synchronize()
    # oracle: one recurrence from zero over (last r prefix tokens + suffix) per sequence
    cu = inp["cu_host"]
    parts = {k: [] for k in ("q", "k", "v", "g", "beta")}
    lens = []
    for n, (L, s, rr) in enumerate(zip(prefix, suffix, replay)):
        b = int(cu[n])
        for k in parts:
            parts[k].append(inp[k][b + L - rr:b + L + s])
        lens.append(rr + s)
    cat = {k: torch.cat(v) for k, v in parts.items()}
    cu_o = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S_ref, o_ref = oracle.prefill(cat["q"], cat["k"], cat["v"], cat["g"], cat["beta"], cu_o,
                                  scale=w.scale)
    eS = eo = 0.0
    row = 0
    Sg, og = oracle.widen(S_f), oracle.widen(o_f)
    for n, (s, rr) in enumerate(zip(suffix, replay)):
        for h in (heads if heads is not None else range(w.h_v)):
            eS = max(eS, rel(Sg[n, h], S_ref[n, h]))
            if s > 0:
                eo = max(eo, rel(og[row:row + s, h], o_ref[int(cu_o[n]) + rr:int(cu_o[n + 1]), h]))
        row += s
    say("  relerr S %.3e  o %.3e" % (eS, eo))
    tol = TOL[w.dtype]
    assert eS <= tol and eo <= tol


def test_replay_then_suffix_varlen_bf16():
    _compose(W.small(W.config(2), L=[1], r=[1], h_qk=2, h_v=4),
             prefix=[700, 130, 64, 1], suffix=[200, 1, 65, 0], replay=[70, 130, 0, 1])


def test_replay_then_suffix_fp32():
    _compose(W.config(0), prefix=[2048], suffix=[300], replay=[205])


def test_replay_then_suffix_stack_layer_shape():
    # one layer of the 36-layer stack's shape: L = 32768, r = 3277, 1024 new tokens
    w = W.config(2).with_(layers=1)
    _compose(w, prefix=[32768], suffix=[1024], replay=[3277], heads=[0, 1, 17, 31])
