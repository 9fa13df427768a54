"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Each compute call only enqueues kernels on the caller's stream (no allocation, no memset,
no synchronisation; the caller owns every buffer), so a serving loop can capture it once
and replay it.  Here gdn_replay with outputs, gdn_prefill continuing from the replayed
state, and gdn_replay_segmented (setup, map, combine and output launches) go into one
graph, which is replayed three times with unrelated eager work, synchronisations and
overwritten outputs between the replays.  Every replay must reproduce the eager results
bit for bit (the kernels are deterministic), and the eager replay is checked against the
oracle.
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


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_captured_calls_replay_bit_for_bit(dtype, d):
    import gated_deltanet_state_gdn_amd as gdn
    base = W.config(1) if dtype == "bf16" else W.config(0)
    w = W.small(base, [900, 200, 64, 333], [777, 130, 64, 0], h_qk=2, h_v=4, d_k=d, d_v=d, dtype=dtype,
                seed=8080 + d)
    inp = W.make_inputs(w, device="cuda")
    say("case", dtype, "d", d, "graph capture of replay, prefill, segmented replay")
    n = len(inp["r_host"])
    tot = int(inp["r_host"].sum())
    T = int(inp["q"].shape[0])
    dev = inp["q"].device
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"])
    desc_r = gdn.make_desc(inp["q"], inp["v"], n, tot, w.scale)
    desc_p = gdn.make_desc(inp["q"], inp["v"], n, T, w.scale)
    odt = inp["q"].dtype
    S_r = torch.empty((n, w.h_v, d, d), dtype=torch.float32, device=dev)
    o_r = torch.empty((tot, w.h_v, d), dtype=odt, device=dev)
    c_r = torch.empty((n + 1,), dtype=torch.int32, device=dev)
    S_p = torch.empty_like(S_r)
    o_p = torch.empty((T, w.h_v, d), dtype=odt, device=dev)
    S_s = torch.empty_like(S_r)
    o_s = torch.empty_like(o_r)
    c_s = torch.empty_like(c_r)
    ws_r = gdn.workspace(desc_r, dev)
    ws_p = gdn.workspace(desc_p, dev)
    ws_s = torch.zeros(gdn.gdn_segmented_workspace_bytes(desc_r, 3), dtype=torch.uint8, device=dev)

    def calls():
        gdn.gdn_replay(*args, inp["r"], total_out_tokens=tot, S_out=S_r, o_out=o_r, cu_out=c_r, ws=ws_r,
                       scale=w.scale)
        gdn.gdn_prefill(*args, S0=S_r, S_out=S_p, o_out=o_p, ws=ws_p, scale=w.scale)
        gdn.gdn_replay_segmented(*args, inp["r"], total_out_tokens=tot, n_segments=3, S_out=S_s, o_out=o_s,
                                 cu_out=c_s, ws=ws_s, scale=w.scale)

    outs = (S_r, o_r, c_r, S_p, o_p, S_s, o_s, c_s)
    calls()
    torch.cuda.synchronize()
    eager = [x.clone() for x in outs]
    for ws in (ws_r, ws_p, ws_s):
        assert gdn.gdn_device_status(ws) == gdn.GDN_OK

    # the eager replay against the oracle, so that what the graph must reproduce is right
    host = dict(inp)
    for key in ("q", "k", "v", "g", "beta"):
        host[key] = inp[key].cpu()
    S_ref, o_ref = oracle_run(host, "replay")
    eS, eo = compare(host, "replay", eager[0].cpu(), eager[1].cpu(), S_ref, o_ref)
    say("  eager replay relerr S %.3e  o %.3e" % (eS, eo))
    assert eS <= TOL[dtype] and eo <= TOL[dtype]
    assert np.array_equal(eager[2].cpu().numpy(), np.concatenate([[0], np.cumsum(inp["r_host"])]))

    side = torch.cuda.Stream()   # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    a = torch.randn(512, 512, device=dev)
    for rep in range(3):
        for x in outs:
            if x.is_floating_point():
                x.fill_(float("nan"))
            else:
                x.fill_(-7)
        b = (a @ a).sum()   # unrelated eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, e in zip(("S_r", "o_r", "cu_r", "S_p", "o_p", "S_s", "o_s", "cu_s"), outs, eager):
            assert torch.equal(x, e), (rep, name)
        assert torch.isfinite(b)
        say("  replay %d bit-identical to the eager calls" % rep)
    for ws in (ws_r, ws_p, ws_s):
        assert gdn.gdn_device_status(ws) == gdn.GDN_OK
