"""GPU: replay on one stream while a second stream copies a pinned host buffer.

Tail-Replay runs the state rebuild asynchronously, on a stream of its own, next to the
restore of the full-attention KV cache, which it does not touch (gist.science technical
summary, "Mecanismos Principais", the overlap of transfer and replay; "Resultados", 18-42 %
less time to first token than serialised copies).  The overlapped replay must match the
fp64 oracle (3e-3 relative Frobenius error of S and o, bf16 inputs), be bit-identical to
a replay without the copy, and leave the copy exact.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import compare, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_deltanet_state_gdn_amd as gdn
    gdn.load()
    yield


def test_overlapped_copy_replay_matches_oracle():
    import gated_deltanet_state_gdn_amd as gdn
    host_inp = W.make_inputs(W.config(1))          # the 8K workload: 16 heads, r = 410
    inp = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in host_inp.items()}
    tot = int(inp["r_host"].sum())
    main = torch.cuda.current_stream()

    def replay():
        return gdn.gdn_replay(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                              inp["cu_seqlens"], inp["r"], total_out_tokens=tot, stream=main)

    say("case overlap: replay alone")
    S_a, o_a, _ = replay()
    torch.cuda.synchronize()
    nbytes = 64 << 20
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    host.copy_(torch.randint(0, 256, (nbytes,), dtype=torch.uint8,
                             generator=torch.Generator().manual_seed(3)))
    dst = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()          # default priority
    say("case overlap: copy on a second stream during replay")
    start = torch.cuda.Event()
    start.record(main)
    side.wait_event(start)
    with torch.cuda.stream(side):
        dst.copy_(host, non_blocking=True)
    S_b, o_b, _ = replay()
    torch.cuda.synchronize()
    S_ref, o_ref = oracle.replay(host_inp["q"], host_inp["k"], host_inp["v"], host_inp["g"],
                                 host_inp["beta"], host_inp["cu_host"], host_inp["r_host"])
    eS, eo = compare(host_inp, "replay", S_b, o_b, S_ref, o_ref)
    say("  overlapped replay vs oracle: relerr S %.3e  o %.3e (all 16 heads)" % (eS, eo))
    assert eS <= 3e-3 and eo <= 3e-3
    assert torch.equal(S_a, S_b)
    assert torch.equal(o_a.view(torch.int16), o_b.view(torch.int16))
    assert torch.equal(dst.cpu(), host)
