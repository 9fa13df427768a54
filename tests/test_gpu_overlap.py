"""GPU: replay on one stream while a second stream copies a pinned host buffer.

Tail-Replay runs the state rebuild asynchronously, on a stream of its own, next to the
restore of the full-attention KV cache, which it does not touch (arXiv 2608.30310,
abstract; gist.science technical summary, "Reconstrucao de Estado Independente").
The overlapped run must give bit-identical replay results and an exact copy.
"""
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


def test_overlapped_copy_leaves_replay_bit_identical():
    import gated_deltanet_state_gdn_amd as gdn
    inp = W.make_inputs(W.config(1), device="cuda")
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
    assert torch.equal(S_a, S_b)
    assert torch.equal(o_a.view(torch.int16), o_b.view(torch.int16))
    assert torch.equal(dst.cpu(), host)
