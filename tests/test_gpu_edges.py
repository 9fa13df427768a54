"""GPU edge cases, invariants and the error report, against the fp64 oracle.

Tolerances: relative Frobenius error of S and o <= 1e-5 (fp32 inputs), <= 3e-3
(bf16 inputs, fp32 state), max over (sequence, v-head).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, compare, gpu_run, oracle_run, rel, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_deltanet_state_gdn_amd as gdn
    gdn.load()
    yield


def _case(w, mode="replay", **kw):
    inp = W.make_inputs(w)
    say("case", w.name, mode, "L", list(w.lengths), "r", list(w.replay), kw)
    S, o, cu_out = gpu_run(to_dev(inp), mode, **kw)
    torch.cuda.synchronize()
    S_ref, o_ref = oracle_run(inp, mode, with_o=o is not None)
    eS, eo = compare(inp, mode, S, o, S_ref, o_ref)
    say("  relerr S %.3e  o %.3e" % (eS, eo))
    return inp, S, o, cu_out, eS, eo


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_ragged_and_degenerate(dtype):
    # empty sequences, r = 0, r = 1, L < 64, L = 64, L = 65, partial last chunks
    L = [0, 1, 63, 64, 65, 130, 200, 5]
    r = [0, 1, 1, 64, 65, 7, 200, 0]
    if dtype == "bf16":
        w = W.small(W.config(2), L=L, r=r, h_qk=2, h_v=4)
    else:
        w = W.small(W.config(0), L=L, r=r)
    for mode in ("replay", "prefill"):
        inp, S, o, cu_out, eS, eo = _case(w, mode)
        assert eS <= TOL[w.dtype] and eo <= TOL[w.dtype]
        if mode == "replay":
            Sg = S.cpu()
            for n in range(len(L)):
                if r[n] == 0:
                    assert torch.count_nonzero(Sg[n]) == 0      # Zero-Only: S = 0 exactly
            assert np.array_equal(cu_out.cpu().numpy(), np.concatenate([[0], np.cumsum(r)]))


def test_replay_full_window_is_prefill_bitwise():
    w = W.small(W.config(1), L=[300, 64, 129], r=[300, 64, 129], h_qk=4, h_v=4)
    inp = to_dev(W.make_inputs(w))
    S1, o1, _ = gpu_run(inp, "replay")
    S2, o2, _ = gpu_run(inp, "prefill")
    torch.cuda.synchronize()
    assert torch.equal(S1, S2) and torch.equal(o1, o2)


def test_deterministic_repeat():
    w = W.small(W.config(2), L=[500, 333], r=[301, 333], h_qk=2, h_v=4)
    inp = to_dev(W.make_inputs(w))
    runs = [gpu_run(inp, "replay") for _ in range(3)]
    torch.cuda.synchronize()
    for S, o, _ in runs[1:]:
        assert torch.equal(S, runs[0][0]) and torch.equal(o, runs[0][1])


def test_state_only_matches_with_outputs():
    w = W.small(W.config(1), L=[400], r=[250], h_qk=4, h_v=4)
    inp = to_dev(W.make_inputs(w))
    S1, _, _ = gpu_run(inp, "replay", with_o=True)
    S2, o2, _ = gpu_run(inp, "replay", with_o=False)
    torch.cuda.synchronize()
    assert o2 is None
    assert torch.equal(S1, S2)


def test_fp32_outputs_for_bf16_inputs():
    w = W.small(W.config(1), L=[300], r=[200], h_qk=2, h_v=2)
    inp, S, o, _, eS, eo = _case(w, "replay", o_dtype=torch.float32)
    assert o.dtype == torch.float32
    assert eS <= 3e-3 and eo <= 3e-3


def test_scale():
    w = W.small(W.config(1), L=[200], r=[150], h_qk=2, h_v=2, scale=0.125)
    inp, S, o, _, eS, eo = _case(w, "replay")
    assert eS <= 3e-3 and eo <= 3e-3


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (128, 128)])
def test_fp32_head_dims(dk, dv):
    # fp32 inputs with d_v = 128 run as two column blocks per head; d_k = 128 keeps one Q
    # buffer in LDS (refilled once the state waves have read it)
    w = W.small(W.config(0), L=[300, 130, 64], r=[170, 130, 1], h_qk=2, h_v=4, d_k=dk, d_v=dv)
    for mode in ("replay", "prefill"):
        inp, S, o, _, eS, eo = _case(w, mode)
        assert eS <= 1e-5 and eo <= 1e-5, (mode, eS, eo)
    inp, S, o, _, eS, eo = _case(w, "replay", with_o=False)
    assert o is None and eS <= 1e-5


def test_resets_inside_and_before_window():
    # alpha = 0 tokens (g = -inf): one per head at random positions, and forced inside
    # the window in a second case, where replay must equal full prefill.
    w = W.small(W.config(4), L=[700], r=[300], h_qk=4, h_v=4, reset_heads=True)
    inp, S, o, _, eS, eo = _case(w, "replay")
    assert eS <= 3e-3 and eo <= 3e-3
    inp, S, o, _, eS, eo = _case(w, "prefill")
    assert eS <= 3e-3 and eo <= 3e-3
    # with the alpha = 0 token inside the window the replayed state equals the full
    # prefill state exactly (oracle), so the GPU replay must match the full state
    w2 = w.with_(reset_in_window=True)
    inp2 = W.make_inputs(w2)
    Sr, _, _ = gpu_run(to_dev(inp2), "replay")
    torch.cuda.synchronize()
    S_full, _ = oracle_run(inp2, "prefill", with_o=False)
    S_rep, _ = oracle_run(inp2, "replay", with_o=False)
    assert np.array_equal(S_full, S_rep)
    for h in range(4):
        e = rel(oracle.widen(Sr[0, h]), S_full[0, h])
        say("  reset in window, head %d: relerr(GPU replay, full) %.3e" % (h, e))
        assert e <= 3e-3


def test_resets_at_chunk_boundaries():
    w = W.small(W.config(1), L=[320], r=[320], h_qk=2, h_v=2)
    inp = W.make_inputs(w)
    for p in (0, 63, 64, 127, 128, 200, 201, 319):
        inp["g"][p, p % 2] = float("-inf")
    S, o, _ = gpu_run(to_dev(inp), "prefill")
    torch.cuda.synchronize()
    S_ref, o_ref = oracle_run(inp, "prefill")
    eS, eo = compare(inp, "prefill", S, o, S_ref, o_ref)
    say("  resets at chunk edges: relerr S %.3e o %.3e" % (eS, eo))
    assert np.isfinite(eS) and eS <= 3e-3 and eo <= 3e-3


def test_prefill_from_initial_state_composition():
    # prefill(0..m) then prefill(m..L, S0 = S_m) equals prefill(0..L) (within tolerance)
    w = W.small(W.config(2), L=[400], r=[400], h_qk=2, h_v=4)
    inp = W.make_inputs(w)
    m = 150
    import gated_deltanet_state_gdn_amd as gdn
    d = to_dev(inp)
    cu1 = torch.tensor([0, m], dtype=torch.int32, device="cuda")
    cu2 = torch.tensor([0, 400 - m], dtype=torch.int32, device="cuda")
    sl1, sl2 = slice(0, m), slice(m, 400)
    S1, _ = gdn.gdn_prefill(d["q"][sl1], d["k"][sl1], d["v"][sl1], d["g"][sl1], d["beta"][sl1], cu1)
    S2, o2 = gdn.gdn_prefill(d["q"][sl2], d["k"][sl2], d["v"][sl2], d["g"][sl2], d["beta"][sl2], cu2, S0=S1)
    torch.cuda.synchronize()
    S_ref, o_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], [0, 400])
    for h in range(4):
        eS = rel(oracle.widen(S2[0, h]), S_ref[0, h])
        eo = rel(oracle.widen(o2[:, h]), o_ref[m:, h])
        say("  head %d composition relerr S %.3e o %.3e" % (h, eS, eo))
        assert eS <= 3e-3 and eo <= 3e-3


def test_relerr_kernel_against_host():
    import gated_deltanet_state_gdn_amd as gdn
    g = torch.Generator().manual_seed(5)
    A = torch.randn((3, 5, 128, 128), generator=g)
    B = A + 1e-3 * torch.randn(A.shape, generator=g)
    B[1, 2] = 0.0
    A[2, 3, 7, 9] = float("nan")
    rel_d, nf_d = gdn.gdn_state_relerr(A.cuda(), B.cuda())
    torch.cuda.synchronize()
    ref, _ = oracle.state_relerr(A.numpy(), B.numpy())
    got = rel_d.cpu().numpy()
    ok = np.isfinite(ref)
    assert np.allclose(got[ok], ref[ok], rtol=1e-5, atol=0)
    assert np.isnan(got[2, 3])
    nf = nf_d.cpu().numpy()
    assert nf[2, 3] == 1 and nf.sum() == 1
    # reference norm 0 -> absolute norm
    assert abs(got[1, 2] - np.linalg.norm(A[1, 2].numpy())) <= 1e-5 * np.linalg.norm(A[1, 2].numpy())


def test_device_status_reports_bad_device_inputs():
    # the kernels only set bits in the status word; gdn_device_status reads and clears it
    import gated_deltanet_state_gdn_amd as gdn
    w = W.small(W.config(1), L=[100, 50], r=[30, 20], h_qk=2, h_v=2)
    d = to_dev(W.make_inputs(w))
    desc = gdn.make_desc(d["q"], d["v"], 2, 50)
    ws = gdn.workspace(desc, "cuda")
    gdn.gdn_replay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["r"],
                   total_out_tokens=50, ws=ws)
    assert gdn.gdn_device_status(ws) == 0
    bad_r = torch.tensor([30, 51], dtype=torch.int32, device="cuda")        # r > L
    gdn.gdn_replay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], bad_r,
                   total_out_tokens=81, ws=ws)
    assert gdn.gdn_device_status(ws) == 8
    assert gdn.gdn_device_status(ws) == 0          # cleared by the read
    bad_cu = torch.tensor([0, 120, 100], dtype=torch.int32, device="cuda")  # non-monotone
    gdn.gdn_replay(d["q"], d["k"], d["v"], d["g"], d["beta"], bad_cu, d["r"],
                   total_out_tokens=50, ws=ws)
    # a later good call does not erase the recorded error
    gdn.gdn_replay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["r"],
                   total_out_tokens=50, ws=ws)
    assert gdn.gdn_device_status(ws) == 8
    short_out = torch.tensor([30, 20], dtype=torch.int32, device="cuda")   # sum r > rows of o
    gdn.gdn_replay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], short_out,
                   total_out_tokens=40, ws=ws)
    assert gdn.gdn_device_status(ws) == 8
    # without outputs the sum of r is not bounded by total_out_tokens
    gdn.gdn_replay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], short_out,
                   total_out_tokens=0, o_out=None, ws=ws)
    assert gdn.gdn_device_status(ws) == 0


def test_state_only_replay_fed_by_adaptive_lengths():
    # r straight from gdn_adaptive_replay_len (device array, never summed on the host) and
    # no outputs, so total_out_tokens = 0: every sequence still gets its state
    import gated_deltanet_state_gdn_amd as gdn
    w = W.small(W.config(1), L=[900, 300, 1500], r=[1, 1, 1], h_qk=2, h_v=4, g_mu=-3.0)
    host = W.make_inputs(w)
    d = to_dev(host)
    r_dev = gdn.gdn_adaptive_replay_len(d["g"], d["cu_seqlens"], eps=1e-2, r_min=16)
    ws = gdn.workspace(gdn.make_desc(d["q"], d["v"], 3, 0), "cuda")
    S, o, _ = gdn.gdn_replay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], r_dev,
                             total_out_tokens=0, o_out=None, ws=ws)
    assert gdn.gdn_device_status(ws) == 0 and o is None
    r_host = r_dev.cpu().numpy().astype(np.int64)
    say("  adaptive r", list(r_host))
    assert (r_host >= 16).all() and (r_host < np.array(w.lengths)).all()
    S_ref, _ = oracle.replay(host["q"], host["k"], host["v"], host["g"], host["beta"], host["cu_host"],
                             r_host, want_o=False)
    e = max(rel(oracle.widen(S[n, h]), S_ref[n, h]) for n in range(3) for h in range(4))
    say("  state-only adaptive replay: relerr S %.3e" % e)
    assert e <= TOL["bf16"]


def test_column_slices_are_bitwise_equal_to_whole_units():
    # 36 layers x 32 v-heads = 1152 units: 1024 whole-unit blocks plus the last 128 units
    # in two column slices each; one layer per call: every unit in eight slices.
    import gated_deltanet_state_gdn_amd as gdn
    w = W.small(W.config(2), L=[300], r=[130], layers=36)
    inp = W.make_inputs(w, device="cuda")
    say("case column slices vs whole units, 36 layers")
    tot = int(inp["r_host"].sum())
    S_all, o_all, _ = gdn.gdn_replay(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     inp["cu_seqlens"], inp["r"], total_out_tokens=tot)
    for layer in (0, 17, 35):
        sl = slice(300 * layer, 300 * (layer + 1))
        cu1 = torch.tensor([0, 300], dtype=torch.int32, device="cuda")
        r1 = inp["r"][layer:layer + 1].contiguous()
        S1, o1, _ = gdn.gdn_replay(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["g"][sl],
                                   inp["beta"][sl], cu1, r1, total_out_tokens=130)
        torch.cuda.synchronize()
        assert torch.equal(S1[0], S_all[layer])
        assert torch.equal(o1.view(torch.int16), o_all[130 * layer:130 * (layer + 1)].view(torch.int16))


@pytest.mark.parametrize("mu", [-2.0, 0.0, 3.0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fast_decay_renormalises_the_stored_state(mu, dtype):
    # alpha ~ 0.88, 0.5 and 0.05 per token: the decay over a chunk reaches 2^-60 within a
    # few chunks or at once (and underflows to 0 in fp32 for mu = 3), so the kernel
    # renormalises its stored state often; the result must not notice.  At mu = 3 the
    # in-chunk log-gate sums reach a few hundred: the compensated gate scan keeps the
    # differences behind every decay weight exact to their own size (a plain fp32 scan
    # put 1.5e-5 on S here, the CPU model of the kernel's arithmetic pins both)
    base = W.config(0) if dtype == "f32" else W.config(1)
    w = W.small(base, L=[700, 513], r=[650, 200], h_qk=2, h_v=4, g_mu=mu, g_sigma=1.0)
    tol = TOL[dtype]
    for mode in ("replay", "prefill"):
        inp, S, o, cu_out, eS, eo = _case(w, mode)
        assert eS <= tol and eo <= tol, (mode, eS, eo)


@pytest.mark.parametrize("mu", [-5.0, -8.0])
def test_bf16_large_values_inside_the_fp16_operand_range(mu):
    # v scaled by 128 (exact in bf16): state entries of a few hundred, so the stored state
    # S / sig (up to 64 |S| between renormalisations) approaches the fp16 operand range the
    # header states; the error must stay that of unit-scale values
    w = W.small(W.config(1), L=[1500, 700], r=[1200, 300], h_qk=2, h_v=4, g_mu=mu, g_sigma=0.5)
    inp = W.make_inputs(w)
    inp["v"] = (inp["v"].float() * 128.0).to(inp["v"].dtype)
    for mode in ("replay", "prefill"):
        S, o, _ = gpu_run(to_dev(inp), mode)
        torch.cuda.synchronize()
        S_ref, o_ref = oracle_run(inp, mode)
        eS, eo = compare(inp, mode, S, o, S_ref, o_ref)
        say("  mu %.0f %s: max|S| %.1f  relerr S %.3e  o %.3e" % (mu, mode, float(np.abs(S_ref).max()), eS, eo))
        assert np.isfinite(eS) and np.isfinite(eo)
        assert eS <= TOL["bf16"] and eo <= TOL["bf16"], (mode, eS, eo)


def test_bf16_range_contract_edge_and_beyond():
    # The header's range contract for bf16 inputs: state entries below ~10^3.  At its edge
    # (v scaled by 256, exact in bf16) the error must stay that of unit-scale values; far
    # beyond it (v scaled by 2^16, |S| in the 10^5 range, past fp16's 65504) the results
    # turn non-finite, and the error report's non-finite count must show it.
    import gated_deltanet_state_gdn_amd as gdn
    w = W.small(W.config(1), L=[1500, 700], r=[1200, 300], h_qk=2, h_v=4, g_mu=-8.0, g_sigma=0.5)
    base = W.make_inputs(w)
    for scale, inside in ((256.0, True), (65536.0, False)):
        inp = dict(base)
        inp["v"] = (base["v"].float() * scale).to(base["v"].dtype)
        S, o, _ = gpu_run(to_dev(inp), "replay")
        torch.cuda.synchronize()
        S_ref, o_ref = oracle_run(inp, "replay")
        smax = float(np.abs(S_ref).max())
        if inside:
            eS, eo = compare(inp, "replay", S, o, S_ref, o_ref)
            say("  v x %.0f: max|S| %.0f  relerr S %.3e  o %.3e" % (scale, smax, eS, eo))
            assert smax > 500.0
            assert eS <= TOL["bf16"] and eo <= TOL["bf16"], (eS, eo)
        else:
            ref = torch.from_numpy(S_ref.astype(np.float32)).cuda()
            rel, nf = gdn.gdn_state_relerr(S, ref)
            torch.cuda.synchronize()
            say("  v x %.0f: max|S| %.0f  non-finite entries flagged %d" % (scale, smax, int(nf.sum())))
            assert smax > 65504.0 and int(nf.sum()) > 0

