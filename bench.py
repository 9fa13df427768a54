"""Benchmark: Gated DeltaNet state rebuild by tail replay on one MI355X.

Default workload: a stack of 36 independent GDN layers (16 q/k heads shared by 32
v heads, d_k = d_v = 128, bf16 inputs, fp32 state), matched prefix L = 32768,
replay budget 10 % (r = 3277), outputs o emitted.  The 36 layers' replays are
independent (each layer has its own inputs and its own state), so one step is one
gdn_replay call over the 36 layers packed as 36 sequences.

Metric: replayed tokens per second per GDN layer (= 36 * r / step time) and the
state-rebuild time per layer (step time / 36).  Inputs are resident in HBM when the
timed region starts.  A workload of under 1 GiB per step (the single-layer ones) would
be served from the 256 MB MALL on repeated steps, so it is timed step by step after a
1 GiB write, and its step time is the median per-launch time.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload cfg2|cfg1|cfg4|cfg3]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, 8 TB/s
METRIC = "replayed tokens/s per GDN layer; state-rebuild µs at 32K prefix/10% replay"


def algorithmic_bytes(w, tokens: int, n_states: int, with_o: bool) -> int:
    """Bytes a call must move at minimum: q, k (q only with o), v, g, beta read once per
    token; o written once per token; S written once per (sequence, v-head)."""
    b = 2 if w.dtype == "bf16" else 4
    per_tok = (2 if with_o else 1) * w.h_qk * w.d_k * b + w.h_v * w.d_v * b + 8 * w.h_v
    if with_o:
        per_tok += w.h_v * w.d_v * b
    return tokens * per_tok + n_states * w.h_v * w.d_k * w.d_v * 4


def algorithmic_flops(w, tokens: int, with_o: bool, C: int = 64) -> float:
    """Chunked-form flops per token (C = 64): q/k Gram products per q/k head, and the
    UT solve, pseudo-value, output and state products per v-head."""
    o = 1 if with_o else 0
    d = w.d_k
    return tokens * (w.h_qk * (2 + 2 * o) * C * d + w.h_v * ((4 + 2 * o) * C * d + (4 + 2 * o) * d * d))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="cfg2")
    ap.add_argument("--no-o", action="store_true", help="state only (no per-token outputs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-extra", action="store_true", help="skip prefill / per-layer timings")
    ap.add_argument("--no-sweep", action="store_true", help="skip the slow-decay replay-budget sweep")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(1, args.steps))
        return

    if args.gpus != 1:
        print(json.dumps({"error": "the replay benchmark runs on one GPU; --gpus %d is not supported "
                                   "(the path shards by (sequence, v-head) with no exchange, "
                                   "see the design notes)" % args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import gated_deltanet_state_gdn_amd as gdn
    import workloads as W

    gdn.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = {"cfg0": 0, "cfg1": 1, "cfg2": 2, "cfg3": 3, "cfg4": 4}[args.workload]
    w = W.config(cfg)
    with_o = not args.no_o
    t_gen = time.time()
    inp = W.make_inputs(w, device=dev)
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen
    q, k, v, g, beta = inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"]
    cu, r = inp["cu_seqlens"], inp["r"]
    n_seqs = len(inp["r_host"])
    tot = int(inp["r_host"].sum())
    desc = gdn.make_desc(q, v, n_seqs, tot, w.scale)
    ws = gdn.workspace(desc, dev)
    S = torch.empty((n_seqs, w.h_v, w.d_k, w.d_v), dtype=torch.float32, device=dev)
    o = torch.empty((tot, w.h_v, w.d_v), dtype=q.dtype, device=dev) if with_o else None
    stream = torch.cuda.current_stream()

    def step():
        gdn.gdn_replay(q, k, v, g, beta, cu, r, total_out_tokens=tot, S_out=S, o_out=o, ws=ws,
                       scale=w.scale, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    status = gdn.gdn_device_status(ws, stream)
    if status != 0:
        raise RuntimeError("device status %d" % status)

    # A workload whose bytes fit in the 256 MB MALL several times over would be served
    # from it on repeated steps: such workloads flush it before every step and take the
    # step time from the per-launch events (median) instead of the wall clock.
    flush = MallFlush(dev)
    cold = algorithmic_bytes(w, tot, n_seqs, with_o) < (1 << 30)

    # timed region: K steps, per-launch events on the launch stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if cold:
            flush()
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = float(np.median(launch_ms)) if cold else wall * 1e3 / args.steps
    kern_ms = float(np.mean(launch_ms))
    launch_stats = {"mean": kern_ms, "median": float(np.median(launch_ms)),
                    "p10": float(np.percentile(launch_ms, 10)),
                    "p90": float(np.percentile(launch_ms, 90)),
                    "min": float(np.min(launch_ms)), "max": float(np.max(launch_ms))}

    layers = n_seqs if w.layers > 1 else 1
    # per GDN layer: a layer rebuilds r tokens in t_step / layers, so its throughput is
    # (layers * r) / t_step = replayed tokens of the step over the step time.
    value = tot / (ms_per_step * 1e-3)
    abytes = algorithmic_bytes(w, tot, n_seqs, with_o)
    aflops = algorithmic_flops(w, tot, with_o)
    achieved = abytes / (kern_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "n_seqs": n_seqs, "h_qk": w.h_qk,
                   "h_v": w.h_v, "d_k": w.d_k, "d_v": w.d_v, "L": list(w.lengths)[:4],
                   "r": list(w.replay)[:4], "replayed_tokens_per_step": tot, "with_o": with_o,
                   "state": "fp32"},
        "rebuild_us_per_layer": kern_ms * 1e3 / layers,
        "launch_ms": launch_stats,
        "mall_flushed_per_step": cold,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_from_profile(kern_ms),
                     "algorithmic_bytes_per_launch": abytes, "kernel_ms": kern_ms,
                     "algorithmic_tflops": aflops / (kern_ms * 1e-3) / 1e12},
    }

    if not args.no_extra:
        # the same replay without per-token outputs, against its own algorithmic bytes
        if with_o:
            fs = lambda: gdn.gdn_replay(q, k, v, g, beta, cu, r, total_out_tokens=tot, S_out=S,
                                        o_out=None, ws=ws, scale=w.scale, stream=stream)
            ms_s = _time(fs, stream, 10)
            ab_s = algorithmic_bytes(w, tot, n_seqs, False)
            out["state_only"] = {"us_per_layer": ms_s * 1e3 / layers,
                                 "replayed_tokens_per_s": tot / (ms_s * 1e-3),
                                 "algorithmic_bytes_per_launch": ab_s,
                                 "roofline_frac": ab_s / (ms_s * 1e-3) / 1e9 / HBM_PEAK_GBS}
        # one layer per call (latency of a single layer's rebuild)
        if w.layers > 1:
            per = int(inp["cu_host"][1])
            sl = slice(0, per)
            r1 = r[:1]
            cu1 = cu[:2]
            o1 = torch.empty((int(inp["r_host"][0]), w.h_v, w.d_v), dtype=q.dtype, device=dev) if with_o else None
            S1 = torch.empty((1, w.h_v, w.d_k, w.d_v), dtype=torch.float32, device=dev)
            f1 = lambda: gdn.gdn_replay(q[sl], k[sl], v[sl], g[sl], beta[sl], cu1, r1,
                                        total_out_tokens=int(inp["r_host"][0]), S_out=S1, o_out=o1,
                                        ws=ws, scale=w.scale, stream=stream)
            out["single_layer_call_us"] = _time_cold(f1, stream, 10, flush) * 1e3
            out["single_layer_segmented"] = segmented_leg(
                gdn, w, (q[sl], k[sl], v[sl], g[sl], beta[sl], cu1, r1), int(inp["r_host"][0]), 1, dev,
                stream, flush)
        elif n_seqs == 1 and w.d_k == w.d_v:
            out["segmented"] = segmented_leg(gdn, w, (q, k, v, g, beta, cu, r), tot, 1, dev, stream, flush)
        # full prefill of the same packed prefixes (the baseline the replay replaces)
        Sp = torch.empty_like(S)
        op = torch.empty((int(q.shape[0]), w.h_v, w.d_v), dtype=q.dtype, device=dev) if with_o else None
        fp = lambda: gdn.gdn_prefill(q, k, v, g, beta, cu, S_out=Sp, o_out=op, ws=ws,
                                     scale=w.scale, stream=stream)
        fp()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            fp()
        e1.record(stream)
        torch.cuda.synchronize()
        pms = e0.elapsed_time(e1) / 3
        out["prefill_us_per_layer"] = pms * 1e3 / layers
        out["prefill_over_replay"] = pms / kern_ms
        rel, nf = gdn.gdn_state_relerr(S, Sp, stream=stream)
        torch.cuda.synchronize()
        out["relerr_replay_vs_full"] = {"max": float(rel.max()), "median": float(rel.median()),
                                        "nonfinite": int(nf.sum())}
        del op
        if len(set(w.lengths)) == 1:
            out["suffix_prefill"] = suffix_leg(w, inp, gdn, stream, ws, pms / layers, n_seqs)
        out["adaptive_replay_len"] = adaptive_leg(w, inp, gdn, stream, ws, Sp, layers, with_o)
        out["transfer_overlap"] = overlap_leg(step, stream, kern_ms)
        if not args.no_sweep:
            out["gate_sweep"] = gate_sweep_leg(gdn, stream, with_o, flush)
        del Sp

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, with_o, args.cpu_seconds)

    print(json.dumps(out), flush=True)


class MallFlush:
    """Writes 1 GiB (four times the 256 MB last-level MALL) so that the next timed call
    finds none of its inputs in the cache."""

    def __init__(self, device, nbytes=1 << 30):
        import torch
        self.buf = torch.empty(nbytes // 4, dtype=torch.int32, device=device)
        self.k = 0

    def __call__(self):
        self.k += 1
        self.buf.fill_(self.k)


def segmented_leg(gdn, w, args, tot, n_seqs, dev, stream, flush, n_segments=0):
    """One layer's replay cut into segments (gdn_replay_segmented) against the plain call,
    cold (MALL flushed before each call): with outputs and state only, and the relative
    error of the segmented state against the plain one."""
    import torch
    desc = gdn.make_desc(args[0], args[2], n_seqs, tot, w.scale)
    ws = torch.zeros(gdn.gdn_segmented_workspace_bytes(desc, n_segments), dtype=torch.uint8, device=dev)
    ws0 = gdn.workspace(desc, dev)
    S0 = torch.empty((n_seqs, w.h_v, w.d_k, w.d_v), dtype=torch.float32, device=dev)
    S1 = torch.empty_like(S0)
    o = torch.empty((tot, w.h_v, w.d_v), dtype=args[0].dtype, device=dev)
    # (0: the library's choice from the head count and the replay length, see include/gdn.h)
    auto = max(1, min(16, 128 // (n_seqs * w.h_v), ((tot // n_seqs + 63) // 64) // 6))
    res = {"n_segments": n_segments if n_segments else auto}
    for name, oo in (("with_o_us", o), ("state_only_us", None)):
        fp = lambda: gdn.gdn_replay(*args, total_out_tokens=tot, S_out=S0, o_out=oo, ws=ws0, scale=w.scale,
                                    stream=stream)
        fs = lambda: gdn.gdn_replay_segmented(*args, total_out_tokens=tot, n_segments=n_segments, S_out=S1,
                                              o_out=oo, ws=ws, scale=w.scale, stream=stream)
        res[name] = _time_cold(fs, stream, 10, flush) * 1e3
        res["plain_" + name] = _time_cold(fp, stream, 10, flush) * 1e3
    rel, _ = gdn.gdn_state_relerr(S1, S0, stream=stream)
    torch.cuda.synchronize()
    res["relerr_S_vs_plain"] = float(rel.max())
    if gdn.gdn_device_status(ws, stream) != 0:
        raise RuntimeError("segmented replay: device status")
    return res


def _time_cold(fn, stream, reps, flush):
    """Median time (ms) of `reps` single calls, each after a MALL flush, with events on
    the launch stream around the call only."""
    import numpy as np
    import torch
    fn()
    ts = []
    for _ in range(reps):
        with torch.cuda.stream(stream):
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def _time(fn, stream, reps):
    import torch
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def suffix_leg(w, inp, gdn, stream, ws, full_prefill_ms_per_layer, n_seqs, suffix=1024):
    """Replay over a matched prefix of L - suffix tokens (10 % budget, state only) plus a
    prefill of the suffix from the rebuilt state, against the full prefill of all L
    tokens: the linear-attention part of time-to-first-token after a cache hit."""
    import numpy as np
    import torch
    import workloads as W
    L = int(w.lengths[0])
    Lp = L - suffix
    rp = W.replay_len(Lp, 0.10)
    dev = inp["q"].device
    # sequence n's matched prefix ends `suffix` tokens before its end; the prefix of
    # sequence n > 0 starts with the previous layer's suffix, which a replay of rp <= Lp
    # tokens never reads
    cu_p = torch.tensor([0] + [n * L + Lp for n in range(n_seqs)], dtype=torch.int32, device=dev)
    r_p = torch.full((n_seqs,), rp, dtype=torch.int32, device=dev)
    idx = torch.cat([torch.arange(n * L + Lp, (n + 1) * L, device=dev) for n in range(n_seqs)])
    suf = {k: inp[k].index_select(0, idx).contiguous() for k in ("q", "k", "v", "g", "beta")}
    cu_s = torch.arange(0, (n_seqs + 1) * suffix, suffix, dtype=torch.int32, device=dev)
    S_r = torch.empty((n_seqs, w.h_v, w.d_k, w.d_v), dtype=torch.float32, device=dev)
    S_f = torch.empty_like(S_r)
    o_f = torch.empty((n_seqs * suffix, w.h_v, w.d_v), dtype=inp["q"].dtype, device=dev)
    q, k, v, g, beta = (inp[x] for x in ("q", "k", "v", "g", "beta"))

    def rebuild():
        gdn.gdn_replay(q, k, v, g, beta, cu_p, r_p, total_out_tokens=n_seqs * rp, S_out=S_r,
                       o_out=None, ws=ws, scale=w.scale, stream=stream)

    def rest():
        gdn.gdn_prefill(suf["q"], suf["k"], suf["v"], suf["g"], suf["beta"], cu_s, S0=S_r,
                        S_out=S_f, o_out=o_f, ws=ws, scale=w.scale, stream=stream)

    def both():
        rebuild()
        rest()

    reps = 5
    t_rep = _time(rebuild, stream, reps) / n_seqs
    t_suf = _time(rest, stream, reps) / n_seqs
    t_both = _time(both, stream, reps) / n_seqs
    return {"matched_prefix": Lp, "replay_tokens": rp, "suffix_tokens": suffix,
            "replay_state_only_us_per_layer": t_rep * 1e3,
            "suffix_prefill_us_per_layer": t_suf * 1e3,
            "replay_plus_suffix_us_per_layer": t_both * 1e3,
            "full_prefill_us_per_layer": full_prefill_ms_per_layer * 1e3,
            "speedup_vs_full_prefill": full_prefill_ms_per_layer / t_both}


def adaptive_leg(w, inp, gdn, stream, ws, S_full, layers, with_o, eps=1e-3):
    """Replay length chosen per sequence from the gates (prod alpha <= eps in every
    v-head), then the replay with that length, and its error against full prefill."""
    import torch
    g, cu = inp["g"], inp["cu_seqlens"]
    n = int(cu.shape[0]) - 1
    r = torch.empty(n, dtype=torch.int32, device=g.device)
    sel = lambda: gdn.gdn_adaptive_replay_len(g, cu, eps=eps, r_out=r, ws=ws, stream=stream)
    t_sel = _time(sel, stream, 5)
    rh = r.cpu().numpy()
    tot = int(rh.sum())
    S = torch.empty_like(S_full)
    o = torch.empty((tot, w.h_v, w.d_v), dtype=inp["q"].dtype, device=g.device) if with_o else None
    rep = lambda: gdn.gdn_replay(inp["q"], inp["k"], inp["v"], g, inp["beta"], cu, r,
                                 total_out_tokens=tot, S_out=S, o_out=o, ws=ws, scale=w.scale,
                                 stream=stream)
    t_rep = _time(rep, stream, 5)
    rel, nf = gdn.gdn_state_relerr(S, S_full, stream=stream)
    torch.cuda.synchronize()
    return {"eps": eps, "r_mean": float(rh.mean()), "r_min": int(rh.min()), "r_max": int(rh.max()),
            "select_us_per_layer": t_sel * 1e3 / layers,
            "replay_us_per_layer": t_rep * 1e3 / layers,
            "relerr_vs_full": {"max": float(rel.max()), "median": float(rel.median()),
                               "nonfinite": int(nf.sum())}}


def gate_sweep_leg(gdn, stream, with_o, flush):
    """Slow-decay layer (16 heads, d = 128, bf16, L = 32768, alpha ~ 0.9997), without and
    with one alpha = 0 token per head: replay time and error against full prefill at the
    replay budgets 1, 2, 5, 10 and 20 %, and the full prefill itself (each call timed
    alone after a MALL flush, median)."""
    import torch
    import workloads as W
    res = {}
    for variant, resets in (("plain", False), ("reset", True)):
        w = W.config(4).with_(reset_heads=resets)
        inp = W.make_inputs(w, device=stream.device)
        q, k, v, g, beta, cu = (inp[x] for x in ("q", "k", "v", "g", "beta", "cu_seqlens"))
        L = int(w.lengths[0])
        S_full, _ = gdn.gdn_prefill(q, k, v, g, beta, cu, o_out=None, stream=stream)
        t_full = _time_cold(lambda: gdn.gdn_prefill(q, k, v, g, beta, cu, S_out=S_full, o_out=None,
                                                    stream=stream), stream, 2, flush)
        rows = []
        for rho in W.GATE_SWEEP:
            rr = W.replay_len(L, rho)
            r = torch.tensor([rr], dtype=torch.int32, device=q.device)
            S = torch.empty_like(S_full)
            o = torch.empty((rr, w.h_v, w.d_v), dtype=q.dtype, device=q.device) if with_o else None
            fn = lambda: gdn.gdn_replay(q, k, v, g, beta, cu, r, total_out_tokens=rr, S_out=S,
                                        o_out=o, stream=stream)
            t = _time_cold(fn, stream, 5, flush)
            rel, _ = gdn.gdn_state_relerr(S, S_full, stream=stream)
            torch.cuda.synchronize()
            rows.append({"budget": rho, "r": rr, "replay_us": t * 1e3,
                         "replayed_tokens_per_s": rr / (t * 1e-3),
                         "relerr_max": float(rel.max()), "relerr_median": float(rel.median())})
        res[variant] = {"full_prefill_us": t_full * 1e3, "budgets": rows}
        del inp
    return res


def overlap_leg(step, stream, replay_ms, fa_layers=12, kv_heads=2, head_dim=256, tokens=32768):
    """A second stream copies a pinned host buffer the size of a hybrid stack's
    full-attention KV cache (fa_layers x K and V x kv_heads x head_dim, bf16, for the
    matched prefix) to the device while the replay runs on its own stream."""
    import torch
    nbytes = fa_layers * 2 * kv_heads * head_dim * 2 * tokens
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    host.fill_(7)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()              # default priority
    copy = lambda: dst.copy_(host, non_blocking=True)

    def run(overlap):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        if overlap:
            side.wait_event(e0)
            with torch.cuda.stream(side):
                copy()
            step()
            done = torch.cuda.Event()
            done.record(side)
            stream.wait_event(done)
        else:
            with torch.cuda.stream(stream):
                copy()
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    run(False); run(True)
    ser = min(run(False) for _ in range(3))
    ovl = min(run(True) for _ in range(3))
    with torch.cuda.stream(stream):
        t_copy = _time(copy, stream, 3)
    del host, dst
    return {"fa_kv_bytes": nbytes, "copy_ms": t_copy, "replay_ms": replay_ms,
            "serialized_ms": ser, "overlapped_ms": ovl, "saved_frac": 1.0 - ovl / ser}


def copy_calibration(mib: int, reps: int):
    """A plain device-to-device copy of known size (the scale for FETCH_SIZE/WRITE_SIZE)."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n,
                      "launches": reps}), flush=True)


def traffic_from_profile(kernel_ms):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    kernel source as it is now (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gdn_chunk_ws_traffic.json")
    src = os.path.join(ROOT, "gated_deltanet_state_gdn_amd", "csrc", "gdn_chunk_ws.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, with_o, budget_s):
    """The fp64 oracle on this host's cores, on a bounded sample of the same workload:
    whole layers (all v-heads of one packed sequence) replayed until ~budget_s seconds."""
    import oracle
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cu, r = inp["cu_host"], inp["r_host"]
    done_tok, t_used, layers = 0, 0.0, 0
    for n in range(len(r)):
        end = int(cu[n + 1]); s = end - int(r[n])
        sl = slice(s, end)
        q, k, v = (oracle.widen(inp[x][sl]) for x in ("q", "k", "v"))
        g, b = oracle.widen(inp["g"][sl]), oracle.widen(inp["beta"][sl])
        t0 = time.perf_counter()
        oracle.replay(q, k, v, g, b, [0, end - s], [end - s], scale=w.scale, want_o=with_o,
                      threads=threads)
        t_used += time.perf_counter() - t0
        done_tok += end - s
        layers += 1
        if t_used >= budget_s:
            break
    return {"value": done_tok / t_used, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d packed sequences (layers), all %d v-heads, %d replayed tokens, "
                      "fp64 token-by-token, %.1f s" % (layers, len(r), w.h_v, done_tok, t_used)}


if __name__ == "__main__":
    main()
