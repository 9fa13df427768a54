"""Seeded synthetic workloads for the Gated DeltaNet replay / prefill path.

This module only draws inputs. It holds none of the recurrence's arithmetic and is
imported by both sides of every comparison: the fp64 oracle under ``oracle/`` and
the HIP library's Python binding.  The two never import each other.

What the inputs stand in for.  Tail-Replay (arXiv 2608.30310, abstract) evaluates
time-to-first-token at matched prefixes of 8K, 16K and 32K tokens with a replay
budget of 5-10 % of the matched prefix, on Gated-DeltaNet hybrids (OLMo-Hybrid-7B,
Qwen3.5 models; gist.science technical summary, "Resultados").  No dataset or model
weight is used: each linear-attention layer receives synthetic post-projection
inputs q, k, v (per token and head), a log-decay g (alpha = exp(g)) and a write
strength beta.

Recipe (per layer, generator seeded with ``seed``; draw order q, k, v, x_g, x_b):
  * q, k ~ N(0, 1), then L2-normalised per (token, head) in fp32, then rounded to the
    storage dtype (bf16 round-to-nearest-even, or kept fp32);
  * v ~ N(0, 1), rounded to the storage dtype;
  * g = -softplus(mu + sigma * x_g), x_g ~ N(0, 1), kept fp32 (g <= 0, alpha in (0, 1]);
  * beta = sigmoid(x_b), x_b ~ N(0, 1), kept fp32;
  * optional reset: g[p_h, h] = -inf (alpha = 0) at one position per v-head;
  * optional key correlation rho (``key_corr``): k = normalise(a u_h + x_k) with x_k the
    N(0, 1) draw above, u_h a unit direction per q/k head (drawn after x_b) and
    a^2 = rho d_k / (1 - rho), so that keys of one head have mean pairwise cosine ~rho;
    rho = 1 gives every token of a head the same key.  Keys of a real Gated DeltaNet
    layer pass through a short convolution and a SiLU before their L2 norm and are far
    from independent; i.i.d. keys are the best-conditioned case of the UT transform;
  * optional fixed beta (``beta_value``) instead of sigmoid(x_b).
Sequence lengths, replay lengths and reset positions are drawn on the host with
numpy's PCG64 so that they do not depend on the device the tensors are drawn on.
Tensors are drawn with a ``torch.Generator`` on the requested device, so the same
seed gives different (but fixed) values on the CPU and on the GPU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional, Sequence

import numpy as np
import torch

__all__ = ["Workload", "CONFIGS", "replay_len", "make_inputs", "config"]


def replay_len(L: int, rho: float) -> int:
    """Replay length for a matched prefix of L tokens under budget fraction rho.

    The pages state the budget as the last 5-10 % of the matched prefix; the
    number of tokens is taken as clamp(ceil(rho * L), 0, L), which never spends
    less than the budget.  A tiny tolerance absorbs binary representation error
    (0.1 * 2048 = 204.8 must give 205, 0.05 * 8192 = 409.6 must give 410).
    """
    if L <= 0 or rho <= 0.0:
        return 0
    x = rho * L
    r = int(math.ceil(x - 1e-9 * max(1.0, x)))
    return max(0, min(L, r))


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: a batch of packed varlen sequences for one GDN layer.

    ``lengths`` are the matched-prefix lengths L_n and ``replay`` the replay lengths
    r_n of each packed sequence.  ``layers`` > 1 stacks independent layers as extra
    packed sequences (each layer's replay is independent of the others).
    """
    name: str
    h_qk: int
    h_v: int
    d_k: int
    d_v: int
    dtype: str                      # "f32" or "bf16": storage dtype of q, k, v and o
    lengths: Sequence[int]
    replay: Sequence[int]
    g_mu: float
    g_sigma: float
    seed: int
    layers: int = 1
    reset_heads: bool = False       # one alpha = 0 token per (sequence, v-head)
    reset_in_window: bool = False   # force that token inside the replay window
    scale: float = 1.0
    key_corr: float = 0.0           # mean pairwise cosine of one head's keys (1: repeated key)
    beta_value: Optional[float] = None   # fixed beta instead of sigmoid(N(0, 1))
    description: str = ""

    @property
    def n_seqs(self) -> int:
        return len(self.lengths) * self.layers

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths)) * self.layers

    @property
    def total_replay(self) -> int:
        return int(sum(self.replay)) * self.layers

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _cfg3_structure(seed: int, n: int = 64):
    rs = np.random.Generator(np.random.PCG64(seed))
    L = rs.integers(1024, 32768, size=n, endpoint=True)
    rho = rs.uniform(0.05, 0.10, size=n)
    r = [replay_len(int(a), float(b)) for a, b in zip(L, rho)]
    return [int(x) for x in L], r


def _build_configs():
    c = {}
    c[0] = Workload(
        name="gdn_f32_h4_d64_L2048_r10", h_qk=4, h_v=4, d_k=64, d_v=64, dtype="f32",
        lengths=[2048], replay=[replay_len(2048, 0.10)], g_mu=-4.0, g_sigma=1.0, seed=1000,
        description="one GDN layer, 1 sequence, 4 heads, d=64, fp32; L=2048, r=205 (10%)")
    c[1] = Workload(
        name="gdn_bf16_h16_d128_L8192_r5", h_qk=16, h_v=16, d_k=128, d_v=128, dtype="bf16",
        lengths=[8192], replay=[replay_len(8192, 0.05)], g_mu=-5.0, g_sigma=1.0, seed=1100,
        description="one GDN layer, 16 heads, d=128, bf16, fp32 state; L=8192, r=410 (5%)")
    c[2] = Workload(
        name="gdn_stack36_bf16_hqk16_hv32_d128_L32768_r10", h_qk=16, h_v=32, d_k=128, d_v=128,
        dtype="bf16", lengths=[32768], replay=[replay_len(32768, 0.10)], g_mu=-5.0, g_sigma=1.0,
        seed=1200, layers=36,
        description="36 independent GDN layers, 16 q/k heads shared by 32 v heads, d=128, "
                    "bf16; L=32768, r=3277 (10%)")
    L3, r3 = _cfg3_structure(1300)
    c[3] = Workload(
        name="gdn_varlen64_bf16_h16_d128", h_qk=16, h_v=16, d_k=128, d_v=128, dtype="bf16",
        lengths=L3, replay=r3, g_mu=-5.0, g_sigma=1.0, seed=1300,
        description="64 packed cache hits, L~U{1024..32768}, r=ceil(U[.05,.10]*L), "
                    "16 heads, d=128, bf16")
    c[4] = Workload(
        name="gdn_slowdecay_bf16_h16_d128_L32768", h_qk=16, h_v=16, d_k=128, d_v=128,
        dtype="bf16", lengths=[32768], replay=[replay_len(32768, 0.10)], g_mu=-8.0,
        g_sigma=0.5, seed=1400,
        description="slow decay alpha~0.9997, L=32768; replay budgets 1,2,5,10,20% "
                    "(variant: alpha=0 at a random position per head)")
    return c


CONFIGS = _build_configs()
GATE_SWEEP = (0.01, 0.02, 0.05, 0.10, 0.20)


def config(i: int, **overrides) -> Workload:
    w = CONFIGS[i]
    return w.with_(**overrides) if overrides else w


def _round_storage(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x.to(torch.float32)
    raise ValueError(dtype)


def _draw_layer(w: Workload, L_total: int, seed: int, device) -> dict:
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    f32 = torch.float32
    q = torch.randn((L_total, w.h_qk, w.d_k), generator=gen, device=device, dtype=f32)
    k = torch.randn((L_total, w.h_qk, w.d_k), generator=gen, device=device, dtype=f32)
    v = torch.randn((L_total, w.h_v, w.d_v), generator=gen, device=device, dtype=f32)
    xg = torch.randn((L_total, w.h_v), generator=gen, device=device, dtype=f32)
    xb = torch.randn((L_total, w.h_v), generator=gen, device=device, dtype=f32)
    q = q / q.norm(dim=-1, keepdim=True)
    if w.key_corr > 0.0:
        u = torch.randn((w.h_qk, w.d_k), generator=gen, device=device, dtype=f32)
        u = u / u.norm(dim=-1, keepdim=True)
        if w.key_corr >= 1.0:
            k = k[:1].expand_as(k).clone()
        else:
            k = k + math.sqrt(w.key_corr * w.d_k / (1.0 - w.key_corr)) * u
    k = k / k.norm(dim=-1, keepdim=True)
    g = -torch.nn.functional.softplus(w.g_mu + w.g_sigma * xg)
    beta = torch.sigmoid(xb) if w.beta_value is None else torch.full_like(xb, float(w.beta_value))
    return dict(q=_round_storage(q, w.dtype), k=_round_storage(k, w.dtype),
                v=_round_storage(v, w.dtype), g=g.contiguous(), beta=beta.contiguous())


def reset_positions(w: Workload, layer: int = 0) -> Optional[np.ndarray]:
    """Positions (relative to each sequence start) of the alpha = 0 token, [n_seq, h_v]."""
    if not w.reset_heads:
        return None
    rs = np.random.Generator(np.random.PCG64(w.seed * 7919 + layer))
    out = np.zeros((len(w.lengths), w.h_v), dtype=np.int64)
    for n, (L, r) in enumerate(zip(w.lengths, w.replay)):
        if w.reset_in_window and r > 0:
            out[n] = rs.integers(L - r, L, size=w.h_v)
        else:
            out[n] = rs.integers(0, L, size=w.h_v)
    return out


def make_inputs(w: Workload, device="cpu") -> dict:
    """Draw the packed varlen inputs of workload ``w`` on ``device``.

    Returns a dict with q, k ([T, h_qk, d_k]), v ([T, h_v, d_v]) in the storage dtype,
    g, beta ([T, h_v], fp32), cu_seqlens ([N+1], int32), r ([N], int32), all on
    ``device``, plus host copies ``cu_host``/``r_host`` (int64 numpy) and ``resets``.
    Layers are stacked as consecutive packed sequences, layer-major.
    """
    device = torch.device(device)
    Ls = list(w.lengths)
    per_layer = int(sum(Ls))
    T = per_layer * w.layers
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q = torch.empty((T, w.h_qk, w.d_k), dtype=tdt, device=device)
    k = torch.empty((T, w.h_qk, w.d_k), dtype=tdt, device=device)
    v = torch.empty((T, w.h_v, w.d_v), dtype=tdt, device=device)
    g = torch.empty((T, w.h_v), dtype=torch.float32, device=device)
    beta = torch.empty((T, w.h_v), dtype=torch.float32, device=device)
    resets = []
    for layer in range(w.layers):
        d = _draw_layer(w, per_layer, w.seed + layer, device)
        sl = slice(layer * per_layer, (layer + 1) * per_layer)
        q[sl] = d["q"]; k[sl] = d["k"]; v[sl] = d["v"]
        gl = d["g"]
        pos = reset_positions(w, layer)
        if pos is not None:
            starts = np.concatenate([[0], np.cumsum(Ls)[:-1]])
            rows = torch.as_tensor((starts[:, None] + pos).reshape(-1), device=device)
            cols = torch.as_tensor(np.tile(np.arange(w.h_v), len(Ls)), device=device)
            gl[rows, cols] = float("-inf")
            resets.append(pos)
        g[sl] = gl; beta[sl] = d["beta"]
        del d
    lengths = Ls * w.layers
    rr = list(w.replay) * w.layers
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    r = np.asarray(rr, dtype=np.int64)
    return dict(q=q, k=k, v=v, g=g, beta=beta,
                cu_seqlens=torch.as_tensor(cu.astype(np.int32), device=device),
                r=torch.as_tensor(r.astype(np.int32), device=device),
                cu_host=cu, r_host=r, resets=resets, workload=w)


def small(w: Workload, L: Sequence[int], r: Sequence[int], layers: int = 1, **kw) -> Workload:
    """A reduced copy of ``w`` with other lengths, for tests the oracle finishes quickly."""
    return w.with_(lengths=list(L), replay=list(r), layers=layers, **kw)
