"""Seeded synthetic inputs for the replay workloads.

This module only draws random inputs with the workloads' shapes and
distributions; it contains none of the replay arithmetic (no tail rule, no
recurrence, no projections).  Both the test oracle and the GPU library consume
what it produces.

Distributions (the workload descriptions of the replay benchmark):
  q, k   ~ N(0, 1), each head vector scaled to unit L2 norm; q further x dk^-1/2
  v      ~ N(0, 1)
  g      = log alpha = -softplus(z), z ~ N(-4, 1)
  beta   = sigmoid(N(0, 1))
  hidden ~ N(0, 1) (bf16), weights ~ N(0, 0.02) (bf16), one seed per (group, layer)
  matched prefix lengths m ~ U{4096 .. 131072} (integers, inclusive)

Two back ends draw the same distributions: ``numpy`` (PCG64, reproducible on any
host; the default) and ``torch`` (the device's Philox generator, for inputs too
large to draw quickly on the host).  A given (seed, back end) pair always gives
the same bits.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


def _softplus_np(z):
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def _normal(shape, rng, backend, device, gen):
    if backend == "numpy":
        return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32))
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _unit_heads(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)


@dataclass
class GdnInputs:
    q: torch.Tensor          # [T, Hqk, dk]
    k: torch.Tensor          # [T, Hqk, dk]
    v: torch.Tensor          # [T, Hv, dv]
    g: torch.Tensor          # [T, Hv] fp32, log alpha
    beta: torch.Tensor       # [T, Hv] fp32
    cu_seqlens: torch.Tensor  # [B+1] int32 (host)

    def to(self, device):
        return GdnInputs(self.q.to(device), self.k.to(device), self.v.to(device),
                         self.g.to(device), self.beta.to(device), self.cu_seqlens)


def cu_from_lengths(lengths) -> torch.Tensor:
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(np.asarray(lengths, dtype=np.int64), out=cu[1:])
    return torch.from_numpy(cu.astype(np.int32))


def gdn_inputs(lengths, Hqk, Hv, dk, dv, dtype=torch.bfloat16, seed=0,
               backend="numpy", device="cpu", q_prescaled=True) -> GdnInputs:
    """Packed varlen inputs for one LA layer: one sequence per entry of ``lengths``."""
    cu = cu_from_lengths(lengths)
    T = int(cu[-1])
    rng = np.random.default_rng(seed) if backend == "numpy" else None
    gen = None
    if backend == "torch":
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
    dev = "cpu" if backend == "numpy" else device
    q = _unit_heads(_normal((T, Hqk, dk), rng, backend, dev, gen))
    if q_prescaled:
        q = q * dk ** -0.5
    k = _unit_heads(_normal((T, Hqk, dk), rng, backend, dev, gen))
    v = _normal((T, Hv, dv), rng, backend, dev, gen)
    z = _normal((T, Hv), rng, backend, dev, gen) - 4.0
    g = -torch.nn.functional.softplus(z.double()).float() if backend == "torch" else \
        torch.from_numpy((-_softplus_np(z.numpy().astype(np.float64))).astype(np.float32))
    zb = _normal((T, Hv), rng, backend, dev, gen)
    beta = torch.sigmoid(zb.double()).float()
    out = GdnInputs(q.to(dtype), k.to(dtype), v.to(dtype), g.contiguous(), beta.contiguous(), cu)
    if backend == "numpy" and device != "cpu":
        out = out.to(device)
    return out


def prefix_lengths(n_hits, seed, lo=4096, hi=131072):
    """Matched prefix lengths m ~ U{lo..hi} (inclusive) for concurrent cache hits."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi, size=n_hits, endpoint=True)]


@dataclass
class GroupInputs:
    h_tail: torch.Tensor     # [G, n, d_model] bf16
    weights: list            # [G][L] dict of bf16 tensors ([out, in] row-major)


def group_inputs(G, L, n, d_model, Hqk, Hv, dk, dv, seed=0, w_std=0.02,
                 backend="numpy", device="cpu") -> GroupInputs:
    """Cached FA hiddens h ~ N(0,1) and per-(group, layer) weights ~ N(0, w_std), bf16."""
    shapes = {"w_qk": (2 * Hqk * dk, d_model), "w_v": (Hv * dv, d_model),
              "w_a": (Hv, d_model), "w_b": (Hv, d_model), "w_o": (d_model, Hv * dv)}

    def draw(shape, s, scale):
        if backend == "numpy":
            r = np.random.default_rng(s)
            return (torch.from_numpy(r.standard_normal(shape, dtype=np.float32)) * scale).to(torch.bfloat16)
        gen = torch.Generator(device=device)
        gen.manual_seed(s)
        return (torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * scale).to(torch.bfloat16)

    h = draw((G, n, d_model), seed, 1.0)
    weights = []
    for gi in range(G):
        row = []
        for li in range(L):
            base = 1_000_003 * (seed + 1) + 1009 * gi + 17 * li
            row.append({name: draw(shape, base + j, w_std)
                        for j, (name, shape) in enumerate(shapes.items())})
        weights.append(row)
    if backend == "numpy" and device != "cpu":
        h = h.to(device)
        weights = [[{k: t.to(device) for k, t in d.items()} for d in row] for row in weights]
    return GroupInputs(h, weights)


# Workload shapes.  The replay length of a hit is NOT computed here: callers apply
# the tail rule to the matched prefix length m.
WORKLOADS = {
    "tiny": dict(desc="1 LA layer, 1 head, dk=dv=64, fp32, 256 tokens from zero state",
                 B=1, Hqk=1, Hv=1, dk=64, dv=64, dtype="f32", n_tokens=256),
    "single_hit": dict(desc="1 LA layer, 16 heads, dk=dv=128, bf16, m=32768, r=0.05",
                       B=1, Hqk=16, Hv=16, dk=128, dv=128, dtype="bf16", m=32768, r=(5, 100)),
    "batched": dict(desc="36 (group, LA layer) instances, 32 v-heads / 16 qk-heads, dk=dv=128, "
                         "bf16, m=32768, r=0.10",
                    B=36, Hqk=16, Hv=32, dk=128, dv=128, dtype="bf16", m=32768, r=(10, 100)),
    "batched_r05": dict(desc="as 'batched' at r=0.05 (the 32K-prefix, 5%-replay batched shape)",
                        B=36, Hqk=16, Hv=32, dk=128, dv=128, dtype="bf16", m=32768, r=(5, 100)),
    "group": dict(desc="12 groups x 3 LA layers, d_model=2048, 16 qk / 32 v heads, dk=dv=128, "
                       "m=32768, r=0.05",
                  G=12, L=3, d_model=2048, Hqk=16, Hv=32, dk=128, dv=128, m=32768, r=(5, 100)),
    "varlen": dict(desc="64 hits, m ~ U{4096..131072}, r=0.05, 16 heads, dk=dv=128, bf16",
                   n_hits=64, Hqk=16, Hv=16, dk=128, dv=128, dtype="bf16", r=(5, 100)),
    "fidelity": dict(desc="one 32768-token sequence from zero, 16 heads, dk=dv=128, bf16; tails at "
                          "r=0.05 and 0.10 of the same sequence",
                     B=1, Hqk=16, Hv=16, dk=128, dv=128, dtype="bf16", m=32768, r=(5, 100),
                     rs=[(5, 100), (10, 100)]),
    "full_prefix": dict(desc="the group workload at r=1: 12 groups x 3 LA layers over all 32768 tokens",
                        G=12, L=3, d_model=2048, Hqk=16, Hv=32, dk=128, dv=128, m=32768, r=(100, 100)),
    "decode": dict(desc="one-token step on 36 instances x 32 v-heads (16 qk-heads), dk=dv=128, bf16 "
                        "inputs, fp32 resident states",
                   B=36, Hqk=16, Hv=32, dk=128, dv=128, dtype="bf16", m=32768, r=(5, 100)),
    "overlap": dict(desc="the group workload (r=0.05) replayed while the matched prefix's full-attention "
                         "KV is copied host to device on a second stream; KV widths are parameters",
                    G=12, L=3, d_model=2048, Hqk=16, Hv=32, dk=128, dv=128, m=32768, r=(5, 100),
                    kv_layers=12, kv_heads=2, kv_head_dim=256),
}
