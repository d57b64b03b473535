"""Seeded synthetic inputs for the IceCache decode hot path.

This module draws inputs only; it holds none of the method's arithmetic and
imports neither the HIP binding nor the oracle, so both sides can be fed the
same tensors.

Keys per stream (one stream = one KV head of one layer of one sequence) follow
a Gaussian mixture: C centres drawn from N(0, I_d); each token picks a centre
i.i.d. (uniformly, or with weights proportional to (c+1)^-alpha for a power-law
mix); key = centre + 0.3 * N(0, I_d); then 4 seeded channels of every key are
multiplied by 8 (outlier channels, as seen in real KV caches).  Values are
N(0, 1).  Each query head of a GQA group is a fresh draw from one randomly
chosen centre, made like a key (outlier channels included).  Keys, values and
queries are rounded to the cache dtype (bf16 round-to-nearest-even) or kept in
fp32.  The random DCI directions are Gaussian (d+1)-vectors normalised in fp64
and rounded to the key dtype.

The pages evaluate on LongBench, RULER, passkey retrieval and a 36k-token
latency sequence with real models; those datasets and weights are not used
here.  These synthetic caches stand in for them with the same shapes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    streams: int          # KV heads per layer x batch
    layers: int
    n: int                # context tokens per stream
    d: int
    dtype: str            # "f32" or "bf16"
    clusters: int
    p: int
    k: int
    m: int
    L: int
    g: int                # GQA group (query heads per KV head)
    powerlaw: float = 0.0  # 0: uniform cluster labels
    needle: int = 0        # tokens of a planted needle cluster
    steps: int = 0         # decode steps of the loop workload
    seed: int = 0

    @property
    def mL(self):
        return self.m * self.L


# The five workloads: one fp32 head checked against brute force; a
# Llama-3.1-8B-shaped layer at 36,864 tokens; the 32-layer, 128-step decode
# loop at 36,864; a 131,072-token batch-4 case with a planted needle; and a
# Qwen3-4B-shaped 262,144-token case with power-law cluster sizes.
WORKLOADS = {
    "single_head_4k_f32": Workload("single_head_4k_f32", 1, 1, 4096, 128, "f32", 64, 16, 256,
                                   4, 2, 1, seed=1000),
    "llama8b_layer_36k": Workload("llama8b_layer_36k", 8, 1, 36864, 128, "bf16", 256, 16, 256,
                                  8, 4, 4, seed=1001),
    "llama8b_decode_36k": Workload("llama8b_decode_36k", 8, 32, 36864, 128, "bf16", 256, 16,
                                   256, 8, 4, 4, steps=128, seed=1002),
    "llama8b_needle_131k_b4": Workload("llama8b_needle_131k_b4", 32, 32, 131072, 128, "bf16",
                                       1024, 16, 1024, 10, 4, 4, needle=16, seed=1003),
    "qwen3_4b_262k": Workload("qwen3_4b_262k", 8, 36, 262144, 128, "bf16", 2048, 32, 2048, 12,
                              6, 4, powerlaw=1.5, seed=1004),
}


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _mix(*xs: int) -> int:
    """Deterministic 63-bit seed from a tuple of small integers (SplitMix64 steps)."""
    h = 0x9E3779B97F4A7C15
    for x in xs:
        h = (h ^ (x & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        h = (h + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = h
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        h = z ^ (z >> 31)
    return h & 0x7FFFFFFFFFFFFFFF


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def directions(mL: int, d: int, seed: int, dtype: str = "bf16") -> torch.Tensor:
    """[mL][d+1] unit Gaussian directions, rounded to the key dtype (CPU tensor)."""
    g = _gen(_mix(seed, 7), "cpu")
    u = torch.randn(mL, d + 1, generator=g, dtype=torch.float64)
    u = u / u.norm(dim=1, keepdim=True)
    return u.to(torch_dtype(dtype))


def stream(n: int, d: int, clusters: int, g: int, seed: int, dtype: str = "bf16",
           powerlaw: float = 0.0, needle: int = 0, device="cpu"):
    """One stream's keys [n][d], values [n][d] and query heads [g][d] in `dtype`.

    With needle > 0, `needle` consecutive tokens at a random position get keys
    alpha * qhat + N(0, (0.01 alpha)^2 / d) per element, where qhat is the unit
    mean of the query heads and alpha the largest norm of the other keys: a
    passkey-style target that the search must return.  Also returns the needle's
    first position (-1 without a needle).
    """
    gen = _gen(seed, device)
    f32 = torch.float32
    mu = torch.randn(clusters, d, generator=gen, device=device, dtype=f32)
    if powerlaw > 0:
        w = (torch.arange(clusters, device=device, dtype=torch.float64) + 1.0) ** (-powerlaw)
        z = torch.multinomial(w / w.sum(), n, replacement=True, generator=gen)
    else:
        z = torch.randint(0, clusters, (n,), generator=gen, device=device)
    K = mu[z] + 0.3 * torch.randn(n, d, generator=gen, device=device, dtype=f32)
    ch = torch.randperm(d, generator=gen, device=device)[:4]
    K[:, ch] *= 8.0
    V = torch.randn(n, d, generator=gen, device=device, dtype=f32)
    cstar = int(torch.randint(0, clusters, (1,), generator=gen, device=device).item())
    q = mu[cstar].unsqueeze(0) + 0.3 * torch.randn(g, d, generator=gen, device=device, dtype=f32)
    q[:, ch] *= 8.0
    p0 = -1
    if needle > 0:
        p0 = int(torch.randint(0, n - needle + 1, (1,), generator=gen, device=device).item())
        qm = q.mean(0)
        qhat = qm / qm.norm()
        keep = torch.ones(n, dtype=torch.bool, device=device)
        keep[p0:p0 + needle] = False
        alpha = K[keep].norm(dim=1).max()
        noise = torch.randn(needle, d, generator=gen, device=device, dtype=f32)
        K[p0:p0 + needle] = alpha * qhat + (0.01 * alpha / d ** 0.5) * noise
    td = torch_dtype(dtype)
    return K.to(td), V.to(td), q.to(td), p0


def layer_inputs(w: Workload, layer: int = 0, streams: range | None = None, device="cpu"):
    """Stacked inputs of one layer: K, V [S][n][d]; q [S*g][d]; U [mL][d+1]; needle starts."""
    streams = range(w.streams) if streams is None else streams
    Ks, Vs, qs, p0s = [], [], [], []
    for s in streams:
        K, V, q, p0 = stream(w.n, w.d, w.clusters, w.g, _mix(w.seed, layer, s, 1), w.dtype,
                             w.powerlaw, w.needle, device)
        Ks.append(K)
        Vs.append(V)
        qs.append(q)
        p0s.append(p0)
    U = directions(w.mL, w.d, _mix(w.seed, layer, 2), w.dtype)
    return (torch.stack(Ks), torch.stack(Vs), torch.cat(qs), U.to(device), p0s)


def step_inputs(w: Workload, layer: int, step: int, device="cpu"):
    """Fresh (k, v) per stream for one decode step and a fresh query cluster draw.

    Returns k_new, v_new [S][d] and q [S*g][d].
    """
    gen = _gen(_mix(w.seed, layer, step, 3), device)
    f32 = torch.float32
    S, d, g = w.streams, w.d, w.g
    k_new = torch.randn(S, d, generator=gen, device=device, dtype=f32)
    v_new = torch.randn(S, d, generator=gen, device=device, dtype=f32)
    centre = torch.randn(S, 1, d, generator=gen, device=device, dtype=f32)
    q = (centre + 0.3 * torch.randn(S, g, d, generator=gen, device=device, dtype=f32))
    td = torch_dtype(w.dtype)
    return k_new.to(td), v_new.to(td), q.reshape(S * g, d).to(td)
