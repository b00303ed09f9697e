"""Seeded synthetic inputs for the KDA chunked forward and decode.

This module only draws random numbers and arranges them into the argument
layouts; it holds none of the method's arithmetic, so both the HIP path and
the CPU oracle can be fed from it.  All draws go through one seeded
``torch.Generator`` on the requested device, in a fixed order:
q, k, v, g, beta, [sequence lengths], [initial state or cache],
[state indices].  Large tensors are drawn in token slices so host memory
stays bounded; a slice size never changes the stream.

Recipes (the five standard workloads; ``g_scale`` and the length recipe can
be overridden for stress cases):

* q, k, v ~ N(0, 1); g = -g_scale * sigmoid(N(0, 1)) per (token, head,
  channel); beta logits ~ N(0, 1); drawn in fp32 and rounded (RNE) to the
  input dtype.
* initial states ~ N(0, 0.02^2) fp32 (V-first [N, Hv, 128, 128]).
* varlen lengths: x_i = exp(U(ln lo, ln hi)), L_i = round(x_i * S / sum x),
  clamped to [lo, hi], residual spread +-1 round-robin from i = 0 over
  entries that stay inside the bounds.  Lengths come from their own CPU
  generator (seed + 1) so that shapes never depend on the device.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

D = 128

# name -> recipe.  "T" is per sequence for dense workloads.
WORKLOADS = {
    "tiny_fp32": dict(kind="chunk", B=1, T=256, hqk=1, hv=1, dtype=torch.float32,
                      g_scale=5.0, init=False, final=True),
    "dense_prefill": dict(kind="chunk", B=4, T=4096, hqk=16, hv=16, dtype=torch.bfloat16,
                          g_scale=5.0, init=True, final=True),
    "varlen_gva_paged": dict(kind="chunk_paged", S=32768, N=24, lo=64, hi=8192, hqk=8,
                             hv=32, slots=64, dtype=torch.bfloat16, g_scale=5.0),
    "long_single": dict(kind="chunk", B=1, T=131072, hqk=32, hv=32, dtype=torch.bfloat16,
                        g_scale=0.5, init=True, final=True),
    "decode_paged": dict(kind="decode", N=256, hqk=32, hv=32, slots=1024,
                         dtype=torch.bfloat16, g_scale=5.0),
}

_SLICE = 8192  # tokens per draw slice


@dataclass
class Batch:
    """Device tensors for one call, in the varlen layout [T_tot, H, 128]."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    cu_seqlens: torch.Tensor            # int32 [N+1]
    scale: float = D ** -0.5
    initial_state: torch.Tensor | None = None   # [N, Hv, 128, 128] fp32
    state_cache: torch.Tensor | None = None     # [slots, Hv, 128, 128] fp32
    state_indices: torch.Tensor | None = None   # int32 [N]
    has_initial_state: torch.Tensor | None = None  # uint8 [N]
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return self.cu_seqlens.numel() - 1

    @property
    def total_tokens(self) -> int:
        return self.q.shape[0]


def _normal(gen, shape, device, dtype, std=1.0):
    """N(0, std^2) in fp32 drawn slice by slice along dim 0, stored as dtype."""
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    for s in range(0, rows, _SLICE):
        e = min(rows, s + _SLICE)
        x = torch.randn((e - s,) + tuple(shape[1:]), generator=gen, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[s:e].copy_(x)
    return out


def _gate(gen, shape, device, dtype, g_scale):
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    for s in range(0, rows, _SLICE):
        e = min(rows, s + _SLICE)
        x = torch.randn((e - s,) + tuple(shape[1:]), generator=gen, device=device,
                        dtype=torch.float32)
        out[s:e].copy_(torch.sigmoid(x).mul_(-g_scale))
    return out


def varlen_lengths(gen, S, N, lo, hi, device="cpu"):
    """Log-uniform lengths in [lo, hi] summing exactly to S."""
    if not (N * lo <= S <= N * hi):
        raise ValueError("S out of reach for these bounds")
    u = torch.rand(N, generator=gen, device=device, dtype=torch.float64).cpu()
    x = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    L = [int(round(float(v))) for v in x * S / x.sum()]
    L = [min(hi, max(lo, v)) for v in L]
    i = 0
    guard = 0
    while sum(L) != S:
        step = 1 if sum(L) < S else -1
        if lo <= L[i] + step <= hi:
            L[i] += step
        i = (i + 1) % N
        guard += 1
        if guard > 100 * N * (hi - lo + 1):
            raise RuntimeError("length balancing did not converge")
    return L


def make_chunk(lengths, hqk, hv, dtype=torch.bfloat16, g_scale=5.0, seed=0,
               device="cpu", init=False, paged_slots=0, has_initial=True):
    """A chunk-forward batch with the given per-sequence lengths."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    T = int(sum(lengths))
    N = len(lengths)
    q = _normal(gen, (T, hqk, D), device, dtype)
    k = _normal(gen, (T, hqk, D), device, dtype)
    v = _normal(gen, (T, hv, D), device, dtype)
    g = _gate(gen, (T, hv, D), device, dtype, g_scale)
    beta = _normal(gen, (T, hv), device, dtype)
    cu = torch.zeros(N + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    b = Batch(q, k, v, g, beta, cu.to(device), meta=dict(lengths=list(lengths), hqk=hqk,
                                                         hv=hv, g_scale=g_scale))
    if paged_slots:
        b.state_cache = _normal(gen, (paged_slots, hv, D, D), device, torch.float32, 0.02)
        perm = torch.randperm(paged_slots, generator=gen, device=device)[:N]
        b.state_indices = perm.to(torch.int32)
        b.has_initial_state = torch.full((N,), 1 if has_initial else 0, dtype=torch.uint8,
                                         device=device)
    elif init:
        b.initial_state = _normal(gen, (N, hv, D, D), device, torch.float32, 0.02)
    return b


def make_decode(n, hqk, hv, slots, dtype=torch.bfloat16, g_scale=5.0, seed=0,
                device="cpu"):
    """A T=1 decode batch over a paged cache with distinct random slots."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = _normal(gen, (n, hqk, D), device, dtype)
    k = _normal(gen, (n, hqk, D), device, dtype)
    v = _normal(gen, (n, hv, D), device, dtype)
    g = _gate(gen, (n, hv, D), device, dtype, g_scale)
    beta = _normal(gen, (n, hv), device, dtype)
    cache = _normal(gen, (slots, hv, D, D), device, torch.float32, 0.02)
    idx = torch.randperm(slots, generator=gen, device=device)[:n].to(torch.int32)
    cu = torch.arange(n + 1, dtype=torch.int32, device=device)
    return Batch(q, k, v, g, beta, cu, state_cache=cache, state_indices=idx,
                 meta=dict(hqk=hqk, hv=hv, g_scale=g_scale, slots=slots))


def make_workload(name, device="cpu", seed=0):
    """One of the five standard workloads by name (see WORKLOADS)."""
    r = WORKLOADS[name]
    if r["kind"] == "decode":
        return make_decode(r["N"], r["hqk"], r["hv"], r["slots"], r["dtype"],
                           r["g_scale"], seed, device)
    if r["kind"] == "chunk_paged":
        gen = torch.Generator(device="cpu")
        gen.manual_seed(seed + 1)
        lengths = varlen_lengths(gen, r["S"], r["N"], r["lo"], r["hi"])
        b = make_chunk(lengths, r["hqk"], r["hv"], r["dtype"], r["g_scale"], seed,
                       device, paged_slots=r["slots"])
        b.meta["workload"] = name
        return b
    lengths = [r["T"]] * r["B"]
    b = make_chunk(lengths, r["hqk"], r["hv"], r["dtype"], r["g_scale"], seed, device,
                   init=r["init"])
    b.meta["workload"] = name
    return b


def make_verify(lengths, window, hqk, hv, slots, dtype=torch.bfloat16, g_scale=5.0, seed=0,
                null=(), device="cpu"):
    """A speculative verify batch: request b holds lengths[b] <= window draft
    tokens (rows query_start[b] .. query_start[b+1]) over a paged cache with
    distinct random slots; the requests listed in ``null`` get slot -1.  The
    accepted counts are uniform in [1, lengths[b]] (0 for an empty window).
    Draw order: q, k, v, g, beta, cache, slots, accepted counts."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, T = len(lengths), int(sum(lengths))
    q = _normal(gen, (T, hqk, D), device, dtype)
    k = _normal(gen, (T, hqk, D), device, dtype)
    v = _normal(gen, (T, hv, D), device, dtype)
    g = _gate(gen, (T, hv, D), device, dtype, g_scale)
    beta = _normal(gen, (T, hv), device, dtype)
    cache = _normal(gen, (slots, hv, D, D), device, torch.float32, 0.02)
    idx = torch.randperm(slots, generator=gen, device=device)[:B].to(torch.int32)
    for b in null:
        idx[b] = -1
    u = torch.rand(B, generator=gen, device=device, dtype=torch.float64).cpu()
    acc = torch.tensor([0 if n == 0 else 1 + min(n - 1, int(float(x) * n))
                        for n, x in zip(lengths, u)], dtype=torch.int32)
    qs = torch.tensor([0] + list(lengths), dtype=torch.int64).cumsum(0).to(torch.int32)
    return Batch(q, k, v, g, beta, qs.to(device), state_cache=cache, state_indices=idx,
                 meta=dict(hqk=hqk, hv=hv, g_scale=g_scale, slots=slots, window=window,
                           accepted=acc.to(device)))
