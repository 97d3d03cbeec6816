"""Seeded synthetic inputs for LSH-sampled decode attention.

This module only draws random tensors; it holds none of the method's
arithmetic (no hashing, no probabilities, no attention).  Both the CPU
oracle and the GPU path take their inputs from here.

Geometry (MagicPIG, arXiv 2410.16179v2, Section 3.1 and Figure 2c / Figure 5):
keys sit in a narrow cone, queries point roughly the opposite way, and the
first token is an attention sink whose key points away from the key cone.
The recipe used here:

* a unit cone direction ``mu`` per stream (Gaussian draw, normalised);
* keys ``k = g + 3 mu`` with ``g ~ N(0, I_d)``; token 0 is exactly ``-20 mu``;
* values ``v ~ N(0, I_d)`` (the sink's value too);
* queries ``q = g - 3 mu`` of the KV head the query head reads;
* projections ``W ~ N(0, 1)`` with shape ``[d][K*L]``, fp32, one per layer
  (shared by every head and sequence of that layer, Section 4.4);
* everything drawn in fp32; bf16 workloads are rounded from those draws by
  torch's round-to-nearest-even cast.

Every tensor comes from its own torch generator whose seed is derived from
(config seed, kind, layer, batch, head) with numpy's SeedSequence, so a unit
can be regenerated on its own, on the host or on the device.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np
import torch

_KINDS = {"mu": 1, "k": 2, "v": 3, "q": 4, "w": 5, "step_k": 6, "step_v": 7, "step_q": 8, "codes": 9}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one synthetic workload (one row of the configuration list)."""

    name: str
    layers: int
    batch: int
    hq: int
    hkv: int
    d: int
    n: int
    K: int
    L: int
    dtype: str  # "f32" or "bf16"
    steps: int = 0  # decode steps that append one key each
    cap_extra: int = 64

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def cap(self) -> int:
        c = self.n + max(self.steps, 1) + self.cap_extra
        return (c + 63) // 64 * 64

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    # Tiny single-head decode, sized for the CPU oracle.
    "tiny": Workload("tiny", layers=1, batch=1, hq=1, hkv=1, d=128, n=4096, K=8, L=75, dtype="f32"),
    # Llama-3.1-8B-shaped single layer (32 q heads, 8 KV heads).
    "llama8b_layer": Workload("llama8b_layer", layers=1, batch=1, hq=32, hkv=8, d=128, n=16384, K=8, L=75,
                              dtype="bf16"),
    # Llama-3.1-8B-shaped full depth at 96K context, one decode step with append.
    "llama8b_96k": Workload("llama8b_96k", layers=32, batch=1, hq=32, hkv=8, d=128, n=98304, K=10, L=150,
                            dtype="bf16", steps=1),
    # CodeLlama-13B-shaped batched decode (MHA).
    "codellama13b_b16": Workload("codellama13b_b16", layers=40, batch=16, hq=40, hkv=40, d=128, n=16384, K=9,
                                 L=120, dtype="bf16", steps=1),
    # CodeLlama-34B-shaped code-store build followed by a 64-step decode.
    "codellama34b_b4": Workload("codellama34b_b4", layers=48, batch=4, hq=64, hkv=8, d=128, n=16384, K=10,
                                L=240, dtype="bf16", steps=64),
}


def stream_seed(seed: int, kind: str, layer: int = 0, b: int = 0, head: int = 0, step: int = 0) -> int:
    """64-bit seed for one random stream, derived from the config seed."""
    ss = np.random.SeedSequence([int(seed), _KINDS[kind], int(layer), int(b), int(head), int(step)])
    return int(ss.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn(shape, seed: int, device="cpu") -> torch.Tensor:
    """fp32 standard normal draws from the stream ``seed``."""
    return torch.randn(*shape, generator=_gen(device, seed), device=device, dtype=torch.float32)


def cone_dir(seed: int, layer: int, b: int, head: int, d: int, device="cpu") -> torch.Tensor:
    g = randn((d,), stream_seed(seed, "mu", layer, b, head), device)
    return g / torch.linalg.vector_norm(g)


def unit_kv(seed: int, layer: int, b: int, head: int, n: int, d: int, dtype: torch.dtype, device="cpu",
            out_k: Optional[torch.Tensor] = None, out_v: Optional[torch.Tensor] = None):
    """Keys and values of one (layer, batch, KV head) unit: ``[n][d]`` each.

    Keys follow the cone-plus-sink recipe; values are standard normal.  When
    ``out_k`` / ``out_v`` are given (views of a larger cache) the draws are
    written into them.
    """
    mu = cone_dir(seed, layer, b, head, d, device)
    k = randn((n, d), stream_seed(seed, "k", layer, b, head), device)
    k.add_(3.0 * mu)
    if n > 0:
        k[0] = -20.0 * mu
    v = randn((n, d), stream_seed(seed, "v", layer, b, head), device)
    if out_k is None:
        return k.to(dtype), v.to(dtype)
    out_k.copy_(k.to(dtype))
    out_v.copy_(v.to(dtype))
    return out_k, out_v


def unit_queries(seed: int, layer: int, b: int, kv_head: int, group: int, d: int, dtype: torch.dtype,
                 device="cpu", step: int = 0) -> torch.Tensor:
    """Queries of the ``group`` query heads that read KV head ``kv_head``: ``[group][d]``."""
    mu = cone_dir(seed, layer, b, kv_head, d, device)
    q = randn((group, d), stream_seed(seed, "step_q" if step else "q", layer, b, kv_head, step), device)
    q.sub_(3.0 * mu)
    return q.to(dtype)


def step_kv(seed: int, layer: int, b: int, head: int, d: int, dtype: torch.dtype, step: int, device="cpu"):
    """The key and value a decode step appends to one unit: two ``[d]`` tensors (cone key)."""
    mu = cone_dir(seed, layer, b, head, d, device)
    k = randn((d,), stream_seed(seed, "step_k", layer, b, head, step), device) + 3.0 * mu
    v = randn((d,), stream_seed(seed, "step_v", layer, b, head, step), device)
    return k.to(dtype), v.to(dtype)


def projections(seed: int, layer: int, d: int, K: int, L: int, device="cpu") -> torch.Tensor:
    """Gaussian projection matrix ``W[d][K*L]`` (fp32) of one layer."""
    return randn((d, K * L), stream_seed(seed, "w", layer), device)


def unit_codes(seed: int, layer: int, b: int, head: int, K: int, L: int, cap: int, device="cpu") -> torch.Tensor:
    """Uniform random table codes ``[L][cap]`` (int32 values in [0, 2^K)) for one unit.

    Tests inject them into a code store, on both sides, when the decode is
    checked independently of how codes were made."""
    g = _gen(device, stream_seed(seed, "codes", layer, b, head))
    return torch.randint(0, 1 << K, (L, cap), generator=g, device=device, dtype=torch.int32)


def layer_inputs(w: Workload, seed: int, layer: int, device="cpu", n: Optional[int] = None,
                 cap: Optional[int] = None):
    """All inputs of one layer in the cache layout the library uses.

    Returns a dict with ``K``/``V`` ``[B][Hkv][cap][d]`` (rows >= n zero),
    ``q`` ``[B][Hq][d]`` and ``W`` ``[d][K*L]`` fp32.
    """
    n = w.n if n is None else n
    cap = w.cap if cap is None else cap
    Kc = torch.zeros(w.batch, w.hkv, cap, w.d, dtype=w.torch_dtype, device=device)
    Vc = torch.zeros_like(Kc)
    q = torch.empty(w.batch, w.hq, w.d, dtype=w.torch_dtype, device=device)
    G = w.group
    for b in range(w.batch):
        for h in range(w.hkv):
            unit_kv(seed, layer, b, h, n, w.d, w.torch_dtype, device, Kc[b, h, :n], Vc[b, h, :n])
            q[b, h * G:(h + 1) * G] = unit_queries(seed, layer, b, h, G, w.d, w.torch_dtype, device)
    W = projections(seed, layer, w.d, w.K, w.L, device)
    return {"K": Kc, "V": Vc, "q": q, "W": W, "n": n, "cap": cap}


def digest(t: torch.Tensor) -> str:
    """Short content hash of a tensor (for logging which inputs a run used)."""
    a = t.detach().cpu().contiguous().view(torch.uint8).numpy()
    return hashlib.sha1(a.tobytes()).hexdigest()[:12]
