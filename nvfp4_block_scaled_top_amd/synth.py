"""Seeded synthetic inputs for the routed-expert layer.

This module draws the inputs only: router logits and the top-k routing that
the layer receives, activations, and raw bf16 expert weights.  It holds none
of the layer's arithmetic (no quantization, no GEMM, no combine), so both the
HIP path and the CPU oracle may be fed from it.

Shapes and distributions follow the workloads named for the layer: 384
experts with top-6 routing (CURRENT_BUG.md@2e65594, "Architecture: DeepSeek-V4
MegaMoE"), a 48-expert expert-parallel share at decode and padding to 128
rows ("Test Plan", Phase 2), and activations with std 0.09 and amax 1.27
(CURRENT_BUG.md@2fc81cc, "Key evidence"), plus a +-8 outlier workload ("amax
~2-8", same section).

Recipe (seed = 0 by default; every tensor has its own numpy PCG64 stream
``default_rng([seed, stream])``):

* stream 0: router logits, ``standard_normal((T, E_global), float32)``;
* stream 1: Zipf ranks: ``perm = permutation(E_global)``; expert ``perm[i]`` gets rank i+1 and
  bias ``-1.2 * ln(rank)`` is added to its logits (in float64, the sum rounded to float32);
* stream 2: x, ``standard_normal((T, H), float32) * 0.09``, clipped to +-1.27, rounded to bf16;
* stream 3: outliers, ``choice(T*H, T*H // 1000)`` positions and ``integers(0, 2)`` signs, set to +-8;
* routing itself (softmax and top-k) is a step of the layer, not part of this module: the
  logits go to the router (the GPU router, or the oracle's);
* weights: ``torch.randn`` (float32) * 0.02, rounded to bf16, drawn on the target
  device from a generator seeded per (seed, matrix, global expert).  Expert e's
  weights are the same in every workload that contains expert e.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_experts_global: int
    top_k: int
    hidden: int
    intermediate: int
    tokens: Sequence[int]
    expert_begin: int
    num_experts: int  # local experts held by this GPU
    pad_multiple: int
    zipf: bool = False
    outliers: bool = False
    block_m_hint: str = "auto"


WORKLOADS = {
    0: Workload("tiny", 8, 2, 256, 128, (16,), 0, 8, 1),
    1: Workload("decode_ep48of384", 384, 6, 7168, 2048, (1, 4, 8), 0, 48, 1, block_m_hint="16"),
    2: Workload("small_prefill_t512_pad128", 384, 6, 7168, 2048, (512,), 0, 384, 128),
    3: Workload("prefill_t8192_zipf", 384, 6, 7168, 2048, (8192,), 0, 384, 1, zipf=True),
    4: Workload("large_prefill_t16384_zipf_outliers", 384, 6, 7168, 2048, (16384,), 0, 384, 1,
                zipf=True, outliers=True),
}

X_STD = 0.09
X_CLIP = 1.27
OUTLIER_VALUE = 8.0
W_STD = 0.02
ZIPF_S = 1.2


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def router_logits(w: Workload, T: int, seed: int = 0) -> np.ndarray:
    """Router logits, float32 [T, E_global]."""
    logits = _rng(seed, 0).standard_normal((T, w.num_experts_global), dtype=np.float32)
    if w.zipf:
        perm = _rng(seed, 1).permutation(w.num_experts_global)
        rank = np.empty(w.num_experts_global, dtype=np.int64)
        rank[perm] = np.arange(1, w.num_experts_global + 1)
        bias = -ZIPF_S * np.log(rank.astype(np.float64))
        logits = (logits.astype(np.float64) + bias[None, :]).astype(np.float32)
    return logits


def activations(w: Workload, T: int, seed: int = 0) -> np.ndarray:
    """x as bf16 bit patterns, uint16 [T, H]."""
    x = _rng(seed, 2).standard_normal((T, w.hidden), dtype=np.float32) * np.float32(X_STD)
    np.clip(x, -X_CLIP, X_CLIP, out=x)
    bits = f32_to_bf16_bits(x)
    if w.outliers:
        n = T * w.hidden // 1000
        r = _rng(seed, 3)
        pos = r.choice(T * w.hidden, n, replace=False)
        sign = r.integers(0, 2, size=n)
        vals = np.where(sign == 1, OUTLIER_VALUE, -OUTLIER_VALUE).astype(np.float32)
        bits.reshape(-1)[pos] = f32_to_bf16_bits(vals)
    return bits


def _weight_seed(seed: int, matrix: int, expert: int) -> int:
    return (seed * 1_000_003 + matrix * 10_007 + expert) & 0x7FFF_FFFF_FFFF_FFFF


def expert_weights(w: Workload, global_expert: int, seed: int = 0, device: str = "cpu",
                   which: Optional[str] = None):
    """Raw bf16 weights of one expert as torch tensors: W13 [2I, H] (gate rows, then up) and W2 [H, I]."""
    import torch

    out = []
    for m, shape in ((4, (2 * w.intermediate, w.hidden)), (5, (w.hidden, w.intermediate))):
        if which is not None and which != ("w13" if m == 4 else "w2"):
            out.append(None)
            continue
        g = torch.Generator(device=device)
        g.manual_seed(_weight_seed(seed, m, global_expert))
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        out.append((t * W_STD).to(torch.bfloat16))
    return tuple(out)


def device_normal_bf16(shape, seed: int, stream: int, std: float, device: str = "cuda"):
    """A seeded N(0, std) bf16 tensor drawn on `device` (stand-in stage inputs of full size, e.g.
    h for the L2 stage and y for the combine).  Streams 6 and up; no method arithmetic."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(_weight_seed(seed, stream, 0))
    return (torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)
