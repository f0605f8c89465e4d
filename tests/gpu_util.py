"""Helpers shared by the GPU parity tests: workload setup on both sides and comparison metrics.

Every input comes from the seeded generator (nvfp4_block_scaled_top_amd.synth): the GPU side
quantizes raw bf16 weights with the library, the oracle side quantizes the same raw weights with
oracle.nvfp4_oracle.  Nothing the HIP path computes is fed to the oracle.
"""
from __future__ import annotations

import dataclasses
import sys
from typing import Dict, List, Optional

import numpy as np
import torch

from nvfp4_block_scaled_top_amd import layer, synth
from oracle import nvfp4_oracle as O
from oracle import nvfp4_ref as R

DEV = "cuda:0"


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_t2np(t: torch.Tensor) -> np.ndarray:
    """int16-viewed bf16 torch tensor -> float64 numpy."""
    return O.bf16_from_bits(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def bf16_bits_of(t: torch.Tensor) -> np.ndarray:
    """bf16 (or int16-viewed bf16) torch tensor -> uint16 bit patterns on the host."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def np2bf16_t(a: np.ndarray, device=DEV) -> torch.Tensor:
    """float64 numpy holding exact bf16 values -> int16-viewed bf16 torch tensor."""
    return torch.from_numpy(O.bf16_bits(a).view(np.int16)).to(device)


def rel_frob(got: np.ndarray, ref: np.ndarray) -> float:
    d = np.linalg.norm(got - ref)
    n = np.linalg.norm(ref)
    return float(d / n) if n > 0 else float(d)


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float((a * b).sum() / (na * nb))


@dataclasses.dataclass
class Setup:
    wl: synth.Workload
    T: int
    ids: np.ndarray          # int32 [T, k] global ids
    wts: np.ndarray          # float32 [T, k]
    x_bits: np.ndarray       # uint16 [T, H]
    gpu_w: layer.MoEWeights  # quantized on the GPU
    raw_dev: List            # per local expert (w13, w2) raw bf16 on the GPU (None if not drawn)
    oracle_w: Dict[int, tuple]  # local expert -> (w13 codes, scales, gs, w2 codes, scales, gs)

    @property
    def x(self) -> np.ndarray:
        return O.bf16_from_bits(self.x_bits)

    def dev_inputs(self):
        return (torch.from_numpy(self.x_bits.view(np.int16)).to(DEV), torch.from_numpy(self.ids).to(DEV),
                torch.from_numpy(self.wts).to(DEV))

    def oracle_quantize(self, e: int) -> tuple:
        """The oracle's NVFP4 quantization of expert e's raw weights (the C form of the oracle's
        quantizer, pinned against brute force and the NumPy form)."""
        if e not in self.oracle_w:
            w13, w2 = self.raw_dev[e]
            c13 = R.quantize_bits(bf16_bits_of(w13))
            c2 = R.quantize_bits(bf16_bits_of(w2))
            self.oracle_w[e] = c13 + c2
        return self.oracle_w[e]

    def oracle_weight_arrays(self, experts) -> dict:
        """Oracle weight arrays for all local experts; experts not listed get NaN scales (never read)."""
        E, H, I = self.wl.num_experts, self.wl.hidden, self.wl.intermediate
        w13c = np.zeros((E, 2 * I, H // 2), np.uint8)
        w13s = np.full((E, 2 * I, H // 16), 0x7F, np.uint8)
        w13g = np.full(E, np.nan, np.float32)
        w2c = np.zeros((E, H, I // 2), np.uint8)
        w2s = np.full((E, H, I // 16), 0x7F, np.uint8)
        w2g = np.full(E, np.nan, np.float32)
        for e in experts:
            q = self.oracle_quantize(e)
            w13c[e], w13s[e], w13g[e], w2c[e], w2s[e], w2g[e] = q
        return dict(w13_codes=w13c, w13_scales=w13s, w13_gs=w13g, w2_codes=w2c, w2_scales=w2s, w2_gs=w2g)


def make_setup(wl: synth.Workload, T: int, seed: int = 0, weight_seed: Optional[int] = None,
               weights_from: Optional[Setup] = None) -> Setup:
    ids, wts = O.router_topk(synth.router_logits(wl, T, seed), wl.top_k)
    x_bits = synth.activations(wl, T, seed)
    if weights_from is not None:
        return Setup(wl, T, ids, wts, x_bits, weights_from.gpu_w, weights_from.raw_dev, weights_from.oracle_w)
    E = wl.num_experts
    W = layer.MoEWeights.empty(E, wl.hidden, wl.intermediate, device=DEV)
    raw = []
    for e in range(E):
        w13, w2 = synth.expert_weights(wl, wl.expert_begin + e, seed if weight_seed is None else weight_seed,
                                       device=DEV)
        layer.quantize_expert_into(W, e, w13, w2)
        raw.append((w13, w2))
    torch.cuda.synchronize()
    return Setup(wl, T, ids, wts, x_bits, W, raw, {})


def oracle_chain(s: Setup) -> dict:
    counts, *_ = O.route(s.ids, s.wl.expert_begin, s.wl.num_experts, s.wl.pad_multiple)
    active = [e for e in range(s.wl.num_experts) if counts[e] > 0]
    wa = s.oracle_weight_arrays(active)
    return O.moe_layer(s.x, s.ids, s.wts, s.wl.expert_begin, s.wl.num_experts, s.wl.pad_multiple, **wa)


def run_gpu(s: Setup, block_m_override: int = 0) -> layer.MoELayer:
    wl = s.wl
    L = layer.MoELayer(s.T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, block_m_override=block_m_override, device=DEV)
    x, ids, wts = s.dev_inputs()
    L.forward(x, ids, wts, s.gpu_w)
    torch.cuda.synchronize()
    return L


def np_i32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()
