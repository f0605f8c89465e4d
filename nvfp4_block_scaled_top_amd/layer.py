"""Buffer ownership and call order for one routed-expert layer on the GPU.

PyTorch allocates device memory here; every computation is a call into libmegamoe through
``megamoe``.  ``MoEWeights`` holds NVFP4 expert weights quantized on the GPU by
``nvfp4_quantize_act`` (one global scale per expert and matrix), and ``MoELayer`` holds the
intermediate buffers for a fixed (T, k, E, H, I, P) and runs the six-call forward:
route/permute, quantize x, L1 gate+up + SiLU, quantize h (amax from L1), L2 down, combine.
``forward_logits`` starts one step earlier, from router logits (router + route/permute in one call).
A shared expert (one expert's weights applied to every token, ``MoEWeights`` with E = 1) can be
passed to ``forward``: its dense gate+up+SiLU and down projections run on the same x codes and its
output is added in the combine.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import megamoe as mm


@dataclasses.dataclass
class MoEWeights:
    w13_codes: torch.Tensor   # uint8 [E, 2I, H/2]
    w13_scales: torch.Tensor  # uint8 [E, 2I, H/16]
    w13_gs: torch.Tensor      # float32 [E]
    w2_codes: torch.Tensor    # uint8 [E, H, I/2]
    w2_scales: torch.Tensor   # uint8 [E, H, I/16]
    w2_gs: torch.Tensor       # float32 [E]
    # Optional second copies of the codes in the 16-row kernels' packed layout (pack()); when
    # present the layer's GEMMs read them in the 16-row kernels (same results, bit for bit).
    w13_packed: Optional[torch.Tensor] = None  # uint8 [E * 2I * H/2]
    w2_packed: Optional[torch.Tensor] = None   # uint8 [E * H * I/2]

    @property
    def num_experts(self) -> int:
        return self.w13_codes.shape[0]

    @property
    def hidden(self) -> int:
        return self.w13_codes.shape[2] * 2

    @property
    def intermediate(self) -> int:
        return self.w13_codes.shape[1] // 2

    def nbytes_expert(self) -> int:
        """NVFP4 bytes of one expert (codes + block scales + the two global scales)."""
        return sum(t[0].numel() * t.element_size() for t in
                   (self.w13_codes, self.w13_scales, self.w2_codes, self.w2_scales)) + 8

    @staticmethod
    def empty(E: int, H: int, I: int, device="cuda") -> "MoEWeights":
        u8 = dict(dtype=torch.uint8, device=device)
        return MoEWeights(torch.empty(E, 2 * I, H // 2, **u8), torch.empty(E, 2 * I, H // 16, **u8),
                          torch.empty(E, dtype=torch.float32, device=device),
                          torch.empty(E, H, I // 2, **u8), torch.empty(E, H, I // 16, **u8),
                          torch.empty(E, dtype=torch.float32, device=device))

    def clone(self) -> "MoEWeights":
        return MoEWeights(*(None if t is None else t.clone() for t in dataclasses.astuple(self)))

    def pack(self, stream=None) -> "MoEWeights":
        """(Re)build the packed copies of the codes (nvfp4_pack_weight_codes); call again after the
        codes change.  W2 is packed only when I is a multiple of 256 (the packed layout's chunk)."""
        self.w13_packed = torch.empty(self.w13_codes.numel(), dtype=torch.uint8, device=self.w13_codes.device)
        mm.nvfp4_pack_weight_codes(self.w13_codes, self.w13_packed, stream=stream)
        if self.intermediate % 256 == 0:
            self.w2_packed = torch.empty(self.w2_codes.numel(), dtype=torch.uint8, device=self.w2_codes.device)
            mm.nvfp4_pack_weight_codes(self.w2_codes, self.w2_packed, stream=stream)
        else:
            self.w2_packed = None
        return self


def quantize_matrix(w_bf16: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, gs: torch.Tensor,
                    stream=None) -> None:
    """NVFP4-quantize one bf16 matrix on the GPU (rows = output features, K contiguous)."""
    ws = torch.empty(mm.megamoe_quant_workspace_bytes(*w_bf16.shape), dtype=torch.uint8, device=w_bf16.device)
    mm.nvfp4_quantize_act(w_bf16.view(torch.int16), codes, scales, gs, workspace=ws, stream=stream)


def quantize_expert_into(weights: MoEWeights, e: int, w13_bf16: torch.Tensor, w2_bf16: torch.Tensor) -> None:
    quantize_matrix(w13_bf16, weights.w13_codes[e], weights.w13_scales[e], weights.w13_gs[e:e + 1])
    quantize_matrix(w2_bf16, weights.w2_codes[e], weights.w2_scales[e], weights.w2_gs[e:e + 1])


class MoELayer:
    """Intermediate buffers for T tokens, top-k, E local experts, hidden H, intermediate I, pad P."""

    def __init__(self, T: int, k: int, E: int, H: int, I: int, P: int = 1, expert_begin: int = 0,
                 block_m_override: int = 0, device="cuda"):
        self.T, self.k, self.E, self.H, self.I, self.P = T, k, E, H, I, P
        self.expert_begin, self.block_m_override = expert_begin, block_m_override
        self.M_cap = mm.megamoe_row_capacity(T, k, E, P)
        i32 = dict(dtype=torch.int32, device=device)
        u8 = dict(dtype=torch.uint8, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.counts = torch.empty(E, **i32)
        self.expert_offsets = torch.empty(E + 1, **i32)
        self.padded_offsets = torch.empty(E + 1, **i32)
        self.row_token = torch.empty(max(self.M_cap, 1), **i32)
        self.token_rows = torch.empty(max(T * k, 1), **i32)
        self.sched = torch.empty(mm.megamoe_sched_len(E), **i32)
        self.route_ws = torch.empty(max(mm.megamoe_route_workspace_bytes(T, k, E), 4), **u8)
        self.x_codes = torch.empty(max(T, 1), H // 2, **u8)
        self.x_scales = torch.empty(max(T, 1), H // 16, **u8)
        self.x_gs = torch.empty(1, **f32)
        self.x_ws = torch.empty(mm.megamoe_quant_workspace_bytes(T, H), **u8)
        self.h = torch.empty(max(self.M_cap, 1), I, dtype=torch.int16, device=device)
        self.h_amax = torch.empty(mm.L1_AMAX_PARTS, **f32)  # per-workgroup partial maxima from L1
        self.h_codes = torch.empty(max(self.M_cap, 1), I // 2, **u8)
        self.h_scales = torch.empty(max(self.M_cap, 1), I // 16, **u8)
        self.h_gs = torch.empty(1, **f32)
        self.y = torch.empty(max(self.M_cap, 1), H, dtype=torch.int16, device=device)
        self.out = torch.empty(max(T, 1), H, dtype=torch.int16, device=device)
        self._gs_x, self._gs_h = self.x_gs, self.h_gs            # global scales the GEMMs read
        self.topk_ids = torch.empty(max(T, 1), k, **i32)          # written by route_logits
        self.topk_weights = torch.empty(max(T, 1), k, **f32)

    def _shared_buffers(self, shared: MoEWeights) -> None:
        Is, dev = shared.intermediate, self.out.device
        if getattr(self, "_sh_I", None) == Is:
            return
        T, H = max(self.T, 1), self.H
        self._sh_I = Is
        self.sh_h = torch.empty(T, Is, dtype=torch.int16, device=dev)
        self.sh_h_amax = torch.empty(mm.L1_AMAX_PARTS, dtype=torch.float32, device=dev)
        self.sh_h_codes = torch.empty(T, Is // 2, dtype=torch.uint8, device=dev)
        self.sh_h_scales = torch.empty(T, Is // 16, dtype=torch.uint8, device=dev)
        self.sh_h_gs = torch.empty(1, dtype=torch.float32, device=dev)
        self.sh_y = torch.empty(T, H, dtype=torch.int16, device=dev)
        self.sh_ws = torch.empty(mm.megamoe_dense_workspace_bytes(self.T), dtype=torch.uint8, device=dev)

    def shared_expert(self, shared: MoEWeights, stream=None, h_gs: Optional[torch.Tensor] = None) -> None:
        """Dense gate+up+SiLU on the x codes, requantize its h (own amax), dense down: sh_y [T, H].
        h_gs given: a calibrated global scale for its h, written as NVFP4 by the gate+up GEMM."""
        self._shared_buffers(shared)
        T = self.T
        if h_gs is None:
            mm.nvfp4_linear_gate_up_silu(self._rows(self.x_codes, T), self._rows(self.x_scales, T), self._gs_x,
                                         shared.w13_codes[0], shared.w13_scales[0], shared.w13_gs[0:1],
                                         self._rows(self.sh_h, T), self.sh_h_amax, self.sh_ws, stream=stream)
            mm.nvfp4_quantize_act(self._rows(self.sh_h, T), self._rows(self.sh_h_codes, T),
                                  self._rows(self.sh_h_scales, T), self.sh_h_gs, amax_in=self.sh_h_amax,
                                  stream=stream)
            gs = self.sh_h_gs
        else:
            mm.nvfp4_linear_gate_up_silu_nvfp4(self._rows(self.x_codes, T), self._rows(self.x_scales, T),
                                               self._gs_x, shared.w13_codes[0], shared.w13_scales[0],
                                               shared.w13_gs[0:1], h_gs, self._rows(self.sh_h_codes, T),
                                               self._rows(self.sh_h_scales, T), self.sh_h_amax, self.sh_ws,
                                               stream=stream)
            gs = h_gs
        mm.nvfp4_linear(self._rows(self.sh_h_codes, T), self._rows(self.sh_h_scales, T), gs,
                        shared.w2_codes[0], shared.w2_scales[0], shared.w2_gs[0:1], self._rows(self.sh_y, T),
                        self.sh_ws, stream=stream)

    def _rows(self, t: torch.Tensor, n: int) -> torch.Tensor:
        return t[:n] if n > 0 else t[:0]

    def route(self, topk_ids: torch.Tensor, stream=None) -> None:
        mm.moe_route_permute(topk_ids, self.expert_begin, self.E, self.P, self.counts, self.expert_offsets,
                             self.padded_offsets, self.row_token, self.token_rows, self.sched, self.route_ws,
                             block_m_override=self.block_m_override, stream=stream)

    def route_logits(self, logits: torch.Tensor, stream=None) -> None:
        """Router (softmax top-k over the float32 logits [T, E_global]) and route/permute."""
        mm.moe_route_logits(logits, self.k, self.expert_begin, self.E, self.P, self._rows(self.topk_ids, self.T),
                            self._rows(self.topk_weights, self.T), self.counts, self.expert_offsets,
                            self.padded_offsets, self.row_token, self.token_rows, self.sched, self.route_ws,
                            block_m_override=self.block_m_override, stream=stream)

    def route_quantize(self, topk_ids: torch.Tensor, x_bf16: torch.Tensor, stream=None,
                       gs: Optional[torch.Tensor] = None) -> None:
        """Route/permute and quantize x in one call (one launch at decode sizes); gs given: the
        calibrated quantizer with that global scale."""
        self._gs_x = self.x_gs if gs is None else gs
        mm.moe_route_quantize(topk_ids, self.expert_begin, self.E, self.P, self.counts, self.expert_offsets,
                              self.padded_offsets, self.row_token, self.token_rows, self.sched, self.route_ws,
                              x_bf16, self._rows(self.x_codes, self.T), self._rows(self.x_scales, self.T), self.x_gs,
                              self.x_ws, block_m_override=self.block_m_override, stream=stream, x_gs_in=gs)

    def quantize_x(self, x_bf16: torch.Tensor, stream=None, gs: Optional[torch.Tensor] = None) -> None:
        """gs given (float32 [1] on the device): the calibrated quantizer with that global scale."""
        self._gs_x = self.x_gs if gs is None else gs
        if gs is None:
            mm.nvfp4_quantize_act(x_bf16, self._rows(self.x_codes, self.T), self._rows(self.x_scales, self.T),
                                  self.x_gs, workspace=self.x_ws, stream=stream)
        else:
            mm.nvfp4_quantize_act_gs(x_bf16, gs, self._rows(self.x_codes, self.T), self._rows(self.x_scales, self.T),
                                     stream=stream)

    def l1(self, w: MoEWeights, stream=None) -> None:
        mm.moe_grouped_gemm_l1_silu(self.x_codes, self.x_scales, self._gs_x, self.row_token, self.padded_offsets,
                                    self.counts, self.sched, w.w13_codes, w.w13_scales, w.w13_gs,
                                    self._rows(self.h, self.M_cap), self.h_amax, self.block_m_override,
                                    self.T, stream=stream, w13_packed=w.w13_packed)

    def l1_nvfp4(self, w: MoEWeights, gs: torch.Tensor, stream=None) -> None:
        """L1 writing h as NVFP4 with the calibrated global scale gs (no bf16 h, no quantize_h)."""
        self._gs_h = gs
        mm.moe_grouped_gemm_l1_silu_nvfp4(self.x_codes, self.x_scales, self._gs_x, self.row_token,
                                          self.padded_offsets, self.counts, self.sched, w.w13_codes, w.w13_scales,
                                          w.w13_gs, gs, self._rows(self.h_codes, self.M_cap),
                                          self._rows(self.h_scales, self.M_cap), self.h_amax, self.block_m_override,
                                          self.T, stream=stream, w13_packed=w.w13_packed)

    def quantize_h(self, stream=None, gs: Optional[torch.Tensor] = None) -> None:
        """gs given (float32 [1] on the device): the calibrated quantizer with that global scale."""
        self._gs_h = self.h_gs if gs is None else gs
        if gs is None:
            mm.nvfp4_quantize_act(self._rows(self.h, self.M_cap), self._rows(self.h_codes, self.M_cap),
                                  self._rows(self.h_scales, self.M_cap), self.h_gs,
                                  row_valid=self._rows(self.row_token, self.M_cap), amax_in=self.h_amax, stream=stream)
        else:
            mm.nvfp4_quantize_act_gs(self._rows(self.h, self.M_cap), gs, self._rows(self.h_codes, self.M_cap),
                                     self._rows(self.h_scales, self.M_cap),
                                     row_valid=self._rows(self.row_token, self.M_cap), stream=stream)

    def l2(self, w: MoEWeights, stream=None) -> None:
        mm.moe_grouped_gemm_l2(self.h_codes, self.h_scales, self._gs_h, self.padded_offsets, self.counts, self.sched,
                               w.w2_codes, w.w2_scales, w.w2_gs, self._rows(self.y, self.M_cap),
                               self.block_m_override, self.T, stream=stream, w2_packed=w.w2_packed)

    def ffn_fused(self, w: MoEWeights, stream=None, h_gs: Optional[torch.Tensor] = None) -> None:
        """L1, the requantization of h and L2 in one launch (every expert in 16-row m-tiles: for
        decode).  h_gs given: a calibrated global scale for h; else h_gs is derived from the amax of
        h inside the launch and written to self.h_gs.  Same bits as l1 / quantize_h / l2 with
        16-row tiles."""
        if getattr(self, "ffn_sync", None) is None:  # zero once; every call leaves it zero
            self.ffn_sync = torch.zeros(mm.megamoe_ffn_sync_bytes(self.E) // 4, dtype=torch.int32,
                                        device=self.out.device)
        self._gs_h = self.h_gs if h_gs is None else h_gs
        M = self.M_cap
        mm.moe_grouped_ffn_fused(self.x_codes, self.x_scales, self._gs_x, self.row_token, self.padded_offsets,
                                 self.counts, self.sched, w.w13_codes, w.w13_scales, w.w13_gs, w.w2_codes,
                                 w.w2_scales, w.w2_gs, self.h_amax, self._rows(self.h_codes, M),
                                 self._rows(self.h_scales, M), self._rows(self.y, M), self.ffn_sync,
                                 h_gs_in=h_gs, h_bf16=None if h_gs is not None else self._rows(self.h, M),
                                 h_gs_out=None if h_gs is not None else self.h_gs, stream=stream,
                                 w13_packed=w.w13_packed, w2_packed=w.w2_packed)

    def ffn_sync_error(self) -> int:
        """The fused launch's error word (non-zero once a wait inside it ever expired)."""
        if getattr(self, "ffn_sync", None) is None:
            return 0
        return int(self.ffn_sync[mm.FFN_SYNC_ERROR_WORD].item())

    def combine(self, topk_weights: torch.Tensor, stream=None, shared: bool = False) -> None:
        if shared:
            mm.moe_combine_shared(self._rows(self.y, self.M_cap), self._rows(self.token_rows, self.T * self.k),
                                  topk_weights, self._rows(self.sh_y, self.T), self._rows(self.out, self.T),
                                  stream=stream)
        else:
            mm.moe_combine(self._rows(self.y, self.M_cap), self._rows(self.token_rows, self.T * self.k),
                           topk_weights, self._rows(self.out, self.T), stream=stream)

    def forward(self, x_bf16: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor, w: MoEWeights,
                stream=None, x_gs: Optional[torch.Tensor] = None, h_gs: Optional[torch.Tensor] = None,
                shared: Optional[MoEWeights] = None, shared_h_gs: Optional[torch.Tensor] = None,
                fused: bool = False) -> torch.Tensor:
        """x_bf16 int16-viewed bf16 [T, H], topk_ids int32 [T, k], topk_weights float32 [T, k].
        x_gs / h_gs (float32 [1] on the device): calibrated global scales for x and h (e.g. the
        x_gs / h_gs buffers of a warm-up forward) instead of ones derived from this call's amax.
        shared: a shared expert (E = 1) whose output is added in the combine; shared_h_gs: a
        calibrated global scale for the shared expert's h.
        With h_gs, L1 writes h as NVFP4 itself (no bf16 h and no separate quantization of h).
        fused: L1, the quantization of h and L2 as one launch (ffn_fused; for decode sizes)."""
        self.route_quantize(topk_ids, x_bf16, stream, gs=x_gs)
        if fused:
            self.ffn_fused(w, stream, h_gs=h_gs)
        else:
            if h_gs is None:
                self.l1(w, stream)
                self.quantize_h(stream)
            else:
                self.l1_nvfp4(w, h_gs, stream)
            self.l2(w, stream)
        if shared is not None:
            self.shared_expert(shared, stream, h_gs=shared_h_gs)
        self.combine(topk_weights, stream, shared=shared is not None)
        return self._rows(self.out, self.T)

    def forward_logits(self, x_bf16: torch.Tensor, logits: torch.Tensor, w: MoEWeights, stream=None) -> torch.Tensor:
        """x_bf16 int16-viewed bf16 [T, H], logits float32 [T, E_global]; the chosen ids and weights
        are left in topk_ids / topk_weights."""
        self.route_logits(logits, stream)
        self.quantize_x(x_bf16, stream)
        self.l1(w, stream)
        self.quantize_h(stream)
        self.l2(w, stream)
        self.combine(self._rows(self.topk_weights, self.T), stream)
        return self._rows(self.out, self.T)
