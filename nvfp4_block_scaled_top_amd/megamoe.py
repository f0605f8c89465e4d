"""Thin ctypes binding of libmegamoe.so: the C entry points under the same names.

Argument marshalling only: each function takes torch tensors that already live on the GPU,
passes their device pointers, sizes and the current HIP stream to the C ABI, and raises
``MegaMoEError`` on a non-zero return code.  Every step of the layer runs in the library's HIP
kernels; there is no fallback.  If the library has not been built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmegamoe.so")
_lib = None

#: Slots of per-workgroup h amax written by moe_grouped_gemm_l1_silu (MEGAMOE_L1_AMAX_PARTS).
L1_AMAX_PARTS = 1280

#: Index of the error word in the sync buffer of moe_grouped_ffn_fused (MEGAMOE_FFN_SYNC_ERROR_WORD).
FFN_SYNC_ERROR_WORD = 352

#: Bytes of the static per-GPU scratch of moe_route_permute_noalloc (MEGAMOE_ROUTE_NOALLOC_SCRATCH_BYTES).
ROUTE_NOALLOC_SCRATCH_BYTES = 1 << 20

ERRORS = {
    -1: "MEGAMOE_ERR_NULL",
    -2: "MEGAMOE_ERR_SHAPE",
    -3: "MEGAMOE_ERR_WORKSPACE",
    -4: "MEGAMOE_ERR_LAUNCH",
    -5: "MEGAMOE_ERR_DEVICE",
}

#: Exported symbols and their C signatures (restype, argtypes), as declared in include/megamoe.h.
_P = ctypes.c_void_p
_I32, _I64, _SZ, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "megamoe_row_capacity": (_I64, [_I32, _I32, _I32, _I32]),
    "megamoe_sched_len": (_I64, [_I32]),
    "megamoe_route_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "megamoe_quant_workspace_bytes": (_SZ, [_I64, _I64]),
    "moe_router_topk": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P]),
    "moe_route_logits": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                _SZ, _P]),
    "moe_route_quantize": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _I64,
                                  _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_gemm_l1_silu_nvfp4": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32,
                                              _I32, _P, _P, _P, _P, _P]),
    "moe_route_permute": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_permute_noalloc": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P]),
    "nvfp4_quantize_act": (_I32, [_P, _I64, _I64, _P, _P, _I32, _P, _P, _P, _P, _SZ, _P]),
    "nvfp4_quantize_act_gs": (_I32, [_P, _I64, _I64, _P, _P, _P, _P, _P]),
    "moe_grouped_gemm_l1_silu": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32,
                                        _P, _P, _P]),
    "moe_grouped_gemm_l2": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _P, _P]),
    "nvfp4_pack_weight_codes": (_I32, [_P, _I64, _I64, _P, _P]),
    "moe_grouped_ffn_fused_packed": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32,
                                            _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_gemm_l1_silu_packed": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64,
                                               _I32, _I32, _P, _P, _P]),
    "moe_grouped_gemm_l1_silu_nvfp4_packed": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                                     _I64, _I32, _I32, _P, _P, _P, _P, _P]),
    "moe_grouped_gemm_l2_packed": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32,
                                          _P, _P]),
    "moe_combine": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P, _P]),
    "moe_combine_shared": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P, _P, _P]),
    "megamoe_dense_workspace_bytes": (_SZ, [_I64]),
    "megamoe_ffn_sync_bytes": (_SZ, [_I32]),
    "moe_grouped_ffn_fused": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _P,
                                     _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "nvfp4_linear": (_I32, [_P, _P, _P, _I64, _I32, _P, _P, _P, _I32, _P, _P, _SZ, _P]),
    "nvfp4_linear_gate_up_silu": (_I32, [_P, _P, _P, _I64, _I32, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "nvfp4_linear_gate_up_silu_nvfp4": (_I32, [_P, _P, _P, _I64, _I32, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _SZ,
                                               _P]),
}


class MegaMoEError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libmegamoe.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise MegaMoEError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python -m nvfp4_block_scaled_top_amd.build_lib")
        h = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def _check(name: str, rc: int) -> None:
    if rc != 0:
        raise MegaMoEError(f"{name} returned {rc} ({ERRORS.get(rc, 'unknown')})")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise MegaMoEError("tensors passed to libmegamoe must be on the GPU")
    if not t.is_contiguous():
        raise MegaMoEError("tensors passed to libmegamoe must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


# ---- size helpers ------------------------------------------------------------------------------

def megamoe_row_capacity(T: int, k: int, num_experts: int, pad_multiple: int) -> int:
    return int(lib().megamoe_row_capacity(T, k, num_experts, pad_multiple))


def megamoe_sched_len(num_experts: int) -> int:
    return int(lib().megamoe_sched_len(num_experts))


def megamoe_route_workspace_bytes(T: int, k: int, num_experts: int) -> int:
    return int(lib().megamoe_route_workspace_bytes(T, k, num_experts))


def megamoe_quant_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().megamoe_quant_workspace_bytes(rows, cols))


# ---- entry points --------------------------------------------------------------------------------

def moe_router_topk(logits, k, topk_ids, topk_weights, stream=None):
    T, Eg = logits.shape
    _check("moe_router_topk", lib().moe_router_topk(_ptr(logits), T, Eg, k, _ptr(topk_ids), _ptr(topk_weights),
                                                    _stream(stream)))


def moe_route_logits(logits, k, expert_begin, num_experts, pad_multiple, topk_ids, topk_weights, counts,
                     expert_offsets, padded_offsets, row_token, token_rows, sched, workspace, block_m_override=0,
                     stream=None):
    T, Eg = logits.shape
    _check("moe_route_logits", lib().moe_route_logits(
        _ptr(logits), T, Eg, k, expert_begin, num_experts, pad_multiple, block_m_override, _ptr(topk_ids),
        _ptr(topk_weights), _ptr(counts), _ptr(expert_offsets), _ptr(padded_offsets), _ptr(row_token),
        _ptr(token_rows), _ptr(sched), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def moe_route_permute(topk_ids, expert_begin, num_experts, pad_multiple, counts, expert_offsets, padded_offsets,
                      row_token, token_rows, sched, workspace, block_m_override=0, stream=None):
    T, k = topk_ids.shape
    _check("moe_route_permute", lib().moe_route_permute(
        _ptr(topk_ids), T, k, expert_begin, num_experts, pad_multiple, block_m_override, _ptr(counts),
        _ptr(expert_offsets), _ptr(padded_offsets), _ptr(row_token), _ptr(token_rows), _ptr(sched),
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def moe_route_permute_noalloc(topk_ids, expert_begin, num_experts, pad_multiple, counts, expert_offsets,
                              padded_offsets, row_token, token_rows, sched, block_m_override=0, stream=None):
    """moe_route_permute with the library's static per-GPU scratch instead of a workspace."""
    T, k = topk_ids.shape
    _check("moe_route_permute_noalloc", lib().moe_route_permute_noalloc(
        _ptr(topk_ids), T, k, expert_begin, num_experts, pad_multiple, block_m_override, _ptr(counts),
        _ptr(expert_offsets), _ptr(padded_offsets), _ptr(row_token), _ptr(token_rows), _ptr(sched),
        _stream(stream)))


def moe_route_quantize(topk_ids, expert_begin, num_experts, pad_multiple, counts, expert_offsets, padded_offsets,
                       row_token, token_rows, sched, route_workspace, x_bf16, x_codes, x_scales, x_global_scale,
                       quant_workspace, block_m_override=0, stream=None, x_gs_in=None):
    """x_gs_in (float32 [1] on the device): calibrated global scale; x_global_scale and
    quant_workspace are then not used (may be None)."""
    T, k = topk_ids.shape
    H = x_bf16.shape[1]
    _check("moe_route_quantize", lib().moe_route_quantize(
        _ptr(topk_ids), T, k, expert_begin, num_experts, pad_multiple, block_m_override, _ptr(counts),
        _ptr(expert_offsets), _ptr(padded_offsets), _ptr(row_token), _ptr(token_rows), _ptr(sched),
        _ptr(route_workspace), _nbytes(route_workspace), _ptr(x_bf16), H, _ptr(x_gs_in), _ptr(x_codes),
        _ptr(x_scales), _ptr(x_global_scale), _ptr(quant_workspace), _nbytes(quant_workspace), _stream(stream)))


def nvfp4_quantize_act(x_bf16, codes, scales, global_scale, workspace=None, row_valid=None, amax_in=None,
                       stream=None):
    rows, cols = x_bf16.shape
    n_amax = 0 if amax_in is None else amax_in.numel()
    _check("nvfp4_quantize_act", lib().nvfp4_quantize_act(
        _ptr(x_bf16), rows, cols, _ptr(row_valid), _ptr(amax_in), n_amax, _ptr(codes), _ptr(scales), _ptr(global_scale),
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def nvfp4_quantize_act_gs(x_bf16, global_scale_in, codes, scales, row_valid=None, stream=None):
    rows, cols = x_bf16.shape
    _check("nvfp4_quantize_act_gs", lib().nvfp4_quantize_act_gs(
        _ptr(x_bf16), rows, cols, _ptr(row_valid), _ptr(global_scale_in), _ptr(codes), _ptr(scales), _stream(stream)))


def nvfp4_pack_weight_codes(codes, packed, stream=None):
    """codes: uint8 [..., rows, K/2] (leading dimensions folded into rows); packed: as many bytes."""
    K = 2 * codes.shape[-1]
    rows = codes.numel() // codes.shape[-1]
    if packed.numel() != codes.numel():
        raise MegaMoEError("packed must hold as many bytes as codes")
    _check("nvfp4_pack_weight_codes", lib().nvfp4_pack_weight_codes(_ptr(codes), rows, K, _ptr(packed), _stream(stream)))


def moe_grouped_gemm_l1_silu(x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_codes,
                             w13_scales, w13_gs, h_bf16, h_amax_parts, block_m_override=0, max_rows_per_expert=0,
                             stream=None, w13_packed=None):
    """w13_packed: optional, the codes packed by nvfp4_pack_weight_codes (moe_grouped_gemm_l1_silu_packed)."""
    E, I2, Hh = w13_codes.shape
    M_cap = h_bf16.shape[0]
    if h_amax_parts.numel() < L1_AMAX_PARTS:
        raise MegaMoEError(f"h_amax_parts needs {L1_AMAX_PARTS} floats")
    head = (_ptr(x_codes), _ptr(x_scales), _ptr(x_gs), _ptr(row_token), _ptr(padded_offsets), _ptr(counts),
            _ptr(sched), _ptr(w13_codes), _ptr(w13_scales), _ptr(w13_gs))
    tail = (E, 2 * Hh, I2 // 2, M_cap, block_m_override, max_rows_per_expert, _ptr(h_bf16), _ptr(h_amax_parts),
            _stream(stream))
    if w13_packed is None:
        _check("moe_grouped_gemm_l1_silu", lib().moe_grouped_gemm_l1_silu(*head, *tail))
    else:
        _check("moe_grouped_gemm_l1_silu_packed", lib().moe_grouped_gemm_l1_silu_packed(*head, _ptr(w13_packed), *tail))


def moe_grouped_gemm_l1_silu_nvfp4(x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_codes,
                                   w13_scales, w13_gs, h_gs, h_codes, h_scales, h_amax_parts, block_m_override=0,
                                   max_rows_per_expert=0, stream=None, w13_packed=None):
    E, I2, Hh = w13_codes.shape
    M_cap = h_codes.shape[0]
    if h_amax_parts.numel() < L1_AMAX_PARTS:
        raise MegaMoEError(f"h_amax_parts needs {L1_AMAX_PARTS} floats")
    head = (_ptr(x_codes), _ptr(x_scales), _ptr(x_gs), _ptr(row_token), _ptr(padded_offsets), _ptr(counts),
            _ptr(sched), _ptr(w13_codes), _ptr(w13_scales), _ptr(w13_gs))
    tail = (E, 2 * Hh, I2 // 2, M_cap, block_m_override, max_rows_per_expert, _ptr(h_gs), _ptr(h_codes),
            _ptr(h_scales), _ptr(h_amax_parts), _stream(stream))
    if w13_packed is None:
        _check("moe_grouped_gemm_l1_silu_nvfp4", lib().moe_grouped_gemm_l1_silu_nvfp4(*head, *tail))
    else:
        _check("moe_grouped_gemm_l1_silu_nvfp4_packed",
               lib().moe_grouped_gemm_l1_silu_nvfp4_packed(*head, _ptr(w13_packed), *tail))


def moe_grouped_gemm_l2(h_codes, h_scales, h_gs, padded_offsets, counts, sched, w2_codes, w2_scales, w2_gs, y_bf16,
                        block_m_override=0, max_rows_per_expert=0, stream=None, w2_packed=None):
    E, H, Ih = w2_codes.shape
    M_cap = y_bf16.shape[0]
    head = (_ptr(h_codes), _ptr(h_scales), _ptr(h_gs), _ptr(padded_offsets), _ptr(counts), _ptr(sched),
            _ptr(w2_codes), _ptr(w2_scales), _ptr(w2_gs))
    tail = (E, H, 2 * Ih, M_cap, block_m_override, max_rows_per_expert, _ptr(y_bf16), _stream(stream))
    if w2_packed is None:
        _check("moe_grouped_gemm_l2", lib().moe_grouped_gemm_l2(*head, *tail))
    else:
        _check("moe_grouped_gemm_l2_packed", lib().moe_grouped_gemm_l2_packed(*head, _ptr(w2_packed), *tail))


def megamoe_ffn_sync_bytes(num_experts: int) -> int:
    return int(lib().megamoe_ffn_sync_bytes(num_experts))


def moe_grouped_ffn_fused(x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_codes, w13_scales,
                          w13_gs, w2_codes, w2_scales, w2_gs, h_amax_parts, h_codes, h_scales, y_bf16, sync,
                          h_gs_in=None, h_bf16=None, h_gs_out=None, stream=None, w13_packed=None, w2_packed=None):
    """w13_packed, w2_packed: optional, both weights' packed codes (moe_grouped_ffn_fused_packed)."""
    E, I2, Hh = w13_codes.shape
    M_cap = y_bf16.shape[0]
    if h_amax_parts.numel() < L1_AMAX_PARTS:
        raise MegaMoEError(f"h_amax_parts needs {L1_AMAX_PARTS} floats")
    head = (_ptr(x_codes), _ptr(x_scales), _ptr(x_gs), _ptr(row_token), _ptr(padded_offsets), _ptr(counts),
            _ptr(sched), _ptr(w13_codes), _ptr(w13_scales), _ptr(w13_gs), _ptr(w2_codes), _ptr(w2_scales),
            _ptr(w2_gs))
    tail = (E, 2 * Hh, I2 // 2, M_cap, _ptr(h_gs_in), _ptr(h_bf16), _ptr(h_amax_parts), _ptr(h_codes),
            _ptr(h_scales), _ptr(h_gs_out), _ptr(y_bf16), _ptr(sync), _nbytes(sync), _stream(stream))
    if w13_packed is None or w2_packed is None:
        _check("moe_grouped_ffn_fused", lib().moe_grouped_ffn_fused(*head, *tail))
    else:
        _check("moe_grouped_ffn_fused_packed",
               lib().moe_grouped_ffn_fused_packed(*head, _ptr(w13_packed), _ptr(w2_packed), *tail))


def moe_combine(y_bf16, token_rows, topk_weights, out_bf16, stream=None):
    T, k = topk_weights.shape
    H = out_bf16.shape[1]
    _check("moe_combine", lib().moe_combine(
        _ptr(y_bf16), _ptr(token_rows), _ptr(topk_weights), T, k, H, _ptr(out_bf16), _stream(stream)))


def moe_combine_shared(y_bf16, token_rows, topk_weights, y_shared_bf16, out_bf16, stream=None):
    T, k = topk_weights.shape
    H = out_bf16.shape[1]
    _check("moe_combine_shared", lib().moe_combine_shared(
        _ptr(y_bf16), _ptr(token_rows), _ptr(topk_weights), T, k, H, _ptr(y_shared_bf16), _ptr(out_bf16),
        _stream(stream)))


# ---- dense layers ------------------------------------------------------------------------------

def megamoe_dense_workspace_bytes(M: int) -> int:
    return int(lib().megamoe_dense_workspace_bytes(M))


def nvfp4_linear(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, out_bf16, workspace, stream=None):
    M, Kh = a_codes.shape
    N = w_codes.shape[0]
    _check("nvfp4_linear", lib().nvfp4_linear(
        _ptr(a_codes), _ptr(a_scales), _ptr(a_gs), M, 2 * Kh, _ptr(w_codes), _ptr(w_scales), _ptr(w_gs), N,
        _ptr(out_bf16), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def nvfp4_linear_gate_up_silu(a_codes, a_scales, a_gs, w13_codes, w13_scales, w13_gs, h_bf16, h_amax_parts,
                              workspace, stream=None):
    M, Kh = a_codes.shape
    I = w13_codes.shape[0] // 2
    if h_amax_parts.numel() < L1_AMAX_PARTS:
        raise MegaMoEError(f"h_amax_parts needs {L1_AMAX_PARTS} floats")
    _check("nvfp4_linear_gate_up_silu", lib().nvfp4_linear_gate_up_silu(
        _ptr(a_codes), _ptr(a_scales), _ptr(a_gs), M, 2 * Kh, _ptr(w13_codes), _ptr(w13_scales), _ptr(w13_gs), I,
        _ptr(h_bf16), _ptr(h_amax_parts), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def nvfp4_linear_gate_up_silu_nvfp4(a_codes, a_scales, a_gs, w13_codes, w13_scales, w13_gs, h_gs, h_codes, h_scales,
                                    h_amax_parts, workspace, stream=None):
    M, Kh = a_codes.shape
    I = w13_codes.shape[0] // 2
    if h_amax_parts.numel() < L1_AMAX_PARTS:
        raise MegaMoEError(f"h_amax_parts needs {L1_AMAX_PARTS} floats")
    _check("nvfp4_linear_gate_up_silu_nvfp4", lib().nvfp4_linear_gate_up_silu_nvfp4(
        _ptr(a_codes), _ptr(a_scales), _ptr(a_gs), M, 2 * Kh, _ptr(w13_codes), _ptr(w13_scales), _ptr(w13_gs), I,
        _ptr(h_gs), _ptr(h_codes), _ptr(h_scales), _ptr(h_amax_parts), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))
