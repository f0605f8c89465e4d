"""Plain CPU oracle for the NVFP4 "MegaMoE" routed-expert layer.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library and its Python binding) never imports, calls or links it, and
this module imports nothing from the product package.

What it computes follows the pages of nvfp4-megamoe-kernel ``CURRENT_BUG.md``
(three revisions of the same file, cited here by their commit):

* @2e65594, "Architecture: DeepSeek-V4 MegaMoE": 384 experts, top-6 routing.
* @2e65594, "Test Plan", Phase 1: the runner takes hidden states, top-k ids and
  top-k weights; L1 gate+up GEMM, SiLU, L2 down GEMM; activations are quantized
  to NVFP4 before the grouped GEMMs.
* @2e65594, "Test Plan", Phase 2: expert-parallel share (48 of 384 experts),
  padding of each expert's rows to 128, zero-token experts, ``expert_offsets``
  and ``padded_expert_offsets``.
* @2fc81cc, "Root Cause" and "Key evidence": the FP4 quantizer multiplies the
  activation by a global scale before forming block scales; a global scale that
  ignores the activation's amax overflows the FP8 block scale.

NVFP4 itself (E2M1 codes, one E4M3 scale per 16 consecutive elements along the
reduction dimension, one FP32 global scale) is the format these pages name.
Where the pages leave a step open the plainest reading is taken; every such
reading is listed in the design notes (global scale 448*6/amax, exact
round-to-nearest-even everywhere, stable permutation, weights applied once in
the combine, rounding to bf16 where h, y and out are stored).

Arithmetic: all real-valued work is float64, and the two roundings that decide
integers (block scale, element code) are taken EXACTLY: every product that is
compared is exact in float64 (bf16 x fp32 needs 32 significant bits) and the
comparison is against exact grid midpoints.  The GEMMs use ``numpy.matmul`` on
exactly decoded float64 operands.  Values are rounded to bf16 only where the
method stores them: h after SiLU(gate)*up, y after L2, out after the combine.

Nothing here is blocked, fused or reordered beyond those definitions.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

#: E2M1 magnitudes, indexed by the 3 low bits of a code (bit 3 is the sign).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

#: Midpoints between consecutive E2M1 magnitudes.  A tie at MIDPOINTS[j] lies
#: between codes j and j+1 and goes to the even one, i.e. up when j is odd.
E2M1_MIDPOINTS = (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:]) / 2.0

E2M1_MAX = 6.0
E4M3_MAX = 448.0
#: Largest global scale for which no block scale can exceed E4M3's maximum.
GLOBAL_SCALE_NUMERATOR = E4M3_MAX * E2M1_MAX  # 2688


def e4m3fn_value(codes) -> np.ndarray:
    """Decode OCP E4M3FN bytes (bias 7, no infinities, 0x7F/0xFF = NaN) to float64."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


#: The 127 finite non-negative E4M3FN values, in code order (codes 0x00..0x7E),
#: which is also increasing order.
E4M3_GRID = e4m3fn_value(np.arange(0x7F))


def e2m1_value(codes) -> np.ndarray:
    """Decode 4-bit E2M1 codes (S.EE.M, bias 1) to float64."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c & 0x8, -1.0, 1.0) * E2M1_MAGNITUDES[c & 0x7]


def bf16_round(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16, ties to even (result in float64).

    bf16 keeps 8 significant bits and float32's exponent range; below 2**-126
    the grid is the subnormal one, spaced 2**-133.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)  # v = m * 2**e with 0.5 <= |m| < 1
    e = np.maximum(e, -125)  # subnormal range: fixed quantum 2**-133
    q = np.rint(np.ldexp(v, 8 - e))  # np.rint rounds half to even
    return np.ldexp(q, e - 8)


def bf16_bits(v) -> np.ndarray:
    """uint16 bit patterns of float64 values that are exactly bf16."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value is not exactly representable in bf16"
    return (b >> 16).astype(np.uint16)


def bf16_from_bits(bits) -> np.ndarray:
    """float64 values of uint16 bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# NVFP4 quantization
# ---------------------------------------------------------------------------

def global_scale(amax: float) -> np.float32:
    """FP32 global scale from a tensor's amax: fl32(448*6 / amax); 1.0 when amax == 0.

    The global scale multiplies the activation before block scales are formed
    (CURRENT_BUG.md@2fc81cc, "Root Cause"); deriving it from amax is what keeps
    every block scale within E4M3's range, unlike a fixed checkpoint scale
    ("Key evidence").  IEEE float32 division rounds the exact quotient once.
    """
    if amax == 0.0:
        return np.float32(1.0)
    return np.float32(GLOBAL_SCALE_NUMERATOR) / np.float32(amax)


def e4m3_round_sat(value) -> np.ndarray:
    """E4M3FN code nearest to each non-negative exact value, ties to even, saturating at 448.

    ``value`` must hold exact float64 numbers.  Nearest is decided against
    the exact midpoints of consecutive grid values.
    """
    v = np.asarray(value, dtype=np.float64)
    assert np.all(v >= 0.0)
    hi = np.searchsorted(E4M3_GRID, v, side="left")  # GRID[hi-1] < v <= GRID[hi]
    hi_c = np.minimum(hi, len(E4M3_GRID) - 1)
    lo_c = np.maximum(hi_c - 1, 0)
    mid = (E4M3_GRID[lo_c] + E4M3_GRID[hi_c]) / 2.0  # exact: <= 5 significant bits
    code = np.where(v < mid, lo_c, hi_c)
    code = np.where((v == mid) & (lo_c % 2 == 0), lo_c, code)  # tie -> even code
    code = np.where(v == E4M3_GRID[hi_c], hi_c, code)
    code = np.where(hi >= len(E4M3_GRID), len(E4M3_GRID) - 1, code)  # saturate at 448
    return code.astype(np.uint8)


def block_scale_codes(block_amax, gs) -> np.ndarray:
    """E4M3 block scale codes: RNE_sat(block_amax * gs / 6), from the exact real value.

    ``block_amax * gs`` is exact in float64 (bf16 times fp32).  Rounding p/6 to
    the grid is done by comparing p with 6 times each grid midpoint, which is
    also exact, so no division is rounded.
    """
    p = np.asarray(block_amax, dtype=np.float64) * np.float64(gs)
    six_grid = 6.0 * E4M3_GRID
    hi = np.searchsorted(six_grid, p, side="left")
    hi_c = np.minimum(hi, len(six_grid) - 1)
    lo_c = np.maximum(hi_c - 1, 0)
    six_mid = 3.0 * (E4M3_GRID[lo_c] + E4M3_GRID[hi_c])  # = 6 * midpoint, exact
    code = np.where(p < six_mid, lo_c, hi_c)
    code = np.where((p == six_mid) & (lo_c % 2 == 0), lo_c, code)
    code = np.where(p == six_grid[hi_c], hi_c, code)
    code = np.where(hi >= len(six_grid), len(six_grid) - 1, code)
    return code.astype(np.uint8)


def e2m1_codes(v, gs, block_scale_value) -> np.ndarray:
    """4-bit E2M1 codes of v*gs on the grid scaled by the element's block scale.

    Magnitude: the grid point m*s nearest to |v|*gs, ties to the even code
    index; values beyond 6*s take 6; a zero block scale gives magnitude 0.
    The sign bit is copied from v (so -0 and small negatives give 0x8).
    ``v`` and ``block_scale_value`` broadcast together; all products compared
    here are exact in float64.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v) * np.float64(gs)
    s = np.asarray(block_scale_value, dtype=np.float64)
    mag = np.zeros(np.broadcast(a, s).shape, dtype=np.int64)
    for j, mid in enumerate(E2M1_MIDPOINTS):
        t = mid * s  # exact: midpoint has <= 3 significant bits, s <= 4
        mag += (a > t) | ((a == t) & (j % 2 == 1))
    mag = np.where(s == 0.0, 0, mag)
    sign = np.signbit(v).astype(np.int64) << 3
    return (sign | mag).astype(np.uint8)


def pack_nibbles(codes) -> np.ndarray:
    """[rows, K] 4-bit codes -> [rows, K/2] bytes, the even element in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    """[rows, K/2] bytes -> [rows, K] 4-bit codes (inverse of pack_nibbles)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def quantize_with_global_scale(v, gs):
    """NVFP4-quantize rows of v (exact bf16 values) with a given global scale.

    Returns (packed codes [rows, K/2] uint8, block scale codes [rows, K/16] uint8).
    Blocks are 16 consecutive elements along the last (reduction) axis.
    """
    v = np.asarray(v, dtype=np.float64)
    rows, K = v.shape
    assert K % 16 == 0
    blocks = v.reshape(rows, K // 16, 16)
    block_amax = np.abs(blocks).max(axis=2)
    scodes = block_scale_codes(block_amax, gs)
    svalue = E4M3_GRID[scodes][:, :, None]
    codes = e2m1_codes(blocks, gs, svalue).reshape(rows, K)
    return pack_nibbles(codes), scodes


def quantize_nvfp4(v, valid_rows=None, chunk_rows: int = 4096):
    """NVFP4 quantization of a tensor with an amax-derived global scale.

    amax is taken over the valid rows only (all rows when ``valid_rows`` is
    None); invalid rows get zero codes and zero scales.  Returns (packed codes,
    scale codes, gs as np.float32).
    """
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.isfinite(v)), "non-finite input is outside the contract"
    rows, K = v.shape
    valid = np.ones(rows, dtype=bool) if valid_rows is None else np.asarray(valid_rows, dtype=bool)
    amax = float(np.abs(v[valid]).max()) if valid.any() and K > 0 else 0.0
    gs = global_scale(amax)
    codes = np.zeros((rows, K // 2), dtype=np.uint8)
    scales = np.zeros((rows, K // 16), dtype=np.uint8)
    idx = np.nonzero(valid)[0]
    for s in range(0, len(idx), chunk_rows):
        r = idx[s:s + chunk_rows]
        codes[r], scales[r] = quantize_with_global_scale(v[r], gs)
    return codes, scales, gs


def dequantize_blocks(packed, scale_codes) -> np.ndarray:
    """Exact float64 value of each element before the global scale: e2m1(code) * e4m3(scale)."""
    codes = unpack_nibbles(packed)
    rows, K = codes.shape
    sv = e4m3fn_value(scale_codes)
    return e2m1_value(codes) * np.repeat(sv, 16, axis=-1).reshape(rows, K)


# ---------------------------------------------------------------------------
# Routing: filter, count, offsets, stable permutation
# ---------------------------------------------------------------------------
# Router: logits -> top-k ids and weights
# ---------------------------------------------------------------------------

def router_topk(logits, k: int):
    """Top-k routing from router logits.

    The runner receives ``topk_ids`` and ``topk_weights`` from the router
    (CURRENT_BUG.md@2e65594, "Test Plan", Phase 1); the router is a softmax
    over all global experts followed by the k largest probabilities.  Readings
    (the pages give no formula): the softmax is taken in float64 over the
    float32 logits, max-subtracted; the k probabilities are NOT renormalised;
    weights are the float64 probabilities rounded to float32.  Order is
    descending probability with equal values going to the lower expert index,
    decided on the float32 logits: the exact softmax is strictly increasing in
    the logit, so this is the exact probabilities' order, and it does not
    depend on float64 rounding (far below the largest logit every probability
    underflows to the same 0).  Returns topk_ids int32 [T, k] and topk_weights
    float32 [T, k].
    """
    lg32 = np.asarray(logits, dtype=np.float32)
    lg = lg32.astype(np.float64)
    T, Eg = lg.shape
    if not 1 <= k <= Eg:
        raise ValueError("need 1 <= k <= number of experts")
    z = lg - lg.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    order = np.argsort(-lg32, axis=1, kind="stable")[:, :k]
    return order.astype(np.int32), np.take_along_axis(p, order, axis=1).astype(np.float32)


# ---------------------------------------------------------------------------
# Routing tables
# ---------------------------------------------------------------------------

def row_capacity(T: int, k: int, E: int, P: int) -> int:
    """Rows needed for every local assignment with each expert padded to a multiple of P."""
    return T * k + E * (P - 1)


def route(topk_ids, expert_begin: int, num_experts: int, pad_multiple: int):
    """Local filter, per-expert counts, offsets and the stable token permutation.

    An assignment (t, j) is local when expert_begin <= id < expert_begin + E
    (the expert-parallel share, CURRENT_BUG.md@2e65594, "Test Plan" Phase 2).
    ``expert_offsets`` is the exclusive prefix sum of counts and
    ``padded_offsets`` that of counts rounded up to ``pad_multiple`` (zero
    stays zero).  Within an expert, rows follow ascending token index (then j).
    Returns counts [E], expert_offsets [E+1], padded_offsets [E+1],
    row_token [M_cap] (-1 = padding), token_rows [T, k] (-1 = not local).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    E, P = num_experts, pad_multiple
    local = (ids >= expert_begin) & (ids < expert_begin + E)
    counts = np.bincount((ids - expert_begin)[local], minlength=E).astype(np.int32)
    expert_offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    padded = (counts + P - 1) // P * P
    padded_offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    row_token = np.full(row_capacity(T, k, E, P), -1, dtype=np.int32)
    token_rows = np.full((T, k), -1, dtype=np.int32)
    for e in range(E):
        ts, js = np.nonzero(ids == expert_begin + e)  # row-major: ascending t, then j
        rows = padded_offsets[e] + np.arange(len(ts))
        row_token[rows] = ts
        token_rows[ts, js] = rows
    return counts, expert_offsets, padded_offsets, row_token, token_rows


# ---------------------------------------------------------------------------
# Expert GEMMs and combine
# ---------------------------------------------------------------------------

def silu(z) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z)) in float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_matmul(a_deq, w_deq, gs_a, gs_w):
    """a @ w^T / (gs_a * gs_w) in float64 for block-dequantized operands.

    ``a_deq`` [n, K] and ``w_deq`` [N, K] hold e2m1*e4m3 values (global scales
    not applied); dividing by both global scales gives the real product.
    """
    return (a_deq @ w_deq.T) / (np.float64(gs_a) * np.float64(gs_w))


def silu_mul(acc):
    """SiLU(gate) * up, where the first half of the last axis is gate and the second up."""
    n = acc.shape[-1] // 2
    return silu(acc[..., :n]) * acc[..., n:]


def l1_gate_up_silu(a_deq, w13_deq, gs_a, gs_w):
    """h = bf16(SiLU(gate) * up) for one expert.

    W13 rows 0..I-1 are the gate projection and rows I..2I-1 the up projection
    (CURRENT_BUG.md@2e65594, "Test Plan" Phase 1: L1 gate+up, then SiLU).
    """
    return bf16_round(silu_mul(expert_matmul(a_deq, w13_deq, gs_a, gs_w)))


def l2_down(h_deq, w2_deq, gs_h, gs_w):
    """y = bf16(h @ W2^T / (gs_h * gs_w)) for one expert (the L2 down projection)."""
    return bf16_round(expert_matmul(h_deq, w2_deq, gs_h, gs_w))


def moe_l1(x_codes, x_scales, gs_x, row_token, padded_offsets, counts,
           w13_codes, w13_scales, w13_gs):
    """L1 gate+up + SiLU over every expert with at least one row.

    x is quantized once per token and gathered through ``row_token``.  Returns
    h [M_cap, I] (float64 holding bf16 values; rows that hold no assignment are
    0) and amax_h over the valid rows.
    """
    E = len(counts)
    I = w13_codes.shape[1] // 2
    h = np.zeros((len(row_token), I), dtype=np.float64)
    for e in range(E):
        c = int(counts[e])
        if c == 0:
            continue
        rows = np.arange(padded_offsets[e], padded_offsets[e] + c)
        toks = row_token[rows]
        a = dequantize_blocks(x_codes[toks], x_scales[toks])
        w = dequantize_blocks(w13_codes[e], w13_scales[e])
        h[rows] = l1_gate_up_silu(a, w, gs_x, w13_gs[e])
    valid = row_token >= 0
    amax_h = float(np.abs(h[valid]).max()) if valid.any() else 0.0
    return h, amax_h


def moe_l2(h_codes, h_scales, gs_h, padded_offsets, counts, w2_codes, w2_scales, w2_gs):
    """L2 down projection over every expert with at least one row: y [M_cap, H]."""
    E = len(counts)
    H = w2_codes.shape[1]
    y = np.zeros((h_codes.shape[0], H), dtype=np.float64)
    for e in range(E):
        c = int(counts[e])
        if c == 0:
            continue
        rows = np.arange(padded_offsets[e], padded_offsets[e] + c)
        a = dequantize_blocks(h_codes[rows], h_scales[rows])
        w = dequantize_blocks(w2_codes[e], w2_scales[e])
        y[rows] = l2_down(a, w, gs_h, w2_gs[e])
    return y


def combine(y, token_rows, topk_weights, y_shared=None):
    """out[t] = bf16( sum over j ascending of w[t,j] * y[token_rows[t,j]] ), +0 if none local.

    The routing weight is applied here and only here, once per (token, expert).
    ``y_shared`` [T, H] (the shared expert's output, weight 1) is added to the
    routed sum before the rounding.
    """
    token_rows = np.asarray(token_rows)
    w = np.asarray(topk_weights, dtype=np.float64)
    T, k = token_rows.shape
    acc = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        r = token_rows[:, j]
        m = r >= 0
        acc[m] += w[m, j, None] * y[r[m]]
    if y_shared is not None:
        acc = acc + np.asarray(y_shared, dtype=np.float64)
    return bf16_round(acc)


# ---------------------------------------------------------------------------
# Dense NVFP4 linear layers (one expert for every row) and the shared expert
# ---------------------------------------------------------------------------

def nvfp4_linear(a_codes, a_scales, gs_a, w_codes, w_scales, gs_w):
    """out = bf16(A @ W^T / (gs_a * gs_w)) for NVFP4 A [M, K] and W [N, K]: the down projection of
    one expert applied to every row (the expert GEMM with a single group)."""
    return l2_down(dequantize_blocks(a_codes, a_scales), dequantize_blocks(w_codes, w_scales), gs_a, gs_w)


def nvfp4_linear_gate_up_silu(a_codes, a_scales, gs_a, w13_codes, w13_scales, gs_w):
    """h = bf16(SiLU(gate) * up) for NVFP4 A [M, K] and W13 [2I, K] (gate rows, then up rows)."""
    return l1_gate_up_silu(dequantize_blocks(a_codes, a_scales), dequantize_blocks(w13_codes, w13_scales), gs_a, gs_w)


def shared_expert(x_codes, x_scales, gs_x, w13_codes, w13_scales, w13_gs, w2_codes, w2_scales, w2_gs):
    """A shared expert applied to every token (DeepSeek-style MoE adds one to the routed experts):
    the same x codes, gate+up with SiLU, h requantized with its own amax over all rows, down
    projection.  Weights are one expert's: w13 [2I, K], w2 [H, I] with scalar global scales.
    Returns (y_shared [T, H] bf16 values, h, gs_h)."""
    h = nvfp4_linear_gate_up_silu(x_codes, x_scales, gs_x, w13_codes, w13_scales, w13_gs)
    h_codes, h_scales, gs_h = quantize_nvfp4(h)
    return nvfp4_linear(h_codes, h_scales, gs_h, w2_codes, w2_scales, w2_gs), h, gs_h


def quantize_rows_with_global_scale(v, gs, valid_rows=None):
    """Calibrated quantization: a given global scale (no amax); invalid rows get zero codes and
    scales.  Blocks whose amax * gs / 6 exceeds 448 take the largest scale and their elements
    saturate at +-6 (CURRENT_BUG.md@2fc81cc, "Key evidence": the checkpoint's fixed scale on
    activations with amax 2-8)."""
    v = np.asarray(v, dtype=np.float64)
    rows, K = v.shape
    valid = np.ones(rows, dtype=bool) if valid_rows is None else np.asarray(valid_rows, dtype=bool)
    codes = np.zeros((rows, K // 2), dtype=np.uint8)
    scales = np.zeros((rows, K // 16), dtype=np.uint8)
    idx = np.nonzero(valid)[0]
    if len(idx):
        codes[idx], scales[idx] = quantize_with_global_scale(v[idx], np.float32(gs))
    return codes, scales


def moe_layer(x, topk_ids, topk_weights, expert_begin, num_experts, pad_multiple,
              w13_codes, w13_scales, w13_gs, w2_codes, w2_scales, w2_gs, gs_x=None, gs_h=None, shared=None):
    """The whole routed-expert layer; returns every intermediate in a dict.

    Order (CURRENT_BUG.md@2e65594, "Test Plan" Phase 1): route and permute,
    quantize x, L1 gate+up with SiLU(gate)*up, requantize h over valid rows,
    L2 down, routing-weighted combine.  ``gs_x`` / ``gs_h`` given: the
    calibrated variant, those global scales instead of the amax-derived ones.
    ``shared``: (w13_codes, w13_scales, w13_gs, w2_codes, w2_scales, w2_gs) of a
    shared expert whose output is added in the combine.
    """
    x = np.asarray(x, dtype=np.float64)
    counts, eoff, poff, row_token, token_rows = route(topk_ids, expert_begin, num_experts, pad_multiple)
    if gs_x is None:
        x_codes, x_scales, gs_x = quantize_nvfp4(x)
    else:
        gs_x = np.float32(gs_x)
        x_codes, x_scales = quantize_rows_with_global_scale(x, gs_x)
    h, amax_h = moe_l1(x_codes, x_scales, gs_x, row_token, poff, counts, w13_codes, w13_scales, w13_gs)
    if gs_h is None:
        h_codes, h_scales, gs_h = quantize_nvfp4(h, valid_rows=row_token >= 0)
    else:
        gs_h = np.float32(gs_h)
        h_codes, h_scales = quantize_rows_with_global_scale(h, gs_h, valid_rows=row_token >= 0)
    y = moe_l2(h_codes, h_scales, gs_h, poff, counts, w2_codes, w2_scales, w2_gs)
    y_shared = None
    if shared is not None:
        y_shared, _, _ = shared_expert(x_codes, x_scales, gs_x, *shared)
    out = combine(y, token_rows, topk_weights, y_shared)
    return dict(counts=counts, expert_offsets=eoff, padded_offsets=poff, row_token=row_token,
                token_rows=token_rows, x_codes=x_codes, x_scales=x_scales, gs_x=gs_x,
                h=h, amax_h=amax_h, h_codes=h_codes, h_scales=h_scales, gs_h=gs_h, y=y, y_shared=y_shared,
                out=out)
