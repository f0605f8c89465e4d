"""End-to-end parity at the full prefill sizes, in the launch configuration bench.py times (MoELayer
with automatic tile classes): 384 experts, hidden 7168, intermediate 2048, top-6, for T = 512 with
rows padded to 128, T = 8192 with Zipf routing, and T = 16384 with Zipf routing and +-8 outliers
(the padded shapes and zero-token experts of CURRENT_BUG.md@2e65594 "Test Plan" Phases 1-2; the
outliers are the "amax ~2-8" of CURRENT_BUG.md@2fc81cc "Key evidence").

Every output of every stage is compared, not a sample.  The oracle runs its whole chain over every
active expert, one expert at a time (its weights regenerated from the seeded generator, quantized
by the oracle's C quantizer and decoded exactly, the GEMMs as float64 matrix products):
  * routing tables, x codes / scales / gs and every active expert's weight codes / scales / gs:
    bit-exact;
  * L1: every valid row of h against the oracle's L1 on the same x codes and weights, relative
    Frobenius <= 1e-3;
  * requantization of h: the oracle's quantizer applied to the GPU's own h (valid rows) gives the
    GPU's h codes, scales and gs bit for bit;
  * L2: every valid row of y against the oracle's L2 on the GPU's h codes, <= 1e-3;
  * combine: every token of out against the oracle's combine of the GPU's y, within one bf16 step
    plus the fp32 accumulation error of k terms;
  * end to end: out against the oracle's own chain (its own h, requantization, y, combine),
    relative Frobenius <= 1e-2 and cosine >= 0.9999;
  * the same forward with the packed copy of the weight codes (how bench.py runs it) gives the same
    bits at every stage.
"""
import time

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_top_amd import layer, synth
from oracle import nvfp4_oracle as O
from oracle import nvfp4_ref as R

from gpu_util import DEV, bf16_bits_of, cosine, log, np_i32, rel_frob

pytestmark = pytest.mark.gpu
STAGE_TOL = 1e-3
E2E_TOL = 1e-2
E2E_COS = 0.9999


def _host_bf16(t: torch.Tensor) -> np.ndarray:
    """int16-viewed bf16 device tensor -> float32 host array (exact)."""
    return (bf16_bits_of(t).astype(np.uint32) << 16).view(np.float32)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [2, 3, 4], ids=["t512_pad128", "t8192_zipf", "t16384_zipf_outliers"])
def test_prefill_full_size_end_to_end(cfg):
    t_start = time.time()
    wl = synth.WORKLOADS[cfg]
    T = wl.tokens[0]
    E, H, I, k, P = wl.num_experts, wl.hidden, wl.intermediate, wl.top_k, wl.pad_multiple
    log(f"[fullsize] {wl.name} T={T}")
    ids, wts = O.router_topk(synth.router_logits(wl, T), k)
    x_bits = synth.activations(wl, T)
    counts, eoff, poff, row_token, token_rows = O.route(ids, wl.expert_begin, E, P)
    active = [int(e) for e in np.nonzero(counts)[0]]

    # ---- GPU: weights of the active experts, one forward --------------------------------------
    W = layer.MoEWeights.empty(E, H, I, device=DEV)
    for e in active:
        w13, w2 = synth.expert_weights(wl, wl.expert_begin + e, device=DEV)
        layer.quantize_expert_into(W, e, w13, w2)
        del w13, w2
    L = layer.MoELayer(T, k, E, H, I, P, expert_begin=wl.expert_begin, device=DEV)
    L.forward(torch.from_numpy(x_bits.view(np.int16)).to(DEV), torch.from_numpy(ids).to(DEV),
              torch.from_numpy(wts).to(DEV), W)
    torch.cuda.synchronize()
    M = L.M_cap
    log(f"[fullsize] GPU forward done ({len(active)} active experts, {M} rows), {time.time() - t_start:.0f} s")

    # routing tables
    assert np.array_equal(np_i32(L.counts), counts)
    assert np.array_equal(np_i32(L.expert_offsets), eoff)
    assert np.array_equal(np_i32(L.padded_offsets), poff)
    assert np.array_equal(np_i32(L.row_token)[:M], row_token)
    assert np.array_equal(np_i32(L.token_rows)[:T * k].reshape(T, k), token_rows)
    # x quantization
    xq, xs, gsx = R.quantize_bits(x_bits)
    assert np.array_equal(np_i32(L.x_codes)[:T], xq) and np.array_equal(np_i32(L.x_scales)[:T], xs)
    assert L.x_gs.item() == float(gsx)
    log(f"[fullsize] routing tables and x codes bit-exact, gs_x={float(gsx)}")

    h_gpu = _host_bf16(L.h[:M])
    hq_gpu, hs_gpu = np_i32(L.h_codes[:M]), np_i32(L.h_scales[:M])
    gsh_gpu = L.h_gs.item()
    y_gpu = _host_bf16(L.y[:M])
    out_gpu = _host_bf16(L.out[:T]).astype(np.float64)
    valid = row_token >= 0

    # the same forward on weights that carry the packed copy of their codes (the benchmark's
    # configuration: the 16-row kernels read it): the same bits at every stage
    W.pack()
    Lp = layer.MoELayer(T, k, E, H, I, P, expert_begin=wl.expert_begin, device=DEV)
    Lp.forward(torch.from_numpy(x_bits.view(np.int16)).to(DEV), torch.from_numpy(ids).to(DEV),
               torch.from_numpy(wts).to(DEV), W)
    torch.cuda.synchronize()
    for name, a, b in (("h", L.h, Lp.h), ("h_codes", L.h_codes, Lp.h_codes), ("h_scales", L.h_scales, Lp.h_scales),
                       ("y", L.y, Lp.y)):
        assert np.array_equal(np_i32(a[:M])[valid], np_i32(b[:M])[valid]), name
    assert Lp.h_gs.item() == gsh_gpu
    assert np.array_equal(bf16_bits_of(L.out[:T]), bf16_bits_of(Lp.out[:T]))
    W.w13_packed = W.w2_packed = None
    del Lp
    log("[fullsize] packed weight codes: h, h codes / scales / gs, y and out bit-identical")

    # ---- oracle L1 per expert (weights regenerated, quantized by the oracle, checked bit-exact) ----
    h_ref = np.zeros((M, I), np.float64)
    w2_q = {}
    for e in active:
        w13, w2 = synth.expert_weights(wl, wl.expert_begin + e, device=DEV)
        c13, s13, g13 = R.quantize_bits(bf16_bits_of(w13))
        c2, s2, g2 = R.quantize_bits(bf16_bits_of(w2))
        del w13, w2
        assert np.array_equal(np_i32(W.w13_codes[e]), c13) and np.array_equal(np_i32(W.w13_scales[e]), s13)
        assert np.array_equal(np_i32(W.w2_codes[e]), c2) and np.array_equal(np_i32(W.w2_scales[e]), s2)
        assert W.w13_gs[e].item() == float(g13) and W.w2_gs[e].item() == float(g2)
        w2_q[e] = (c2, s2, g2)
        rows = np.arange(poff[e], poff[e] + counts[e])
        toks = row_token[rows]
        a = R.dequantize(xq[toks], xs[toks])
        h_ref[rows] = O.l1_gate_up_silu(a, R.dequantize(c13, s13), gsx, g13)
    err_h = rel_frob(h_gpu[valid].astype(np.float64), h_ref[valid])
    log(f"[fullsize] weights of {len(active)} experts bit-exact; L1 all {valid.sum()} rows rel_frob={err_h:.2e}, "
        f"{time.time() - t_start:.0f} s")
    assert err_h <= STAGE_TOL

    # ---- requantization of h ----------------------------------------------------------------------
    h_bits_gpu = bf16_bits_of(L.h[:M])
    hq_o, hs_o, gsh_o = R.quantize_bits(h_bits_gpu, valid_rows=valid)
    assert gsh_gpu == float(gsh_o)
    assert np.array_equal(hq_gpu[valid], hq_o[valid]) and np.array_equal(hs_gpu[valid], hs_o[valid])
    log(f"[fullsize] h codes / scales / gs_h={gsh_gpu} bit-exact with the oracle's quantization of the GPU's h")
    hq_ref, hs_ref, gsh_ref = R.quantize_bits(O.bf16_bits(h_ref), valid_rows=valid)

    # ---- oracle L2 per expert: on the GPU's h codes (stage) and on its own chain (end to end) -----
    y_stage = np.zeros((M, H), np.float32)
    y_ref = np.zeros((M, H), np.float32)
    for e in active:
        c2, s2, g2 = w2_q.pop(e)
        w = R.dequantize(c2, s2)
        rows = np.arange(poff[e], poff[e] + counts[e])
        y_stage[rows] = O.l2_down(R.dequantize(hq_gpu[rows], hs_gpu[rows]), w, gsh_gpu, g2)
        y_ref[rows] = O.l2_down(R.dequantize(hq_ref[rows], hs_ref[rows]), w, gsh_ref, g2)
    err_y = rel_frob(y_gpu[valid].astype(np.float64), y_stage[valid].astype(np.float64))
    log(f"[fullsize] L2 all rows rel_frob={err_y:.2e}, {time.time() - t_start:.0f} s")
    assert err_y <= STAGE_TOL

    # ---- combine of the GPU's y, every token ------------------------------------------------------
    ref_c = O.combine(y_gpu, token_rows, wts)
    ulp = np.exp2(np.frexp(ref_c)[1] - 8.0)
    mag = O.combine(np.abs(y_gpu), token_rows, np.abs(wts))
    tol = ulp + (k + 2) * 2.0 ** -24 * mag * 1.01
    assert np.all(np.abs(out_gpu - ref_c) <= tol)
    log(f"[fullsize] combine: {np.mean(out_gpu == ref_c):.4%} of out bit-equal, all within one bf16 step")

    # ---- end to end against the oracle's own chain ------------------------------------------------
    out_ref = O.combine(y_ref, token_rows, wts)
    err, cos = rel_frob(out_gpu, out_ref), cosine(out_gpu, out_ref)
    log(f"[fullsize] end to end rel_frob={err:.2e} cosine={cos:.7f} ({time.time() - t_start:.0f} s)")
    assert np.isfinite(out_gpu).all()
    assert err <= E2E_TOL and cos >= E2E_COS
