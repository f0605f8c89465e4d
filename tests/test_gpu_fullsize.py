"""Parity at the full prefill sizes, in the launch configuration bench.py times (MoELayer with
automatic tile classes): 384 experts, hidden 7168, intermediate 2048, top-6, for T = 512 padded to
128, T = 8192 with Zipf routing and T = 16384 with Zipf routing and +-8 outliers.

The whole-layer oracle is too slow at these sizes, so each stage is checked on outputs the oracle
computes one by one, with the oracle's own inputs for that stage:
  * routing tables and the quantization of x: every output, bit-exact;
  * L1 (the forward's own launch; its inputs are the x codes just shown equal to the oracle's and
    weights shown equal to the oracle's quantization): h rows of sampled experts -- the most loaded,
    a middle one of the large-tile class and the smallest and largest of the 16-row class -- first
    and last rows (ragged tail) plus random rows, relative Frobenius <= 1e-3;
  * L2 on oracle-quantized synthetic h of the full shape: sampled y rows, <= 1e-3;
  * combine on synthetic y of the full shape: sampled tokens, within one bf16 step plus the fp32
    accumulation error of k terms;
  * property of the forward: gs_h = fl32(2688 / max |h|) over the valid rows (the per-workgroup
    maxima of L1 and their reduction in the quantizer at full size).
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_top_amd import layer, megamoe as mm, synth
from oracle import nvfp4_oracle as O

from gpu_util import DEV, bf16_t2np, log, np_i32, rel_frob

pytestmark = pytest.mark.gpu
STAGE_TOL = 1e-3


def _rows_sample(first: int, n: int, rng, k: int = 24) -> np.ndarray:
    picks = {first, first + n - 1}
    if n > 2:
        picks.update((first + rng.choice(n, size=min(k, n), replace=False)).tolist())
    return np.array(sorted(picks), dtype=np.int64)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("cfg", [2, 3, 4], ids=["t512_pad128", "t8192_zipf", "t16384_zipf_outliers"])
def test_prefill_full_size_sampled(cfg):
    wl = synth.WORKLOADS[cfg]
    T = wl.tokens[0]
    E, H, I, k, P = wl.num_experts, wl.hidden, wl.intermediate, wl.top_k, wl.pad_multiple
    rng = np.random.default_rng(1234 + cfg)
    log(f"[fullsize] {wl.name} T={T}")
    ids, wts = O.router_topk(synth.router_logits(wl, T), wl.top_k)
    x_bits = synth.activations(wl, T)
    counts = O.route(ids, wl.expert_begin, E, P)[0]
    active = np.nonzero(counts)[0]
    order = active[np.argsort(counts[active], kind="stable")]
    small = [int(e) for e in order if counts[e] <= 16]
    large = [int(e) for e in order if counts[e] > 16]
    picks = {int(order[-1])}
    if large:
        picks.add(large[len(large) // 2])   # a middle large-tile expert
    if small:
        picks.update((small[0], small[-1]))  # the smallest and the largest 16-row-tile expert
    sampled = sorted(picks)
    log(f"[fullsize] sampled experts {sampled} with counts {[int(counts[e]) for e in sampled]}")

    # GPU weights for the active experts; raw bf16 of the sampled ones kept for the oracle
    W = layer.MoEWeights.empty(E, H, I, device=DEV)
    raw = {}
    for e in active:
        w13, w2 = synth.expert_weights(wl, wl.expert_begin + int(e), device=DEV)
        layer.quantize_expert_into(W, int(e), w13, w2)
        if int(e) in sampled:
            raw[int(e)] = (w13, w2)
    torch.cuda.synchronize()

    L = layer.MoELayer(T, k, E, H, I, P, expert_begin=wl.expert_begin, device=DEV)
    x_dev = torch.from_numpy(x_bits.view(np.int16)).to(DEV)
    ids_dev, wts_dev = torch.from_numpy(ids).to(DEV), torch.from_numpy(wts).to(DEV)
    L.forward(x_dev, ids_dev, wts_dev, W)
    torch.cuda.synchronize()
    M = L.M_cap

    # routing tables
    r_counts, r_eoff, r_poff, r_row_token, r_token_rows = O.route(ids, wl.expert_begin, E, P)
    assert np.array_equal(np_i32(L.counts), r_counts)
    assert np.array_equal(np_i32(L.expert_offsets), r_eoff)
    assert np.array_equal(np_i32(L.padded_offsets), r_poff)
    assert np.array_equal(np_i32(L.row_token)[:M], r_row_token)
    assert np.array_equal(np_i32(L.token_rows)[:T * k], r_token_rows.reshape(-1))
    log("[fullsize] routing tables bit-exact")

    # quantization of x
    xq, xs, gsx = O.quantize_nvfp4(O.bf16_from_bits(x_bits))
    assert np.array_equal(np_i32(L.x_codes)[:T], xq) and np.array_equal(np_i32(L.x_scales)[:T], xs)
    assert L.x_gs.item() == float(gsx)
    log(f"[fullsize] x codes/scales bit-exact, gs_x={float(gsx)}")

    # sampled experts: oracle weights equal the GPU's; L1 rows
    oq = {}
    for e in sampled:
        w13, w2 = raw[e]
        c13, s13, g13 = O.quantize_nvfp4(bf16_t2np(w13.view(torch.int16)))
        c2, s2, g2 = O.quantize_nvfp4(bf16_t2np(w2.view(torch.int16)))
        assert np.array_equal(np_i32(W.w13_codes[e]), c13) and np.array_equal(np_i32(W.w13_scales[e]), s13)
        assert np.array_equal(np_i32(W.w2_codes[e]), c2) and np.array_equal(np_i32(W.w2_scales[e]), s2)
        assert W.w13_gs[e].item() == float(g13) and W.w2_gs[e].item() == float(g2)
        oq[e] = (O.dequantize_blocks(c13, s13), g13, O.dequantize_blocks(c2, s2), g2)
    h_got, h_ref = [], []
    for e in sampled:
        rows = _rows_sample(int(r_poff[e]), int(r_counts[e]), rng)
        toks = r_row_token[rows]
        a = O.dequantize_blocks(xq[toks], xs[toks])
        h_ref.append(O.l1_gate_up_silu(a, oq[e][0], gsx, oq[e][1]))
        h_got.append(bf16_t2np(L.h[torch.from_numpy(rows).to(DEV)]))
    err_h = rel_frob(np.concatenate(h_got), np.concatenate(h_ref))
    log(f"[fullsize] L1 sampled rows rel_frob={err_h:.2e}")
    assert err_h <= STAGE_TOL

    # property: gs_h from the forward's own h (amax slots of L1 + the quantizer's reduction)
    valid_dev = L.row_token[:M] >= 0
    amax = L.h[:M][valid_dev].view(torch.bfloat16).float().abs().max().item()
    assert L.h_gs.item() == float(np.float32(2688.0) / np.float32(amax))

    # L2 on oracle-quantized synthetic h of the full shape
    h_syn = synth.device_normal_bf16((M, I), 0, 6, 0.05, device=DEV)
    valid = r_row_token >= 0
    hq, hs, gsh = O.quantize_nvfp4(bf16_t2np(h_syn.view(torch.int16)), valid_rows=valid)
    del h_syn
    hq_d, hs_d = torch.from_numpy(hq).to(DEV), torch.from_numpy(hs).to(DEV)
    gsh_d = torch.tensor([float(gsh)], dtype=torch.float32, device=DEV)
    y = torch.empty(M, H, dtype=torch.int16, device=DEV)
    mm.moe_grouped_gemm_l2(hq_d, hs_d, gsh_d, L.padded_offsets, L.counts, L.sched, W.w2_codes, W.w2_scales,
                           W.w2_gs, y, max_rows_per_expert=T)
    torch.cuda.synchronize()
    y_got, y_ref = [], []
    for e in sampled:
        rows = _rows_sample(int(r_poff[e]), int(r_counts[e]), rng)
        y_ref.append(O.l2_down(O.dequantize_blocks(hq[rows], hs[rows]), oq[e][2], gsh, oq[e][3]))
        y_got.append(bf16_t2np(y[torch.from_numpy(rows).to(DEV)]))
    err_y = rel_frob(np.concatenate(y_got), np.concatenate(y_ref))
    log(f"[fullsize] L2 sampled rows rel_frob={err_y:.2e}")
    assert err_y <= STAGE_TOL
    del y, hq_d, hs_d

    # combine on synthetic y of the full shape, sampled tokens
    y_syn = synth.device_normal_bf16((M, H), 0, 7, 0.05, device=DEV).view(torch.int16)
    out = torch.empty(T, H, dtype=torch.int16, device=DEV)
    mm.moe_combine(y_syn, L.token_rows[:T * k], wts_dev, out)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=min(256, T), replace=False)]))
    tr = r_token_rows.reshape(T, k)[toks]
    need = np.unique(tr[tr >= 0])
    y_rows = bf16_t2np(y_syn[torch.from_numpy(need).to(DEV)]) if len(need) else np.zeros((0, H))
    remap = np.full(M, -1, np.int64)
    remap[need] = np.arange(len(need))
    tr_sub = np.where(tr >= 0, remap[np.maximum(tr, 0)], -1).astype(np.int32)
    ref = O.combine(y_rows, tr_sub, wts[toks])
    got = bf16_t2np(out[torch.from_numpy(toks).to(DEV)])
    # one bf16 step of the result, plus the fp32 accumulation error of k fused multiply-adds
    # (at most (k + 2) * 2^-24 * sum |w * y|, which matters where the terms nearly cancel)
    ulp = np.exp2(np.frexp(ref)[1] - 8.0)
    mag = O.combine(np.abs(y_rows), tr_sub, np.abs(wts[toks]))
    tol = ulp + (k + 2) * 2.0 ** -24 * mag * 1.01
    assert np.all(np.abs(got - ref) <= tol)
    exact = np.mean(got == ref)
    log(f"[fullsize] combine on {len(toks)} sampled tokens: {exact:.4%} bit-equal, the rest within tolerance")
