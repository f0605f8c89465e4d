"""Calibrated global scales (nvfp4_quantize_act_gs and the layer's x_gs / h_gs): the quantizer
with a caller-given global scale is bit-exact with the oracle's, including blocks that saturate
(scale 448, elements +-6) when the scale is too large for the data; the layer with calibrated
scales matches the oracle's calibrated layer, and with the amax-derived scales passed in gives
the same bits as the uncalibrated forward."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_top_amd import layer, megamoe as mm, synth
from oracle import nvfp4_oracle as O

from gpu_util import DEV, bf16_t2np, log, make_setup, np2bf16_t, np_i32, rel_frob

pytestmark = pytest.mark.gpu


def gpu_quant_gs(x64, gs, row_valid=None):
    rows, cols = x64.shape
    codes = torch.full((rows, cols // 2), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((rows, cols // 16), 0xCD, dtype=torch.uint8, device=DEV)
    g = torch.tensor([gs], dtype=torch.float32, device=DEV)
    rv = None if row_valid is None else torch.from_numpy(np.where(row_valid, 0, -1).astype(np.int32)).to(DEV)
    mm.nvfp4_quantize_act_gs(np2bf16_t(x64), g, codes, scales, row_valid=rv)
    torch.cuda.synchronize()
    return np_i32(codes), np_i32(scales)


@pytest.mark.parametrize("factor", [1.0, 0.31, 3.0, 64.0])
@pytest.mark.parametrize("shape", [(5, 64), (37, 7168), (300, 2048)])
def test_quantizer_given_scale(factor, shape):
    rng = np.random.default_rng(int(factor * 10) + shape[0])
    x = O.bf16_round(rng.standard_normal(shape) * 0.09)
    x[0, :16] = 0.0
    valid = rng.random(shape[0]) > 0.2
    gs = np.float32(O.global_scale(float(np.abs(x).max())) * np.float32(factor))
    ref_c, ref_s = O.quantize_rows_with_global_scale(x, gs, valid_rows=valid)
    c, s = gpu_quant_gs(x, float(gs), valid)
    assert np.array_equal(c, ref_c) and np.array_equal(s, ref_s)
    log(f"[calibrated] {shape} x{factor}: {int((ref_s == 0x7E).sum())} saturated blocks, bit-exact")


def test_checkpoint_scale_saturates_instead_of_nan():
    """The pages' fixed checkpoint scale (1/input_scale = 3977.6) on activations with amax up to
    8 (std 0.09 with +-8 outliers): every block scale stays finite (<= 0x7E), bit-exact."""
    rng = np.random.default_rng(9)
    x = O.bf16_round(np.clip(rng.standard_normal((64, 7168)) * 0.09, -1.27, 1.27))
    pos = rng.choice(x.size, x.size // 1000, replace=False)
    x.reshape(-1)[pos] = np.where(rng.integers(0, 2, pos.size) == 1, 8.0, -8.0)
    gs = np.float32(3977.6)
    ref_c, ref_s = O.quantize_rows_with_global_scale(x, gs)
    c, s = gpu_quant_gs(x, float(gs))
    assert np.array_equal(c, ref_c) and np.array_equal(s, ref_s)
    assert s.max() == 0x7E and (s == 0x7E).sum() >= pos.size // 16


@pytest.mark.parametrize("i,T", [(0, 16), (1, 8)], ids=["tiny", "decode_t8"])
def test_layer_calibrated(i, T):
    wl = synth.WORKLOADS[i]
    s = make_setup(wl, T)
    x, ids, wts = s.dev_inputs()
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=DEV)
    base = L.forward(x, ids, wts, s.gpu_w).clone()
    torch.cuda.synchronize()
    gx, gh = L.x_gs.clone(), L.h_gs.clone()
    # the amax-derived scales passed back in: the same bits
    same = L.forward(x, ids, wts, s.gpu_w, x_gs=gx, h_gs=gh).clone()
    torch.cuda.synchronize()
    assert np.array_equal(np_i32(same.view(torch.int16)), np_i32(base.view(torch.int16)))
    # warm-up scales off by factors (x: 4x too large -> saturation; h: 0.5x)
    gx2 = gx * 4.0
    gh2 = gh * 0.5
    out = bf16_t2np(L.forward(x, ids, wts, s.gpu_w, x_gs=gx2, h_gs=gh2))
    torch.cuda.synchronize()
    counts = O.route(s.ids, wl.expert_begin, wl.num_experts, wl.pad_multiple)[0]
    q = s.oracle_weight_arrays([e for e in range(wl.num_experts) if counts[e] > 0])
    ref = O.moe_layer(s.x, s.ids, s.wts, wl.expert_begin, wl.num_experts, wl.pad_multiple, **q,
                      gs_x=float(gx2.item()), gs_h=float(gh2.item()))
    assert np.array_equal(np_i32(L.x_codes[:T]), ref["x_codes"]) and np.array_equal(np_i32(L.x_scales[:T]),
                                                                                    ref["x_scales"])
    err = rel_frob(out, ref["out"])
    log(f"[calibrated] layer {wl.name} T={T}: rel_frob {err:.2e}")
    assert err <= 1e-2


MID = synth.Workload("mid_zipf_e24", 32, 4, 512, 256, (300,), 0, 24, 1, zipf=True)
# experts with up to 10 m-tiles of 256 rows: the large-tile kernel's tile order with NVFP4 h
MANY_MT = synth.Workload("many_mtiles_e4", 4, 1, 1024, 512, (4000,), 0, 4, 1, zipf=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl,T", [(synth.WORKLOADS[0], 16), (synth.WORKLOADS[1], 8), (MID, 300),
                                  (synth.WORKLOADS[2], 512), (MANY_MT, 4000), (synth.WORKLOADS[3], 8192)],
                         ids=["tiny", "decode_t8", "mid", "t512_pad128", "many_mtiles", "t8192_zipf"])
def test_l1_nvfp4_equals_l1_then_quantizer(wl, T):
    """moe_grouped_gemm_l1_silu_nvfp4 (h quantized in the GEMM epilogue) gives, on every row that
    holds an assignment, the bits nvfp4_quantize_act_gs writes for the bf16 h of the plain L1; the
    other rows are left alone; the amax slots are those of the plain L1.  Scales: the amax-derived
    one, and 4x it (saturating blocks).  The 8192-token Zipf routing runs the 256-row kernel's
    epilogue over the full prefill tile list (53 experts, full and tail tiles)."""
    s = make_setup(wl, T)
    x, ids, _ = s.dev_inputs()
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=DEV)
    L.route_quantize(ids, x)
    L.l1(s.gpu_w)
    L.quantize_h()
    torch.cuda.synchronize()
    M, I = L.M_cap, wl.intermediate
    valid = np_i32(L.row_token[:M]) >= 0
    amax_plain = L.h_amax.clone()
    for factor in (1.0, 4.0):
        gs = L.h_gs * factor
        ref_c = torch.empty(M, I // 2, dtype=torch.uint8, device=DEV)
        ref_s = torch.empty(M, I // 16, dtype=torch.uint8, device=DEV)
        mm.nvfp4_quantize_act_gs(L.h[:M], gs, ref_c, ref_s, row_valid=L.row_token[:M])
        codes = torch.full((M, I // 2), 0xAB, dtype=torch.uint8, device=DEV)
        scales = torch.full((M, I // 16), 0xCD, dtype=torch.uint8, device=DEV)
        amax = torch.full((mm.L1_AMAX_PARTS,), -1.0, dtype=torch.float32, device=DEV)
        mm.moe_grouped_gemm_l1_silu_nvfp4(L.x_codes, L.x_scales, L.x_gs, L.row_token, L.padded_offsets, L.counts,
                                          L.sched, s.gpu_w.w13_codes, s.gpu_w.w13_scales, s.gpu_w.w13_gs, gs, codes,
                                          scales, amax, max_rows_per_expert=T)
        torch.cuda.synchronize()
        c, sc = np_i32(codes), np_i32(scales)
        assert np.array_equal(c[valid], np_i32(ref_c)[valid]) and np.array_equal(sc[valid], np_i32(ref_s)[valid])
        assert np.all(c[~valid] == 0xAB) and np.all(sc[~valid] == 0xCD)
        assert amax.min().item() >= 0.0 and amax.max().item() == amax_plain.max().item()  # every slot written; max |h| as the plain L1's
        log(f"[calibrated] fused L1 {wl.name} T={T} x{factor}: {int(valid.sum())} rows bit-exact, "
            f"{int((sc[valid] == 0x7E).sum())} saturated blocks")


@pytest.mark.parametrize("T,H", [(8, 7168), (1, 7168), (300, 2048)])
def test_route_quantize_with_scale(T, H):
    """moe_route_quantize with a calibrated scale (one launch at decode sizes, two calls above)
    equals moe_route_permute + nvfp4_quantize_act_gs, bit for bit, and leaves x_global_scale alone."""
    rng = np.random.default_rng(T + 3)
    k, E = 6, 48
    ids = np.array([rng.permutation(384)[:k] for _ in range(T)], np.int32)
    x = O.bf16_round(rng.standard_normal((T, H)) * 0.09)
    xd, idd = np2bf16_t(x), torch.from_numpy(ids).to(DEV)
    gs = torch.tensor([float(O.global_scale(float(np.abs(x).max())) * 2.0)], dtype=torch.float32, device=DEV)
    La = layer.MoELayer(T, k, E, H, 128, 1, device=DEV)
    Lb = layer.MoELayer(T, k, E, H, 128, 1, device=DEV)
    La.x_gs.fill_(-5.0)
    La.route_quantize(idd, xd, gs=gs)
    Lb.route(idd)
    Lb.quantize_x(xd, gs=gs)
    torch.cuda.synchronize()
    assert La.x_gs.item() == -5.0
    for name in ("counts", "expert_offsets", "padded_offsets", "sched"):
        assert torch.equal(getattr(La, name), getattr(Lb, name)), name
    assert torch.equal(La.row_token[:La.M_cap], Lb.row_token[:Lb.M_cap])
    assert torch.equal(La.x_codes[:T], Lb.x_codes[:T]) and torch.equal(La.x_scales[:T], Lb.x_scales[:T])
    ref_c, ref_s = O.quantize_rows_with_global_scale(x, np.float32(gs.item()))
    assert np.array_equal(np_i32(La.x_codes[:T]), ref_c) and np.array_equal(np_i32(La.x_scales[:T]), ref_s)
