"""Dense NVFP4 layers (nvfp4_linear, nvfp4_linear_gate_up_silu: the grouped GEMMs with one group of
every row), the combine with a shared expert's term, and the layer with a shared expert, against
the oracle.  Operands are quantized by the oracle (bit-exact inputs); outputs are compared by
relative Frobenius norm (1e-3 per GEMM, as for the grouped GEMMs; 1e-2 end to end)."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_top_amd import layer, megamoe as mm, synth
from oracle import nvfp4_oracle as O

from gpu_util import DEV, bf16_t2np, log, make_setup, np2bf16_t, np_i32, rel_frob

pytestmark = pytest.mark.gpu


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


def f32(v):
    return torch.tensor([float(v)], dtype=torch.float32, device=DEV)


def quantized(rng, rows, K, std):
    return O.quantize_nvfp4(O.bf16_round(rng.standard_normal((rows, K)) * std))


@pytest.mark.parametrize("M,K,N", [(0, 2048, 256), (1, 2048, 7168), (5, 128, 256), (16, 7168, 2048),
                                   (17, 2048, 7168), (300, 7168, 2048), (1000, 256, 512), (8, 640, 512),
                                   (3, 1152, 256), (12, 1024, 768)])
def test_linear(M, K, N):
    rng = np.random.default_rng(M + K + N)
    ac, as_, ag = quantized(rng, M, K, 0.09)
    wc, ws, wg = quantized(rng, N, K, 0.02)
    out = torch.full((max(M, 1), N), 0x7FC0, dtype=torch.int16, device=DEV)
    wsp = torch.empty(mm.megamoe_dense_workspace_bytes(M), dtype=torch.uint8, device=DEV)
    mm.nvfp4_linear(u8(ac), u8(as_), f32(ag), u8(wc), u8(ws), f32(wg), out[:M], wsp)
    torch.cuda.synchronize()
    if M == 0:
        assert np.all(np_i32(out) == 0x7FC0)  # nothing written
        return
    ref = O.nvfp4_linear(ac, as_, ag, wc, ws, wg)
    err = rel_frob(bf16_t2np(out[:M]), ref)
    log(f"[dense] linear M={M} K={K} N={N}: rel_frob {err:.2e}")
    assert err <= 1e-3


@pytest.mark.parametrize("M,K,I", [(1, 7168, 2048), (7, 256, 128), (16, 2048, 256), (40, 7168, 2048),
                                   (513, 2048, 1024), (3, 1024, 640)])
def test_gate_up_silu(M, K, I):
    rng = np.random.default_rng(M * 7 + K + I)
    ac, as_, ag = quantized(rng, M, K, 0.09)
    wc, ws, wg = quantized(rng, 2 * I, K, 0.02)
    h = torch.empty(M, I, dtype=torch.int16, device=DEV)
    amax = torch.full((mm.L1_AMAX_PARTS,), -1.0, dtype=torch.float32, device=DEV)
    wsp = torch.empty(mm.megamoe_dense_workspace_bytes(M), dtype=torch.uint8, device=DEV)
    mm.nvfp4_linear_gate_up_silu(u8(ac), u8(as_), f32(ag), u8(wc), u8(ws), f32(wg), h, amax, wsp)
    torch.cuda.synchronize()
    ref = O.nvfp4_linear_gate_up_silu(ac, as_, ag, wc, ws, wg)
    got = bf16_t2np(h)
    err = rel_frob(got, ref)
    log(f"[dense] gate_up_silu M={M} K={K} I={I}: rel_frob {err:.2e}")
    assert err <= 1e-3
    a = amax.cpu().numpy()
    assert a.min() >= 0 and a.max() == np.abs(got).max()  # every slot written; max = max |h|


def test_linear_full_size_sampled():
    """M=8192, K=7168, N=2048 (large tiles): 64 sampled rows against the oracle."""
    rng = np.random.default_rng(77)
    M, K, N = 8192, 7168, 2048
    ac, as_, ag = quantized(rng, M, K, 0.09)
    wc, ws, wg = quantized(rng, N, K, 0.02)
    out = torch.empty(M, N, dtype=torch.int16, device=DEV)
    wsp = torch.empty(mm.megamoe_dense_workspace_bytes(M), dtype=torch.uint8, device=DEV)
    mm.nvfp4_linear(u8(ac), u8(as_), f32(ag), u8(wc), u8(ws), f32(wg), out, wsp)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(M, 64, replace=False))
    ref = O.nvfp4_linear(ac[rows], as_[rows], ag, wc, ws, wg)
    err = rel_frob(bf16_t2np(out)[rows], ref)
    log(f"[dense] linear full size, 64 sampled rows: rel_frob {err:.2e}")
    assert err <= 1e-3


def test_combine_shared():
    rng = np.random.default_rng(4)
    T, k, H, Mc = 37, 6, 512, 300
    y = O.bf16_round(rng.standard_normal((Mc, H)))
    ys = O.bf16_round(rng.standard_normal((T, H)))
    rows = rng.integers(-1, Mc, (T, k)).astype(np.int32)
    w = rng.uniform(0, 0.4, (T, k)).astype(np.float32)
    out = torch.empty(T, H, dtype=torch.int16, device=DEV)
    mm.moe_combine_shared(np2bf16_t(y), torch.from_numpy(rows.reshape(-1)).to(DEV), torch.from_numpy(w).to(DEV),
                          np2bf16_t(ys), out)
    torch.cuda.synchronize()
    ref = O.combine(y, rows, w, ys)
    got = bf16_t2np(out)
    # fp32 accumulation against the float64 sum: within one bf16 step of the reference
    step = np.abs(ref) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(got - ref) <= step)


@pytest.mark.parametrize("i,T", [(0, 16), (1, 8)], ids=["tiny", "decode_t8"])
def test_layer_with_shared_expert(i, T):
    wl = synth.WORKLOADS[i]
    s = make_setup(wl, T)
    x, ids, wts = s.dev_inputs()
    # shared expert: weights drawn like a routed expert's, under an id no routed expert uses
    sh = layer.MoEWeights.empty(1, wl.hidden, wl.intermediate, device=DEV)
    w13, w2 = synth.expert_weights(wl, 100000, device=DEV)
    layer.quantize_expert_into(sh, 0, w13, w2)
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=DEV)
    out = bf16_t2np(L.forward(x, ids, wts, s.gpu_w, shared=sh))
    torch.cuda.synchronize()
    counts = O.route(s.ids, wl.expert_begin, wl.num_experts, wl.pad_multiple)[0]
    q = s.oracle_weight_arrays([e for e in range(wl.num_experts) if counts[e] > 0])
    q13 = O.quantize_nvfp4(O.bf16_from_bits(w13.cpu().view(torch.int16).numpy().view(np.uint16)))
    q2 = O.quantize_nvfp4(O.bf16_from_bits(w2.cpu().view(torch.int16).numpy().view(np.uint16)))
    assert np.array_equal(np_i32(sh.w13_codes[0]), q13[0]) and np.array_equal(np_i32(sh.w2_scales[0]), q2[1])
    ref = O.moe_layer(s.x, s.ids, s.wts, wl.expert_begin, wl.num_experts, wl.pad_multiple, **q,
                      shared=(q13[0], q13[1], q13[2], q2[0], q2[1], q2[2]))
    err = rel_frob(out, ref["out"])
    err_sh = rel_frob(bf16_t2np(L.sh_y[:T]), ref["y_shared"])
    log(f"[dense] layer {wl.name} T={T} with a shared expert: out rel_frob {err:.2e}, shared y {err_sh:.2e}")
    assert err <= 1e-2 and err_sh <= 1e-2


@pytest.mark.parametrize("M,K,I", [(1, 7168, 2048), (7, 256, 128), (40, 7168, 2048), (513, 2048, 1024)])
def test_gate_up_silu_nvfp4_equals_gate_up_then_quantizer(M, K, I):
    """nvfp4_linear_gate_up_silu_nvfp4 (h quantized in the epilogue with a given scale) equals
    nvfp4_linear_gate_up_silu followed by nvfp4_quantize_act_gs, bit for bit on every row; the
    max over the amax slots is that of the plain call."""
    rng = np.random.default_rng(M * 5 + K + I)
    ac, as_, ag = quantized(rng, M, K, 0.09)
    wc, ws, wg = quantized(rng, 2 * I, K, 0.02)
    wsp = torch.empty(mm.megamoe_dense_workspace_bytes(M), dtype=torch.uint8, device=DEV)
    h = torch.empty(M, I, dtype=torch.int16, device=DEV)
    amax = torch.empty(mm.L1_AMAX_PARTS, dtype=torch.float32, device=DEV)
    mm.nvfp4_linear_gate_up_silu(u8(ac), u8(as_), f32(ag), u8(wc), u8(ws), f32(wg), h, amax, wsp)
    torch.cuda.synchronize()
    gs = f32(O.global_scale(float(np.abs(bf16_t2np(h)).max())) * np.float32(2.0))  # some blocks saturate
    ref_c = torch.empty(M, I // 2, dtype=torch.uint8, device=DEV)
    ref_s = torch.empty(M, I // 16, dtype=torch.uint8, device=DEV)
    mm.nvfp4_quantize_act_gs(h, gs, ref_c, ref_s)
    codes = torch.full((M, I // 2), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((M, I // 16), 0xCD, dtype=torch.uint8, device=DEV)
    amax2 = torch.full((mm.L1_AMAX_PARTS,), -1.0, dtype=torch.float32, device=DEV)
    mm.nvfp4_linear_gate_up_silu_nvfp4(u8(ac), u8(as_), f32(ag), u8(wc), u8(ws), f32(wg), gs, codes, scales, amax2,
                                       wsp)
    torch.cuda.synchronize()
    assert torch.equal(codes, ref_c) and torch.equal(scales, ref_s)
    assert amax2.min().item() >= 0.0 and amax2.max().item() == amax.max().item()  # every slot written; same max |h|
    log(f"[dense] gate_up_silu_nvfp4 M={M} K={K} I={I}: bit-exact, "
        f"{int((np_i32(scales) == 0x7E).sum())} saturated blocks")


@pytest.mark.parametrize("i,T", [(0, 16), (1, 8)], ids=["tiny", "decode_t8"])
def test_layer_with_calibrated_shared_expert(i, T):
    """The layer with a shared expert and calibrated scales everywhere (x, routed h, shared h):
    the scales the uncalibrated forward derived, passed back in, give the same bits."""
    wl = synth.WORKLOADS[i]
    s = make_setup(wl, T)
    x, ids, wts = s.dev_inputs()
    sh = layer.MoEWeights.empty(1, wl.hidden, wl.intermediate, device=DEV)
    w13, w2 = synth.expert_weights(wl, 100000, device=DEV)
    layer.quantize_expert_into(sh, 0, w13, w2)
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=DEV)
    base = L.forward(x, ids, wts, s.gpu_w, shared=sh).clone()
    torch.cuda.synchronize()
    gx, gh, gsh = L.x_gs.clone(), L.h_gs.clone(), L.sh_h_gs.clone()
    same = L.forward(x, ids, wts, s.gpu_w, shared=sh, x_gs=gx, h_gs=gh, shared_h_gs=gsh).clone()
    torch.cuda.synchronize()
    assert torch.equal(same, base)
