"""The packed copy of the weight codes (nvfp4_pack_weight_codes) and the GEMM calls that read it.

The layout matches its definition in include/megamoe.h byte for byte, and a layer forward on packed
weights gives the same bits as on the row-major codes alone: h (bf16, or its NVFP4 codes and scales
with a calibrated global scale), y and out, on the decode share of 48 experts, on a routing whose
L2 takes 4-block groups, and on a mid-size routing with both tile classes."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_top_amd import megamoe as mm
from nvfp4_block_scaled_top_amd import synth

from gpu_util import DEV, log, make_setup, np_i32, run_gpu

pytestmark = pytest.mark.gpu


def packed_reference(codes: np.ndarray) -> np.ndarray:
    """The header's layout written out in storage order: 16-row block, 256-element chunk, half of
    the chunk's 2 KB, lane L = 16 g + r holding 16 bytes of row r of the block."""
    rows, kh = codes.shape
    out = np.empty(rows * kh, dtype=np.uint8)
    pos = 0
    for b in range(rows // 16):
        for c in range(2 * kh // 256):
            for q in range(2):
                for lane in range(64):
                    r, g = lane % 16, lane // 16
                    start = 128 * c + 32 * g + 16 * q
                    out[pos:pos + 16] = codes[16 * b + r, start:start + 16]
                    pos += 16
    return out


@pytest.mark.parametrize("shape", [(16, 128), (48, 384), (3, 32, 256)], ids=["16x256", "48x768", "3x32x512"])
def test_pack_layout_matches_definition(shape):
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=shape, dtype=np.uint8)
    log(f"[packed] layout {shape}")
    dev = torch.from_numpy(codes).to(DEV)
    packed = torch.empty(codes.size, dtype=torch.uint8, device=DEV)
    mm.nvfp4_pack_weight_codes(dev, packed)
    torch.cuda.synchronize()
    ref = packed_reference(codes.reshape(-1, shape[-1]))
    assert np.array_equal(packed.cpu().numpy(), ref)


def _valid_rows(L, t: torch.Tensor) -> np.ndarray:
    """Rows of a [M_cap, ...] buffer that hold an assignment (row_token >= 0), as bytes."""
    rt = np_i32(L.row_token[:L.M_cap])
    rows = np.nonzero(rt >= 0)[0]
    a = t[:L.M_cap].contiguous().view(torch.uint8).cpu().numpy()
    return a[rows]


def _forward_bits(s, packed: bool, h_gs=None) -> dict:
    w = s.gpu_w.clone()
    if packed:
        w.pack()
        assert w.w13_packed is not None and w.w2_packed is not None
    saved = s.gpu_w
    s.gpu_w = w
    try:
        if h_gs is None:
            L = run_gpu(s)
        else:
            wl = s.wl
            from nvfp4_block_scaled_top_amd import layer
            L = layer.MoELayer(s.T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                               expert_begin=wl.expert_begin, device=DEV)
            x, ids, wts = s.dev_inputs()
            L.forward(x, ids, wts, w, h_gs=h_gs)
            torch.cuda.synchronize()
    finally:
        s.gpu_w = saved
    res = {"out": L.out[:L.T].contiguous().view(torch.uint8).cpu().numpy(), "y": _valid_rows(L, L.y),
           "h_codes": _valid_rows(L, L.h_codes), "h_scales": _valid_rows(L, L.h_scales)}
    if h_gs is None:
        res["h"] = _valid_rows(L, L.h)
        res["h_gs"] = L.h_gs.cpu().numpy()
    return res


PK_MID = synth.Workload("packed_mid_e16", 16, 4, 2048, 2048, (400,), 0, 16, 1, zipf=True)
PK_WIDE = synth.Workload("packed_wide_l2_e4", 4, 1, 7168, 2048, (1280,), 0, 4, 1)
CASES = [(synth.WORKLOADS[1], 8), (synth.WORKLOADS[1], 4), (PK_WIDE, 1280), (PK_MID, 400)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl,T", CASES, ids=[f"{w.name}_t{t}" for w, t in CASES])
def test_layer_packed_equals_unpacked(wl, T):
    log(f"[packed] layer {wl.name} T={T}")
    s = make_setup(wl, T)
    a = _forward_bits(s, packed=False)
    b = _forward_bits(s, packed=True)
    assert a["y"].shape[0] > 0
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl,T", CASES[:1] + CASES[3:], ids=[f"{w.name}_t{t}" for w, t in CASES[:1] + CASES[3:]])
def test_layer_packed_equals_unpacked_calibrated(wl, T):
    """With a calibrated global scale for h, L1 writes NVFP4 h itself (the NVFP4-output epilogue of
    the 16-row kernels, whose blocks then pair 16 gate rows with the 16 up rows)."""
    log(f"[packed] calibrated layer {wl.name} T={T}")
    s = make_setup(wl, T)
    gs = torch.from_numpy(_forward_bits(s, packed=False)["h_gs"]).to(DEV)
    a = _forward_bits(s, packed=False, h_gs=gs)
    b = _forward_bits(s, packed=True, h_gs=gs)
    assert a["h_codes"].shape[0] > 0
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def _fused_bits(s, packed: bool, h_gs=None) -> dict:
    from nvfp4_block_scaled_top_amd import layer
    w = s.gpu_w.clone()
    if packed:
        w.pack()
    wl = s.wl
    L = layer.MoELayer(s.T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=DEV)
    x, ids, wts = s.dev_inputs()
    L.forward(x, ids, wts, w, h_gs=h_gs, fused=True)
    torch.cuda.synchronize()
    assert L.ffn_sync_error() == 0
    return {"out": L.out[:L.T].contiguous().view(torch.uint8).cpu().numpy(), "y": _valid_rows(L, L.y),
            "h_codes": _valid_rows(L, L.h_codes), "h_scales": _valid_rows(L, L.h_scales)}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("calibrated", [False, True], ids=["amax_scale", "calibrated_scale"])
def test_fused_packed_equals_unpacked(calibrated):
    """moe_grouped_ffn_fused_packed against moe_grouped_ffn_fused on the decode share (T=8)."""
    wl, T = synth.WORKLOADS[1], 8
    log(f"[packed] fused {wl.name} T={T} calibrated={calibrated}")
    s = make_setup(wl, T)
    gs = torch.from_numpy(_forward_bits(s, packed=False)["h_gs"]).to(DEV) if calibrated else None
    a = _fused_bits(s, packed=False, h_gs=gs)
    b = _fused_bits(s, packed=True, h_gs=gs)
    assert a["y"].shape[0] > 0
    for k in a:
        assert np.array_equal(a[k], b[k]), k
