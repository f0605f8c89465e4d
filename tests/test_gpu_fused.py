"""moe_grouped_ffn_fused: L1 gate+up with SiLU, the requantization of h and L2 down as one persistent
launch.  Its results are those of the three separate calls with every expert in 16-row m-tiles,
bit for bit: h codes and scales, the global scale of h, the amax slots' maximum and y, with the
amax-derived scale (the launch waits for every L1 group before quantizing h) and with a calibrated
one (an expert's L2 waits for its own L1 groups only).  Workloads: decode at T = 1, 4 and 8 on
the 48-expert share, the tiny and odd-K shapes (128-element chunks), padded rows,
experts of up to 50 rows (several 16-row m-tiles each), a single expert, 1024 local experts, and two
routings with enough m-tiles that the separate L2 kernel takes 4-block groups, with 256- and
128-element chunks and at the layer's real shape with staged scales (the fused launch keeps 2-block
ones, so these compare the two group widths bit for bit).  The sync words are back
at zero after every call, no wait expired, a second call right after the first gives the same bits,
the layer's fused forward matches the oracle's layer, and replays of a captured graph equal the
eager result."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_top_amd import layer, megamoe as mm, synth
from oracle import nvfp4_oracle as O

from gpu_util import DEV, bf16_t2np, log, make_setup, np_i32, rel_frob

pytestmark = pytest.mark.gpu

MID = synth.Workload("mid_zipf_e24", 32, 4, 512, 256, (300,), 0, 24, 1, zipf=True)
MID_PAD = synth.Workload("mid_zipf_e16_pad128", 32, 4, 512, 256, (150,), 8, 16, 128, zipf=True)
ODD_K = synth.Workload("odd_k640_e16", 128, 6, 1024, 640, (8,), 0, 16, 1)
SINGLE = synth.Workload("single_expert_top1", 1, 1, 256, 128, (40,), 0, 1, 1)
# the most local experts one call takes: 24.6 KB of per-expert tables in LDS, 1024 expert counters
# in the sync buffer
WIDE = synth.Workload("wide_e1024", 2048, 8, 512, 256, (24,), 512, 1024, 1)
# The separate L2 kernel's 4-block groups (from 32 two-block groups per workgroup of the 512):
# 1280 tokens top-1 over 4 experts at hidden 7168 (>= 80 regular m-tiles x 224 groups, staged weight
# scales), and 1024 tokens top-2 over 1024 experts at hidden 1024 (mostly m-tiles of 1-2 rows, the
# tiny phase, x 32 groups).
WIDE_REG = synth.Workload("l2_4block_regular_e4", 4, 1, 7168, 2048, (1280,), 0, 4, 1)
WIDE_TINY = synth.Workload("l2_4block_tiny_e1024", 1024, 2, 1024, 256, (1024,), 0, 1024, 1)
# ... and with 128-element chunks (intermediate 640, an odd multiple of 128): 3072 tokens top-2
# over 256 experts at hidden 2048 (about 24 rows per expert, two 16-row m-tiles, x 64 groups).
WIDE_CH128 = synth.Workload("l2_4block_ch128_e256", 256, 2, 2048, 640, (3072,), 0, 256, 1)
# ... and at the layer's real shape with staged weight scales: 32 tokens top-6 over all 384 experts
# (about 160 m-tiles, mostly of one row: the tiny phase, x 224 groups).
WIDE_TINY_REAL = synth.Workload("l2_4block_tiny_e384", 384, 6, 7168, 2048, (32,), 0, 384, 1)
DEC = synth.WORKLOADS[1]

CASES = [(synth.WORKLOADS[0], 16), (DEC, 1), (DEC, 4), (DEC, 8), (MID, 300), (MID_PAD, 150), (ODD_K, 8),
         (SINGLE, 40), (WIDE, 24), (WIDE_REG, 1280), (WIDE_TINY, 1024), (WIDE_CH128, 3072), (WIDE_TINY_REAL, 32)]
IDS = ["tiny", "decode_t1", "decode_t4", "decode_t8", "mid", "mid_pad128", "odd_k640", "single_expert",
       "wide_e1024", "l2_4block_regular", "l2_4block_tiny", "l2_4block_ch128", "l2_4block_tiny_e384"]


def make_layer(wl, T):
    s = make_setup(wl, T)
    x, ids, wts = s.dev_inputs()
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=DEV)
    L.route_quantize(ids, x)
    return s, L, (x, ids, wts)


def separate(L, w, gs_h=None):
    """The three calls in 16-row m-tiles; returns (h codes, h scales, gs_h, amax max, y) on the host."""
    M = L.M_cap
    if gs_h is None:
        mm.moe_grouped_gemm_l1_silu(L.x_codes, L.x_scales, L._gs_x, L.row_token, L.padded_offsets, L.counts,
                                    L.sched, w.w13_codes, w.w13_scales, w.w13_gs, L.h[:M], L.h_amax,
                                    block_m_override=16)
        mm.nvfp4_quantize_act(L.h[:M], L.h_codes[:M], L.h_scales[:M], L.h_gs, row_valid=L.row_token[:M],
                              amax_in=L.h_amax)
        gs = L.h_gs
    else:
        mm.moe_grouped_gemm_l1_silu_nvfp4(L.x_codes, L.x_scales, L._gs_x, L.row_token, L.padded_offsets, L.counts,
                                          L.sched, w.w13_codes, w.w13_scales, w.w13_gs, gs_h, L.h_codes[:M],
                                          L.h_scales[:M], L.h_amax, block_m_override=16)
        gs = gs_h
    mm.moe_grouped_gemm_l2(L.h_codes, L.h_scales, gs, L.padded_offsets, L.counts, L.sched, w.w2_codes, w.w2_scales,
                           w.w2_gs, L.y[:M], block_m_override=16)
    torch.cuda.synchronize()
    return (np_i32(L.h_codes[:M]).copy(), np_i32(L.h_scales[:M]).copy(), float(gs.item()),
            float(L.h_amax.max().item()), np_i32(L.y[:M]).copy())


def poison(L):
    L.h_codes.fill_(0xAB)
    L.h_scales.fill_(0xCD)
    L.y.fill_(0x7FC0)
    L.h_amax.fill_(-1.0)
    L.h_gs.fill_(-5.0)


def check_fused(L, ref, gs_h, tag):
    M = L.M_cap
    rc, rs, rgs, ramax, ry = ref
    valid = np_i32(L.row_token[:M]) >= 0
    c, sc, y = np_i32(L.h_codes[:M]), np_i32(L.h_scales[:M]), np_i32(L.y[:M])
    if gs_h is None:
        # every row written (rows without an assignment zero), like the separate quantizer
        assert np.array_equal(c, rc) and np.array_equal(sc, rs), tag
        assert L.h_gs.item() == rgs, tag
    else:
        assert np.array_equal(c[valid], rc[valid]) and np.array_equal(sc[valid], rs[valid]), tag
        assert np.all(c[~valid] == 0xAB) and np.all(sc[~valid] == 0xCD), tag
    assert L.h_amax.min().item() >= 0.0 and L.h_amax.max().item() == ramax, tag  # every slot written
    assert np.array_equal(y[valid], ry[valid]), tag
    assert np.all(y[~valid] == 0x7FC0), tag                                      # not written
    assert int(L.ffn_sync.abs().sum().item()) == 0, tag                          # counters back at 0, no error


@pytest.mark.parametrize("calibrated", [False, True], ids=["amax_scale", "calibrated"])
@pytest.mark.parametrize("wl,T", CASES, ids=IDS)
def test_fused_equals_separate(wl, T, calibrated):
    s, L, _ = make_layer(wl, T)
    w = s.gpu_w
    torch.cuda.synchronize()
    if wl in (WIDE_REG, WIDE_TINY, WIDE_CH128, WIDE_TINY_REAL):  # enough 16-row m-tiles for 4-block L2 groups
        assert int(((L.counts + 15) // 16).sum().item()) * (wl.hidden // 32) >= 32 * 512
    gs_h = None
    if calibrated:
        separate(L, w)  # the amax scale, times 0.75 (a warm-up scale off by a factor)
        gs_h = L.h_gs.clone() * 0.75
    poison(L)
    ref = separate(L, w, gs_h)
    for rep in range(2):  # the second call checks that the first left the sync words at zero
        poison(L)
        L.ffn_fused(w, h_gs=gs_h)
        torch.cuda.synchronize()
        check_fused(L, ref, gs_h, f"{wl.name} T={T} call {rep}")
    valid = int((np_i32(L.row_token[:L.M_cap]) >= 0).sum())
    log(f"[fused] {wl.name} T={T} {'calibrated' if calibrated else 'amax'}: {valid} rows, h and y bit-exact, "
        f"sync words zero")


def test_fused_consecutive_different_inputs():
    """Two decode calls in a row on different routings (T=8, then T=4 through another layer sharing
    nothing but the weights): each equals its separate calls."""
    for T, seed_wl in ((8, DEC), (4, DEC)):
        s, L, _ = make_layer(seed_wl, T)
        ref = separate(L, s.gpu_w)
        poison(L)
        L.ffn_fused(s.gpu_w)
        torch.cuda.synchronize()
        check_fused(L, ref, None, f"consecutive T={T}")


@pytest.mark.parametrize("calibrated", [False, True], ids=["amax_scale", "calibrated"])
@pytest.mark.parametrize("wl,T", [(synth.WORKLOADS[0], 16), (DEC, 8)], ids=["tiny", "decode_t8"])
def test_fused_layer_matches_oracle(wl, T, calibrated):
    """The layer's fused forward (route+quantize x, the fused launch, combine) against the oracle's
    layer with the same global scales."""
    s = make_setup(wl, T)
    x, ids, wts = s.dev_inputs()
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=DEV)
    gh = None
    if calibrated:
        L.forward(x, ids, wts, s.gpu_w)
        torch.cuda.synchronize()
        gh = L.h_gs.clone() * 0.5
    out = bf16_t2np(L.forward(x, ids, wts, s.gpu_w, h_gs=gh, fused=True))
    torch.cuda.synchronize()
    assert L.ffn_sync_error() == 0
    counts = O.route(s.ids, wl.expert_begin, wl.num_experts, wl.pad_multiple)[0]
    q = s.oracle_weight_arrays([e for e in range(wl.num_experts) if counts[e] > 0])
    kw = {} if gh is None else {"gs_h": float(gh.item())}
    ref = O.moe_layer(s.x, s.ids, s.wts, wl.expert_begin, wl.num_experts, wl.pad_multiple, **q, **kw)
    if gh is None:
        assert L.h_gs.item() == np.float32(ref["gs_h"])
    err = rel_frob(out, ref["out"])
    log(f"[fused] layer {wl.name} T={T} {'calibrated' if calibrated else 'amax'}: rel_frob {err:.2e}")
    assert err <= 1e-2


@pytest.mark.parametrize("calibrated", [False, True], ids=["amax_scale", "calibrated"])
def test_fused_graph_replays(calibrated):
    """The fused decode forward captured once: every replay equals the eager result, with the
    outputs poisoned by eager work in between (the launch resets its own counters, no memset)."""
    wl, T = DEC, 8
    s = make_setup(wl, T)
    x, ids, wts = s.dev_inputs()
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=DEV)
    L.forward(x, ids, wts, s.gpu_w)
    torch.cuda.synchronize()
    gh = L.h_gs.clone() if calibrated else None
    L.forward(x, ids, wts, s.gpu_w, h_gs=gh, fused=True)
    torch.cuda.synchronize()
    eager = np_i32(L.out[:T].view(torch.int16)).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.forward(x, ids, wts, s.gpu_w, h_gs=gh, fused=True)
    for r in range(4):
        L.out.fill_(0x7FC0)
        L.h_codes.fill_(0xAB)
        L.y.fill_(0x7FC0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np_i32(L.out[:T].view(torch.int16)), eager), r
        assert int(L.ffn_sync.abs().sum().item()) == 0, r


def test_fused_empty_input():
    """T = 0 (no rows): the call only writes the amax slots (0) and gs_h = 1."""
    L = layer.MoELayer(0, 6, 48, 256, 128, 1, device=DEV)
    w = layer.MoEWeights.empty(48, 256, 128, device=DEV)
    L.x_gs.fill_(1.0)
    L._gs_x = L.x_gs
    L.h_amax.fill_(-1.0)
    L.h_gs.fill_(-5.0)
    L.counts.zero_()
    L.padded_offsets.zero_()
    L.sched.zero_()
    L.ffn_fused(w)
    torch.cuda.synchronize()
    assert L.h_amax.abs().max().item() == 0.0 and L.h_gs.item() == 1.0
