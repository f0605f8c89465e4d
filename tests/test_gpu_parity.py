"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bars: bit-exact for routing tables, FP4 codes, E4M3 scales and global scales; relative Frobenius
<= 1e-3 for h (L1) and y (L2) when fed the same quantized inputs; <= 1e-2 with cosine >= 0.9999
end to end.  Workloads: the tiny workload, three medium workloads that mix both tile classes with
ragged tails, non-local ids, a zero-token expert and padding to 128 (one with hidden 2048 and
intermediate 1024, long enough in K for the staged-scale path of the 16-row kernels), experts
with up to 8 m-tiles of 256 rows (the large-tile kernels' tile order), a single expert with top-1
routing, an empty input (T = 0), and the decode workload at its full size (48 local experts of 384,
hidden 7168, intermediate 2048, T = 1, 4, 8).
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_top_amd import layer, megamoe as mm, synth
from oracle import nvfp4_oracle as O

from gpu_util import (DEV, bf16_t2np, cosine, log, make_setup, np2bf16_t, np_i32, oracle_chain, rel_frob,
                      run_gpu)

pytestmark = pytest.mark.gpu

MID = synth.Workload("mid_zipf_e24", 32, 4, 512, 256, (300,), 0, 24, 1, zipf=True)
MID_PAD = synth.Workload("mid_zipf_e16_pad128", 32, 4, 512, 256, (150,), 8, 16, 128, zipf=True)
# K of at least 4 chunks of 256 in both GEMMs (hidden 2048, intermediate 1024): the 16-row tile
# kernels take the path with weight scales staged in LDS; Zipf routing leaves both tile classes.
MID_K = synth.Workload("mid_k_e12", 24, 4, 2048, 1024, (160,), 4, 12, 1, zipf=True)
# L2 reduction length 640 = five 128-element chunks (the 16-row kernel's 128-chunk path with its
# weight scales read from HBM; staged scales cover whole 256-element chunks only).
ODD_K = synth.Workload("odd_k640_e16", 128, 6, 1024, 640, (8,), 0, 16, 1)
# Experts with many 256-row m-tiles (top-1 over 4 Zipf-biased experts, T=4000) and 4 n-tiles per
# m-tile in both GEMMs (intermediate 512, hidden 1024): the large-tile kernels' bands of m-tiles,
# whole and ragged, and tail tiles.
MANY_MT = synth.Workload("many_mtiles_e4", 4, 1, 1024, 512, (4000,), 0, 4, 1, zipf=True)
# Many 16-row m-tiles with a short L2 reduction (intermediate 1024 = four 256-element chunks, one
# per wave of the 16-row kernel) and hidden 7168: with block_m 16 forced, 40 m-tiles x 224 L2 groups
# put ~17 groups on every workgroup of the 16-row L2 kernel (the weight-scale copies of its loader
# run ahead of the compute across group boundaries).
SMALL_K1024 = synth.Workload("small_k1024_e4", 4, 2, 7168, 1024, (320,), 0, 4, 1)
# Enough 16-row m-tiles for the 16-row L2 kernel's 4-block groups: top-1 over 4 experts, 1280 tokens
# with block_m 16 forced, at least 80 m-tiles x 224 two-block groups of 7168 output columns, i.e.
# at least 32 per workgroup of the 512 (reduction length 2048 with staged weight scales).
SMALL_WIDE = synth.Workload("small_wide_l2_e4", 4, 1, 7168, 2048, (1280,), 0, 4, 1)
# The degenerate routing: one expert, top-1 (every token's weight is 1), 40 tokens in one 256-row
# tile whose rows 40..255 are padding, no tail tiles (intermediate 128, hidden 256).
SINGLE = synth.Workload("single_expert_top1", 1, 1, 256, 128, (40,), 0, 1, 1)
TINY = synth.WORKLOADS[0]
DECODE = synth.WORKLOADS[1]

STAGE_TOL = 1e-3
E2E_TOL = 1e-2
E2E_COS = 0.9999

_cache = {}


def setup_for(wl, T):
    """Seeded inputs for (workload, T); expert weights are drawn once per workload and shared."""
    key = (wl.name, T)
    if key not in _cache:
        log(f"[setup] {wl.name} T={T}")
        other = next((v for (n, _), v in _cache.items() if n == wl.name), None)
        _cache[key] = make_setup(wl, T, weights_from=other)
    return _cache[key]


def check_tables(L, ref):
    E = L.E
    assert np.array_equal(np_i32(L.counts), ref["counts"])
    assert np.array_equal(np_i32(L.expert_offsets), ref["expert_offsets"])
    assert np.array_equal(np_i32(L.padded_offsets), ref["padded_offsets"])
    assert np.array_equal(np_i32(L.row_token)[:L.M_cap], ref["row_token"])
    assert np.array_equal(np_i32(L.token_rows)[:L.T * L.k].reshape(L.T, L.k), ref["token_rows"])
    sched = np_i32(L.sched)
    bm = sched[4:4 + E]
    counts = ref["counts"]
    assert np.all((bm == 0) == (counts == 0))
    small = np.where(bm == 16, (counts + 15) // 16, 0)
    large = np.where(bm == 256, (counts + 255) // 256, 0)
    assert np.array_equal(sched[4 + E:5 + 2 * E], np.concatenate([[0], np.cumsum(small)]))
    assert np.array_equal(sched[5 + 2 * E:6 + 3 * E], np.concatenate([[0], np.cumsum(large)]))
    assert sched[1] == small.sum() and sched[2] == large.sum()


@pytest.mark.parametrize("wl,T", [(TINY, 16), (MID, 300), (MID_PAD, 150), (MID_K, 160), (ODD_K, 8), (MANY_MT, 4000),
                                  (SINGLE, 40)],
                         ids=["tiny", "mid", "mid_pad128", "mid_k2048", "odd_k640", "many_mtiles", "single_expert"])
def test_layer_end_to_end_and_stages(wl, T):
    s = setup_for(wl, T)
    log(f"[run] {wl.name} T={T}: GPU layer")
    L = run_gpu(s)
    log(f"[oracle] {wl.name} T={T}")
    ref = oracle_chain(s)
    check_tables(L, ref)
    # x quantization: bit-exact
    assert np.array_equal(np_i32(L.x_codes)[:T], ref["x_codes"])
    assert np.array_equal(np_i32(L.x_scales)[:T], ref["x_scales"])
    assert L.x_gs.item() == float(ref["gs_x"])
    # weights quantized on the GPU equal the oracle's
    for e in range(wl.num_experts):
        if ref["counts"][e] > 0:
            q = s.oracle_quantize(e)
            assert np.array_equal(np_i32(s.gpu_w.w13_codes[e]), q[0])
            assert np.array_equal(np_i32(s.gpu_w.w13_scales[e]), q[1])
            assert s.gpu_w.w13_gs[e].item() == float(q[2])
            assert np.array_equal(np_i32(s.gpu_w.w2_codes[e]), q[3])
            assert np.array_equal(np_i32(s.gpu_w.w2_scales[e]), q[4])
            assert s.gpu_w.w2_gs[e].item() == float(q[5])
    valid = ref["row_token"] >= 0
    # L1 (same quantized inputs on both sides)
    h = bf16_t2np(L.h[:L.M_cap])
    err_h = rel_frob(h[valid], ref["h"][valid])
    # the L1 amax is the max over the rows the kernel wrote
    assert L.h_amax.max().item() == np.abs(h[valid]).max()
    log(f"[l1] rel_frob={err_h:.2e}")
    assert err_h <= STAGE_TOL
    # end to end
    out = bf16_t2np(L.out[:T])
    err, cos = rel_frob(out, ref["out"]), cosine(out, ref["out"])
    log(f"[e2e] rel_frob={err:.2e} cosine={cos:.7f}")
    assert np.isfinite(out).all() and err <= E2E_TOL and cos >= E2E_COS
    none_local = np.all(ref["token_rows"] < 0, axis=1)
    assert np.all(np_i32(L.out[:T].view(torch.int16))[none_local] == 0)


def test_layer_empty_input():
    """T = 0: every launch of the forward runs with no work.  The routing tables are empty, both
    global scales are the amax-zero value 1 (oracle.global_scale), and there is no output row."""
    s = setup_for(TINY, 0)
    L = run_gpu(s)
    ref = oracle_chain(s)
    assert np.array_equal(np_i32(L.counts), ref["counts"]) and ref["counts"].sum() == 0
    assert L.x_gs.item() == float(ref["gs_x"]) == 1.0
    assert L.h_gs.item() == float(ref["gs_h"]) == 1.0
    assert L.out[:0].shape[0] == 0 and ref["out"].shape[0] == 0


@pytest.mark.parametrize("wl,T", [(TINY, 16), (MID, 300), (MID_PAD, 150), (MID_K, 160)],
                         ids=["tiny", "mid", "mid_pad128", "mid_k2048"])
def test_stage_inputs_from_oracle(wl, T):
    """Requantize h, L2 and combine, each fed the oracle's own inputs for that stage."""
    s = setup_for(wl, T)
    ref = oracle_chain(s)
    L = run_gpu(s)  # routing tables (bit-exact with the oracle's) and buffers
    valid = ref["row_token"] >= 0
    M = L.M_cap
    # S4: the GPU quantizer on the oracle's h with the oracle's amax
    h_dev = np2bf16_t(ref["h"])
    amax = torch.tensor([ref["amax_h"]], dtype=torch.float32, device=DEV)
    codes = torch.empty(M, wl.intermediate // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(M, wl.intermediate // 16, dtype=torch.uint8, device=DEV)
    gs = torch.empty(1, dtype=torch.float32, device=DEV)
    mm.nvfp4_quantize_act(h_dev, codes, scales, gs, row_valid=L.row_token[:M], amax_in=amax)
    torch.cuda.synchronize()
    assert np.array_equal(np_i32(codes), ref["h_codes"]) and np.array_equal(np_i32(scales), ref["h_scales"])
    assert gs.item() == float(ref["gs_h"])
    # S5: L2 on the oracle's quantized h
    y = torch.empty(M, wl.hidden, dtype=torch.int16, device=DEV)
    mm.moe_grouped_gemm_l2(codes, scales, gs, L.padded_offsets, L.counts, L.sched, s.gpu_w.w2_codes,
                           s.gpu_w.w2_scales, s.gpu_w.w2_gs, y, max_rows_per_expert=T)
    torch.cuda.synchronize()
    err_y = rel_frob(bf16_t2np(y)[valid], ref["y"][valid])
    log(f"[l2] rel_frob={err_y:.2e}")
    assert err_y <= STAGE_TOL
    # S6: combine on the oracle's y
    out = torch.empty(T, wl.hidden, dtype=torch.int16, device=DEV)
    mm.moe_combine(np2bf16_t(ref["y"]), L.token_rows[:T * wl.top_k], torch.from_numpy(s.wts).to(DEV), out)
    torch.cuda.synchronize()
    got = bf16_t2np(out)
    # fp32 vs float64 accumulation of <= k terms: at most one bf16 rounding step apart
    ulp = np.exp2(np.frexp(ref["out"])[1] - 8.0)
    assert np.all(np.abs(got - ref["out"]) <= ulp)
    assert rel_frob(got, ref["out"]) <= STAGE_TOL


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [1, 4, 8])
def test_decode_full_size(T):
    """48 local experts of 384 at hidden 7168 / intermediate 2048 (the expert-parallel decode share)."""
    s = setup_for(DECODE, T)
    L = run_gpu(s)
    log(f"[oracle] decode T={T}")
    ref = oracle_chain(s)
    check_tables(L, ref)
    assert np.array_equal(np_i32(L.x_codes)[:T], ref["x_codes"])
    assert np.array_equal(np_i32(L.x_scales)[:T], ref["x_scales"])
    out = bf16_t2np(L.out[:T])
    if np.linalg.norm(ref["out"]) == 0:
        assert T == 1 and np.all(np_i32(L.out[:T].view(torch.int16)) == 0)
        return
    valid = ref["row_token"] >= 0
    h = bf16_t2np(L.h[:L.M_cap])
    err_h = rel_frob(h[valid], ref["h"][valid])
    err, cos = rel_frob(out, ref["out"]), cosine(out, ref["out"])
    log(f"[decode T={T}] l1 rel_frob={err_h:.2e} e2e rel_frob={err:.2e} cosine={cos:.7f}")
    assert err_h <= STAGE_TOL and err <= E2E_TOL and cos >= E2E_COS


def test_quantizer_edge_cases():
    """Zeros, ties at every E2M1 midpoint, every E4M3 scale code, ragged valid rows, amax_in."""
    rng = np.random.default_rng(21)
    rows, cols = 160, 256
    x = O.bf16_round(rng.standard_normal((rows, cols)) * 0.05)
    x[0, 0] = 2688.0  # amax 2688 -> gs exactly 1, so x*gs/s is x/s
    # rows 1..127: block amax 6*s for every E4M3 value s, elements on the exact midpoints m*s
    grid = O.E4M3_GRID
    for c in range(1, 127):
        r = c
        s = grid[c]
        blk = np.array([6 * s] + [m * s * (-1) ** j for j, m in enumerate(O.E2M1_MIDPOINTS)] +
                       [0.0, -0.0] + list(O.E2M1_MAGNITUDES[1:7] * s))
        blk = O.bf16_round(blk)
        x[r, 16:32] = blk
    x[130] = 0.0
    x[131] = -0.0
    valid = np.ones(rows, np.int32)
    valid[[5, 77, 140, 159]] = -1
    for row_valid in (None, valid):
        ref_c, ref_s, ref_g = O.quantize_nvfp4(x, None if row_valid is None else row_valid >= 0)
        xd = np2bf16_t(x)
        codes = torch.empty(rows, cols // 2, dtype=torch.uint8, device=DEV)
        scales = torch.empty(rows, cols // 16, dtype=torch.uint8, device=DEV)
        gs = torch.empty(1, dtype=torch.float32, device=DEV)
        ws = torch.empty(mm.megamoe_quant_workspace_bytes(rows, cols), dtype=torch.uint8, device=DEV)
        rv = None if row_valid is None else torch.from_numpy(row_valid).to(DEV)
        mm.nvfp4_quantize_act(xd, codes, scales, gs, workspace=ws, row_valid=rv)
        torch.cuda.synchronize()
        assert gs.item() == float(ref_g)
        assert np.array_equal(np_i32(scales), ref_s)
        assert np.array_equal(np_i32(codes), ref_c)
        assert len(set(np_i32(scales).ravel().tolist())) > 120  # nearly every scale code occurs
        # amax passed in instead of computed: same result
        amax = torch.tensor([np.abs(x[(valid >= 0) if row_valid is not None else slice(None)]).max()],
                            dtype=torch.float32, device=DEV)
        mm.nvfp4_quantize_act(xd, codes, scales, gs, row_valid=rv, amax_in=amax)
        torch.cuda.synchronize()
        assert np.array_equal(np_i32(codes), ref_c) and gs.item() == float(ref_g)
    # all zeros: gs = 1, zero scales
    z = torch.zeros(4, 64, dtype=torch.int16, device=DEV)
    codes = torch.empty(4, 32, dtype=torch.uint8, device=DEV)
    scales = torch.empty(4, 4, dtype=torch.uint8, device=DEV)
    gs = torch.empty(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(mm.megamoe_quant_workspace_bytes(4, 64), dtype=torch.uint8, device=DEV)
    mm.nvfp4_quantize_act(z, codes, scales, gs, workspace=ws)
    torch.cuda.synchronize()
    assert gs.item() == 1.0 and int(scales.sum()) == 0 and int(codes.sum()) == 0


def test_quantizer_hand_built_bytes():
    """The GPU quantizer writes the bytes worked out by hand from the format definition
    (tests/golden/nvfp4_layout_literal.txt: exact ties, -0, a zero block, scales 448/112/224/0)."""
    import os

    g = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "nvfp4_layout_literal.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, *vals = line.split()
                g[key] = [float(v) for v in vals] if key[0] in "xg" else [int(v, 16) for v in vals]
    x = np.array([g["x0"], g["x1"]])
    codes = torch.empty(2, 16, dtype=torch.uint8, device=DEV)
    scales = torch.empty(2, 2, dtype=torch.uint8, device=DEV)
    gs = torch.empty(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(mm.megamoe_quant_workspace_bytes(2, 32), dtype=torch.uint8, device=DEV)
    mm.nvfp4_quantize_act(np2bf16_t(x), codes, scales, gs, workspace=ws)
    torch.cuda.synchronize()
    assert gs.item() == g["gs"][0]
    assert np_i32(codes).tolist() == [g["codes0"], g["codes1"]]
    assert np_i32(scales).tolist() == [g["scales0"], g["scales1"]]


@pytest.mark.parametrize("wl,T,wide", [(SMALL_K1024, 320, False), (SMALL_WIDE, 1280, True)],
                         ids=["k1024_2block_groups", "k2048_4block_l2_groups"])
def test_small_class_many_groups(wl, T, wide):
    """16-row kernels only (block_m 16 forced): L2 with K = 1024 and ~17 two-block groups per
    workgroup, and L2 with K = 2048 and enough m-tiles for 4-block groups; every stage against the
    oracle (h, y within 1e-3; end to end 1e-2 / 0.9999)."""
    s = setup_for(wl, T)
    ref = oracle_chain(s)
    L = run_gpu(s, block_m_override=16)
    check_tables(L, ref)
    sched = np_i32(L.sched)
    assert sched[1] >= 40 and sched[2] == 0  # >= 40 small m-tiles, no large ones
    # the L2 kernel takes 4-block groups from 32 two-block groups (32 columns) per workgroup
    assert (int(sched[1]) * (wl.hidden // 32) >= 32 * 512) == wide
    valid = ref["row_token"] >= 0
    err_h = rel_frob(bf16_t2np(L.h[:L.M_cap])[valid], ref["h"][valid])
    # L2 on the oracle's quantized h
    hq = torch.from_numpy(ref["h_codes"]).to(DEV)
    hs = torch.from_numpy(ref["h_scales"]).to(DEV)
    hg = torch.tensor([float(ref["gs_h"])], dtype=torch.float32, device=DEV)
    y = torch.empty_like(L.y[:L.M_cap])
    w = s.gpu_w
    mm.moe_grouped_gemm_l2(hq, hs, hg, L.padded_offsets, L.counts, L.sched, w.w2_codes, w.w2_scales, w.w2_gs, y,
                           16, 0)
    torch.cuda.synchronize()
    err_y = rel_frob(bf16_t2np(y)[valid], ref["y"][valid])
    out = bf16_t2np(L.out[:L.T])
    err, cos = rel_frob(out, ref["out"]), cosine(out, ref["out"])
    log(f"[small {wl.name}] l1 {err_h:.2e} l2 {err_y:.2e} e2e {err:.2e} cos {cos:.7f}")
    assert err_h <= STAGE_TOL and err_y <= STAGE_TOL and err <= E2E_TOL and cos >= E2E_COS


def test_quantizer_random_global_scales():
    """Many tensors with different amax: the fp32 global scale division is correctly rounded."""
    rng = np.random.default_rng(22)
    for i in range(40):
        scale = float(np.exp2(rng.uniform(-20, 10)))
        x = O.bf16_round(rng.standard_normal((3, 32)) * scale)
        ref_c, ref_s, ref_g = O.quantize_nvfp4(x)
        codes = torch.empty(3, 16, dtype=torch.uint8, device=DEV)
        scales = torch.empty(3, 2, dtype=torch.uint8, device=DEV)
        gs = torch.empty(1, dtype=torch.float32, device=DEV)
        ws = torch.empty(mm.megamoe_quant_workspace_bytes(3, 32), dtype=torch.uint8, device=DEV)
        mm.nvfp4_quantize_act(np2bf16_t(x), codes, scales, gs, workspace=ws)
        torch.cuda.synchronize()
        assert gs.item() == float(ref_g), (i, scale)
        assert np.array_equal(np_i32(codes), ref_c) and np.array_equal(np_i32(scales), ref_s)


@pytest.mark.parametrize("T,k,E,e0,P,Eg", [(0, 6, 8, 0, 4, 16), (1, 6, 48, 0, 1, 384), (1000, 6, 384, 0, 128, 384),
                                           (5000, 4, 7, 3, 5, 12), (3000, 8, 1024, 0, 1, 1100)])
def test_route_random(T, k, E, e0, P, Eg):
    rng = np.random.default_rng(T + E)
    ids = np.array([rng.permutation(Eg)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
    ref = dict(zip(["counts", "expert_offsets", "padded_offsets", "row_token", "token_rows"], O.route(ids, e0, E, P)))
    L = layer.MoELayer(T, k, E, 256, 128, P, expert_begin=e0, device=DEV)
    L.route(torch.from_numpy(ids).to(DEV))
    torch.cuda.synchronize()
    check_tables(L, ref)


@pytest.mark.parametrize("i", [2, 3, 4])
def test_route_full_size_workloads(i):
    wl = synth.WORKLOADS[i]
    T = wl.tokens[0]
    ids, _ = O.router_topk(synth.router_logits(wl, T), wl.top_k)
    ref = dict(zip(["counts", "expert_offsets", "padded_offsets", "row_token", "token_rows"],
                   O.route(ids, wl.expert_begin, wl.num_experts, wl.pad_multiple)))
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple, device=DEV)
    L.route(torch.from_numpy(ids).to(DEV))
    torch.cuda.synchronize()
    check_tables(L, ref)


def test_gemm_extreme_block_scales():
    """Weight blocks spanning ~24 binades: subnormal and tiny E4M3 block scales reach the GEMM decode."""
    rng = np.random.default_rng(23)
    E, H, I, T, k = 2, 256, 128, 40, 1
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    wts = np.ones((T, k), np.float32)
    x = O.bf16_round(rng.standard_normal((T, H)) * 0.09)

    def weights(shape):
        w = rng.standard_normal(shape) * 0.02
        blk = np.exp2(-rng.integers(0, 24, (shape[0], shape[1] // 16)).astype(np.float64))
        return O.bf16_round(w * np.repeat(blk, 16, axis=1))

    W13 = [weights((2 * I, H)) for _ in range(E)]
    W2 = [weights((H, I)) for _ in range(E)]
    q13 = [O.quantize_nvfp4(w) for w in W13]
    q2 = [O.quantize_nvfp4(w) for w in W2]
    assert min(int(q[1][q[1] > 0].min()) for q in q13) < 8  # subnormal scale codes present
    ref = O.moe_layer(x, ids, wts, 0, E, 1, np.stack([q[0] for q in q13]), np.stack([q[1] for q in q13]),
                      np.array([q[2] for q in q13], np.float32), np.stack([q[0] for q in q2]),
                      np.stack([q[1] for q in q2]), np.array([q[2] for q in q2], np.float32))
    Wg = layer.MoEWeights.empty(E, H, I, device=DEV)
    for e in range(E):
        layer.quantize_expert_into(Wg, e, np2bf16_t(W13[e]), np2bf16_t(W2[e]))
    L = layer.MoELayer(T, k, E, H, I, 1, device=DEV)
    L.forward(np2bf16_t(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(wts).to(DEV), Wg)
    torch.cuda.synchronize()
    for e in range(E):
        assert np.array_equal(np_i32(Wg.w13_scales[e]), q13[e][1]) and np.array_equal(np_i32(Wg.w2_codes[e]), q2[e][0])
    valid = ref["row_token"] >= 0
    err_h = rel_frob(bf16_t2np(L.h[:L.M_cap])[valid], ref["h"][valid])
    out = bf16_t2np(L.out[:T])
    err, cos = rel_frob(out, ref["out"]), cosine(out, ref["out"])
    log(f"[extreme scales] l1 {err_h:.2e} e2e {err:.2e} cos {cos:.7f}")
    assert err_h <= STAGE_TOL and err <= E2E_TOL and cos >= E2E_COS
