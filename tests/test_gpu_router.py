"""GPU router (moe_router_topk, moe_route_logits) against the oracle's router on the same float32
logits: top-k ids bit for bit; weights within one float32 unit, since the two float64 softmax
denominators are summed in different orders and may differ in the last bit (nearly every weight
comes out bit-identical, and the test reports how many do not).  The permutation tables that
moe_route_logits writes equal the oracle's route() of the oracle's ids, bit for bit."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_top_amd import layer, megamoe as mm, synth
from oracle import nvfp4_oracle as O

from gpu_util import DEV, log, make_setup, np_i32

pytestmark = pytest.mark.gpu


def gpu_router(logits: np.ndarray, k: int):
    T = logits.shape[0]
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(DEV)
    ids = torch.full((max(T, 1), k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((max(T, 1), k), -1.0, dtype=torch.float32, device=DEV)
    mm.moe_router_topk(lg, k, ids[:T], w[:T])
    torch.cuda.synchronize()
    return np_i32(ids[:T]), w[:T].cpu().numpy(), np_i32(ids[T:]), w[T:].cpu().numpy()


def check_router(logits, k, label):
    ids, w, ids_tail, w_tail = gpu_router(logits, k)
    ref_ids, ref_w = O.router_topk(logits, k)
    assert np.array_equal(ids, ref_ids), label
    ulps = np.abs(w.view(np.int32).astype(np.int64) - ref_w.view(np.int32).astype(np.int64))
    log(f"[router] {label}: T={logits.shape[0]} E={logits.shape[1]} k={k} ids equal, weights "
        f"{int((ulps == 0).sum())}/{ulps.size} bit-identical, max {int(ulps.max(initial=0))} ulp")
    assert ulps.max(initial=0) <= 1, label
    if logits.shape[0] == 0:  # nothing written past the (empty) output
        assert np.all(ids_tail == -7) and np.all(w_tail == -1.0)


@pytest.mark.parametrize("i", [0, 1, 2, 3, 4])
def test_router_workloads(i):
    wl = synth.WORKLOADS[i]
    for T in wl.tokens:
        check_router(synth.router_logits(wl, T), wl.top_k, f"{wl.name} T={T}")


def test_router_decode_seeds():
    wl = synth.WORKLOADS[1]
    lg = np.concatenate([synth.router_logits(wl, 8, seed) for seed in range(64)])
    check_router(lg, wl.top_k, "decode logits of 64 seeds")


@pytest.mark.parametrize("T,E,k", [(0, 384, 6), (1, 1, 1), (3, 100, 7), (13, 1024, 64), (5, 64, 64),
                                   (257, 257, 9)])
def test_router_shapes(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    check_router(rng.standard_normal((T, E)).astype(np.float32) * np.float32(3), k, f"shape T={T} E={E} k={k}")


def test_router_ties_and_extremes():
    rng = np.random.default_rng(5)
    lg = (np.round(rng.standard_normal((40, 384)) * 4) / 4).astype(np.float32)  # many exact ties
    lg[0] = 0.5                                    # all equal: the lowest ids, 1/E each
    lg[1, 100:200] = lg[1].max()                   # a hundred-way tie for the maximum
    lg[2] *= np.float32(2000.0)                    # most probabilities underflow to 0
    lg[3, ::2] = -np.float32(1e30)                 # half the experts far below the rest
    check_router(lg, 6, "ties and extremes")
    ids, w, _, _ = gpu_router(lg[:2], 6)
    assert ids[0].tolist() == list(range(6)) and np.all(w[0] == np.float32(1 / 384))
    assert ids[1].tolist() == list(range(100, 106))


@pytest.mark.parametrize("wl,T", [(synth.WORKLOADS[1], 8), (synth.WORKLOADS[2], 512),
                                  (synth.WORKLOADS[3], 8192)], ids=["decode_t8", "t512_pad128", "t8192_zipf"])
def test_route_logits_tables(wl, T):
    lg = synth.router_logits(wl, T)
    ref_ids, ref_w = O.router_topk(lg, wl.top_k)
    ref = O.route(ref_ids, wl.expert_begin, wl.num_experts, wl.pad_multiple)
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=DEV)
    L.route_logits(torch.from_numpy(lg).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(np_i32(L.topk_ids[:T]), ref_ids)
    ulps = np.abs(L.topk_weights[:T].cpu().numpy().view(np.int32).astype(np.int64)
                  - ref_w.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    got = [np_i32(L.counts), np_i32(L.expert_offsets), np_i32(L.padded_offsets), np_i32(L.row_token[:L.M_cap]),
           np_i32(L.token_rows[:T * wl.top_k]).reshape(T, wl.top_k)]
    for g, r, name in zip(got, ref, ["counts", "expert_offsets", "padded_offsets", "row_token", "token_rows"]):
        assert np.array_equal(g, r), name


@pytest.mark.parametrize("i,T", [(0, 16), (1, 8)], ids=["tiny", "decode_t8"])
def test_forward_logits_equals_forward_from_ids(i, T):
    """The layer from logits gives the same bits as the layer from the GPU router's ids and weights."""
    wl = synth.WORKLOADS[i]
    s = make_setup(wl, T)
    lg = torch.from_numpy(synth.router_logits(wl, T)).to(DEV)
    x, _, _ = s.dev_inputs()
    La = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                        expert_begin=wl.expert_begin, device=DEV)
    out_a = La.forward_logits(x, lg, s.gpu_w).clone()
    Lb = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                        expert_begin=wl.expert_begin, device=DEV)
    out_b = Lb.forward(x, La.topk_ids[:T].clone(), La.topk_weights[:T].clone(), s.gpu_w)
    torch.cuda.synchronize()
    assert np.array_equal(np_i32(out_a.view(torch.int16)), np_i32(out_b.view(torch.int16)))


@pytest.mark.parametrize("T,E,H,k", [(1, 48, 7168, 6), (8, 48, 7168, 6), (16, 8, 256, 2), (170, 384, 256, 6),
                                     (171, 384, 256, 6), (300, 384, 7168, 6), (0, 48, 7168, 6)])
def test_route_quantize_equals_separate_calls(T, E, H, k):
    """moe_route_quantize (one launch at decode sizes, two calls above them) gives the bits of
    moe_route_permute and nvfp4_quantize_act; T=170/171 straddle the one-launch limit."""
    rng = np.random.default_rng(T + H)
    ids = np.array([rng.permutation(384)[:k] for _ in range(T)], np.int32).reshape(T, k)
    x = O.bf16_round(rng.standard_normal((T, H)) * 0.09)
    from gpu_util import np2bf16_t
    xd, idd = np2bf16_t(x), torch.from_numpy(ids).to(DEV)
    La = layer.MoELayer(T, k, E, H, 128, 1, device=DEV)
    Lb = layer.MoELayer(T, k, E, H, 128, 1, device=DEV)
    for t in (La.row_token, La.token_rows, La.x_codes, Lb.row_token, Lb.token_rows, Lb.x_codes):
        t.fill_(0x55)
    La.route_quantize(idd, xd)
    Lb.route(idd)
    Lb.quantize_x(xd)
    torch.cuda.synchronize()
    for name in ("counts", "expert_offsets", "padded_offsets", "sched", "x_gs"):
        assert np.array_equal(getattr(La, name).cpu().numpy(), getattr(Lb, name).cpu().numpy()), name
    assert np.array_equal(np_i32(La.row_token[:La.M_cap]), np_i32(Lb.row_token[:Lb.M_cap]))
    assert np.array_equal(np_i32(La.token_rows[:T * k]), np_i32(Lb.token_rows[:T * k]))
    assert np.array_equal(np_i32(La.x_codes[:T]), np_i32(Lb.x_codes[:T]))
    assert np.array_equal(np_i32(La.x_scales[:T]), np_i32(Lb.x_scales[:T]))
    if T:
        ref_c, ref_s, ref_g = O.quantize_nvfp4(x)
        assert np.array_equal(np_i32(La.x_codes[:T]), ref_c) and La.x_gs.item() == float(ref_g)
