"""HIP-graph capture of one layer forward (mid-size, decode T=8, and the 8192- and 512-token
prefills): every replay equals the eager result bit for bit, with eager work and synchronizations
between replays (the benchmark replays captured steps)."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_top_amd import layer, synth

from gpu_util import DEV, make_setup, np_i32

pytestmark = pytest.mark.gpu

MID = synth.Workload("mid_zipf_e24", 32, 4, 512, 256, (300,), 0, 24, 1, zipf=True)


# the prefill launch sequences bench.py replays: three-kernel routing, the amax pass, both tile
# classes (the 512-token one with 4-block L2 groups)
PREFILL = [(synth.WORKLOADS[3], 8192), (synth.WORKLOADS[2], 512)]
CASES = [(MID, 300), (synth.WORKLOADS[1], 8)] + PREFILL
IDS = ["mid", "decode_t8", "t8192_zipf", "t512_pad128"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl,T", CASES, ids=IDS)
def test_graph_replays_match_eager(wl, T):
    s = make_setup(wl, T)
    x, ids, wts = s.dev_inputs()
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=DEV)
    L.forward(x, ids, wts, s.gpu_w)
    torch.cuda.synchronize()
    eager = np_i32(L.out[:T].view(torch.int16)).copy()
    eager_h = np_i32(L.h[:L.M_cap].view(torch.int16)).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.forward(x, ids, wts, s.gpu_w)
    for r in range(4):
        L.out.fill_(0x7FC0)   # eager work between replays: poison outputs
        L.h_amax.fill_(123.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np_i32(L.out[:T].view(torch.int16)), eager), r
        valid = np_i32(L.row_token[:L.M_cap]) >= 0
        assert np.array_equal(np_i32(L.h[:L.M_cap].view(torch.int16))[valid], eager_h[valid]), r


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl,T", CASES[1:], ids=IDS[1:])
def test_graph_replays_packed_weights(wl, T):
    """The benchmark's configuration: weights with the packed copy of their codes.  Every replay
    equals the eager forward on the row-major codes alone, bit for bit."""
    s = make_setup(wl, T)
    x, ids, wts = s.dev_inputs()
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=DEV)
    L.forward(x, ids, wts, s.gpu_w)
    torch.cuda.synchronize()
    eager = np_i32(L.out[:T].view(torch.int16)).copy()
    w = s.gpu_w.clone().pack()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.forward(x, ids, wts, w)
    for r in range(3):
        L.out.fill_(0x7FC0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np_i32(L.out[:T].view(torch.int16)), eager), r


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl,T", CASES, ids=IDS)
def test_graph_replays_calibrated(wl, T):
    """The calibrated forward (x quantized in the routing launch, h written as NVFP4 by L1)
    captured once: every replay equals the eager result, with h's codes poisoned in between."""
    s = make_setup(wl, T)
    x, ids, wts = s.dev_inputs()
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=DEV)
    L.forward(x, ids, wts, s.gpu_w)
    torch.cuda.synchronize()
    gx, gh = L.x_gs.clone(), L.h_gs.clone()
    L.forward(x, ids, wts, s.gpu_w, x_gs=gx, h_gs=gh)
    torch.cuda.synchronize()
    eager = np_i32(L.out[:T].view(torch.int16)).copy()
    valid = np_i32(L.row_token[:L.M_cap]) >= 0
    eager_hc = np_i32(L.h_codes[:L.M_cap])[valid].copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.forward(x, ids, wts, s.gpu_w, x_gs=gx, h_gs=gh)
    for r in range(4):
        L.out.fill_(0x7FC0)
        L.h_codes.fill_(0xEE)
        L.x_codes.fill_(0xEE)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np_i32(L.out[:T].view(torch.int16)), eager), r
        assert np.array_equal(np_i32(L.h_codes[:L.M_cap])[valid], eager_hc), r
