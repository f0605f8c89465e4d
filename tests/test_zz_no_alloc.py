"""moe_route_permute_noalloc (static per-GPU scratch, no workspace argument) against
moe_route_permute (caller's workspace) through the C ABI: every routing table bit for bit, on two
calls in a row, the second with fewer assignments and fewer experts than the first (the static
array keeps the first call's histograms, which the second must not depend on)."""
import ctypes

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_top_amd import megamoe as mm

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _tables(T, k, E, P, device=DEV):
    i32 = dict(dtype=torch.int32, device=device)
    M = mm.megamoe_row_capacity(T, k, E, P)
    return dict(counts=torch.full((E,), -7, **i32), expert_offsets=torch.full((E + 1,), -7, **i32),
                padded_offsets=torch.full((E + 1,), -7, **i32), row_token=torch.full((max(M, 1),), -7, **i32),
                token_rows=torch.full((max(T * k, 1),), -7, **i32),
                sched=torch.full((mm.megamoe_sched_len(E),), -7, **i32))


def _call_c(fn, ids, T, k, e0, E, P, tb, extra):
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    return fn(p(ids), T, k, e0, E, P, 0, p(tb["counts"]), p(tb["expert_offsets"]), p(tb["padded_offsets"]),
              p(tb["row_token"]), p(tb["token_rows"]), p(tb["sched"]), *extra,
              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_route_matches_workspace_route(order):
    lib = mm.lib()
    rng = np.random.default_rng(77)
    cases = [(16384, 6, 384, 0, 1, 384), (3000, 4, 96, 8, 128, 128)]  # second: fewer assignments, experts
    for T, k, E, e0, P, Eg in cases:
        print(f"[noalloc] T={T} k={k} E={E} e0={e0} P={P}", flush=True)
        ids = torch.from_numpy(np.stack([rng.permutation(Eg)[:k] for _ in range(T)]).astype(np.int32)).to(DEV)
        need = mm.megamoe_route_workspace_bytes(T, k, E)
        assert 0 < need <= mm.ROUTE_NOALLOC_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        ref = _tables(T, k, E, P)
        got = _tables(T, k, E, P)
        assert _call_c(lib.moe_route_permute, ids, T, k, e0, E, P, ref,
                       [ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(need)]) == 0
        assert _call_c(lib.moe_route_permute_noalloc, ids, T, k, e0, E, P, got, []) == 0
        torch.cuda.synchronize()
        for name in ref:
            assert torch.equal(ref[name], got[name]), name
        assert int(got["counts"].sum()) > 0
