"""The C-ABI library loads, exports every symbol include/megamoe.h declares, and rejects bad
arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

from nvfp4_block_scaled_top_amd import megamoe as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "megamoe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:int32_t|int64_t|size_t)\s+(\w+)\s*\(", src, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mm.library_path()):
        from nvfp4_block_scaled_top_amd import build_lib
        build_lib.build()
    return mm.lib()


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert set(names) == set(mm.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n)


def test_constants_match_header():
    src = open(HEADER).read()
    assert re.search(rf"#define MEGAMOE_L1_AMAX_PARTS {mm.L1_AMAX_PARTS}\b", src)


def test_error_codes_match_header():
    src = open(HEADER).read()
    for code, name in mm.ERRORS.items():
        assert re.search(rf"#define {name} \({code}\)", src), name


def test_size_helpers(lib):
    assert mm.megamoe_row_capacity(8192, 6, 384, 1) == 49152
    assert mm.megamoe_row_capacity(512, 6, 384, 128) == 3072 + 384 * 127
    assert mm.megamoe_row_capacity(-1, 6, 384, 1) == -1
    assert mm.megamoe_sched_len(48) == 6 + 3 * 48
    assert mm.megamoe_sched_len(0) == -1
    assert mm.megamoe_route_workspace_bytes(8, 6, 48) == 48 * 4
    assert mm.megamoe_route_workspace_bytes(16384, 6, 384) == 96 * 384 * 4
    assert mm.megamoe_quant_workspace_bytes(16, 256) == 4
    assert mm.megamoe_quant_workspace_bytes(16384, 7168) == 1024 * 4


def _c(v):
    return ctypes.c_void_p(v)


FAKE = 0x1000  # never dereferenced: every call below must fail its host-side checks


def test_route_rejects_bad_args(lib):
    f = lib.moe_route_permute
    ok = [FAKE] * 6
    assert f(FAKE, 4, 0, 0, 48, 1, 0, *ok, FAKE, 4096, None) == -2            # k < 1
    assert f(FAKE, 4, 6, 0, 0, 1, 0, *ok, FAKE, 4096, None) == -2             # E < 1
    assert f(FAKE, 4, 6, 0, 2000, 1, 0, *ok, FAKE, 1 << 20, None) == -2       # E too large
    assert f(FAKE, 4, 6, 0, 48, 0, 0, *ok, FAKE, 4096, None) == -2            # P < 1
    assert f(FAKE, 4, 6, 0, 48, 1, 48, *ok, FAKE, 4096, None) == -2           # unsupported block_m
    assert f(FAKE, -1, 6, 0, 48, 1, 0, *ok, FAKE, 4096, None) == -2           # T < 0
    assert f(None, 4, 6, 0, 48, 1, 0, *ok, FAKE, 4096, None) == -1            # ids NULL
    assert f(FAKE, 4, 6, 0, 48, 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 4096, None) == -1  # sched NULL
    assert f(FAKE, 4, 6, 0, 48, 1, 0, *ok, FAKE, 4, None) == -3               # workspace too small


def test_route_noalloc_rejects_bad_args_and_oversize(lib):
    """The no-allocation routing entry point makes moe_route_permute's checks and rejects sizes whose
    scratch would exceed its static per-GPU array, all before any HIP call."""
    f = lib.moe_route_permute_noalloc
    ok = [FAKE] * 6
    assert f(FAKE, 4, 0, 0, 48, 1, 0, *ok, None) == -2             # k < 1
    assert f(FAKE, 4, 6, 0, 48, 0, 0, *ok, None) == -2             # P < 1
    assert f(None, 4, 6, 0, 48, 1, 0, *ok, None) == -1             # ids NULL
    assert f(FAKE, 4, 6, 0, 48, 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -1  # sched NULL
    cap = mm.ROUTE_NOALLOC_SCRATCH_BYTES
    assert re.search(rf"#define MEGAMOE_ROUTE_NOALLOC_SCRATCH_BYTES \(1 << 20\)", open(HEADER).read())
    assert cap == 1 << 20
    # 384 experts: 682 chunks of 1024 assignments fit (682 * 384 * 4 <= 1 MiB), 683 do not
    assert mm.megamoe_route_workspace_bytes(682 * 1024 // 8, 8, 384) <= cap
    assert mm.megamoe_route_workspace_bytes(683 * 1024 // 8, 8, 384) > cap
    assert f(FAKE, 683 * 1024 // 8, 8, 0, 384, 1, 0, *ok, None) == -3  # scratch too small


def test_router_rejects_bad_args(lib):
    f = lib.moe_router_topk
    assert f(FAKE, 4, 384, 0, FAKE, FAKE, None) == -2        # k < 1
    assert f(FAKE, 4, 384, 65, FAKE, FAKE, None) == -2       # k > 64
    assert f(FAKE, 4, 4, 6, FAKE, FAKE, None) == -2          # k > number of experts
    assert f(FAKE, 4, 2048, 6, FAKE, FAKE, None) == -2       # too many experts
    assert f(FAKE, -1, 384, 6, FAKE, FAKE, None) == -2       # T < 0
    assert f(None, 4, 384, 6, FAKE, FAKE, None) == -1        # logits NULL
    assert f(FAKE, 4, 384, 6, FAKE, None, None) == -1        # weights NULL
    g = lib.moe_route_logits
    ok = [FAKE] * 6
    assert g(FAKE, 4, 384, 0, 0, 48, 1, 0, FAKE, FAKE, *ok, FAKE, 4096, None) == -2         # k < 1
    assert g(FAKE, 4, 384, 6, 0, 0, 1, 0, FAKE, FAKE, *ok, FAKE, 4096, None) == -2          # E < 1
    assert g(None, 4, 384, 6, 0, 48, 1, 0, FAKE, FAKE, *ok, FAKE, 4096, None) == -1         # logits NULL
    assert g(FAKE, 4, 384, 6, 0, 48, 1, 0, FAKE, FAKE, *ok, FAKE, 4, None) == -3            # workspace too small

    h = lib.moe_route_quantize
    r = [FAKE] * 6 + [FAKE, 1 << 20]
    assert h(FAKE, 4, 0, 0, 48, 1, 0, *r, FAKE, 7168, None, FAKE, FAKE, FAKE, FAKE, 4096, None) == -2    # k < 1
    assert h(FAKE, 4, 6, 0, 48, 1, 0, *r, FAKE, 48, None, FAKE, FAKE, FAKE, FAKE, 4096, None) == -2      # H % 32
    assert h(FAKE, 4, 6, 0, 48, 1, 0, *r, FAKE, 0, None, FAKE, FAKE, FAKE, FAKE, 4096, None) == -2       # H 0
    assert h(FAKE, 4, 6, 0, 48, 1, 0, *r, None, 7168, None, FAKE, FAKE, FAKE, FAKE, 4096, None) == -1    # x NULL
    assert h(FAKE, 4, 6, 0, 48, 1, 0, *r, FAKE, 7168, None, FAKE, FAKE, None, FAKE, 4096, None) == -1    # scale NULL
    assert h(FAKE, 4, 6, 0, 48, 1, 0, *[FAKE] * 6, FAKE, 4, FAKE, 7168, None, FAKE, FAKE, FAKE, FAKE, 4096,
             None) == -3                                                                         # route ws
    # calibrated scale given: x_global_scale and the quantizer workspace are not needed
    assert h(FAKE, 4, 6, 0, 48, 1, 0, *r, FAKE, 48, FAKE, FAKE, FAKE, None, None, 0, None) == -2  # H % 32
    assert h(FAKE, 4, 6, 0, 48, 1, 0, *r, None, 7168, FAKE, FAKE, FAKE, None, None, 0, None) == -1  # x NULL
    assert h(FAKE, 100000, 6, 0, 48, 1, 0, *r, FAKE, 7168, None, FAKE, FAKE, FAKE, FAKE, 64, None) == -3  # quant ws
    assert h(FAKE, 100000, 6, 0, 48, 1, 0, *r, FAKE, 7168, None, FAKE, FAKE, FAKE, None, 4096, None) == -1


def test_quant_rejects_bad_args(lib):
    f = lib.nvfp4_quantize_act
    assert f(FAKE, 4, 48, None, None, 0, FAKE, FAKE, FAKE, FAKE, 64, None) == -2   # cols % 32
    assert f(FAKE, 4, 0, None, None, 0, FAKE, FAKE, FAKE, FAKE, 64, None) == -2    # cols 0
    assert f(FAKE, -2, 64, None, None, 0, FAKE, FAKE, FAKE, FAKE, 64, None) == -2  # rows < 0
    assert f(FAKE, 4, 64, None, FAKE, 0, FAKE, FAKE, FAKE, FAKE, 64, None) == -2   # amax_in_count 0
    assert f(None, 4, 64, None, None, 0, FAKE, FAKE, FAKE, FAKE, 64, None) == -1
    assert f(FAKE, 4, 64, None, None, 0, FAKE, FAKE, None, FAKE, 64, None) == -1
    assert f(FAKE, 4, 64, None, None, 0, FAKE, FAKE, FAKE, FAKE, 0, None) == -3
    assert f(FAKE, 4, 64, None, None, 0, FAKE, FAKE, FAKE, None, 64, None) == -1   # workspace NULL


def test_gemm_rejects_bad_args(lib):
    l1, l2 = lib.moe_grouped_gemm_l1_silu, lib.moe_grouped_gemm_l2
    p10 = [FAKE] * 10
    assert l1(*p10, 8, 384, 128, 64, 0, 0, FAKE, FAKE, None) == -2      # H not a multiple of 256
    assert l1(*p10, 8, 256, 96, 64, 0, 0, FAKE, FAKE, None) == -2       # I not a multiple of 128
    assert l1(*p10, 0, 256, 128, 64, 0, 0, FAKE, FAKE, None) == -2      # E < 1
    assert l1(*p10, 8, 256, 128, -1, 0, 0, FAKE, FAKE, None) == -2      # M_cap < 0
    assert l1(*p10, 8, 256, 128, 64, 48, 0, FAKE, FAKE, None) == -2     # unsupported block_m
    assert l1(*p10, 8, 256, 128, 64, 0, -1, FAKE, FAKE, None) == -2     # negative row bound
    assert l1(*p10, 8, 256, 128, 64, 0, 0, FAKE, None, None) == -1      # h_amax NULL
    assert l1(None, *p10[1:], 8, 256, 128, 64, 0, 0, FAKE, FAKE, None) == -1
    q = lib.moe_grouped_gemm_l1_silu_nvfp4
    assert q(*p10, 8, 384, 128, 64, 0, 0, FAKE, FAKE, FAKE, FAKE, None) == -2   # H not a multiple of 256
    assert q(*p10, 8, 256, 128, 64, 0, 0, None, FAKE, FAKE, FAKE, None) == -1   # h_gs NULL
    assert q(*p10, 8, 256, 128, 64, 0, 0, FAKE, None, FAKE, FAKE, None) == -1   # h_codes NULL
    assert q(*p10, 8, 256, 128, 64, 0, 0, FAKE, FAKE, FAKE, None, None) == -1   # h_amax NULL
    p9 = [FAKE] * 9
    assert l2(*p9, 8, 256, 100, 64, 0, 0, FAKE, None) == -2
    assert l2(*p9, 8, 128, 128, 64, 0, 0, FAKE, None) == -2
    assert l2(*p9, 8, 256, 128, 64, 32, 0, FAKE, None) == -2
    assert l2(*p9, 8, 256, 128, 64, 0, 0, None, None) == -1
    # M_cap == 0: the row arrays may be NULL, the small fixed-size ones may not
    pl1 = [FAKE] * 10
    pl1[0] = pl1[1] = pl1[3] = None                                         # x_codes, x_scales, row_token
    assert l1(*pl1, 8, 256, 128, 0, 0, 0, FAKE, None, None) == -1          # h_amax still required
    assert l1(*pl1, 8, 256, 128, 64, 0, 0, FAKE, FAKE, None) == -1         # rows present: required
    pnull_gs = [FAKE] * 10
    pnull_gs[2] = None                                                      # x_gs
    assert l1(*pnull_gs, 8, 256, 128, 0, 0, 0, None, FAKE, None) == -1
    pl2 = [FAKE] * 9
    pl2[0] = pl2[1] = None                                                  # h_codes, h_scales
    assert l2(*pl2, 8, 256, 128, 64, 0, 0, None, None) == -1               # rows present: required
    pl2[2] = None                                                           # h_gs
    assert l2(*pl2, 8, 256, 128, 0, 0, 0, None, None) == -1


def test_packed_entry_points_reject_bad_args(lib):
    """nvfp4_pack_weight_codes and the *_packed GEMMs: shape and NULL checks, before any HIP call."""
    pk = lib.nvfp4_pack_weight_codes
    assert pk(FAKE, 24, 256, FAKE, None) == -2    # rows not a multiple of 16
    assert pk(FAKE, 0, 256, FAKE, None) == -2
    assert pk(FAKE, 16, 384, FAKE, None) == -2    # K not a multiple of 256
    assert pk(None, 16, 256, FAKE, None) == -1
    assert pk(FAKE, 16, 256, None, None) == -1
    p10 = [FAKE] * 10
    l1p = lib.moe_grouped_gemm_l1_silu_packed
    assert l1p(*p10, None, 8, 256, 128, 64, 0, 0, FAKE, FAKE, None) == -1    # packed codes NULL
    assert l1p(*p10, FAKE, 8, 384, 128, 64, 0, 0, FAKE, FAKE, None) == -2    # H not a multiple of 256
    assert l1p(*p10, FAKE, 8, 256, 128, 64, 0, 0, FAKE, None, None) == -1    # h_amax NULL
    qp = lib.moe_grouped_gemm_l1_silu_nvfp4_packed
    assert qp(*p10, None, 8, 256, 128, 64, 0, 0, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert qp(*p10, FAKE, 8, 256, 128, 64, 0, 0, None, FAKE, FAKE, FAKE, None) == -1   # h_gs NULL
    p9 = [FAKE] * 9
    l2p = lib.moe_grouped_gemm_l2_packed
    assert l2p(*p9, FAKE, 8, 256, 128, 64, 0, 0, FAKE, None) == -2    # I not a multiple of 256
    assert l2p(*p9, None, 8, 256, 256, 64, 0, 0, FAKE, None) == -1
    assert l2p(*p9, FAKE, 8, 256, 256, 64, 0, 0, None, None) == -1    # y NULL
    fp = lib.moe_grouped_ffn_fused_packed
    need = mm.megamoe_ffn_sync_bytes(8)
    p13 = [FAKE] * 13
    tail = (FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, need, None)
    assert fp(*p13, FAKE, FAKE, 8, 256, 128, 64, *tail) == -2     # I not a multiple of 256
    assert fp(*p13, None, FAKE, 8, 256, 256, 64, *tail) == -1     # w13 packed NULL
    assert fp(*p13, FAKE, None, 8, 256, 256, 64, *tail) == -1     # w2 packed NULL


def test_ffn_fused_rejects_bad_args(lib):
    """moe_grouped_ffn_fused: shape, NULL and sync-size checks, all before any HIP call."""
    f = lib.moe_grouped_ffn_fused
    need = mm.megamoe_ffn_sync_bytes(8)
    assert need == (384 + 8 * 32) * 4
    assert mm.megamoe_ffn_sync_bytes(0) == 0 and mm.megamoe_ffn_sync_bytes(1025) == 0
    p13 = [FAKE] * 13

    def call(p=p13, E=8, H=256, I=128, M=64, gs_in=FAKE, hbf=None, amax=FAKE, codes=FAKE, scales=FAKE,
             gs_out=None, y=FAKE, sync=FAKE, nbytes=need):
        return f(*p, E, H, I, M, gs_in, hbf, amax, codes, scales, gs_out, y, sync, nbytes, None)

    assert call(H=384) == -2                         # H not a multiple of 256
    assert call(I=96) == -2                          # I not a multiple of 128
    assert call(E=0) == -2
    assert call(M=-1) == -2
    assert call(nbytes=need - 1) == -3               # sync too small
    assert call(sync=None) == -1
    assert call(amax=None) == -1
    assert call(gs_in=None) == -1                    # neither a calibrated scale nor h_gs_out
    assert call(gs_in=None, gs_out=FAKE) == -1       # no calibrated scale: h_bf16 required
    assert call(codes=None) == -1
    assert call(y=None) == -1
    pn = list(p13)
    pn[10] = None                                    # w2_codes
    assert call(p=pn) == -1
    pr = list(p13)
    pr[0] = pr[1] = pr[3] = None                     # x_codes, x_scales, row_token
    assert call(p=pr) == -1                          # rows present: required
    assert call(p=pr, M=0, codes=None, scales=None, y=None, sync=FAKE, amax=None) == -1  # amax still required


def test_ffn_error_word_matches_header():
    src = open(HEADER).read()
    assert re.search(rf"#define MEGAMOE_FFN_SYNC_ERROR_WORD {mm.FFN_SYNC_ERROR_WORD}\b", src)


def test_combine_rejects_bad_args(lib):
    f = lib.moe_combine
    assert f(FAKE, FAKE, FAKE, 4, 0, 256, FAKE, None) == -2
    assert f(FAKE, FAKE, FAKE, 4, 6, 12, FAKE, None) == -2
    assert f(None, FAKE, FAKE, 4, 6, 256, FAKE, None) == -1


def test_dense_nvfp4_rejects_bad_args(lib):
    f = lib.nvfp4_linear_gate_up_silu_nvfp4
    need = mm.megamoe_dense_workspace_bytes(4)
    assert f(FAKE, FAKE, FAKE, 4, 200, FAKE, FAKE, FAKE, 128, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == -2  # K
    assert f(FAKE, FAKE, FAKE, 4, 256, FAKE, FAKE, FAKE, 100, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == -2  # I
    assert f(FAKE, FAKE, FAKE, 4, 256, FAKE, FAKE, FAKE, 128, None, FAKE, FAKE, FAKE, FAKE, need, None) == -1  # h_gs
    assert f(FAKE, FAKE, FAKE, 4, 256, FAKE, FAKE, FAKE, 128, FAKE, None, FAKE, FAKE, FAKE, need, None) == -1  # codes
    assert f(FAKE, FAKE, FAKE, 4, 256, FAKE, FAKE, FAKE, 128, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == -3


def test_probe_lib_exports_and_rejects_bad_args():
    """bench.py's measurement kernels (csrc/probe.hip): the library loads, exports its entry points
    and rejects bad arguments before any launch (no GPU is touched)."""
    from nvfp4_block_scaled_top_amd import build_lib

    if not os.path.exists(build_lib.PROBE_LIB_PATH):
        pytest.skip("libmegamoe_probe.so not built")
    h = ctypes.CDLL(build_lib.PROBE_LIB_PATH)
    h.megamoe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    h.megamoe_probe_placement.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    fake = ctypes.c_void_p(16)  # never dereferenced: the checks fail first
    assert h.megamoe_probe_read(None, 1024, 0, 512, 1, fake, None) == -1        # null buffer
    assert h.megamoe_probe_read(fake, 1000, 0, 512, 1, fake, None) == -1        # bytes % 16
    assert h.megamoe_probe_read(fake, 1024, 3, 512, 1, fake, None) == -1        # order
    assert h.megamoe_probe_read(fake, 1024, 0, 500, 1, fake, None) == -1        # grid % 8
    assert h.megamoe_probe_read(fake, 1024, 0, 512, 2, fake, None) == -1        # unroll
    assert h.megamoe_probe_placement(fake, 513, None) == -1                     # grid > 512
    assert h.megamoe_probe_placement(None, 512, None) == -1
    h.megamoe_probe_gemm_stream.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p]
    need = 9 * 4096 * 3584
    assert h.megamoe_probe_gemm_stream(fake, need - 16, 9, 0, fake, None) == -1   # buffer too small
    assert h.megamoe_probe_gemm_stream(fake, need, 9, 3, fake, None) == -1        # pattern
    assert h.megamoe_probe_gemm_stream(fake, need, 0, 0, fake, None) == -1        # experts
    assert h.megamoe_probe_gemm_stream(None, need, 9, 1, fake, None) == -1


def test_build_spill_check_parses_remarks():
    """The build refuses kernels that spill: it reads the compiler's resource-usage remarks."""
    from nvfp4_block_scaled_top_amd import build_lib
    text = ("a.hip:1:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]\n"
            "a.hip:1:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]\n"
            "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 1028 [-Rpass-analysis=kernel-resource-usage]\n"
            "b.hip:9:1: remark: Function Name: _Z1jv [-Rpass-analysis=kernel-resource-usage]\n"
            "b.hip:9:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n")
    assert build_lib.kernel_scratch(text) == {"_Z1kv": 1028, "_Z1jv": 0}
