"""Pins for the CPU oracle: each test checks the oracle against something other than itself.

Kinds of pin used here: exhaustive brute force with exact rational arithmetic
(``fractions.Fraction``), library routines for the number formats
(``torch.float8_e4m3fn`` casts, ``torch.bfloat16`` casts), closed forms and
invariants, the pages' printed numbers (``tests/golden``), and the seed-0
routing statistics of the synthetic workloads.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from nvfp4_block_scaled_top_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            vals[k] = float(v)
    return vals


# ---------------------------------------------------------------------------
# brute-force references (exact rationals, no shared code with the oracle)
# ---------------------------------------------------------------------------

def e4m3_fraction(code):
    """E4M3FN value from its bit fields, as an exact Fraction (finite codes only)."""
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return Fraction(m, 512)
    return Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


E4M3_FR = [e4m3_fraction(c) for c in range(0x7F)]
E2M1_FR = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def brute_nearest(value, grid):
    """Index of the grid point nearest to value; ties to the even index; beyond the end -> last."""
    best = None
    for i, g in enumerate(grid):
        d = abs(value - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0 and best[1] % 2 == 1):
            best = (d, i)
    return best[1]


def brute_block_scale(amax_b, gs):
    v = Fraction(float(amax_b)) * Fraction(float(gs)) / 6
    if v > E4M3_FR[-1]:
        return 0x7E
    return brute_nearest(v, E4M3_FR)


def brute_code(x, gs, s_code):
    s = E4M3_FR[s_code]
    if s == 0:
        mag = 0
    else:
        a = abs(Fraction(float(x))) * Fraction(float(gs))
        mag = brute_nearest(a, [g * s for g in E2M1_FR])
    return (8 if math.copysign(1.0, float(x)) < 0 else 0) | mag


def bf16_values(rng, n, scale=1.0):
    return O.bf16_round(rng.standard_normal(n) * scale)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3fn_value(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert O.E4M3_GRID[-1] == 448.0 and np.all(np.diff(O.E4M3_GRID) > 0)


def test_e2m1_decode_matches_bitfields():
    # E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal (m * 0.5).
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        assert O.e2m1_value(c) == (-mag if s else mag)


# ---------------------------------------------------------------------------
# byte layout: literal bytes written out by hand (tests/golden/nvfp4_layout_literal.txt)
# ---------------------------------------------------------------------------

def read_layout_literal():
    rows = {}
    with open(os.path.join(GOLDEN, "nvfp4_layout_literal.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key.startswith("x"):
                rows[key] = np.array([float(v) for v in vals])
            elif key == "gs":
                rows[key] = float(vals[0])
            else:
                rows[key] = [int(v, 16) for v in vals]
    return rows


def test_pack_nibbles_literal_bytes():
    """The even element goes in the low nibble: codes (1, 2, 0xF, 0x8) are the bytes 0x21, 0x8F."""
    assert O.pack_nibbles(np.array([[1, 2, 0xF, 0x8]], np.uint8)).tolist() == [[0x21, 0x8F]]
    assert O.unpack_nibbles(np.array([[0x21, 0x8F]], np.uint8)).tolist() == [[1, 2, 0xF, 0x8]]
    # a byte's low nibble is element 0 of the pair after decoding as well
    assert O.dequantize_blocks(np.array([[0x71] + [0] * 7], np.uint8), np.array([[0x38]], np.uint8))[0, :2].tolist() \
        == [0.5, 6.0]  # scale 0x38 = 1.0


def test_hand_built_tensor_bytes():
    """The quantizer reproduces bytes worked out by hand from the format's definition (codes with
    exact ties, -0, a zero block, block scales 448 / 112 / 224 / 0, gs = 448)."""
    g = read_layout_literal()
    x = np.stack([g["x0"], g["x1"]])
    assert np.signbit(x[0, 15]) and np.signbit(x[1, 31])  # "-0" is -0.0
    codes, scales, gs = O.quantize_nvfp4(x)
    assert float(gs) == g["gs"]
    assert codes.tolist() == [g["codes0"], g["codes1"]]
    assert scales.tolist() == [g["scales0"], g["scales1"]]
    # decoding the bytes: row 0 lies on its blocks' grids, row 1's ties went to the even code
    dec = O.dequantize_blocks(codes, scales) / float(gs)
    assert np.array_equal(dec[0], x[0])
    assert dec[1, :16].tolist() == [3, 1, 0.25, 0.75, -2, 0.5, 1, 0, 0.5, 2, 2, 0, -1, -0.5, 0.5, -3]
    assert not dec[1, 16:].any()


def test_decode_products_exact_in_f16_and_bf16():
    """Every E2M1 x finite E4M3 product is exact in fp16 and bf16 (why the GPU decodes to fp16)."""
    prods = (O.E2M1_MAGNITUDES[:, None] * O.E4M3_GRID[None, :]).ravel()
    assert np.array_equal(prods.astype(np.float16).astype(np.float64), prods)
    assert np.array_equal(O.bf16_round(prods), prods)
    # and they are normal fp16 numbers (no fp16 subnormal reaches the MFMA)
    nz = prods[prods > 0]
    assert nz.min() >= 2.0 ** -14 and nz.max() <= 2688.0
    # whereas E4M3 itself cannot hold them all (an FP8 MFMA would round)
    e4 = torch.tensor(prods, dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.sum(e4 != prods) > 0


def test_bf16_round_matches_torch_on_float32():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(200000) * np.exp2(rng.integers(-30, 30, 200000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(v.astype(np.float64)), ref)


def test_bf16_round_ties_and_float64_bruteforce():
    rng = np.random.default_rng(2)
    base = O.bf16_round(rng.standard_normal(300))
    ulp = np.exp2(np.frexp(base)[1] - 8.0)
    ties = base + ulp / 2  # exact midpoints between bf16 neighbours
    offs = base + ulp * rng.uniform(-0.49, 0.49, 300)
    for v in np.concatenate([ties, offs]):
        f = Fraction(float(v))
        m, e = math.frexp(float(v))
        q = Fraction(2) ** (e - 8)
        lo = (f / q).__floor__()
        cand = [lo * q, (lo + 1) * q]
        d0, d1 = abs(f - cand[0]), abs(f - cand[1])
        want = cand[0] if d0 < d1 or (d0 == d1 and lo % 2 == 0) else cand[1]
        assert Fraction(float(O.bf16_round(v))) == want


# ---------------------------------------------------------------------------
# quantizer
# ---------------------------------------------------------------------------

def test_e4m3_round_matches_torch_cast():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.uniform(0, 448, 100000),
        rng.uniform(0, 2 ** -6, 20000),
        (O.E4M3_GRID[:-1] + O.E4M3_GRID[1:]) / 2,  # every midpoint: ties
        O.E4M3_GRID,
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_round_sat(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_global_scale_is_correctly_rounded():
    rng = np.random.default_rng(4)
    for a in np.concatenate([bf16_values(rng, 2000, 1.0), [1.27, 8.0, 2.0 ** -20, 300.0]]):
        a = float(O.bf16_round(abs(a)))
        if a == 0:
            continue
        gs = O.global_scale(a)
        exact = Fraction(2688) / Fraction(a)
        f = Fraction(float(gs))
        # no float32 is closer to the exact quotient
        up = Fraction(float(np.nextafter(gs, np.float32(np.inf))))
        dn = Fraction(float(np.nextafter(gs, np.float32(0))))
        assert abs(f - exact) <= abs(up - exact) and abs(f - exact) <= abs(dn - exact)
    assert O.global_scale(0.0) == np.float32(1.0)


def test_block_scale_bruteforce_random_and_ties():
    rng = np.random.default_rng(5)
    amaxes = np.abs(bf16_values(rng, 3000, 0.3))
    gss = np.array([O.global_scale(float(a) * 1.7 + 1e-3) for a in amaxes], dtype=np.float32)
    got = O.block_scale_codes(amaxes, gss)
    for a, g, c in zip(amaxes, gss, got):
        assert c == brute_block_scale(a, g)
    # exact ties: amax_b * gs / 6 equal to a midpoint of the E4M3 grid (gs a power of two)
    mids = (O.E4M3_GRID[:-1] + O.E4M3_GRID[1:]) / 2
    for mid in mids:
        a = 6 * mid / 4.0
        assert O.bf16_round(a) == a
        c = O.block_scale_codes(np.array([a]), np.float32(4.0))[0]
        assert c == brute_block_scale(a, np.float32(4.0))
        assert c % 2 == 0  # ties go to the even code
    # saturation above 448
    assert O.block_scale_codes(np.array([1000.0]), np.float32(6.0))[0] == 0x7E


def test_element_codes_bruteforce_random_and_ties():
    rng = np.random.default_rng(6)
    for trial in range(60):
        x = bf16_values(rng, 64, 0.09)
        if trial % 3 == 0:
            x[rng.integers(0, 64, 4)] = -0.0
        codes, scales, gs = O.quantize_nvfp4(x.reshape(4, 16))
        c = O.unpack_nibbles(codes).reshape(-1)
        for i, xv in enumerate(x):
            assert c[i] == brute_code(xv, gs, scales.reshape(-1)[i // 16])
    # exact ties between E2M1 grid points: x * gs = mid * s with gs = 1
    for s_code in (0x30, 0x38, 0x3B, 0x41, 0x01, 0x07):
        s = O.E4M3_GRID[s_code]
        for mid in O.E2M1_MIDPOINTS:
            for sign in (1.0, -1.0):
                xv = sign * mid * s
                assert O.bf16_round(xv) == xv
                got = O.e2m1_codes(np.array([xv]), np.float32(1.0), np.array([s]))[0]
                assert got == brute_code(xv, np.float32(1.0), s_code)
                assert (got & 7) % 2 == 0
    # a zero block scale gives code magnitude 0; the sign bit follows x
    assert O.e2m1_codes(np.array([-1e-9]), np.float32(1.0), np.array([0.0]))[0] == 0x8


def test_amax_block_closed_form():
    """The block holding the tensor amax gets scale 448 (0x7E) and that element encodes as +-6."""
    rng = np.random.default_rng(7)
    for _ in range(20):
        x = bf16_values(rng, 32 * 64, 0.09).reshape(32, 64)
        codes, scales, gs = O.quantize_nvfp4(x)
        r, k = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert scales[r, k // 16] == 0x7E
        assert O.unpack_nibbles(codes)[r, k] & 7 == 7
        assert scales.max() <= 0x7E


def test_scaling_invariance():
    rng = np.random.default_rng(8)
    x = bf16_values(rng, 16 * 128, 0.09).reshape(16, 128)
    c0, s0, g0 = O.quantize_nvfp4(x)
    for k in (-3, -1, 1, 4):
        c1, s1, g1 = O.quantize_nvfp4(x * 2.0 ** k)
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
        assert float(g1) == float(g0) * 2.0 ** -k


def test_sign_symmetry():
    rng = np.random.default_rng(9)
    x = bf16_values(rng, 8 * 64, 0.09).reshape(8, 64)
    x[x == 0] = 0.5  # avoid +-0 ambiguity
    c0, s0, g0 = O.quantize_nvfp4(x)
    c1, s1, g1 = O.quantize_nvfp4(-x)
    assert np.array_equal(c0 ^ 0x88, c1) and np.array_equal(s0, s1) and g0 == g1


def test_reconstruction_within_half_grid_step():
    rng = np.random.default_rng(10)
    x = bf16_values(rng, 64 * 256, 0.09).reshape(64, 256)
    codes, scales, gs = O.quantize_nvfp4(x)
    deq = O.dequantize_blocks(codes, scales)
    s = np.repeat(O.e4m3fn_value(scales), 16, axis=1)
    a = np.abs(x) * float(gs)
    mag = np.abs(deq) / np.where(s == 0, 1, s)
    steps = np.diff(O.E2M1_MAGNITUDES)
    idx = np.searchsorted(O.E2M1_MAGNITUDES, mag)
    half_gap = np.where(idx < 7, steps[np.minimum(idx, 6)], steps[-1]) / 2
    half_gap = np.maximum(half_gap, np.where(idx > 0, steps[np.maximum(idx - 1, 0)], 0) / 2)
    err = np.abs(a - np.abs(deq))
    sat = a > 6 * s
    assert np.all(err[~sat] <= half_gap[~sat] * s[~sat] * (1 + 1e-12))
    assert np.all(np.sign(deq[deq != 0]) == np.sign(x[deq != 0]))


def test_invalid_rows_zero_and_excluded_from_amax():
    rng = np.random.default_rng(11)
    x = bf16_values(rng, 6 * 32, 0.09).reshape(6, 32)
    x[2] = 100.0  # large but invalid: must not move gs
    valid = np.array([1, 1, 0, 1, 0, 1], bool)
    c, s, gs = O.quantize_nvfp4(x, valid)
    assert gs == O.global_scale(float(np.abs(x[valid]).max()))
    assert np.all(c[~valid] == 0) and np.all(s[~valid] == 0)
    cz, sz, gz = O.quantize_nvfp4(np.zeros((3, 32)))
    assert gz == 1.0 and np.all(sz == 0) and np.all((cz & 0x77) == 0)


def test_overflow_contrast_pages_numbers():
    """The pages' overflow: a checkpoint global scale 1/input_scale applied to amax 1.27-8."""
    g = read_golden("overflow_evidence.txt")
    inv_qa = 1.0 / g["q_a_proj_input_scale"]
    inv_qb = 1.0 / g["q_b_proj_input_scale"]
    assert abs(inv_qa - g["q_a_proj_inv_printed"]) < 0.05
    # the printed 16287.1 is the reciprocal of the scale before it was rounded to 4 digits
    assert abs(inv_qb - g["q_b_proj_inv_printed"]) < 1.0
    for amax, want in ((g["embedding_amax"], 842), (g["activation_amax_low"], 1326), (g["activation_amax_high"], 5303)):
        block_scale = amax * inv_qa / 6
        assert round(block_scale) == want and block_scale > O.E4M3_MAX
        assert torch.isnan(torch.tensor([block_scale], dtype=torch.float32).to(torch.float8_e4m3fn).float()).all()
    # no-overflow threshold under the checkpoint scale: amax <= 448*6/3977.6 = 0.676
    assert abs(O.GLOBAL_SCALE_NUMERATOR / inv_qa - 0.676) < 1e-3
    # the amax-derived global scale never exceeds E4M3, even with +-8 outliers
    w = synth.WORKLOADS[4]
    x = np.random.default_rng(12).standard_normal((8, 256)) * g["embedding_std"]
    x[0, 3], x[5, 100] = g["activation_amax_high"], -g["activation_amax_high"]
    x = O.bf16_round(x)
    c, s, gs = O.quantize_nvfp4(x)
    assert s.max() == 0x7E and not np.isnan(O.e4m3fn_value(s)).any()
    assert w.outliers


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E,e0,P", [(16, 2, 8, 0, 1), (50, 6, 48, 0, 1), (37, 6, 24, 100, 128),
                                        (1, 6, 48, 0, 1), (0, 6, 8, 0, 4), (200, 4, 7, 3, 5)])
def test_route_matches_sorted(T, k, E, e0, P):
    rng = np.random.default_rng(T * 7 + k)
    Eg = max(E + e0 + 20, k)
    ids = np.array([rng.permutation(Eg)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
    counts, eoff, poff, row_token, token_rows = O.route(ids, e0, E, P)
    # brute force: sort local assignments by (expert, token, j)
    local = sorted((int(ids[t, j]) - e0, t, j) for t in range(T) for j in range(k) if e0 <= ids[t, j] < e0 + E)
    assert int(counts.sum()) == len(local)
    seen = {}
    for e, t, j in local:
        r = poff[e] + seen.get(e, 0)
        seen[e] = seen.get(e, 0) + 1
        assert row_token[r] == t and token_rows[t, j] == r
    assert np.all(np.diff(eoff) == counts) and eoff[0] == 0
    assert np.all(np.diff(poff) == (counts + P - 1) // P * P)
    assert len(row_token) == T * k + E * (P - 1)
    nonlocal_mask = (ids < e0) | (ids >= e0 + E)
    assert np.all(token_rows[nonlocal_mask] == -1)
    valid = row_token >= 0
    assert valid.sum() == len(local)
    # inverse maps agree
    tr = token_rows[token_rows >= 0]
    assert np.array_equal(np.sort(tr), np.sort(np.nonzero(valid)[0]))


# ---------------------------------------------------------------------------
# GEMMs, SiLU, combine
# ---------------------------------------------------------------------------

def test_expert_matmul_bruteforce_fractions():
    rng = np.random.default_rng(13)
    a = O.bf16_round(rng.standard_normal((3, 32)) * 0.1)
    w = O.bf16_round(rng.standard_normal((8, 32)) * 0.02)
    ac, as_, ag = O.quantize_nvfp4(a)
    wc, ws, wg = O.quantize_nvfp4(w)
    ad, wd = O.dequantize_blocks(ac, as_), O.dequantize_blocks(wc, ws)
    got = O.expert_matmul(ad, wd, ag, wg)
    # exact rational dot products from codes and scales, decoded independently
    acodes, wcodes = O.unpack_nibbles(ac), O.unpack_nibbles(wc)

    def dec(code, sc):
        mag = E2M1_FR[code & 7] * E4M3_FR[sc]
        return -mag if code & 8 else mag

    for i in range(3):
        for n in range(8):
            s = sum(dec(int(acodes[i, k]), int(as_[i, k // 16])) * dec(int(wcodes[n, k]), int(ws[n, k // 16]))
                    for k in range(32))
            exact = s / (Fraction(float(ag)) * Fraction(float(wg)))
            assert abs(got[i, n] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def test_silu_identities():
    z = np.linspace(-30, 30, 1201)
    s = O.silu(z)
    assert np.allclose(s - O.silu(-z), z, rtol=0, atol=1e-12)  # z*sig(z) - (-z)*sig(-z) = z
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - 1 / (1 + math.exp(-1))) < 1e-15
    assert O.silu(np.array([-1000.0]))[0] == 0.0
    acc = np.array([[2.0, -1.0, 3.0, 0.5]])  # gate = [2, -1], up = [3, 0.5]
    assert np.allclose(O.silu_mul(acc), [[O.silu(2.0) * 3.0, O.silu(-1.0) * 0.5]])


def _tiny_layer_inputs(seed=0, E=4, k=2, H=64, I=64, T=10, e0=0, Eg=None, P=1, identical=False):
    rng = np.random.default_rng(seed)
    Eg = Eg or E
    ids = np.stack([rng.permutation(Eg)[:k] for _ in range(T)]).astype(np.int32)
    wts = rng.uniform(0.05, 0.5, (T, k)).astype(np.float32)
    x = O.bf16_round(rng.standard_normal((T, H)) * 0.09)
    W13, W2 = [], []
    for e in range(E):
        r = np.random.default_rng(1000 + (0 if identical else e))
        W13.append(O.bf16_round(r.standard_normal((2 * I, H)) * 0.02))
        W2.append(O.bf16_round(r.standard_normal((H, I)) * 0.02))
    q13 = [O.quantize_nvfp4(w) for w in W13]
    q2 = [O.quantize_nvfp4(w) for w in W2]
    return dict(x=x, topk_ids=ids, topk_weights=wts, expert_begin=e0, num_experts=E, pad_multiple=P,
                w13_codes=np.stack([q[0] for q in q13]), w13_scales=np.stack([q[1] for q in q13]),
                w13_gs=np.array([q[2] for q in q13], np.float32),
                w2_codes=np.stack([q[0] for q in q2]), w2_scales=np.stack([q[1] for q in q2]),
                w2_gs=np.array([q[2] for q in q2], np.float32))


def test_layer_dense_special_case():
    """E=1, k=1, weight 1: the layer is a dense NVFP4 MLP and out == y row for row."""
    inp = _tiny_layer_inputs(E=1, k=1, T=7)
    inp["topk_weights"][:] = 1.0
    r = O.moe_layer(**inp)
    assert np.array_equal(r["out"], r["y"][r["token_rows"][:, 0]])
    # and y is that of a dense MLP computed step by step
    xd = O.dequantize_blocks(r["x_codes"], r["x_scales"])
    w13 = O.dequantize_blocks(inp["w13_codes"][0], inp["w13_scales"][0])
    h = O.bf16_round(O.silu_mul(xd @ w13.T / (float(r["gs_x"]) * float(inp["w13_gs"][0]))))
    assert np.array_equal(h, r["h"][r["token_rows"][:, 0]])


def test_layer_identical_experts():
    """Identical experts: out = bf16(sum_j w_j * y) with the same y for every slot."""
    inp = _tiny_layer_inputs(E=4, k=3, T=9, identical=True)
    r = O.moe_layer(**inp)
    y0 = r["y"][r["token_rows"][:, 0]]
    for j in range(3):
        assert np.array_equal(r["y"][r["token_rows"][:, j]], y0)
    want = O.bf16_round(inp["topk_weights"].astype(np.float64).sum(1, keepdims=True) * y0)
    ulp = np.exp2(np.frexp(want)[1] - 8.0)
    assert np.all(np.abs(r["out"] - want) <= ulp)


def test_zero_token_experts_are_never_read():
    inp = _tiny_layer_inputs(E=6, k=2, T=3, Eg=6, seed=3)
    r0 = O.moe_layer(**inp)
    empty = np.nonzero(r0["counts"] == 0)[0]
    assert len(empty) > 0
    for e in empty:
        inp["w13_scales"][e] = 0x7F  # NaN block scales
        inp["w2_scales"][e] = 0x7F
        inp["w13_gs"][e] = np.nan
    r1 = O.moe_layer(**inp)
    assert np.array_equal(r0["out"], r1["out"]) and not np.isnan(r1["out"]).any()


def test_weights_applied_once():
    inp = _tiny_layer_inputs(E=4, k=2, T=8, seed=4)
    r1 = O.moe_layer(**inp)
    inp["topk_weights"] = inp["topk_weights"] * np.float32(2)
    r2 = O.moe_layer(**inp)
    assert np.array_equal(r2["out"], 2 * r1["out"])
    assert np.array_equal(r2["y"], r1["y"])


def test_nonlocal_tokens_are_plus_zero():
    inp = _tiny_layer_inputs(E=4, k=2, T=12, Eg=10, e0=3, seed=5)
    r = O.moe_layer(**inp)
    none = np.all(r["token_rows"] < 0, axis=1)
    assert none.any()
    assert np.all(O.bf16_bits(r["out"][none]) == 0)


@pytest.mark.parametrize("P", [3, 4, 128])
def test_padded_layer_equals_unpadded(P):
    """Padding each expert's rows to a multiple of P (padded_expert_offsets, CURRENT_BUG.md@2e65594
    "Test Plan" Phase 2) moves rows, never values: with a local share starting at e0 > 0, out is
    bitwise that of P = 1, every assignment's h and y row is the unpadded run's row, gs_h is the
    same, and padded rows hold -1 / zero codes / zero scales."""
    base = _tiny_layer_inputs(E=5, k=2, T=13, Eg=9, e0=2, seed=11)
    r1 = O.moe_layer(**base)
    rP = O.moe_layer(**dict(base, pad_multiple=P))
    counts = rP["counts"]
    assert np.array_equal(counts, r1["counts"]) and counts.sum() > 0
    assert np.array_equal(rP["padded_offsets"], np.concatenate([[0], np.cumsum((counts + P - 1) // P * P)]))
    assert not np.array_equal(rP["padded_offsets"], rP["expert_offsets"])  # padding is really there
    assert np.array_equal(rP["out"], r1["out"])
    assert float(rP["gs_h"]) == float(r1["gs_h"])
    t1, tP = r1["token_rows"], rP["token_rows"]
    assert np.array_equal(t1 >= 0, tP >= 0)
    m = t1 >= 0
    for key in ("h", "y", "h_codes", "h_scales"):
        assert np.array_equal(rP[key][tP[m]], r1[key][t1[m]])
    pad = rP["row_token"] < 0
    assert pad.sum() == len(rP["row_token"]) - counts.sum()
    assert not rP["h"][pad].any() and not rP["y"][pad].any()
    assert not rP["h_codes"][pad].any() and not rP["h_scales"][pad].any()


def test_padded_rows_are_never_read():
    """L1 reads only rows padded_offsets[e] .. + counts[e] of each expert, through row_token, and
    L2 only those rows of h: poisoning every padding row (NaN block scales, -1 tokens) changes
    nothing."""
    inp = _tiny_layer_inputs(E=5, k=2, T=13, Eg=9, e0=2, seed=12, P=8)
    r = O.moe_layer(**inp)
    pad = r["row_token"] < 0
    assert pad.any()
    hc, hs = r["h_codes"].copy(), r["h_scales"].copy()
    hc[pad], hs[pad] = 0xFF, 0x7F
    y = O.moe_l2(hc, hs, r["gs_h"], r["padded_offsets"], r["counts"], inp["w2_codes"], inp["w2_scales"],
                 inp["w2_gs"])
    assert np.array_equal(y, r["y"])
    # padding rows of row_token pointed at a poisoned extra token row of x are not followed either
    T = r["x_codes"].shape[0]
    xc = np.concatenate([r["x_codes"], np.full((1, r["x_codes"].shape[1]), 0xFF, np.uint8)])
    xs = np.concatenate([r["x_scales"], np.full((1, r["x_scales"].shape[1]), 0x7F, np.uint8)])
    rt = np.where(pad, T, r["row_token"]).astype(np.int32)
    h, amax = O.moe_l1(xc, xs, r["gs_x"], rt, r["padded_offsets"], r["counts"],
                       inp["w13_codes"], inp["w13_scales"], inp["w13_gs"])
    assert np.array_equal(h, r["h"]) and amax == r["amax_h"]


def test_decode_t1_has_no_local_work():
    w = synth.WORKLOADS[1]
    ids, _ = O.router_topk(synth.router_logits(w, 1), w.top_k)
    counts, *_ = O.route(ids, w.expert_begin, w.num_experts, w.pad_multiple)
    assert counts.sum() == 0


# ---------------------------------------------------------------------------
# generator recipe and the pages' shapes
# ---------------------------------------------------------------------------

def test_generator_seed0_statistics():
    def counts(i, T):
        w = synth.WORKLOADS[i]
        ids, _ = O.router_topk(synth.router_logits(w, T), w.top_k)
        loc = ids[(ids >= w.expert_begin) & (ids < w.expert_begin + w.num_experts)] - w.expert_begin
        return np.bincount(loc, minlength=w.num_experts)

    c0 = counts(0, 16)
    assert c0.tolist() == [3, 6, 3, 3, 4, 4, 5, 4]
    _, wts = O.router_topk(synth.router_logits(synth.WORKLOADS[0], 16), 2)
    assert abs(wts[0, 0] - 0.3327) < 5e-5 and abs(wts[0, 1] - 0.1985) < 5e-5
    assert [counts(1, T).sum() for T in (1, 4, 8)] == [0, 5, 10]
    assert (counts(1, 8) > 0).sum() == 9
    c2 = counts(2, 512)
    assert (c2 == 0).sum() == 0 and c2.max() == 16 and c2.min() == 2 and np.median(c2) == 8
    c3 = counts(3, 8192)
    assert (c3 == 0).sum() == 261
    assert sorted(c3.tolist())[::-1][:10] == [7916, 6874, 5726, 4670, 3758, 3029, 2493, 2121, 1728, 1396]
    assert ((c3 >= 1) & (c3 <= 15)).sum() == 69
    c4 = counts(4, 16384)
    assert (c4 == 0).sum() == 245 and c4.max() == 15843


def test_generator_activations_distribution():
    g = read_golden("overflow_evidence.txt")
    w = synth.WORKLOADS[3]
    x = synth.bf16_bits_to_f32(synth.activations(w, 64))
    assert abs(x.std() - g["embedding_std"]) < 2e-3
    assert np.abs(x).max() <= g["embedding_amax"]
    w4 = synth.WORKLOADS[4]
    x4 = synth.bf16_bits_to_f32(synth.activations(w4, 16))
    assert (np.abs(x4) == 8.0).sum() == 16 * w4.hidden // 1000


def test_workloads_follow_pages_shapes():
    g = read_golden("megamoe_shapes.txt")
    for i in (1, 2, 3, 4):
        w = synth.WORKLOADS[i]
        assert w.num_experts_global == g["num_experts"] and w.top_k == g["top_k"]
    w1 = synth.WORKLOADS[1]
    assert w1.num_experts == g["num_experts"] / g["ep_degree"] == g["ep_local_experts"]
    assert max(w1.tokens) == g["decode_tokens_max"]
    assert synth.WORKLOADS[2].pad_multiple == g["pad_multiple"]


# ---------------------------------------------------------------------------
# router: softmax over all experts, top-k, ties to the lower index
# ---------------------------------------------------------------------------

def _router_brute(row, k):
    """Independent reference: order by (-logit, index) on Python floats, probabilities from
    math.exp and an exactly rounded sum (math.fsum)."""
    vals = [float(v) for v in np.asarray(row, np.float32)]
    m = max(vals)
    ex = [math.exp(v - m) for v in vals]
    s = math.fsum(ex)
    order = sorted(range(len(vals)), key=lambda j: (-vals[j], j))[:k]
    return order, [np.float32(ex[j] / s) for j in order]


@pytest.mark.parametrize("T,E,k,seed", [(40, 7, 3, 0), (25, 64, 6, 1), (9, 384, 6, 2), (5, 130, 130, 3)])
def test_router_matches_brute_force(T, E, k, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32) * np.float32(2.5)
    logits[0, : min(4, E)] = logits[0, 0]          # exact ties in one row
    logits[1, -1] = logits[1].max()                 # a tie for the maximum at the highest index
    ids, w = O.router_topk(logits, k)
    assert ids.dtype == np.int32 and w.dtype == np.float32 and ids.shape == (T, k) == w.shape
    for t in range(T):
        order, ref = _router_brute(logits[t], k)
        assert ids[t].tolist() == order
        # float64 sums in different orders may differ in the last bit, which can move a float32
        # rounding by one unit at most
        np.testing.assert_allclose(w[t], np.array(ref, np.float32), rtol=2.0 ** -23, atol=0)


def test_router_invariants():
    rng = np.random.default_rng(7)
    # logits on a 2^-10 grid, so that adding 4.0 below is exact in float32
    logits = (np.round(rng.standard_normal((64, 48)) * 1024) / 1024).astype(np.float32)
    ids, w = O.router_topk(logits, 48)                       # k = E: the full softmax, sorted
    assert np.all(np.sort(ids, axis=1) == np.arange(48))
    assert np.all(np.diff(w, axis=1) <= 0) and np.all(w > 0)
    np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), 1.0, rtol=1e-6)
    ids6, w6 = O.router_topk(logits, 6)                      # not renormalised: a prefix of the full list
    assert np.array_equal(ids6, ids[:, :6]) and np.array_equal(w6, w[:, :6])
    assert np.all(w6.sum(axis=1) < 1)
    ids_s, w_s = O.router_topk(logits + np.float32(4.0), 6)   # shift invariance
    assert np.array_equal(ids_s, ids6)
    np.testing.assert_allclose(w_s, w6, rtol=2.0 ** -22)
    flat = np.full((3, 10), 0.25, np.float32)                # all equal: the k lowest indices, 1/E each
    ids_f, w_f = O.router_topk(flat, 4)
    assert np.all(ids_f == np.arange(4)) and np.all(w_f == np.float32(0.1))


def test_router_order_survives_underflow():
    """Far below the largest logit the float64 probabilities all underflow to 0; the order stays
    that of the logits (the exact probabilities'), not the index order of equal zeros."""
    logits = np.array([[0.0, -900.0, -800.0, -1000.0, -850.0]], np.float32)
    ids, w = O.router_topk(logits, 4)
    assert ids.tolist() == [[0, 2, 4, 1]]
    assert w[0, 0] == 1 and np.all(w[0, 1:] == 0)


def test_router_large_logits_do_not_overflow():
    logits = np.array([[1000.0, 999.0, -1000.0, 998.0]], np.float32)
    ids, w = O.router_topk(logits, 2)
    assert ids.tolist() == [[0, 1]]
    e = [math.exp(0.0), math.exp(-1.0), math.exp(-2000.0), math.exp(-2.0)]
    np.testing.assert_allclose(w[0], np.array([e[0], e[1]]) / math.fsum(e), rtol=2.0 ** -23)


# ---------------------------------------------------------------------------
# calibrated variant: a given global scale, saturating block scales and codes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("factor", [0.37, 4.0, 40.0])
def test_calibrated_quantizer_vs_brute_force(factor):
    rng = np.random.default_rng(int(factor * 100))
    x = O.bf16_round(rng.standard_normal((4, 64)) * 0.09)
    x[1, :16] = 0.0
    gs = np.float32(O.global_scale(float(np.abs(x).max())) * np.float32(factor))
    valid = np.array([True, True, False, True])
    codes, scales = O.quantize_rows_with_global_scale(x, gs, valid_rows=valid)
    unpacked = O.unpack_nibbles(codes)
    for r in range(4):
        for b in range(4):
            blk = x[r, 16 * b: 16 * b + 16]
            if not valid[r]:
                assert scales[r, b] == 0 and np.all(unpacked[r, 16 * b: 16 * b + 16] == 0)
                continue
            sc = brute_block_scale(np.abs(blk).max(), gs)
            assert scales[r, b] == sc
            for i, v in enumerate(blk):
                assert unpacked[r, 16 * b + i] == brute_code(v, gs, sc)
    if factor > 1:  # the scale is too large for the data: saturated blocks and elements occur
        assert (scales == 0x7E).sum() > 0 and (unpacked[valid.repeat(64).reshape(4, 64)] & 7 == 7).sum() > 0


def test_calibrated_equals_amax_derived_at_the_amax_scale():
    rng = np.random.default_rng(3)
    x = O.bf16_round(rng.standard_normal((6, 96)))
    c, s, gs = O.quantize_nvfp4(x)
    c2, s2 = O.quantize_rows_with_global_scale(x, gs)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


# ---------------------------------------------------------------------------
# dense NVFP4 linear layers, the shared expert and its term in the combine
# ---------------------------------------------------------------------------

def test_nvfp4_linear_bruteforce_fractions():
    """out = bf16 of the exact rational A.W^T / (gs_a gs_w), from codes and scales decoded here."""
    rng = np.random.default_rng(31)
    a = O.bf16_round(rng.standard_normal((3, 48)) * 0.1)
    w = O.bf16_round(rng.standard_normal((5, 48)) * 0.02)
    ac, as_, ag = O.quantize_nvfp4(a)
    wc, ws, wg = O.quantize_nvfp4(w)
    got = O.nvfp4_linear(ac, as_, ag, wc, ws, wg)
    acodes, wcodes = O.unpack_nibbles(ac), O.unpack_nibbles(wc)

    def dec(code, sc):
        mag = E2M1_FR[code & 7] * E4M3_FR[sc]
        return -mag if code & 8 else mag

    for i in range(3):
        for n in range(5):
            s = sum(dec(int(acodes[i, k]), int(as_[i, k // 16])) * dec(int(wcodes[n, k]), int(ws[n, k // 16]))
                    for k in range(48))
            exact = s / (Fraction(float(ag)) * Fraction(float(wg)))
            # bf16 of the exact value: the nearest of the two bf16 neighbours of float(exact)
            want = float(O.bf16_round(np.array([float(exact)]))[0])
            assert got[i, n] == want or abs(Fraction(got[i, n]) - exact) <= abs(Fraction(want) - exact)


def test_gate_up_silu_dense_is_the_single_expert_l1():
    inp = _tiny_layer_inputs(E=1, k=1, T=9, seed=8)
    r = O.moe_layer(**inp)
    h = O.nvfp4_linear_gate_up_silu(r["x_codes"], r["x_scales"], r["gs_x"], inp["w13_codes"][0],
                                    inp["w13_scales"][0], inp["w13_gs"][0])
    rows = r["token_rows"][:, 0]
    assert np.array_equal(h, r["h"][rows])


def test_shared_expert_equals_routed_single_expert():
    """A shared expert with expert 0's weights equals the routed layer's y when every token goes
    to expert 0 alone with weight 1 (E=1, k=1): same x codes, same h amax, same GEMMs."""
    inp = _tiny_layer_inputs(E=1, k=1, T=11, seed=9)
    inp["topk_weights"][:] = 1.0
    r = O.moe_layer(**inp)
    shared = tuple(inp[n][0] for n in ("w13_codes", "w13_scales", "w13_gs", "w2_codes", "w2_scales", "w2_gs"))
    ys, h, gs_h = O.shared_expert(r["x_codes"], r["x_scales"], r["gs_x"], *shared)
    rows = r["token_rows"][:, 0]
    assert np.array_equal(ys, r["y"][rows]) and gs_h == r["gs_h"]
    # with it as a shared expert on top of the same routing, out = bf16(y + y) = 2 y exactly
    r2 = O.moe_layer(**inp, shared=shared)
    assert np.array_equal(r2["out"], 2 * r["out"])


def test_combine_shared_term():
    rng = np.random.default_rng(10)
    y = O.bf16_round(rng.standard_normal((12, 32)))
    ys = O.bf16_round(rng.standard_normal((5, 32)))
    rows = np.array([[0, 3], [-1, 5], [-1, -1], [7, 8], [11, 2]], np.int32)
    w = rng.uniform(0.1, 0.5, (5, 2)).astype(np.float32)
    out = O.combine(y, rows, np.zeros_like(w), ys)
    assert np.array_equal(out, ys)  # zero routing weights: the shared output alone
    out = O.combine(y, rows, w, ys)
    for t in range(5):
        for c in range(32):
            s = Fraction(float(ys[t, c])) + sum(Fraction(float(w[t, j])) * Fraction(float(y[rows[t, j], c]))
                                                for j in range(2) if rows[t, j] >= 0)
            want = float(O.bf16_round(np.array([float(s)]))[0])
            assert out[t, c] == want or abs(Fraction(out[t, c]) - s) <= abs(Fraction(want) - s)
