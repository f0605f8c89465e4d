// Device code of the NVFP4 activation quantizer shared by quant.hip, the fused decode kernel in
// route.hip and the GEMM epilogues that write NVFP4 h (gemm.hip): block scale and element code
// rules (bit-exact with the real-number definition, see quant.hip), one 16-element block, and the
// single-launch small-tensor forms.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace megamoe {

__device__ __forceinline__ uint32_t bf16_abs_max8(u32x4 v) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = v[j] & 0x7FFFu, hi = (v[j] >> 16) & 0x7FFFu;
    m = m > lo ? m : lo;
    m = m > hi ? m : hi;
  }
  return m;
}

// E4M3FN code of the non-negative double q, round to nearest even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_code_rne(double q) {
  if (q >= 464.0) return 0x7Eu;
  if (q < 0.015625) return (uint32_t)rint(q * 512.0);  // subnormal grid m * 2^-9 (m = 8 is 2^-6)
  int ex;
  (void)frexp(q, &ex);  // q in [2^(ex-1), 2^ex)
  const int E = ex - 1;
  double mant = rint(ldexp(q, 3 - E));  // in [8, 16]
  int Eq = E;
  if (mant >= 16.0) {
    mant = 8.0;
    Eq += 1;
  }
  const uint32_t code = ((uint32_t)(Eq + 7) << 3) | ((uint32_t)mant - 8u);
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  return e == 0 ? (float)m * 0x1p-9f : ldexpf((float)(8u + m), (int)e - 10);
}

// 4-bit code of one element: sign of x, magnitude = nearest E2M1 index with ties to even.  The
// magnitude is the number of midpoints t[i] = m_i * s that x * gs passes (">=" where the tie goes
// up to the even code: 0.75, 1.75, 3.5; ">" elsewhere).  The thresholds increase, so passing one
// implies passing every lower one, and a binary search over them (3 tests instead of 7) gives the
// same count; each test is the sign of one exactly-rounded fma residual.
__device__ __forceinline__ uint32_t e2m1_code(uint32_t xbits, float gs, const float t[7], bool zero_scale) {
  const float a = bf16_bits_to_f32(xbits & 0x7FFFu);
  uint32_t mag = 0;
  if (!zero_scale) {
    const bool b2 = fmaf(a, gs, -t[3]) >= 0.0f;                     // >= 1.75 s: magnitude >= 4
    const bool b1 = fmaf(a, gs, -(b2 ? t[5] : t[1])) >= 0.0f;       // >= 3.5 s or >= 0.75 s
    const float t0 = b2 ? (b1 ? t[6] : t[4]) : (b1 ? t[2] : t[0]);  // 5, 2.5, 1.25 or 0.25 s
    const bool b0 = fmaf(a, gs, -t0) > 0.0f;
    mag = (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
  }
  return ((xbits >> 12) & 8u) | mag;
}

// Block scale of a 16-element block whose largest magnitude has bf16 bits bmax: returns the E4M3
// code and fills the element thresholds t (the E2M1 midpoints times the scale value).
__device__ __forceinline__ uint32_t block_scale(uint32_t bmax, float gs, float (&t)[7]) {
  const double q = ((double)bf16_bits_to_f32(bmax) * (double)gs) / 6.0;
  const uint32_t sc = e4m3_code_rne(q);
  const float s = e4m3_value(sc);
  t[0] = 0.25f * s;
  t[1] = 0.75f * s;
  t[2] = 1.25f * s;
  t[3] = 1.75f * s;
  t[4] = 2.5f * s;
  t[5] = 3.5f * s;
  t[6] = 5.0f * s;
  return sc;
}

// Quantize 16 bf16 elements (v0: elements 0-7, v1: 8-15, two per word, the lower element in the
// low half) with global scale gs: returns the E4M3 scale code; codes[0..1] receive the 8 code
// bytes (element 2i in the low nibble of byte i).
__device__ __forceinline__ uint32_t quant16(u32x4 v0, u32x4 v1, float gs, uint32_t (&out)[2]) {
  uint32_t bmax = bf16_abs_max8(v0);
  const uint32_t bm1 = bf16_abs_max8(v1);
  bmax = bmax > bm1 ? bmax : bm1;
  float t[7];
  const uint32_t sc = block_scale(bmax, gs, t);
  const bool zs = sc == 0;
  out[0] = out[1] = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w = j < 4 ? v0[j] : v1[j - 4];
    const uint32_t c0 = e2m1_code(w & 0xFFFFu, gs, t, zs);
    const uint32_t c1 = e2m1_code(w >> 16, gs, t, zs);
    out[j >> 2] |= (c0 | (c1 << 4)) << (8 * (j & 3));
  }
  return sc;
}

// Quantize one 16-element block b of the tensor (row-major blocks) with global scale gs.
__device__ __forceinline__ void quant_block(const uint16_t* __restrict__ x, int64_t b, float gs,
                                            uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const u32x4 v0 = *reinterpret_cast<const u32x4*>(x + b * 16);
  const u32x4 v1 = *reinterpret_cast<const u32x4*>(x + b * 16 + 8);
  uint32_t out[2];
  const uint32_t sc = quant16(v0, v1, gs, out);
  *reinterpret_cast<u32x2*>(codes + b * 8) = u32x2{out[0], out[1]};
  scales[b] = (uint8_t)sc;
}

__device__ __forceinline__ float global_scale_of(float amax) {
  return amax > 0.0f ? 2688.0f / amax : 1.0f;  // IEEE division (correctly rounded)
}

// Small tensors (decode activations, up to 2^16 elements): one launch of ceil(blocks / 256)
// workgroups of 1024 threads.  Every workgroup reduces the amax of the whole tensor itself (at most
// 8 loads of 16 bytes per thread, all in flight, from L2 after the first workgroup), so no
// workgroup waits for another; then each quad of threads quantizes one 16-element block, 4
// elements per thread (the per-element tests are most of the work, and a workgroup runs on one CU).
constexpr int kQuantSmallThreads = 1024;
constexpr int kQuantSmallLoads = 8;
constexpr int64_t kQuantSmallElems = (int64_t)kQuantSmallThreads * kQuantSmallLoads * 8;
constexpr int kQuantQuad = 4;                                          // threads per block
constexpr int kQuantSmallBlocks = kQuantSmallThreads / kQuantQuad;    // blocks per workgroup

// Elements 4q..4q+3 of block b (q = lane % 4; the four lanes of a quad call it together with the
// same b, so they share the block maximum through quad swaps): the block's scale (written by lane
// q = 0) and its 4 codes (2 bytes).  !valid: zero codes and scale.  Same bits as quant_block.
__device__ __forceinline__ void quant_block_quarter(const uint16_t* __restrict__ x, int64_t b, float gs, bool valid,
                                                    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int q = (int)(threadIdx.x % kQuantQuad);
  if (!valid) {
    *reinterpret_cast<uint16_t*>(codes + b * 8 + 2 * q) = 0;
    if (q == 0) scales[b] = 0;
    return;
  }
  const u32x2 v = *reinterpret_cast<const u32x2*>(x + b * 16 + 4 * q);
  uint32_t m = (v.x & 0x7FFFu) > ((v.x >> 16) & 0x7FFFu) ? (v.x & 0x7FFFu) : ((v.x >> 16) & 0x7FFFu);
  const uint32_t m1 = (v.y & 0x7FFFu) > ((v.y >> 16) & 0x7FFFu) ? (v.y & 0x7FFFu) : ((v.y >> 16) & 0x7FFFu);
  m = m > m1 ? m : m1;
  uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false);  // lane ^ 1
  m = m > o ? m : o;
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false);  // lane ^ 2
  m = m > o ? m : o;
  float t[7];
  const uint32_t sc = block_scale(m, gs, t);
  const bool zs = sc == 0;
  const uint32_t c = e2m1_code(v.x & 0xFFFFu, gs, t, zs) | (e2m1_code(v.x >> 16, gs, t, zs) << 4) |
                     (e2m1_code(v.y & 0xFFFFu, gs, t, zs) << 8) | (e2m1_code(v.y >> 16, gs, t, zs) << 12);
  *reinterpret_cast<uint16_t*>(codes + b * 8 + 2 * q) = (uint16_t)c;
  if (q == 0) scales[b] = (uint8_t)sc;
}

// Workgroup `wg` of the single-launch form with a caller-given global scale: one block per quad.
__device__ __forceinline__ void quant_gs_small_body(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                    float gs, uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales, int wg) {
  const int64_t b = (int64_t)wg * kQuantSmallBlocks + threadIdx.x / kQuantQuad;
  if (b < rows * (cols / 16)) quant_block_quarter(x, b, gs, true, codes, scales);
}

// Workgroup `wg` of the small-tensor quantizer (1024 threads); red: [kQuantSmallThreads / kWave].
__device__ __forceinline__ void quant_small_body(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                 const int32_t* __restrict__ row_valid, uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales, float* __restrict__ gs_out, int wg,
                                                 uint32_t* red) {
  const int nvec = (int)(rows * cols / 8);
  u32x4 d[kQuantSmallLoads];
#pragma unroll
  for (int j = 0; j < kQuantSmallLoads; ++j) {
    const int v = (int)threadIdx.x + j * kQuantSmallThreads;
    d[j] = u32x4{0u, 0u, 0u, 0u};
    if (v < nvec && (row_valid == nullptr || row_valid[((int64_t)v * 8) / cols] >= 0))
      d[j] = *reinterpret_cast<const u32x4*>(x + (int64_t)v * 8);
  }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < kQuantSmallLoads; ++j) {
    const uint32_t t = bf16_abs_max8(d[j]);
    m = m > t ? m : t;
  }
  m = wave_max_u32(m);
  if (lane_id() == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  m = red[0];
  for (int j = 1; j < kQuantSmallThreads / kWave; ++j) m = m > red[j] ? m : red[j];
  const float gs = global_scale_of(bf16_bits_to_f32(m));
  if (wg == 0 && threadIdx.x == 0) *gs_out = gs;
  const int64_t bpr = cols / 16;
  const int64_t b = (int64_t)wg * kQuantSmallBlocks + threadIdx.x / kQuantQuad;
  if (b >= rows * bpr) return;  // whole quads leave together
  quant_block_quarter(x, b, gs, row_valid == nullptr || row_valid[b / bpr] >= 0, codes, scales);
}

}  // namespace megamoe
