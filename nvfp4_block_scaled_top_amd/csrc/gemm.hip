// NVFP4 x NVFP4 grouped GEMMs over experts: L1 gate+up with SiLU(gate)*up, and L2 down.
//
// Grouped GEMM with per-expert shapes, a per-expert tile height chosen from the token count
// (small at decode, large at prefill), persistent tile scheduling across experts, and experts
// with no tokens skipped (nvfp4-megamoe-kernel CURRENT_BUG.md@2e65594, "Architecture: DeepSeek-V4
// MegaMoE", "Test Plan" Phases 1-2 and "Key References").  The B200 design on those pages
// updates TMA tensor maps per expert; gfx950 has no TMA, so each tile simply computes its
// expert's base pointers.
//
// Arithmetic.  Both operands are NVFP4 and are decoded exactly to fp16 (e2m1 * e4m3 is always a
// normal fp16 number), multiplied on the fp16 MFMA (v_mfma_f32_16x16x32_f16) and accumulated in
// fp32; the product of the two global scales is divided out in the epilogue.
//
// Two tile classes, both persistent over a tile list taken from the routing step's table:
//  * small (16-row tiles, used for experts with few tokens, e.g. decode): weights are streamed
//    from HBM straight into registers, 16 B per lane per 128-element chunk of the reduction
//    dimension; the reduction dimension is split over the 4 waves of a workgroup and the partial
//    sums are added in a fixed order through LDS (deterministic);
//  * large (128x128 tiles): both operands are decoded into fp16 tiles in LDS (double-buffered,
//    register-prefetched), and each wave computes a 64x64 block with 16 MFMAs per 32-K step.
// Tiles are ordered expert-major, then m-tile, then n-tile (n fastest), and workgroup ids are
// remapped so that the workgroups on one XCD take consecutive tiles (the same A rows stay in that
// XCD's L2).
//
// Reduction-order permutation.  In the small class, lane l of a fragment holds 8 consecutive
// elements at k = chunk + 32*(l/16) + 8*j for MFMA step j = 0..3 (instead of the MFMA's natural
// 8*(l/16) within each 32-K step).  A and B use the same permutation, so each dot product is
// unchanged; it lets a lane read 16 contiguous bytes of codes per chunk.
#include "device_common.h"
#include "internal.h"

namespace megamoe {

constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// XCD-aware persistent tile loop.  Workgroups are dispatched round-robin over the 8 XCDs, so
// workgroup b runs on XCD b % 8.  The tile list is cut into 8 contiguous segments and XCD x's
// workgroups walk segment x with stride grid/8: consecutive tiles (which share A rows or weight
// rows) stay in one XCD's L2, and every XCD gets an equal share even when tiles < grid.
struct XcdTiles {
  int t, end, stride;
  __device__ XcdTiles(int total) {
    const int b = blockIdx.x, per = gridDim.x / kXcds, x = b % kXcds;
    const int seg = (total + kXcds - 1) / kXcds;
    t = x * seg + b / kXcds;
    end = min((x + 1) * seg, total);
    stride = per;
  }
};

// Find the expert owning tile t: pref (in LDS) is the exclusive prefix of m-tiles per expert.
// Returns the expert; every thread of the workgroup calls it with the same t.
__device__ __forceinline__ int find_expert(const int* s_pref, int E, int ntn, int t) {
  int lo = 0, hi = E;  // invariant: pref[lo]*ntn <= t < pref[hi]*ntn
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] * ntn <= t) lo = mid; else hi = mid;
  }
  return lo;
}

struct TileInfo {
  int e, mt, nt, row0, rows_left;
};

__device__ __forceinline__ TileInfo decode_tile(const int* s_pref, int E, int ntn, int t, int bm,
                                                const int32_t* __restrict__ poff, const int32_t* __restrict__ counts) {
  TileInfo ti;
  ti.e = find_expert(s_pref, E, ntn, t);
  const int local = t - s_pref[ti.e] * ntn;
  ti.mt = local / ntn;
  ti.nt = local - ti.mt * ntn;
  ti.row0 = poff[ti.e] + ti.mt * bm;
  ti.rows_left = counts[ti.e] - ti.mt * bm;
  return ti;
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// ============================================================================================
// Small class: 16 rows x 32 weight rows per tile, K split over 4 waves.
// L1: weight rows {nt*16 + r (gate), I + nt*16 + r (up)} -> 16 h columns.  L2: rows nt*32 + r.
// ============================================================================================
constexpr int kSmallBn = 32;
constexpr int kChunk = 128;

template <bool kL1>
__global__ __launch_bounds__(kGemmThreads) void gemm_small_kernel(GemmArgs p) {
  __shared__ int s_pref[kMaxExperts + 1];
  __shared__ f32x4 s_red[4][2][kWave];
  const int E = p.E;
  const int32_t* __restrict__ sched = p.sched;
  for (int j = threadIdx.x; j <= E; j += blockDim.x) s_pref[j] = sched[sched_pref_small(E) + j];
  __syncthreads();
  const int ntn = kL1 ? p.N / 16 : p.N / kSmallBn;
  const int total = s_pref[E] * ntn;
  const int K = p.K, Kh = K / 2, Ks = K / 16;
  const int Nw = kL1 ? 2 * p.N : p.N;  // weight rows per expert
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int nc = K / kChunk;
  const int c_begin = wave * nc / 4, c_end = (wave + 1) * nc / 4;
  const float gs_a = *p.a_gs;
  uint32_t amax_bits = 0;

  const XcdTiles tl(total);
  for (int t = tl.t; t < tl.end; t += tl.stride) {
    const TileInfo ti = decode_tile(s_pref, E, ntn, t, kBlockMSmall, p.padded_offsets, p.counts);
    const bool a_ok = r16 < ti.rows_left;
    int64_t a_row = ti.row0 + r16;
    if (kL1) a_row = a_ok ? p.row_token[a_row] : 0;
    const uint8_t* __restrict__ a_c = p.a_codes + a_row * Kh + g * 16;
    const uint8_t* __restrict__ a_s = p.a_scales + a_row * Ks + g * 2;
    int64_t b_row0, b_row1;
    if (kL1) {
      b_row0 = (int64_t)ti.e * Nw + ti.nt * 16 + r16;
      b_row1 = b_row0 + p.N;
    } else {
      b_row0 = (int64_t)ti.e * Nw + ti.nt * kSmallBn + r16;
      b_row1 = b_row0 + 16;
    }
    const uint8_t* __restrict__ b0_c = p.w_codes + b_row0 * Kh + g * 16;
    const uint8_t* __restrict__ b1_c = p.w_codes + b_row1 * Kh + g * 16;
    const uint8_t* __restrict__ b0_s = p.w_scales + b_row0 * Ks + g * 2;
    const uint8_t* __restrict__ b1_s = p.w_scales + b_row1 * Ks + g * 2;

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    // Register double-buffering of the next chunk's raw codes and scales.
    u32x4 ac = {0u, 0u, 0u, 0u}, bc0 = {0u, 0u, 0u, 0u}, bc1 = {0u, 0u, 0u, 0u};
    uint32_t as = 0, bs0 = 0, bs1 = 0;
    if (c_begin < c_end) {
      const int64_t off = (int64_t)c_begin * (kChunk / 2);
      const int64_t soff = (int64_t)c_begin * (kChunk / 16);
      if (a_ok) {
        ac = *reinterpret_cast<const u32x4*>(a_c + off);
        as = *reinterpret_cast<const uint16_t*>(a_s + soff);
      }
      bc0 = *reinterpret_cast<const u32x4*>(b0_c + off);
      bc1 = *reinterpret_cast<const u32x4*>(b1_c + off);
      bs0 = *reinterpret_cast<const uint16_t*>(b0_s + soff);
      bs1 = *reinterpret_cast<const uint16_t*>(b1_s + soff);
    }
    for (int c = c_begin; c < c_end; ++c) {
      const u32x4 cac = ac, cb0 = bc0, cb1 = bc1;
      const uint32_t cas = as, cbs0 = bs0, cbs1 = bs1;
      if (c + 1 < c_end) {
        const int64_t off = (int64_t)(c + 1) * (kChunk / 2);
        const int64_t soff = (int64_t)(c + 1) * (kChunk / 16);
        if (a_ok) {
          ac = *reinterpret_cast<const u32x4*>(a_c + off);
          as = *reinterpret_cast<const uint16_t*>(a_s + soff);
        }
        bc0 = *reinterpret_cast<const u32x4*>(b0_c + off);
        bc1 = *reinterpret_cast<const u32x4*>(b1_c + off);
        bs0 = *reinterpret_cast<const uint16_t*>(b0_s + soff);
        bs1 = *reinterpret_cast<const uint16_t*>(b1_s + soff);
      }
      const f16x2 sa = e4m3x2_to_f16(cas, false);
      const f16x2 sb0 = e4m3x2_to_f16(cbs0, false);
      const f16x2 sb1 = e4m3x2_to_f16(cbs1, false);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x8 a = decode8(cac[j], j < 2 ? bcast_lo(sa) : bcast_hi(sa));
        const f16x8 w0 = decode8(cb0[j], j < 2 ? bcast_lo(sb0) : bcast_hi(sb0));
        const f16x8 w1 = decode8(cb1[j], j < 2 ? bcast_lo(sb1) : bcast_hi(sb1));
        acc0 = mfma16(a, w0, acc0);
        acc1 = mfma16(a, w1, acc1);
      }
    }
    // Fixed-order reduction of the 4 K-partials.
    s_red[wave][0][lane] = acc0;
    s_red[wave][1][lane] = acc1;
    __syncthreads();
    if (wave == 0) {
      f32x4 r0 = s_red[0][0][lane], r1 = s_red[0][1][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        r0 += s_red[w][0][lane];
        r1 += s_red[w][1][lane];
      }
      const float inv = (float)(1.0 / ((double)gs_a * (double)p.w_gs[ti.e]));
      uint16_t* __restrict__ out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * g + q;
        if (r < ti.rows_left) {
          const int64_t orow = (int64_t)(ti.row0 + r) * p.N;
          if (kL1) {
            const float gt = r0[q] * inv, up = r1[q] * inv;
            const uint32_t hb = f32_to_bf16_bits(silu_f32(gt) * up);
            out[orow + ti.nt * 16 + r16] = (uint16_t)hb;
            const uint32_t mag = hb & 0x7FFFu;
            amax_bits = amax_bits > mag ? amax_bits : mag;
          } else {
            out[orow + ti.nt * kSmallBn + r16] = (uint16_t)f32_to_bf16_bits(r0[q] * inv);
            out[orow + ti.nt * kSmallBn + 16 + r16] = (uint16_t)f32_to_bf16_bits(r1[q] * inv);
          }
        }
      }
    }
    __syncthreads();
  }
  if (kL1) {
    amax_bits = wave_max_u32(amax_bits);
    if (threadIdx.x == 0 && amax_bits != 0) atomicMax(reinterpret_cast<unsigned int*>(p.amax_out), amax_bits << 16);
  }
}

// ============================================================================================
// Large class: 128x128 tiles, K step 64, LDS-staged fp16 operands.
// L1: B tile rows 0..63 = gate rows nt*64.., rows 64..127 = up rows I + nt*64.. -> 64 h columns.
// L2: B tile rows = weight rows nt*128..+128 -> 128 y columns.
// ============================================================================================
constexpr int kLBm = kBlockMLarge, kLBn = 128, kLKt = 64, kLLd = kLKt + 8;  // LDS row pitch (fp16)

template <bool kL1>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_large_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][kLBm * kLLd];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][kLBn * kLLd];
  __shared__ int s_pref[kMaxExperts + 1];
  const int E = p.E;
  for (int j = threadIdx.x; j <= E; j += blockDim.x) s_pref[j] = p.sched[sched_pref_large(E) + j];
  __syncthreads();
  const int ntn = kL1 ? p.N / 64 : p.N / kLBn;
  const int total = s_pref[E] * ntn;
  const int K = p.K, Kh = K / 2, Ks = K / 16;
  const int Nw = kL1 ? 2 * p.N : p.N;
  const int nk = K / kLKt;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, g = lane >> 4;
  const int ld_row = tid >> 1, ld_half = tid & 1;  // global->LDS: 128 rows x 2 halves of 32 K
  const float gs_a = *p.a_gs;
  uint32_t amax_bits = 0;
  // LDS row of B fragment f for this wave.
  int brow[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) brow[f] = kL1 ? (f < 2 ? wn * 32 + 16 * f : 64 + wn * 32 + 16 * (f - 2)) : wn * 64 + 16 * f;

  const XcdTiles tl(total);
  for (int t = tl.t; t < tl.end; t += tl.stride) {
    const TileInfo ti = decode_tile(s_pref, E, ntn, t, kLBm, p.padded_offsets, p.counts);
    // This thread's A and B source rows for the global->LDS copy.
    const bool a_ok = ld_row < ti.rows_left;
    int64_t a_row = ti.row0 + ld_row;
    if (kL1) a_row = a_ok ? p.row_token[a_row] : 0;
    const uint8_t* __restrict__ a_c = p.a_codes + a_row * Kh + ld_half * 16;
    const uint8_t* __restrict__ a_s = p.a_scales + a_row * Ks + ld_half * 2;
    int64_t b_row;
    if (kL1) b_row = (int64_t)ti.e * Nw + (ld_row < 64 ? ti.nt * 64 + ld_row : p.N + ti.nt * 64 + ld_row - 64);
    else b_row = (int64_t)ti.e * Nw + ti.nt * kLBn + ld_row;
    const uint8_t* __restrict__ b_c = p.w_codes + b_row * Kh + ld_half * 16;
    const uint8_t* __restrict__ b_s = p.w_scales + b_row * Ks + ld_half * 2;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ac = {0u, 0u, 0u, 0u}, bc = {0u, 0u, 0u, 0u};
    uint32_t as = 0, bs = 0;
    auto load = [&](int kt) {
      const int64_t off = (int64_t)kt * (kLKt / 2), soff = (int64_t)kt * (kLKt / 16);
      if (a_ok) {
        ac = *reinterpret_cast<const u32x4*>(a_c + off);
        as = *reinterpret_cast<const uint16_t*>(a_s + soff);
      }
      bc = *reinterpret_cast<const u32x4*>(b_c + off);
      bs = *reinterpret_cast<const uint16_t*>(b_s + soff);
    };
    auto store = [&](int buf) {
      const f16x2 sa = e4m3x2_to_f16(as, false), sb = e4m3x2_to_f16(bs, false);
      _Float16* ad = &As[buf][ld_row * kLLd + ld_half * 32];
      _Float16* bd = &Bs[buf][ld_row * kLLd + ld_half * 32];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<f16x8*>(ad + 8 * j) = decode8(ac[j], j < 2 ? bcast_lo(sa) : bcast_hi(sa));
        *reinterpret_cast<f16x8*>(bd + 8 * j) = decode8(bc[j], j < 2 ? bcast_lo(sb) : bcast_hi(sb));
      }
    };
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) load(kt + 1);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        f16x8 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a[i] = *reinterpret_cast<const f16x8*>(&As[buf][(wm * 64 + 16 * i + r16) * kLLd + s * 32 + 8 * g]);
#pragma unroll
        for (int f = 0; f < 4; ++f)
          b[f] = *reinterpret_cast<const f16x8*>(&Bs[buf][(brow[f] + r16) * kLLd + s * 32 + 8 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[i][f] = mfma16(a[i], b[f], acc[i][f]);
      }
      if (kt + 1 < nk) store(buf ^ 1);
      __syncthreads();
    }

    const float inv = (float)(1.0 / ((double)gs_a * (double)p.w_gs[ti.e]));
    uint16_t* __restrict__ out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = wm * 64 + 16 * i + 4 * g + q;
        if (r < ti.rows_left) {
          const int64_t orow = (int64_t)(ti.row0 + r) * p.N;
          if (kL1) {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
              const float gt = acc[i][f][q] * inv, up = acc[i][f + 2][q] * inv;
              const uint32_t hb = f32_to_bf16_bits(silu_f32(gt) * up);
              out[orow + ti.nt * 64 + wn * 32 + 16 * f + r16] = (uint16_t)hb;
              const uint32_t mag = hb & 0x7FFFu;
              amax_bits = amax_bits > mag ? amax_bits : mag;
            }
          } else {
#pragma unroll
            for (int f = 0; f < 4; ++f)
              out[orow + ti.nt * kLBn + wn * 64 + 16 * f + r16] = (uint16_t)f32_to_bf16_bits(acc[i][f][q] * inv);
          }
        }
      }
    }
  }
  if (kL1) {
    amax_bits = wave_max_u32(amax_bits);
    if (lane == 0 && amax_bits != 0) atomicMax(reinterpret_cast<unsigned int*>(p.amax_out), amax_bits << 16);
  }
}

__global__ void zero_f32_kernel(float* p) { *p = 0.0f; }

constexpr int kSmallGrid = 1024;  // persistent grids (multiples of kXcds)
constexpr int kLargeGrid = 512;

template <bool kL1>
static hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(gemm_large_kernel<kL1>, dim3(kLargeGrid), dim3(kGemmThreads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(gemm_small_kernel<kL1>, dim3(kSmallGrid), dim3(kGemmThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm_l1(const GemmArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(zero_f32_kernel, dim3(1), dim3(1), 0, stream, a.amax_out);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_gemm<true>(a, stream);
}

hipError_t launch_gemm_l2(const GemmArgs& a, hipStream_t stream) { return launch_gemm<false>(a, stream); }

}  // namespace megamoe
