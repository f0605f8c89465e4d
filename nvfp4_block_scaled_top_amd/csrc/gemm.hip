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
// normal fp16 number), multiplied on the fp16 MFMA (16x16x32 in the small class, 32x32x16 in the
// large class) and accumulated in
// fp32; the product of the two global scales is divided out in the epilogue.
//
// Two tile classes, both persistent over a work list taken from the routing step's table:
//  * small (m-tiles of 16 token rows, for experts with few tokens, e.g. decode): weights are
//    streamed from HBM straight into registers; every workgroup takes an equal share of the
//    output columns, its 4 waves split K and add their partial sums in a fixed order through LDS
//    (deterministic);
//  * large (256x256 tiles): raw NVFP4 staged in an LDS ring and decoded per wave; 8 waves (4x2)
//    each compute a 64x128 block, 2 waves per SIMD (details below).
// Workgroup ids are remapped so that the workgroups on one XCD take neighbouring work (the same A
// rows stay in that XCD's L2).
//
// Reduction-order permutation.  In the small class, lane l of a fragment holds CH/8 consecutive
// code bytes of its row (elements chunk + (CH/4)*(l/16) ..) and feeds element group st of them to
// MFMA step st (instead of the MFMA's natural 8*(l/16) within each 32-K step).  A and B use the
// same permutation, so each dot product is unchanged; it lets a lane read contiguous bytes.
#include "device_common.h"
#include "internal.h"

namespace megamoe {

constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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

// SiLU in fp32 with the hardware exp2 and reciprocal (a few ulp); h is rounded to bf16 right after.
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}

// ============================================================================================
// Small class (m-tiles of 16 token rows; experts with few tokens, e.g. decode).  Each weight byte
// feeds one 16-row MFMA block, so the kernel streams weights, and decoding NVFP4 to fp16 costs
// about 2 VALU instructions per weight byte and lane -- the VALU, not HBM, is what runs out
// first.  The design keeps the VALU work per weight byte low and every workgroup equally busy:
//  * work unit = one output column of one m-tile (L1: an h column, i.e. a gate row and its up
//    row; L2: a y column, i.e. a weight row).  The units of all small m-tiles are laid end to end
//    and each workgroup takes an equal contiguous range (workgroups on one XCD get neighbouring
//    ranges, so the A rows of an m-tile stay in that XCD's L2);
//  * a workgroup walks its range in groups of up to kSNb (small_nb) 16-column MFMA blocks (one
//    m-tile per group).  Its 4 waves split the reduction dimension K in four and stream the same
//    groups: one decoded A fragment feeds kSNb MFMAs;
//  * weight codes come straight into registers (CH/8 bytes per lane per CH-element chunk)
//    through a kSDepth-deep ring that runs on across group boundaries; the weights' block scales
//    are copied per group into LDS by direct-to-LDS loads (kStaged, see below);
//  * at the end of a group each wave leaves its kSNb partial blocks in LDS (double-buffered by
//    group parity) and, after one LDS-only barrier (the weight loads stay in flight), wave w adds
//    the 4 partials of blocks j = w mod 4 in wave order (deterministic) and stores them.
// Lanes whose row lies outside the group or m-tile load a valid row of the same tile instead; the
// MFMA outputs they feed are never stored.
// L1 block j of a group: MFMA columns 0-7 are gate rows of h columns j0+8j.., columns 8-15 the
// matching up rows, paired after the reduction with a lane shuffle.  L2 block j: weight rows
// j0+16j..+16.
// ============================================================================================
#ifndef MEGAMOE_SMALL_NB_L1
#define MEGAMOE_SMALL_NB_L1 2
#endif
#ifndef MEGAMOE_SMALL_NB_L2
#define MEGAMOE_SMALL_NB_L2 2
#endif
#ifndef MEGAMOE_SMALL_DEPTH
#define MEGAMOE_SMALL_DEPTH 2
#endif
#ifndef MEGAMOE_SMALL_OCC
#define MEGAMOE_SMALL_OCC 2
#endif
template <bool kL1>
constexpr int small_nb() { return kL1 ? MEGAMOE_SMALL_NB_L1 : MEGAMOE_SMALL_NB_L2; }  // blocks per group
constexpr int kSDepth = MEGAMOE_SMALL_DEPTH;  // ring slots (chunks in flight per wave)
constexpr int kSOcc = MEGAMOE_SMALL_OCC;      // workgroups (of 4 waves) per CU
constexpr int kSWaves = kGemmThreads / kWave; // K split
constexpr int kLargeGrid = 256;               // large class: one workgroup per CU (LDS ~148 KB)
constexpr int kSmallGrid = 256 * kSOcc;       // small class: resident workgroups
constexpr int kAmaxSmallSlots = MEGAMOE_L1_AMAX_PARTS - kLargeGrid;  // slots [kLargeGrid, PARTS)
#ifndef MEGAMOE_SMALL_STAGED_KB
#define MEGAMOE_SMALL_STAGED_KB 48
#endif
constexpr size_t kSmallStagedMaxLds = MEGAMOE_SMALL_STAGED_KB * 1024;  // 3 staged scale buffers
static_assert(kSmallGrid <= kAmaxSmallSlots, "one amax slot per small workgroup");
static_assert(kSmallGrid % kXcds == 0, "grid split");

template <bool kL1>
constexpr int small_group_units() { return kL1 ? 8 * small_nb<kL1>() : 16 * small_nb<kL1>(); }

struct SmallGroup {
  int e;          // expert
  int row0;       // first padded row of the m-tile
  int rows_left;  // token rows of the m-tile (>= 1)
  int j0;         // first unit of the group (L1: h column, L2: output column)
  int n;          // units in the group
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Direct global -> LDS loads.  Issued through inline assembly so that the compiler does not track
// them as LDS writes (it would otherwise wait for every outstanding load before any LDS read it
// cannot prove disjoint, draining the prefetch each stage).  Their ordering is explicit instead:
// wait_vmcnt() for this wave's loads, then s_barrier for everyone's.  The compiler's own vmcnt
// waits stay correct because loads retire in order.  Nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is written only here (checked in the ISA)
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}
__device__ __forceinline__ void dma16(const uint8_t* src, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform; must live in an SGPR for M0
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const uint8_t* src, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(n), other counters unconstrained (gfx9 encoding: vmcnt bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One chunk of the reduction dimension for one lane: CH/8 code bytes (CH/32 MFMA steps) and
// CH/64 scale bytes of its A row and of each of its kSNb weight rows.
template <int CH, int NB>
struct SmallSlot {
  static constexpr int kQ = CH / 128;  // u32x4 words per lane and row (1 or 2)
  u32x4 a[kQ];
  uint32_t as;
  u32x4 b[NB][kQ];
  uint32_t bs[NB];
};

// Wave-uniform read through the scalar data cache (the index must be wave-uniform).  Scalar
// loads are counted by lgkmcnt, so waiting for one does not wait for the vector loads of the
// weight stream (vmcnt counts vector memory operations in issue order).
template <typename T>
__device__ __forceinline__ T sload(const T* p, int i) {
  i = __builtin_amdgcn_readfirstlane(i);
  return ((const __attribute__((address_space(4))) T*)(uintptr_t)p)[i];
}

// Workgroup barrier that orders LDS only: vector memory loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// CH (128 or 256) is the chunk of K a wave step covers: a lane loads CH/8 contiguous code bytes
// (CH/32 MFMA steps) and CH/64 scale bytes per row.  256 halves the scale loads per weight byte
// (one u32 instead of one u16 per 128 elements); 128 serves K that is an odd multiple of 128.
// Weight scales staged in LDS (kStaged): a group's rows of weight block scales (row-contiguous in
// HBM) are copied by full-line direct-to-LDS loads when the loader enters the group, into buffer
// (group index) % 3, rows padded by 16 bytes so that the 4-byte reads of 16 rows x 4 lanes hit
// distinct banks.  The steady state then issues no scale loads for the weights (they carried 4
// bytes per lane and cost as much issue as the 16-byte code loads).  With a ring of kSDepth
// steps the loader runs at most 2 groups ahead of the compute (one step per group at least), so 3
// buffers suffice; every wave has issued at least kSDepth steps of loads after its copy of group
// q+1 when group q ends, so vmcnt <= kSDepth * (loads per step) there (before the group's
// barrier) means the copy has landed.
template <bool kL1, int CH, bool kStaged>
__global__ __launch_bounds__(kGemmThreads, kSOcc) void gemm_small_kernel(GemmArgs p) {
  constexpr int kSNb = small_nb<kL1>();
  using Slot = SmallSlot<CH, kSNb>;
  constexpr int kQ = Slot::kQ;
  constexpr int kLaneBytes = CH / 8, kLaneScales = CH / 64;
  constexpr int kLoadsPerStep = kQ * (1 + kSNb) + 1 + (kStaged ? 0 : kSNb);
  extern __shared__ __attribute__((aligned(16))) uint8_t s_scl[];  // [3][scale buffer] if kStaged
  // Per-expert tables in LDS: reading them inside the loop must not wait on the weight stream.
  __shared__ int s_pref[kMaxExperts + 1];
  __shared__ int s_poff[kMaxExperts];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ float s_wgs[kMaxExperts];
  __shared__ f32x4 s_red[2][kSWaves][kSNb][kWave];
  __shared__ uint32_t s_amax[kSWaves];
  const int E = p.E;
  const int32_t* __restrict__ sched = p.sched;
  for (int j = threadIdx.x; j <= E; j += blockDim.x) {
    s_pref[j] = sched[sched_pref_small(E) + j];
    if (j < E) {
      s_poff[j] = p.padded_offsets[j];
      s_cnt[j] = p.counts[j];
      s_wgs[j] = p.w_gs[j];
    }
  }
  __syncthreads();
  const int NU = p.N;  // units per m-tile: L1 h columns (I), L2 output columns (H)
  constexpr int GU = small_group_units<kL1>();
  const int64_t U = (int64_t)s_pref[E] * NU;
  const int K = p.K, Kh = K / 2, Ks = K / 16;
  const int Nw = kL1 ? 2 * p.N : p.N;  // weight rows per expert
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int nch = K / CH;
  const int ks = nch < kSWaves ? nch : kSWaves;  // waves sharing K (all 4 unless K < 512)
  const int c0 = wave < ks ? wave * nch / ks : 0, c1 = wave < ks ? (wave + 1) * nch / ks : 0;
  const float gs_a = *p.a_gs;
  uint32_t amax_bits = 0;

  // This workgroup's unit range; workgroup b runs on XCD b % 8.
  const int G = gridDim.x, b = blockIdx.x;
  const int64_t lb = (int64_t)(b % kXcds) * (G / kXcds) + b / kXcds;
  const int64_t u_begin = lb * U / G, u_end = (lb + 1) * U / G;

  // Number of groups in [u_begin, u_end): groups never cross an m-tile.
  int64_t ngroups = 0;
  if (u_begin < u_end) {
    const int64_t ma = u_begin / NU, mb = (u_end - 1) / NU;
    if (ma == mb) {
      ngroups = (u_end - u_begin + GU - 1) / GU;
    } else {
      ngroups = ((ma + 1) * NU - u_begin + GU - 1) / GU + (mb - ma - 1) * ((NU + GU - 1) / GU) +
                (u_end - mb * NU + GU - 1) / GU;
    }
  }

  auto group_at = [&](int64_t u) {
    SmallGroup q;
    const int mtg = (int)(u / NU);
    q.e = find_expert(s_pref, E, 1, mtg);
    const int mt = mtg - s_pref[q.e];
    q.row0 = s_poff[q.e] + mt * kBlockMSmall;
    q.rows_left = s_cnt[q.e] - mt * kBlockMSmall;
    q.j0 = (int)(u - (int64_t)mtg * NU);
    int64_t n = u_end - u;
    if (n > NU - q.j0) n = NU - q.j0;
    if (n > GU) n = GU;
    q.n = (int)n;
    return q;
  };

  if (c1 == c0) {
    // K has fewer than 4 chunks and this wave has none: it only keeps the barrier count.
    for (int64_t q = 0; q < ngroups; ++q) lds_barrier();
  } else {
    // ---- loader cursor: group being loaded, this lane's row pointers, next chunk --------------
    // Past the last step the loader keeps re-reading its last group's first chunk (valid memory,
    // never consumed), so every step issues the same loads.
    int64_t lu = u_begin;
    int lc = c0, ln = 0;
    const uint8_t* la_c = p.a_codes;
    const uint8_t* la_s = p.a_scales;
    const uint8_t* lb_c[kSNb];
    const uint8_t* lb_s[kSNb];
#pragma unroll
    for (int j = 0; j < kSNb; ++j) {
      lb_c[j] = p.w_codes;
      lb_s[j] = p.w_scales;
    }
    // Staged scales: buffer geometry (pieces of 16 bytes; P per padded row).
    const int P = Ks / 16 + 1, SRB = 16 * P;
    const int npieces = kSNb * 16 * P, ndma = (npieces + 63) / 64;
    const int buf_bytes = ndma * 1024;
    int lq = 0;  // loader's group index
    auto weight_row = [&](const SmallGroup& q, int col) -> int64_t {  // MFMA column -> weight row
      if (kL1) {
        const int j = col / 16, c = col % 16;
        const int hc = 8 * j + (c & 7);
        const int hcol = q.j0 + (hc < q.n ? hc : 0);
        return (int64_t)q.e * Nw + (c < 8 ? hcol : p.N + hcol);
      }
      return (int64_t)q.e * Nw + q.j0 + (col < q.n ? col : 0);
    };
    auto stage_scales = [&](const SmallGroup& q, int buf) {
      const uint32_t base = lds_addr(s_scl + buf * buf_bytes);
      for (int i = wave; i < ndma; i += kSWaves) {
        const int pc = 64 * i + lane;
        const int cr = pc / P, pi = pc - cr * P;
        const bool real = cr < kSNb * 16 && pi < P - 1;
        const uint8_t* src = p.w_scales + weight_row(q, real ? cr : 0) * Ks + (real ? 16 * pi : 0);
        dma16(src, base + 1024 * i);
      }
    };
    auto loader_enter = [&](int64_t u) {
      const SmallGroup q = group_at(u);
      if (kStaged) stage_scales(q, lq % 3);
      ++lq;
      int64_t arow;
      if (kL1) {
        int tok = sload(p.row_token, q.row0);
        for (int i = 1; i < kBlockMSmall; ++i) {
          if (i < q.rows_left) {
            const int t = sload(p.row_token, q.row0 + i);
            tok = r16 == i ? t : tok;
          }
        }
        arow = tok;
      } else {
        arow = q.row0 + (r16 < q.rows_left ? r16 : 0);
      }
      la_c = p.a_codes + arow * Kh + g * kLaneBytes;
      la_s = p.a_scales + arow * Ks + g * kLaneScales;
#pragma unroll
      for (int j = 0; j < kSNb; ++j) {
        int64_t brow;
        if (kL1) {
          const int hc = 8 * j + (r16 & 7);
          const int col = q.j0 + (hc < q.n ? hc : 0);
          brow = (int64_t)q.e * Nw + (r16 < 8 ? col : p.N + col);
        } else {
          const int rc = 16 * j + r16;
          brow = (int64_t)q.e * Nw + q.j0 + (rc < q.n ? rc : 0);
        }
        lb_c[j] = p.w_codes + brow * Kh + g * kLaneBytes;
        lb_s[j] = p.w_scales + brow * Ks + g * kLaneScales;
      }
      ln = q.n;
    };
    if (u_begin < u_end) loader_enter(u_begin);
    auto load_scale = [](const uint8_t* q) -> uint32_t {
      if (kLaneScales == 4) return *reinterpret_cast<const uint32_t*>(q);
      return *reinterpret_cast<const uint16_t*>(q);
    };
    auto load = [&](Slot& d) {
      const int64_t off = (int64_t)lc * (CH / 2), soff = (int64_t)lc * (CH / 16);
#pragma unroll
      for (int q = 0; q < kQ; ++q) d.a[q] = *reinterpret_cast<const u32x4*>(la_c + off + 16 * q);
      d.as = load_scale(la_s + soff);
#pragma unroll
      for (int j = 0; j < kSNb; ++j) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) d.b[j][q] = *reinterpret_cast<const u32x4*>(lb_c[j] + off + 16 * q);
        if (!kStaged) d.bs[j] = load_scale(lb_s[j] + soff);
      }
      if (++lc == c1) {
        lc = c0;
        if (lu + ln < u_end) {
          lu += ln;
          loader_enter(lu);
        }
      }
    };

    // ---- compute cursor ---------------------------------------------------------------------------
    int64_t cu = u_begin;
    int cc = c0, parity = 0, cq = 0;  // cq: compute cursor's group index
    SmallGroup cg{0, 0, 1, 0, 0};
    if (cu < u_end) cg = group_at(cu);
    f32x4 acc[kSNb];
#pragma unroll
    for (int j = 0; j < kSNb; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // MFMA step st takes the lane's code word st (8 elements, scale block st / 2).
    auto compute = [&](const Slot& d) {
      uint32_t bsw[kSNb];
      if (kStaged) {
        // this lane's scale bytes of chunk cc for its row in each block (LDS, padded rows)
        const uint8_t* sb0 = s_scl + (cq % 3) * buf_bytes + r16 * SRB + cc * (CH / 16) + g * kLaneScales;
#pragma unroll
        for (int j = 0; j < kSNb; ++j) {
          if (kLaneScales == 4) bsw[j] = *reinterpret_cast<const uint32_t*>(sb0 + 16 * j * SRB);
          else bsw[j] = *reinterpret_cast<const uint16_t*>(sb0 + 16 * j * SRB);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kSNb; ++j) bsw[j] = d.bs[j];
      }
      f16x2 sa[kQ];
      f16x2 sb[kSNb][kQ];
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        sa[q] = e4m3x2_to_f16(d.as, q == 1);
#pragma unroll
        for (int j = 0; j < kSNb; ++j) sb[j][q] = e4m3x2_to_f16(bsw[j], q == 1);
      }
#pragma unroll
      for (int st = 0; st < CH / 32; ++st) {
        const int q = st / 4, w4 = st % 4;
        const f16x8 a = decode8(d.a[q][w4], w4 < 2 ? bcast_lo(sa[q]) : bcast_hi(sa[q]));
#pragma unroll
        for (int j = 0; j < kSNb; ++j) {
          const f16x8 w = decode8(d.b[j][q][w4], w4 < 2 ? bcast_lo(sb[j][q]) : bcast_hi(sb[j][q]));
          acc[j] = mfma16(a, w, acc[j]);
        }
      }
    };

    // End of a group: publish the partial blocks, then wave w finishes blocks j = w (mod ks).
    // (Staged scales: the next group's copy has landed for this wave once vmcnt <= kSDepth steps
    // of loads; in the predicated tail fewer loads follow it, so wait for all.)
    auto group_end = [&](bool tail) {
#pragma unroll
      for (int j = 0; j < kSNb; ++j) {
        s_red[parity][wave][j][lane] = acc[j];
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (kStaged) {
        if (tail) wait_vmcnt<0>();
        else wait_vmcnt<kSDepth * kLoadsPerStep>();
      }
      lds_barrier();
      const float inv = (float)(1.0 / ((double)gs_a * (double)s_wgs[cg.e]));
      uint16_t* __restrict__ out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
      for (int j = 0; j < kSNb; ++j) {
        if (j % ks != wave) continue;
        f32x4 r = s_red[parity][0][j][lane];
        for (int w = 1; w < ks; ++w) r += s_red[parity][w][j][lane];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 4 * g + q;
          if (kL1) {
            const float up_raw = __shfl(r[q], lane + 8, kWave);  // column c+8 holds the up row of c
            const int hc = 8 * j + r16;
            if (r16 < 8 && hc < cg.n && row < cg.rows_left) {
              const float gt = r[q] * inv, up = up_raw * inv;
              const uint32_t hb = f32_to_bf16_bits(silu_f32(gt) * up);
              out[(int64_t)(cg.row0 + row) * p.N + cg.j0 + hc] = (uint16_t)hb;
              const uint32_t mag = hb & 0x7FFFu;
              amax_bits = amax_bits > mag ? amax_bits : mag;
            }
          } else {
            const int rc = 16 * j + r16;
            if (rc < cg.n && row < cg.rows_left)
              out[(int64_t)(cg.row0 + row) * p.N + cg.j0 + rc] = (uint16_t)f32_to_bf16_bits(r[q] * inv);
          }
        }
      }
      parity ^= 1;
    };
    auto step_done = [&](bool tail) {
      if (++cc == c1) {
        group_end(tail);
        cc = c0;
        ++cq;
        cu += cg.n;
        if (cu < u_end) cg = group_at(cu);
      }
    };

    // Steady state: step s computes ring slot s % kSDepth and refills it with step s + kSDepth.
    // Loads are unconditional in the prologue and the main loop (so the compiler's in-order vmcnt
    // waits keep kSDepth - 1 steps in flight); only the last < 2 kSDepth steps are predicated.
    const int64_t S = ngroups * (c1 - c0);
    Slot ring[kSDepth];
#pragma unroll
    for (int k = 0; k < kSDepth; ++k) load(ring[k]);
    if (kStaged) {  // the first group's scales (issued before the prologue loads) have landed
      wait_vmcnt<kSDepth * kLoadsPerStep>();
      lds_barrier();
    }
    int64_t s0 = 0;
    for (; s0 + 2 * kSDepth <= S; s0 += kSDepth) {
#pragma unroll
      for (int k = 0; k < kSDepth; ++k) {
        compute(ring[k]);
        load(ring[k]);
        step_done(false);
      }
    }
#pragma unroll
    for (int i = 0; i < 2 * kSDepth - 1; ++i) {
      if (s0 + i < S) {
        compute(ring[i % kSDepth]);
        if (s0 + i + kSDepth < S) load(ring[i % kSDepth]);
        step_done(true);
      }
    }
  }

  if (kL1) {
    amax_bits = wave_max_u32(amax_bits);
    if (lane == 0) s_amax[wave] = amax_bits;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t m = s_amax[0];
      for (int w = 1; w < kSWaves; ++w) m = m > s_amax[w] ? m : s_amax[w];
      p.amax_out[kLargeGrid + b] = bf16_bits_to_f32(m);
      for (int j = b + G; j < kAmaxSmallSlots; j += G) p.amax_out[kLargeGrid + j] = 0.0f;
      if (p.clear_other)
        for (int j = b; j < kLargeGrid; j += G) p.amax_out[j] = 0.0f;
    }
  }
}

// ============================================================================================
// Large class: 256x256 tiles, stages of raw NVFP4 streamed straight into an LDS ring.
//
// Global -> LDS: gfx950's global_load_lds_dwordx4 writes each lane's 16 bytes into LDS without a
// register round trip (lane i of an instruction lands at base + 16*i).  Stage ks+kLAhead is
// requested while stage ks is computed; a stage is consumed after an explicit s_waitcnt vmcnt
// (this wave's loads) and one s_barrier (everyone's).  The slot being refilled was last read two
// stages earlier, so that single barrier per stage orders both directions.  (__syncthreads()
// would also wait for every load still in flight.)  Measured on the 8192-token prefill, 128-K
// stages with 4 slots were faster than 64-K stages with 8 slots and six stages in flight.
//
// LDS holds raw codes and scales (0.5625 B/element) and each wave decodes the fragments it needs
// right before its MFMAs.  Decoding into fp16 tiles in LDS instead would move ~3.5x more LDS
// bytes per MFMA; per-wave decoding costs 4 VALU instructions per 32-cycle
// v_mfma_f32_32x32x16_f16, which the VALU issues while the matrix core runs (the 32x32x16 shape
// sustains ~97% of the fp16 peak on gfx950, the 16x16x32 shape only ~55%).
//
// Stage layout (per operand): codes row-major, kLRowBytes per tile row R, with the 16-byte chunk
// c (elements 32c..32c+31 of the stage) stored in slot c ^ swizzle(R) so that the 16-byte
// fragment reads of 8 consecutive rows hit distinct banks; a DMA instruction covers 1024 / 
// kLRowBytes rows with kLChunks lanes per row (row-contiguous global bytes).  Scales: the stage's 8
// block scales of row R at R * 8 (lane half h reads the 4 bytes at R * 8 + 4h).
// Lane (p = lane % 32, h = lane / 32) of a 32-row fragment owns elements [h * kLKs/2, +kLKs/2) of
// its row and feeds [h * kLKs/2 + 8s, +8) to MFMA step s as the MFMA's k = 8h..8h+7.  A and B use
// the same map, so each dot product runs over every element once.
//
// Waves are kLWM x 2 (4 x 2 by default), each (256/kLWM) x 128 of the tile: kLMI x 4 MFMA blocks
// of 32x32 (128 fp32 accumulators).  Two waves per SIMD hide each other's LDS waits and barrier
// skew; the price is 6 decode VALU per MFMA instead of 4 with 2 x 2 waves of 128 x 128.
// L1: tile weight rows 0..127 are gate rows nt*128.., 128..255 the matching up rows, so a wave
// holds gate and up of the same 64 h columns and applies SiLU(gate)*up in registers.
// L2: tile weight rows are output rows nt*256..+256.
// The epilogue stages the bf16 tile in LDS and writes it with 16-byte row-contiguous stores.
// ============================================================================================
#ifndef MEGAMOE_LARGE_WM
#define MEGAMOE_LARGE_WM 4
#endif
constexpr int kLBm = kBlockMLarge, kLBn = 256;
constexpr int kLWM = MEGAMOE_LARGE_WM, kLWN = 2;                 // waves along M and N
constexpr int kLWaves = kLWM * kLWN, kLThreads = kLWaves * kWave;
constexpr int kLMI = kLBm / 32 / kLWM;                           // 32-row MFMA blocks per wave
constexpr int kLRowsPerWave = kLBm / kLWaves;                    // DMA rows per wave and operand
constexpr int kLKs = 128, kLSlots = 4, kLAhead = 2;               // stage depth, ring slots, prefetch
constexpr int kLRowBytes = kLKs / 2;                             // code bytes of one row per stage
constexpr int kLChunks = kLRowBytes / 16;                        // 16-byte chunks per row (2 or 4)
constexpr int kLSwzShift = kLChunks == 2 ? 2 : 1;                // row bits that pick the swizzle
constexpr int kLScaleRow = kLKs / 16;                            // scale bytes of one row per stage
constexpr int kLSteps = kLKs / 16;                               // 32x32x16 MFMA steps per stage
constexpr int kLCodeBytes = kLBm * kLRowBytes;
constexpr int kLScaleBytes = kLBm * kLScaleRow;
constexpr int kLOpBytes = kLCodeBytes + kLScaleBytes;            // one operand, one stage
constexpr int kLStageBytes = 2 * kLOpBytes;
constexpr int kLLdsBytes = kLSlots * kLStageBytes;
constexpr int kLCodeDma = kLRowsPerWave * kLRowBytes / 1024;     // 16-byte DMA per wave and operand
constexpr int kLScaleDma = kLRowsPerWave * kLScaleRow / 256;     // 4-byte DMA per wave and operand
constexpr int kLDmaPerWave = 2 * (kLCodeDma + kLScaleDma);
constexpr int kLOutPitchL1 = 128 * 2 + 16, kLOutPitchL2 = 256 * 2 + 16;  // bf16 staging pitches
static_assert(kLKs == 64 || kLKs == 128, "stage depth");
static_assert(kLBm == 256 && kLBn == 256, "large tiles are 256x256");
static_assert(kLWM == 2 || kLWM == 4, "2x2 or 4x2 waves");
static_assert(kLCodeDma >= 1 && kLScaleDma >= 1 && kLRowsPerWave * kLScaleRow % 256 == 0, "DMA split");
static_assert(kLAhead <= kLSlots - 2, "refilled slot must have been read two stages earlier");
static_assert(kLBm * kLOutPitchL2 <= kLLdsBytes && kLBm * kLOutPitchL1 <= kLLdsBytes, "staging fits");

// Wait until at most `stages_after` (<= kLAhead) later stages' loads are outstanding for this wave.
template <int K = kLAhead>
__device__ __forceinline__ void wait_stage(int stages_after) {
  if constexpr (K == 0) {
    wait_vmcnt<0>();
  } else {
    if (stages_after >= K) wait_vmcnt<K * kLDmaPerWave>();
    else wait_stage<K - 1>(stages_after);
  }
}

template <bool kL1>
__global__ __launch_bounds__(kLThreads, 1) void gemm_large_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLLdsBytes];
  __shared__ int s_pref[kMaxExperts + 1];
  __shared__ uint32_t s_amax[kLWaves];
  const int E = p.E;
  for (int j = threadIdx.x; j <= E; j += blockDim.x) s_pref[j] = p.sched[sched_pref_large(E) + j];
  __syncthreads();
  const int ntn = kL1 ? p.N / 128 : p.N / kLBn;
  const int total = s_pref[E] * ntn;
  const int K = p.K, Kh = K / 2, Ks = K / 16;
  const int Nw = kL1 ? 2 * p.N : p.N;
  const int nks = K / kLKs;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int wm = wave / kLWN, wn = wave % kLWN;
  const int p32 = lane & 31, h2 = lane >> 5;
  const float gs_a = *p.a_gs;
  uint32_t amax_bits = 0;

  // first tile weight row of this wave's 32-column fragment f
  auto brow_of = [&](int f) {
    return kL1 ? (f < 2 ? wn * 64 + 32 * f : 128 + wn * 64 + 32 * (f - 2)) : wn * 128 + 32 * f;
  };

  const XcdTiles tl(total);
  for (int t = tl.t; t < tl.end; t += tl.stride) {
    const TileInfo ti = decode_tile(s_pref, E, ntn, t, kLBm, p.padded_offsets, p.counts);
    // ---- DMA sources of this lane --------------------------------------------------------------
    // codes: instruction j covers tile rows kLRowsPerWave*wave + j*rows_per + lane/kLChunks;
    // lane%kLChunks picks the LDS slot and the global chunk (lane%kLChunks) ^ swizzle(row) goes
    // there; scales: instruction j covers rows kLRowsPerWave*wave + 32j + lane/2, lane%2 picking
    // the 4-byte half (LDS scale layout: 8 bytes per row).
    auto a_row_of = [&](int R) -> int64_t {
      const int Rv = R < ti.rows_left ? R : 0;  // rows past the expert read row 0; never stored
      const int64_t r = ti.row0 + Rv;
      return kL1 ? (int64_t)p.row_token[r] : r;
    };
    auto b_row_of = [&](int R) -> int64_t {
      if (kL1) return (int64_t)ti.e * Nw + (R < 128 ? ti.nt * 128 + R : p.N + ti.nt * 128 + R - 128);
      return (int64_t)ti.e * Nw + ti.nt * kLBn + R;
    };
    constexpr int rows_per = 1024 / kLRowBytes;
    const uint8_t* a_code_src[kLCodeDma];
    const uint8_t* b_code_src[kLCodeDma];
#pragma unroll
    for (int j = 0; j < kLCodeDma; ++j) {
      const int R = kLRowsPerWave * wave + rows_per * j + lane / kLChunks;
      const int chunk = (lane % kLChunks) ^ ((R >> kLSwzShift) & (kLChunks - 1));
      a_code_src[j] = p.a_codes + a_row_of(R) * Kh + 16 * chunk;
      b_code_src[j] = p.w_codes + b_row_of(R) * Kh + 16 * chunk;
    }
    static_assert(kLScaleRow == 8, "scale DMA assumes 128-K stages");
    const uint8_t* a_scale_src[kLScaleDma];
    const uint8_t* b_scale_src[kLScaleDma];
#pragma unroll
    for (int j = 0; j < kLScaleDma; ++j) {
      const int R = kLRowsPerWave * wave + 32 * j + lane / 2;
      a_scale_src[j] = p.a_scales + a_row_of(R) * Ks + 4 * (lane & 1);
      b_scale_src[j] = p.w_scales + b_row_of(R) * Ks + 4 * (lane & 1);
    }

    f32x16 acc[kLMI][4];
#pragma unroll
    for (int i = 0; i < kLMI; ++i)
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.f;

    // kLDmaPerWave DMA instructions per wave: this wave's kLRowsPerWave rows of both operands.
    auto issue_stage = [&](int ks, int slot) {
      const uint32_t lb = lds_addr(smem + slot * kLStageBytes);
      const int64_t off = (int64_t)ks * kLRowBytes, soff = (int64_t)ks * kLScaleRow;
#pragma unroll
      for (int j = 0; j < kLCodeDma; ++j) {
        dma16(a_code_src[j] + off, lb + (kLRowsPerWave * wave + rows_per * j) * kLRowBytes);
        dma16(b_code_src[j] + off, lb + kLOpBytes + (kLRowsPerWave * wave + rows_per * j) * kLRowBytes);
      }
#pragma unroll
      for (int j = 0; j < kLScaleDma; ++j) {
        const int so = kLCodeBytes + (kLRowsPerWave * wave + 32 * j) * kLScaleRow;
        dma4(a_scale_src[j] + soff, lb + so);
        dma4(b_scale_src[j] + soff, lb + kLOpBytes + so);
      }
    };
    auto compute_stage = [&](int slot) {
      const uint8_t* base = smem + slot * kLStageBytes;
      const uint8_t* a_codes = base;
      const uint8_t* a_scales = base + kLCodeBytes;
      const uint8_t* b_codes = base + kLOpBytes;
      const uint8_t* b_scales = b_codes + kLCodeBytes;
      constexpr int CPL = kLChunks / 2;  // chunks per lane half
      // rows 32i + p and brow_of(f) + p share (row >> shift) with p: offsets are multiples of 32
      const int swz = (p32 >> kLSwzShift) & (kLChunks - 1);
      // scale bytes of this lane half: 2 (64-K stages) or 4 (128-K stages) per row
      auto scale_word = [&](const uint8_t* sp, int row) -> uint32_t {
        return *reinterpret_cast<const uint32_t*>(sp + row * kLScaleRow + 4 * h2);
      };
      u32x4 araw[kLMI][CPL], braw[4][CPL];
      uint32_t asw[kLMI], bsw[4];
#pragma unroll
      for (int i = 0; i < kLMI; ++i) {
        const int row = wm * (32 * kLMI) + 32 * i + p32;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
          araw[i][j] = *reinterpret_cast<const u32x4*>(a_codes + row * kLRowBytes + 16 * ((CPL * h2 + j) ^ swz));
        asw[i] = scale_word(a_scales, row);
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int row = brow_of(f) + p32;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
          braw[f][j] = *reinterpret_cast<const u32x4*>(b_codes + row * kLRowBytes + 16 * ((CPL * h2 + j) ^ swz));
        bsw[f] = scale_word(b_scales, row);
      }
      // fp16 scale pairs: pair q covers steps 4q..4q+3 (blocks 2q, 2q+1 of this lane half)
      f16x2 asc[kLMI][CPL], bsc[4][CPL];
#pragma unroll
      for (int i = 0; i < kLMI; ++i) {
        asc[i][0] = e4m3x2_to_f16(asw[i], false);
        if (CPL == 2) asc[i][CPL - 1] = e4m3x2_to_f16(asw[i], true);
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        bsc[f][0] = e4m3x2_to_f16(bsw[f], false);
        if (CPL == 2) bsc[f][CPL - 1] = e4m3x2_to_f16(bsw[f], true);
      }
      auto sc = [](const f16x2 (&pr)[CPL], int step) {
        const f16x2 v = pr[step >> 2];
        return (step & 2) ? bcast_hi(v) : bcast_lo(v);
      };
      auto word = [](const u32x4 (&r)[CPL], int step) { return r[step >> 2][step & 3]; };
      // Software pipeline: B fragments of step s+1 are decoded between the MFMAs of step s.
      constexpr int kBPerI = 4 / kLMI;             // B fragments decoded per A row block
      constexpr int kVPerM = 2 + 8 * kBPerI / 4;   // VALU per MFMA: (8 for A + 8 per B) / 4 MFMAs
      f16x8 b[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) b[f] = decode8(word(braw[f], 0), sc(bsc[f], 0));
#pragma unroll
      for (int st = 0; st < kLSteps; ++st) {
        f16x8 bn[4];
#pragma unroll
        for (int i = 0; i < kLMI; ++i) {
          const f16x8 a = decode8(word(araw[i], st), sc(asc[i], st));
          if (st + 1 < kLSteps) {
#pragma unroll
            for (int q = 0; q < kBPerI; ++q) {
              const int f = kBPerI * i + q;
              bn[f] = decode8(word(braw[f], st + 1), sc(bsc[f], st + 1));
            }
          }
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[i][f] = mfma32(a, b[f], acc[i][f]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, kVPerM, 0);  // its share of the decode
          }
        }
        if (st + 1 < kLSteps) {
#pragma unroll
          for (int f = 0; f < 4; ++f) b[f] = bn[f];
        }
      }
    };

    for (int ks = 0; ks < kLAhead && ks < nks; ++ks) issue_stage(ks, ks);
    for (int ks = 0; ks < nks; ++ks) {
      // Request stage ks+kLAhead into the slot last read by stage ks-2 (every wave has passed the
      // barrier of stage ks-1 since), then wait until this wave's stage-ks loads have landed.
      if (ks + kLAhead < nks) issue_stage(ks + kLAhead, (ks + kLAhead) % kLSlots);
      const int after = nks - 1 - ks;
      wait_stage(after < kLAhead ? after : kLAhead);
      __builtin_amdgcn_s_barrier();  // everyone's stage-ks loads have landed
      compute_stage(ks % kLSlots);
    }
    __syncthreads();  // all waves are done reading the ring before it is reused for staging

    // ---- epilogue: scale, (SiLU*up), bf16, stage in LDS, coalesced stores ----------------------
    // accumulator r of block (i, f) is row 32i + 8(r/4) + 4h + r%4, column 32f + p of the wave tile
    const float inv = (float)(1.0 / ((double)gs_a * (double)p.w_gs[ti.e]));
    constexpr int pitch = kL1 ? kLOutPitchL1 : kLOutPitchL2;
#pragma unroll
    for (int i = 0; i < kLMI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * (32 * kLMI) + 32 * i + 8 * (r >> 2) + 4 * h2 + (r & 3);
        const bool ok = row < ti.rows_left;
        if (kL1) {
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            const float gt = acc[i][f][r] * inv, up = acc[i][f + 2][r] * inv;
            const uint32_t hb = f32_to_bf16_bits(silu_f32(gt) * up);
            *reinterpret_cast<uint16_t*>(smem + row * pitch + 2 * (wn * 64 + 32 * f + p32)) = (uint16_t)hb;
            const uint32_t mag = ok ? (hb & 0x7FFFu) : 0u;
            amax_bits = amax_bits > mag ? amax_bits : mag;
          }
        } else {
#pragma unroll
          for (int f = 0; f < 4; ++f)
            *reinterpret_cast<uint16_t*>(smem + row * pitch + 2 * (wn * 128 + 32 * f + p32)) =
                (uint16_t)f32_to_bf16_bits(acc[i][f][r] * inv);
        }
      }
    }
    __syncthreads();
    {
      constexpr int cols = kL1 ? 128 : 256;
      constexpr int chunks = cols * 2 / 16;  // 16-byte chunks per row
      const int nrows = ti.rows_left < kLBm ? ti.rows_left : kLBm;
      uint16_t* __restrict__ out = reinterpret_cast<uint16_t*>(p.out);
      const int col0 = ti.nt * cols;
      for (int idx = tid; idx < nrows * chunks; idx += kLThreads) {
        const int r = idx / chunks, c = idx - r * chunks;
        const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * pitch + 16 * c);
        *reinterpret_cast<u32x4*>(out + (int64_t)(ti.row0 + r) * p.N + col0 + 8 * c) = v;
      }
    }
    __syncthreads();  // staging reads done before the next tile's DMA refills the ring
  }
  if (kL1) {
    amax_bits = wave_max_u32(amax_bits);
    if (lane == 0) s_amax[wave] = amax_bits;
    __syncthreads();
    if (tid == 0) {
      uint32_t m = s_amax[0];
      for (int w = 1; w < kLWaves; ++w) m = m > s_amax[w] ? m : s_amax[w];
      p.amax_out[blockIdx.x] = bf16_bits_to_f32(m);
      if (p.clear_other)
        for (int j = (int)blockIdx.x; j < kAmaxSmallSlots; j += kLargeGrid) p.amax_out[kLargeGrid + j] = 0.0f;
    }
  }
}

// Launch the tile classes the call may contain.  When only one class runs, its kernel also
// zeroes the other class's amax slots (clear_other), so every slot is written on every call.
template <bool kL1>
static hipError_t launch_gemm(GemmArgs a, GemmClasses c, hipStream_t stream) {
  a.clear_other = !(c.large && c.small);
  if (c.large) {
    hipLaunchKernelGGL(gemm_large_kernel<kL1>, dim3(kLargeGrid), dim3(kLThreads), 0, stream, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (c.small) {
    // Staged weight scales need every wave on K (K >= 4 chunks) and 3 buffers within 48 KB.
    const int Ks = a.K / 16, P = Ks / 16 + 1;
    const size_t buf = (size_t)((small_nb<kL1>() * 16 * P + 63) / 64) * 1024;
    const int ch = a.K % 256 == 0 ? 256 : 128;
    const bool staged = a.K / ch >= kSWaves && 3 * buf <= kSmallStagedMaxLds;
    const size_t dyn = staged ? 3 * buf : 0;
    if (ch == 256 && staged)
      hipLaunchKernelGGL((gemm_small_kernel<kL1, 256, true>), dim3(kSmallGrid), dim3(kGemmThreads), dyn, stream, a);
    else if (ch == 256)
      hipLaunchKernelGGL((gemm_small_kernel<kL1, 256, false>), dim3(kSmallGrid), dim3(kGemmThreads), 0, stream, a);
    else if (staged)
      hipLaunchKernelGGL((gemm_small_kernel<kL1, 128, true>), dim3(kSmallGrid), dim3(kGemmThreads), dyn, stream, a);
    else
      hipLaunchKernelGGL((gemm_small_kernel<kL1, 128, false>), dim3(kSmallGrid), dim3(kGemmThreads), 0, stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_gemm_l1(const GemmArgs& a, GemmClasses c, hipStream_t stream) { return launch_gemm<true>(a, c, stream); }

hipError_t launch_gemm_l2(const GemmArgs& a, GemmClasses c, hipStream_t stream) { return launch_gemm<false>(a, c, stream); }

}  // namespace megamoe
