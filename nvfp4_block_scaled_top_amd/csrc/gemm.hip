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
#include <atomic>

#include "device_common.h"
#include "internal.h"
#include "quant_device.h"

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
// about 2 VALU instructions per weight byte and lane; the design keeps every other VALU cost per
// weight byte small and every CU equally busy:
//  * work unit = a group: kSNb (small_nb) 16-column MFMA blocks of one m-tile over the whole K
//    (L1 blocks 2i and 2i+1: the gate rows and the up rows of h columns j0+16i..+15, so that
//    every weight load instruction reads 16 consecutive rows and gate and up of an h column meet
//    in the same lane after the reduction; L2 block j: weight rows j0+16j..);
//    L2 takes kSNbWide blocks per group when there are many groups per workgroup (see kSNbWide).
//    The width changes neither the K split nor any summation order: both give the same bits.
//    The groups of all small m-tiles are laid end to end and each workgroup takes an equal
//    contiguous range of whole groups.  The two workgroups that share a CU take neighbouring
//    ranges and the workgroups of one XCD a contiguous eighth (the A rows of an m-tile stay in
//    that XCD's L2);
//  * the 4 waves of a workgroup split K four ways and stream the same groups: weight codes come
//    straight into registers (CH/8 bytes per lane per CH-element chunk) through a kSDepth-deep
//    ring that runs on across group boundaries; the weights' block scales are copied per group
//    into LDS by direct-to-LDS loads (kStaged, see below);
//  * the A operand takes one of two forms.  M-tiles with at most kTinyRows = 512/CH token rows
//    (every m-tile at decode) run first, as the "tiny" phase: a lane loads one code word and one
//    scale byte of a dense [rows x CH] A chunk, decodes its 8 elements once, and the MFMA
//    fragments are read back from a per-wave LDS buffer (rows past the m-tile read row 0), so the
//    A operand costs 9 VALU per chunk instead of 8 per MFMA step.  The other m-tiles ("regular"
//    phase) gather each lane's A row and decode it per MFMA step, shared by the group's blocks;
//  * at the end of a group each wave leaves its partial blocks in LDS (double-buffered by group
//    parity) and, after one LDS-only barrier (the weight loads stay in flight), wave w adds the
//    partials of accumulator row w of every block in wave order (deterministic) and stores them
//    (L1 with a given global scale for h: each row's 16 h columns of a block pair are gathered
//    into one lane and stored as one NVFP4 block).
// Lanes whose row lies outside the group or m-tile load a valid row of the same tile instead; the
// MFMA outputs they feed are never stored.
// ============================================================================================
#ifndef MEGAMOE_SMALL_NB_L1
#define MEGAMOE_SMALL_NB_L1 2
#endif
#ifndef MEGAMOE_SMALL_NB_L2
#define MEGAMOE_SMALL_NB_L2 2
#endif
#ifndef MEGAMOE_SMALL_NB_L2_WIDE
#define MEGAMOE_SMALL_NB_L2_WIDE 4
#endif
#ifndef MEGAMOE_SMALL_DEPTH
#define MEGAMOE_SMALL_DEPTH 2
#endif
#ifndef MEGAMOE_SMALL_OCC
#define MEGAMOE_SMALL_OCC 2
#endif
#ifndef MEGAMOE_SMALL_STAGED
#define MEGAMOE_SMALL_STAGED 1
#endif
template <bool kL1>
constexpr int small_nb() { return kL1 ? MEGAMOE_SMALL_NB_L1 : MEGAMOE_SMALL_NB_L2; }  // blocks per group
// L2 with many groups per workgroup takes wider groups: the regular phase decodes each A row once
// per MFMA step for all blocks of a group, so 4 blocks halve that cost per weight byte (the
// 512-token prefill's L2: 757 -> 676 us), while with few groups per workgroup the coarser split
// balances worse (decode T=8: 22.0 -> 23.1 us).  The kernel takes the wide width when the narrow
// grouping gives every workgroup at least kWideMinGroups groups.
constexpr int kSNbWide = MEGAMOE_SMALL_NB_L2_WIDE;
constexpr int kWideMinGroups = 32;
constexpr int kSDepth = MEGAMOE_SMALL_DEPTH;  // ring slots (chunks in flight per wave)
constexpr int kSOcc = MEGAMOE_SMALL_OCC;      // workgroups (of 4 waves) per CU
constexpr int kSWaves = kGemmThreads / kWave; // K split
constexpr int kLargeGrid = 256;               // large class: one workgroup per CU (LDS ~148 KB)
constexpr int kSmallGrid = 256 * kSOcc;       // small class: resident workgroups
constexpr int kAmaxSmallSlots = MEGAMOE_L1_AMAX_PARTS - kLargeGrid;  // slots [kLargeGrid, PARTS)
// Dynamic LDS of the small class: the per-expert tables, then 3 staged scale buffers if kStaged.
// With kSOcc = 2 a workgroup may use 80 KB; the static arrays of a kernel whose groups have at
// most nb blocks take 8 KB per block (the double-buffered group-end partials) plus about 5 KB.
constexpr size_t small_dyn_max_lds(int nb) { return 160 * 1024 / kSOcc - (size_t)nb * 8 * 1024 - 6 * 1024; }
static_assert(kSmallGrid <= kAmaxSmallSlots, "one amax slot per small workgroup");
static_assert(kSmallGrid % kXcds == 0 && (kSmallGrid / kXcds) % kSOcc == 0, "grid split");

template <bool kL1, int NB = small_nb<kL1>()>
constexpr int small_group_units() { return kL1 ? 8 * NB : 16 * NB; }

// Bytes of the per-expert tables at the start of the small class's dynamic LDS (16-aligned).
__host__ __device__ constexpr size_t small_table_bytes(int E) { return (((size_t)5 * E + 1) * 4 + 15) / 16 * 16; }
static_assert(small_table_bytes(MEGAMOE_MAX_EXPERTS) <= small_dyn_max_lds(kSNbWide), "the tables fit beside wide groups");
// Bytes of one staged scale buffer: kSNb x 16 weight rows of Ks scale bytes, each row padded to
// (Ks/16 + 1) pieces of 16 bytes, rounded up to whole 1024-byte DMA instructions.
__host__ __device__ inline size_t small_scale_buf_bytes(int nb, int K) {
  const int P = K / 256 + 1;
  return (size_t)((nb * 16 * P + 63) / 64) * 1024;
}

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
// The same with the non-temporal hint: for bytes read once per call (the 16-row kernels' weight
// scales when they stream the packed codes).
__device__ __forceinline__ void dma16nt(const uint8_t* src, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds), "v"(src) : "memory", "m0");
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

// One chunk of the reduction dimension for one lane: CH/8 code bytes (CH/32 MFMA steps) of each
// of its kSNb weight rows, and its A operand: regular phase, CH/8 code bytes and CH/64 scale
// bytes of its A row; tiny phase, one code word (8 elements) and one scale byte of the dense
// A chunk.
template <int CH, int NB, bool kTiny>
struct SmallSlot {
  static constexpr int kQ = CH / 128;  // u32x4 words per lane and weight row (1 or 2)
  static constexpr int kAQ = kTiny ? 1 : kQ;
  u32x4 a[kAQ];  // tiny: a[0].x only
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

template <bool V>
struct BoolTag {
  static constexpr bool value = V;
};

// CH (128 or 256) is the chunk of K a wave step covers: a lane loads CH/8 contiguous code bytes
// (CH/32 MFMA steps) per weight row.  256 halves the scale traffic per weight byte; 128 serves K
// that is an odd multiple of 128.
// Weight scales staged in LDS (kStaged): a group's rows of weight block scales (row-contiguous in
// HBM) are copied by full-line direct-to-LDS loads when the loader enters the group, into buffer
// (group index) % 3, rows padded by 16 bytes so that the 4-byte reads of 16 rows x 4 lanes hit
// distinct banks.  The steady state then issues no scale loads for the weights.  The loader runs
// kSDepth = 2 steps ahead of the compute and enters group g right after loading the last chunk of
// group g-1, i.e. while the compute is at step C*g - 3 for a wave with C chunks per group: in group
// g-1 or g-2 when C >= 2.  Buffer g % 3 was last read in group g-3, whose barrier every wave has
// passed by then, so 3 buffers suffice -- only if every wave has at least 2 chunks per group (with
// C = 1 the copy of group g would land during group g-3's compute); the launch enables staging only
// then.  Every wave has issued at least kSDepth steps of loads after its copy of group q+1 when
// group q ends, so vmcnt <= kSDepth * (loads per step) there (before the group's barrier) means the
// copy has landed.
// LDS of the small class, owned by the kernels and handed to the passes: the per-expert tables
// (dynamic LDS, identical for L1 and L2 since both walk the routing step's m-tiles) and the
// group-end reduction buffers.
template <int NB>
struct SmallLds {
  int* pref;     // [E+1] exclusive prefix of regular small m-tiles
  int* poff;     // [E] first padded row
  int* cnt;      // [E] tokens
  int* tiny;     // experts whose one m-tile is tiny
  int* ntiny;    // [1] their number
  uint8_t* scl;  // [3][scale buffer] if staged
  f32x4 (*red)[kSWaves][NB][kWave];  // [2] partial blocks at a group end (by group parity)
  f16x8 (*afrag)[kWave];             // [kSWaves] tiny phase: the chunk's decoded A pieces
};

// Device-scope (every XCD) accesses.  The fused kernel below hands h from the workgroups that
// compute it to those that read it within one launch; the 8 XCDs' L2 caches are not coherent with
// each other, so those stores and loads are relaxed atomics at agent scope (gfx950: the sc1 bit;
// no cache-wide write-back or invalidate).
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u16(const uint8_t* p) {
  return __hip_atomic_load(reinterpret_cast<const uint16_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u8(const uint8_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x4 ld_dev_x4(const uint8_t* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Order of the handoff.  The producer's device-scope stores complete (s_waitcnt: vmcnt counts
// stores on gfx9) before its counter increment is issued; the consumer issues its device-scope
// loads only after its poll has seen the final count.  The hardware keeps both orders; a
// compiler-only fence at each end keeps the compiler from moving the relaxed accesses across them
// (no cache write-back or invalidate is emitted).
__device__ __forceinline__ void publish_fence() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Waits until the device-scope counter *c reaches target (wave-uniform; every lane of the wave
// calls it).  Bounded: after about a quarter of a second it sets *err and returns, so a broken
// dependency shows as an error word instead of a hang.
constexpr int kSpinLimit = 1 << 18;
__device__ __forceinline__ void wait_count(const uint32_t* c, uint32_t target, uint32_t* err) {
  for (int it = 0; it < kSpinLimit; ++it) {
    if ((uint32_t)__builtin_amdgcn_readfirstlane(ld_dev(c)) >= target) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      return;
    }
    __builtin_amdgcn_s_sleep(8);
  }
  st_dev(err, 1u);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The part of one phase's group list that work item `part` of `nparts` takes.
__device__ __forceinline__ void phase_part(int64_t part, int64_t nparts, int64_t groups, int64_t& begin,
                                           int64_t& end) {
  begin = part * groups / nparts;
  end = (part + 1) * groups / nparts;
}

// Fills the per-expert tables from the routing step's table and inv[e] = 1 / (gs_a * gs_w[e]) for
// the experts with small m-tiles (and inv2 likewise with gs_a2 and w_gs2 when inv2 is given).
// Small m-tiles are split into tiny ones (the expert's only m-tile, at most 512/CH rows) and
// regular ones.  Ends with a workgroup barrier.
template <int CH, int NB>
__device__ __forceinline__ void small_tables(const GemmArgs& p, const SmallLds<NB>& L, float* inv, float gs_a,
                                             float* inv2 = nullptr, float gs_a2 = 0.0f,
                                             const float* w_gs2 = nullptr) {
  constexpr int kTinyRows = kWave / (CH / 8);
  const int E = p.E;
  const int32_t* __restrict__ pref = p.sched + sched_pref_small(E);
  const int32_t* __restrict__ bm = p.sched + sched_block_m(E);
  for (int j = threadIdx.x; j < E; j += blockDim.x) {
    const int cnt = p.counts[j];
    L.poff[j] = p.padded_offsets[j];
    L.cnt[j] = cnt;
    // small m-tiles of expert j (scanned below); when the 256-row kernel is not launched, an
    // expert the routing step gave 256-row tiles is covered here in 16-row m-tiles
    int nt = pref[j + 1] - pref[j];
    if (p.small_covers_large && bm[j] == kBlockMLarge) nt = (cnt + kBlockMSmall - 1) / kBlockMSmall;
    L.pref[j] = nt;
    inv[j] = nt > 0 ? (float)(1.0 / ((double)gs_a * (double)p.w_gs[j])) : 0.0f;
    if (inv2) inv2[j] = nt > 0 ? (float)(1.0 / ((double)gs_a2 * (double)w_gs2[j])) : 0.0f;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {  // wave 0: split the small m-tiles into tiny and regular
    const int lane = lane_id();
    int reg_carry = 0, tiny_carry = 0;
    for (int c = 0; c < E; c += kWave) {
      const int e = c + lane;
      const int nt = e < E ? L.pref[e] : 0;
      const int cnt = e < E ? L.cnt[e] : 0;
      const bool tiny = nt == 1 && cnt <= kTinyRows;
      const int reg = tiny ? 0 : nt;
      int incl = reg;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
      }
      const uint64_t mask = __ballot(tiny);
      const int tpos = tiny_carry + __popcll(mask & ((1ull << lane) - 1));
      if (e < E) L.pref[e] = reg_carry + incl - reg;
      if (tiny) L.tiny[tpos] = e;
      reg_carry += __shfl(incl, kWave - 1, kWave);
      tiny_carry += __popcll(mask);
    }
    if (lane == 0) {
      L.pref[E] = reg_carry;
      *L.ntiny = tiny_carry;
    }
  }
  __syncthreads();
}

// What the fused kernel adds to a pass.  L2 (ready != NULL): before a group's A rows (h) are
// loaded, wait until the L1 groups of its expert are done (ready[e * kSyncStride] counts them;
// gm1 L1 groups per m-tile).  kDev: h is read (L2) or written (L1) with device-scope accesses.
constexpr int kSyncStride = kFfnSyncStride;  // words between per-expert counters (a 128-byte line)
struct SmallSync {
  const uint32_t* ready = nullptr;
  int gm1 = 0;
  uint32_t* err = nullptr;
};

// One pass of the small class over part `part` of `nparts` of its group lists (tiny m-tiles,
// then regular ones), for one workgroup.  inv: the pass's 1 / (gs_a * gs_w[e]).
// kPacked: the weight codes come from the packed copy (p.w_packed, see pack_codes16_kernel) with
// non-temporal loads, 1 KB contiguous per load instruction, instead of from the row-major codes.
template <bool kL1, int NB, int CH, bool kStaged, bool kQOut, bool kDev, bool kPacked = false>
__device__ __forceinline__ void small_pass(const GemmArgs& p, const SmallLds<NB>& L, const float* inv,
                                           int64_t part, int64_t nparts, uint32_t& amax_bits, int& parity,
                                           const SmallSync& sync) {
  static_assert(!kStaged || CH == 256, "staged scales copy whole 16-byte pieces: one per 256-element chunk");
  static_assert(!kPacked || CH == 256, "the packed codes are laid out in 256-element chunks");
  static_assert(!kL1 || NB % 2 == 0, "L1 NVFP4 h: a group holds whole 16-column blocks of h");
  constexpr int kSNb = NB;
  constexpr int kQ = CH / 128;
  constexpr int kLaneBytes = CH / 8, kLaneScales = CH / 64;
  constexpr int kPieces = CH / 8;               // 8-element pieces per row and chunk
  constexpr int kTinyRows = kWave / kPieces;    // rows of a dense A chunk (2 or 4)
  constexpr bool kDevA = kDev && !kL1;          // A (h) written by other workgroups of this launch
  constexpr bool kDevOut = kDev && kL1;         // h read by other workgroups of this launch
  const int E = p.E;
  const int* s_pref = L.pref;
  const int* s_poff = L.poff;
  const int* s_cnt = L.cnt;
  const int* s_tiny = L.tiny;
  uint8_t* s_scl = L.scl;
  constexpr bool quant_out = kL1 && kQOut;  // L1: NVFP4 h (q_codes, q_scales) instead of bf16 h
  const float gs_q = quant_out ? *p.q_gs : 1.0f;
  const int NU = p.N;  // units per m-tile: L1 h columns (I), L2 output columns (H)
  constexpr int GU = small_group_units<kL1, NB>();
  const int Gm = (NU + GU - 1) / GU;  // groups per m-tile
  const int K = p.K, Kh = K / 2, Ks = K / 16;
  const int Nw = kL1 ? 2 * p.N : p.N;  // weight rows per expert
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int nch = K / CH;
  const int ks = nch < kSWaves ? nch : kSWaves;  // waves sharing K (all 4 unless K < 4 chunks)
  const int c0 = wave < ks ? wave * nch / ks : 0, c1 = wave < ks ? (wave + 1) * nch / ks : 0;

  // Staged scales: buffer geometry (pieces of 16 bytes; P per padded row).
  const int P = Ks / 16 + 1, SRB = 16 * P;
  const int ndma = (kSNb * 16 * P + 63) / 64;
  const int buf_bytes = ndma * 1024;
  const float invP = 1.0f / (float)P;

  // One phase: the tiny m-tiles (kTiny) or the regular ones, as a list of groups.
  auto run_phase = [&](auto tiny_tag) {
    constexpr bool kTiny = decltype(tiny_tag)::value;
    using Slot = SmallSlot<CH, kSNb, kTiny>;
    constexpr int kLoadsPerStep =
        (kTiny ? 2 : (kDevA ? 2 * kQ : kQ) + 1) + kSNb * kQ + (kStaged ? 0 : kSNb);
    const int nm = kTiny ? *L.ntiny : s_pref[E];
    int64_t g_begin, g_end;
    phase_part(part, nparts, (int64_t)nm * Gm, g_begin, g_end);
    const int ngroups = (int)(g_end - g_begin);
    if (ngroups == 0) return;

    // Group cursor: m-tile mt (index in this phase's list), group gi within it, and its expert.
    struct Cursor {
      int mt, gi, e;
    };
    auto cursor_at = [&](int64_t gidx) {
      Cursor c;
      c.mt = (int)(gidx / Gm);
      c.gi = (int)(gidx - (int64_t)c.mt * Gm);
      c.e = kTiny ? s_tiny[c.mt] : find_expert(s_pref, E, 1, c.mt);
      return c;
    };
    auto cursor_next = [&](Cursor& c) {
      if (++c.gi == Gm) {
        c.gi = 0;
        ++c.mt;
        if (kTiny) c.e = s_tiny[c.mt];
        else
          while (s_pref[c.e + 1] <= c.mt) ++c.e;
      }
    };
    auto group_of = [&](const Cursor& c) {
      SmallGroup q;
      q.e = c.e;
      const int local = kTiny ? 0 : c.mt - s_pref[c.e];
      q.row0 = s_poff[c.e] + local * kBlockMSmall;
      q.rows_left = s_cnt[c.e] - local * kBlockMSmall;
      q.j0 = c.gi * GU;
      q.n = NU - q.j0 < GU ? NU - q.j0 : GU;
      return q;
    };

    // End of a group: publish the partial blocks; after the barrier wave w adds accumulator row
    // w of every block in wave order and writes it out.
    auto group_epilogue = [&](const SmallGroup& cg) {
      const float invg = inv[cg.e];
      const float* red = reinterpret_cast<const float*>(&L.red[parity][0][0][0]);
      uint16_t* __restrict__ out = reinterpret_cast<uint16_t*>(p.out);
      const int row = 4 * g + wave;  // MFMA output row of accumulator element `wave`
      // partial sums of block j, column `lane`, accumulator row `wave`, added in wave order
      auto reduced = [&](int j) {
        float r = red[((0 * kSNb + j) * kWave + lane) * 4 + wave];
        for (int w = 1; w < ks; ++w) r += red[((w * kSNb + j) * kWave + lane) * 4 + wave];
        return r;
      };
      if constexpr (kL1) {
        // block 2i holds the gate rows and block 2i+1 the up rows of h columns j0 + 16i + r16:
        // gate and up of a column meet in the same lane
        uint32_t hq[kSNb / 2];  // bf16 h of column 16i + r16
#pragma unroll
        for (int i = 0; i < kSNb / 2; ++i) {
          const float rg = reduced(2 * i), ru = reduced(2 * i + 1);
          const int hc = 16 * i + r16;
          const uint32_t hb = f32_to_bf16_bits(silu_f32(rg * invg) * (ru * invg));
          hq[i] = hb;
          if (hc < cg.n && row < cg.rows_left) {
            if (!quant_out) {
              uint16_t* dst = out + (int64_t)(cg.row0 + row) * p.N + cg.j0 + hc;
              if (kDevOut) st_dev(dst, (uint16_t)hb);
              else *dst = (uint16_t)hb;
            }
            const uint32_t mag = hb & 0x7FFFu;
            amax_bits = amax_bits > mag ? amax_bits : mag;
          }
        }
        if constexpr (quant_out) {
          // NVFP4 h: the 16 columns 16i.. of row `row` (one 16-element block) are the 16 lanes
          // 16g + e, register i.  The 16 lanes reduce the block's amax, each derives the block
          // scale and codes its own element (the quantizer's block_scale / e2m1_code), and the
          // codes are gathered into lane 16g (element 2k in the low nibble of byte k), which stores
          // the block.
#pragma unroll
          for (int i = 0; i < kSNb / 2; ++i) {
            const uint32_t e0 = hq[i] & 0xFFFFu;
            uint32_t m = e0 & 0x7FFFu;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
              const uint32_t t = __shfl_xor(m, o, kWave);
              m = m > t ? m : t;
            }
            float th[7];
            const uint32_t sc = block_scale(m, gs_q, th);
            const uint32_t c = e2m1_code(e0, gs_q, th, sc == 0);
            const uint32_t b1 = c | (__shfl_xor(c, 1, kWave) << 4);     // lane 2k: byte k
            const uint32_t b2 = b1 | (__shfl_xor(b1, 2, kWave) << 8);   // lane 4k: bytes 2k, 2k+1
            const uint32_t b4 = b2 | (__shfl_xor(b2, 4, kWave) << 16);  // lane 8k: bytes 4k..4k+3
            const uint32_t hi = __shfl_xor(b4, 8, kWave);               // lane 16g: bytes 4..7
            if (r16 == 0 && 16 * i < cg.n && row < cg.rows_left) {
              const int64_t orow = cg.row0 + row;
              const int col = cg.j0 + 16 * i;
              uint8_t* cdst = p.q_codes + orow * (p.N / 2) + col / 2;
              uint8_t* sdst = p.q_scales + orow * (p.N / 16) + col / 16;
              if (kDevOut) {
                st_dev(reinterpret_cast<uint64_t*>(cdst), (uint64_t)b4 | ((uint64_t)hi << 32));
                st_dev(sdst, (uint8_t)sc);
              } else {
                *reinterpret_cast<u32x2*>(cdst) = u32x2{b4, hi};
                *sdst = (uint8_t)sc;
              }
            }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < kSNb; ++j) {
          const float r = reduced(j);
          const int rc = 16 * j + r16;
          if (rc < cg.n && row < cg.rows_left)
            out[(int64_t)(cg.row0 + row) * p.N + cg.j0 + rc] = (uint16_t)f32_to_bf16_bits(r * invg);
        }
      }
      parity ^= 1;
    };

    if (c1 == c0) {
      // K has fewer than 4 chunks and this wave has none: it keeps the barrier count and takes
      // its share of the epilogues.
      Cursor cc = cursor_at(g_begin);
      for (int q = 0; q < ngroups; ++q) {
        lds_barrier();
        group_epilogue(group_of(cc));
        if (q + 1 < ngroups) cursor_next(cc);
      }
      return;
    }

    // ---- loader: group being loaded, this lane's row pointers, next chunk ----------------------
    // Past the last step the loader keeps re-reading its last group's first chunk (valid memory,
    // never consumed), so every step issues the same loads.
    Cursor lcur = cursor_at(g_begin);
    int lgrp = 0, lc = c0;
    int ready_e = -1;  // fused L2: the last expert whose h is known to be complete
    const uint8_t* la_c = p.a_codes;
    const uint8_t* la_s = p.a_scales;
    const uint8_t* lb_c[kSNb];
    const uint8_t* lb_s[kSNb];
#pragma unroll
    for (int j = 0; j < kSNb; ++j) {
      lb_c[j] = p.w_codes;
      lb_s[j] = p.w_scales;
    }
    auto weight_row = [&](const SmallGroup& q, int col) -> int64_t {  // MFMA column -> weight row
      if (kL1) {
        const int j = col / 16, c = col % 16;
        const int hc = 16 * (j / 2) + c;
        const int hcol = q.j0 + (hc < q.n ? hc : 0);
        return (int64_t)q.e * Nw + ((j & 1) ? p.N + hcol : hcol);
      }
      return (int64_t)q.e * Nw + q.j0 + (col < q.n ? col : 0);
    };
    auto stage_scales = [&](const SmallGroup& q, int buf) {
      const uint32_t base = lds_addr(s_scl + buf * buf_bytes);
      for (int i = wave; i < ndma; i += kSWaves) {
        const int pc = 64 * i + lane;
        const int cr = (int)(((float)pc + 0.5f) * invP);  // pc / P (exact for pc < 2^21)
        const int pi = pc - cr * P;
        const bool real = cr < kSNb * 16 && pi < P - 1;
        const uint8_t* src = p.w_scales + weight_row(q, real ? cr : 0) * Ks + (real ? 16 * pi : 0);
        if constexpr (kPacked) dma16nt(src, base + 1024 * i);  // read once, like the packed codes
        else dma16(src, base + 1024 * i);
      }
    };
    auto loader_enter = [&]() {
      const SmallGroup q = group_of(lcur);
      if (kStaged) stage_scales(q, lgrp % 3);
      ++lgrp;
      if (kDevA && sync.ready != nullptr && q.e != ready_e) {
        // the h rows of this expert are written by the L1 groups of its m-tiles
        const int nmt = kTiny ? 1 : s_pref[q.e + 1] - s_pref[q.e];
        wait_count(sync.ready + q.e * kSyncStride, (uint32_t)(sync.gm1 * nmt), sync.err);
        ready_e = q.e;
      }
      if (kTiny) {
        // dense A: lane -> (row lane / kPieces, piece lane % kPieces); rows past the m-tile read
        // row 0
        const int rr = lane / kPieces, pc = lane % kPieces;
        int64_t arow;
        if (kL1) {
          int tok = sload(p.row_token, q.row0);
#pragma unroll
          for (int i = 1; i < kTinyRows; ++i) {
            if (i < q.rows_left) {
              const int t = sload(p.row_token, q.row0 + i);
              tok = rr == i ? t : tok;
            }
          }
          arow = tok;
        } else {
          arow = q.row0 + (rr < q.rows_left ? rr : 0);
        }
        la_c = p.a_codes + arow * Kh + 4 * pc;
        la_s = p.a_scales + arow * Ks + pc / 2;
      } else {
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
      }
#pragma unroll
      for (int j = 0; j < kSNb; ++j) {
        int64_t brow;
        if (kL1) {
          const int hc = 16 * (j / 2) + r16;
          const int col = q.j0 + (hc < q.n ? hc : 0);
          brow = (int64_t)q.e * Nw + ((j & 1) ? p.N + col : col);
        } else {
          const int rc = 16 * j + r16;
          brow = (int64_t)q.e * Nw + q.j0 + (rc < q.n ? rc : 0);
        }
        if constexpr (kPacked) {
          // the block's 16 consecutive weight rows (whole: N % 16 == 0); a block past the
          // group's units re-reads the group's first block
          const int u0 = kL1 ? 16 * (j / 2) : 16 * j;
          const int64_t r0 = (int64_t)q.e * Nw + ((kL1 && (j & 1)) ? p.N : 0) + q.j0 + (u0 < q.n ? u0 : 0);
          lb_c[j] = p.w_packed + r0 * Kh + 16 * lane;
        } else {
          lb_c[j] = p.w_codes + brow * Kh + g * kLaneBytes;
        }
        lb_s[j] = p.w_scales + brow * Ks + g * kLaneScales;
      }
    };
    loader_enter();
    auto load_scale = [](const uint8_t* q) -> uint32_t {
      if (kDevA) return kLaneScales == 4 ? ld_dev(reinterpret_cast<const uint32_t*>(q)) : ld_dev_u16(q);
      if (kLaneScales == 4) return *reinterpret_cast<const uint32_t*>(q);
      return *reinterpret_cast<const uint16_t*>(q);
    };
    auto load = [&](Slot& d) {
      const int64_t off = (int64_t)lc * (CH / 2), soff = (int64_t)lc * (CH / 16);
      if (kTiny) {
        if (kDevA) {
          d.a[0].x = ld_dev(reinterpret_cast<const uint32_t*>(la_c + off));
          d.as = ld_dev_u8(la_s + soff);
        } else {
          d.a[0].x = *reinterpret_cast<const uint32_t*>(la_c + off);
          d.as = *(la_s + soff);
        }
      } else {
#pragma unroll
        for (int q = 0; q < kQ; ++q)
          d.a[q] = kDevA ? ld_dev_x4(la_c + off + 16 * q) : *reinterpret_cast<const u32x4*>(la_c + off + 16 * q);
        d.as = load_scale(la_s + soff);
      }
#pragma unroll
      for (int j = 0; j < kSNb; ++j) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          // packed: chunk lc of a block is 2 KB, instruction q its q-th KB
          if constexpr (kPacked)
            d.b[j][q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(lb_c[j] + 16 * off + 1024 * q));
          else
            d.b[j][q] = *reinterpret_cast<const u32x4*>(lb_c[j] + off + 16 * q);
        }
        if (!kStaged) d.bs[j] = load_scale(lb_s[j] + soff);
      }
      if (++lc == c1) {
        lc = c0;
        if (lgrp < ngroups) {
          cursor_next(lcur);
          loader_enter();
        }
      }
    };

    // ---- compute cursor ---------------------------------------------------------------------------
    Cursor ccur = cursor_at(g_begin);
    SmallGroup cg = group_of(ccur);
    int cc = c0, cgrp = 0;  // chunk, group index
    f32x4 acc[kSNb];
#pragma unroll
    for (int j = 0; j < kSNb; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Tiny phase: MFMA step st of lane L takes piece (CH/32)*(L/16) + st of row (L % 16), or of
    // row 0 when that row is past the m-tile.
    int tsrc = (r16 < cg.rows_left ? r16 : 0) * kPieces + (CH / 32) * g;

    // MFMA step st takes the lane's code word st (8 elements, scale block st / 2).
    auto compute = [&](const Slot& d) {
      uint32_t bsw[kSNb];
      if (kStaged) {
        // this lane's scale bytes of chunk cc for its row in each block (LDS, padded rows)
        const uint8_t* sb0 = s_scl + (cgrp % 3) * buf_bytes + r16 * SRB + cc * (CH / 16) + g * kLaneScales;
#pragma unroll
        for (int j = 0; j < kSNb; ++j) {
          if (kLaneScales == 4) bsw[j] = *reinterpret_cast<const uint32_t*>(sb0 + 16 * j * SRB);
          else bsw[j] = *reinterpret_cast<const uint16_t*>(sb0 + 16 * j * SRB);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kSNb; ++j) bsw[j] = d.bs[j];
      }
      f16x2 sb[kSNb][kQ];
#pragma unroll
      for (int q = 0; q < kQ; ++q)
#pragma unroll
        for (int j = 0; j < kSNb; ++j) sb[j][q] = e4m3x2_to_f16(bsw[j], q == 1);
      if (kTiny) {
        L.afrag[wave][lane] = decode8(d.a[0].x, bcast_lo(e4m3x2_to_f16(d.as, false)));
#pragma unroll
        for (int st = 0; st < CH / 32; ++st) {
          const int q = st / 4, w4 = st % 4;
          const f16x8 a = L.afrag[wave][tsrc + st];
#pragma unroll
          for (int j = 0; j < kSNb; ++j) {
            const f16x8 w = decode8(d.b[j][q][w4], w4 < 2 ? bcast_lo(sb[j][q]) : bcast_hi(sb[j][q]));
            acc[j] = mfma16(a, w, acc[j]);
          }
        }
      } else {
        f16x2 sa[kQ];
#pragma unroll
        for (int q = 0; q < kQ; ++q) sa[q] = e4m3x2_to_f16(d.as, q == 1);
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
      }
    };

    // (Staged scales: the next group's copy has landed for this wave once vmcnt <= kSDepth steps
    // of loads; in the predicated tail fewer loads follow it, so wait for all.)
    auto group_end = [&](bool tail) {
#pragma unroll
      for (int j = 0; j < kSNb; ++j) {
        L.red[parity][wave][j][lane] = acc[j];
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (kStaged) {
        if (tail) wait_vmcnt<0>();
        else wait_vmcnt<kSDepth * kLoadsPerStep>();
      }
      lds_barrier();
      group_epilogue(cg);
    };
    auto step_done = [&](bool tail) {
      if (++cc == c1) {
        group_end(tail);
        cc = c0;
        ++cgrp;
        if (cgrp < ngroups) {
          cursor_next(ccur);
          cg = group_of(ccur);
          if (kTiny) tsrc = (r16 < cg.rows_left ? r16 : 0) * kPieces + (CH / 32) * g;
        }
      }
    };

    // Steady state: step s computes ring slot s % kSDepth and refills it with step s + kSDepth.
    // Loads are unconditional in the prologue and the main loop (so the compiler's in-order vmcnt
    // waits keep kSDepth - 1 steps in flight); only the last < 2 kSDepth steps are predicated.
    const int S = ngroups * (c1 - c0);
    Slot ring[kSDepth];
#pragma unroll
    for (int k = 0; k < kSDepth; ++k) load(ring[k]);
    if (kStaged) {  // the first group's scales (issued before the prologue loads) have landed
      wait_vmcnt<kSDepth * kLoadsPerStep>();
      lds_barrier();
    }
    int s0 = 0;
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
  };

  run_phase(BoolTag<true>{});
  run_phase(BoolTag<false>{});
}

// kNbMax: the widest group the kernel may take (L2: kSNbWide when the launch sized the staged
// scale buffers for it, else the narrow width); the dynamic LDS holds scale buffers of that width.
template <bool kL1, int CH, bool kStaged, bool kQOut, int kNbMax, bool kPacked = false>
__global__ __launch_bounds__(kGemmThreads, kSOcc) void gemm_small_kernel(GemmArgs p) {
  constexpr int kSNb = small_nb<kL1>();
  static_assert(kNbMax >= kSNb && (kL1 ? kNbMax == kSNb : kNbMax % kSNb == 0), "group widths");
  extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
  __shared__ f32x4 s_red[2][kSWaves][kNbMax][kWave];
  __shared__ f16x8 s_afrag[kSWaves][kWave];  // tiny phase: this chunk's decoded A pieces
  __shared__ uint32_t s_amax[kSWaves];
  __shared__ int s_ntiny;
  const int E = p.E;
  // Per-expert tables (LDS; reading them inside the loop must not wait on the weight stream).
  SmallLds<kSNb> L;
  L.pref = reinterpret_cast<int*>(s_dyn);
  L.poff = L.pref + E + 1;
  L.cnt = L.poff + E;
  float* s_inv = reinterpret_cast<float*>(L.cnt + E);  // [E] 1 / (gs_a * gs_w[e])
  L.tiny = reinterpret_cast<int*>(s_inv + E);
  L.ntiny = &s_ntiny;
  L.scl = s_dyn + small_table_bytes(E);
  L.red = reinterpret_cast<f32x4 (*)[kSWaves][kSNb][kWave]>(&s_red[0][0][0][0]);
  L.afrag = s_afrag;

  // This workgroup's position: workgroup b runs on XCD b % 8; the kSOcc workgroups of a CU (XCD-
  // local indices i and i + 256/8) get neighbouring positions.
  const int G = kSmallGrid, b = blockIdx.x;
  constexpr int kPerXcd = kSmallGrid / kXcds, kCusPerXcd = kPerXcd / kSOcc;
  const int xi = b / kXcds;
  const int64_t lb = (int64_t)(b % kXcds) * kPerXcd + (xi % kCusPerXcd) * kSOcc + xi / kCusPerXcd;

  uint32_t amax_bits = 0;
  int parity = 0;  // s_red buffer of the next group end (continues across phases)
  // The m-tile totals of the routing step's table header: with none for this class (e.g. a decode
  // step without a local token) the tables are not built and only the amax slots are written.
  if (sload(p.sched, 1) + (p.small_covers_large ? sload(p.sched, 2) : 0) > 0) {
    small_tables<CH>(p, L, s_inv, *p.a_gs);
    bool wide = false;
    if constexpr (kNbMax > kSNb) {  // every workgroup derives the same choice from the same tables
      constexpr int GU = small_group_units<kL1>();
      const int64_t narrow_groups = (int64_t)(s_ntiny + L.pref[E]) * ((p.N + GU - 1) / GU);
      wide = narrow_groups >= (int64_t)kWideMinGroups * G;
    }
    if (wide) {
      const SmallLds<kNbMax> W{L.pref, L.poff, L.cnt, L.tiny, L.ntiny, L.scl,
                               reinterpret_cast<f32x4 (*)[kSWaves][kNbMax][kWave]>(&s_red[0][0][0][0]), s_afrag};
      small_pass<kL1, kNbMax, CH, kStaged, kQOut, false, kPacked>(p, W, s_inv, lb, G, amax_bits, parity, SmallSync{});
    } else {
      small_pass<kL1, kSNb, CH, kStaged, kQOut, false, kPacked>(p, L, s_inv, lb, G, amax_bits, parity, SmallSync{});
    }
  }

  if (kL1) {
    const int wave = threadIdx.x / kWave, lane = lane_id();
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
// L1 -> requantization of h -> L2 of the small class in one persistent launch (decode).
//
// The layer's S3, S4 and S5 (CURRENT_BUG.md@2e65594, "Test Plan" Phase 1) as one kernel, so that a
// decode step pays one kernel boundary fewer with a calibrated global scale for h (S4 is then the
// L1 epilogue) and two fewer without.  Work items, taken in order from a device-scope ticket
// counter of the workgroup's XCD (each XCD takes a contiguous eighth of every kind of item):
//  1. the L1 parts: the group lists of gemm_small_kernel cut into at most 512 parts, computed by
//     the same pass (same groups, same K split and reduction order: bit-identical results);
//  2. without a calibrated scale, the quantization parts of h: the global scale of h needs the
//     amax of all of h, so they wait until every L1 part is done (the method's grid-wide barrier)
//     and then quantize a share of h's rows each, as nvfp4_quantize_act does;
//  3. the L2 parts.  With a calibrated scale a group waits only until the L1 groups of its expert
//     are done (per-expert counters); otherwise until every quantization part is done.
// A workgroup claims an item only while it runs, and only after finishing the previous one; an item
// waits only for L1 (or quantization) items.  A workgroup of XCD x waits only once every L1 item
// of x is claimed, by a running workgroup that will finish it without waiting, and the slots of XCD
// y can hold only y's workgroups, which take y's L1 items before anything else: the launch needs no
// co-residency (no cooperative launch) and cannot deadlock, as long as every XCD receives
// workgroups (512 of them over the 8 XCDs of the GPU).  Claiming the next item while computing the
// current one was slower: the items are as large as a workgroup's share of a GEMM, and workgroups
// that started first took a second one.  h and the amax slots go from workgroup to
// workgroup through device-scope stores and loads, after which the counters are incremented; the
// waits are bounded (an expired wait sets the error word).  The sync words start at zero and the
// last workgroup to leave sets them back to zero, so replays of a captured graph need no reset.
// ============================================================================================
// Sync words: the ticket counter of XCD x at 32x (x < 8), then the exit, L1-done and
// quantization-done counters and the error word, each on a 128-byte line of its own; per-expert
// counters from kSyncHeader on.
constexpr int kSyncExit = 256, kSyncL1 = 288, kSyncQ = 320, kSyncHeader = kFfnSyncHeader;
constexpr int kFfnQuantBlocks = 256;  // 16-element blocks of h per quantization part (one per thread)
constexpr int kFfnMaxQuantParts = 512;
static_assert(MEGAMOE_FFN_SYNC_ERROR_WORD == 352 && kSyncHeader >= 384, "sync word layout");

// Bytes of the fused kernel's per-expert tables: those of the small class plus the L2 inv.
__host__ __device__ inline size_t ffn_table_bytes(int E) { return (((size_t)6 * E + 1) * 4 + 15) / 16 * 16; }

template <int CH, bool kStaged, bool kCal, bool kPacked = false>
__global__ __launch_bounds__(kGemmThreads, kSOcc) void ffn_small_kernel(FfnArgs a) {
  constexpr int kSNb = small_nb<true>();
  static_assert(small_nb<false>() == kSNb, "the two passes share the reduction buffers");
  extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
  __shared__ f32x4 s_red[2][kSWaves][kSNb][kWave];
  __shared__ f16x8 s_afrag[kSWaves][kWave];
  __shared__ uint32_t s_amax[kSWaves];
  __shared__ int s_ntiny;
  __shared__ uint32_t s_ticket;
  uint32_t* const sync = a.sync;
  uint32_t* const err = sync + MEGAMOE_FFN_SYNC_ERROR_WORD;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  // This workgroup's XCD (hardware register XCC_ID), among the nxcd of the device.
  const int xcd = (int)((__builtin_amdgcn_s_getreg((31 << 11) | 20) & 0xFu) % (uint32_t)a.nxcd);
  uint32_t* const ticket = sync + 32 * xcd;
  const GemmArgs& p1 = a.l1;
  const GemmArgs& p2 = a.l2;
  const int E = p1.E;
  if (sload(p1.sched, 1) + sload(p1.sched, 2) == 0) {
    // No m-tile (a decode step without a local token): no counter is touched.  The amax slots
    // are zero; without a calibrated scale h's codes are zero on every row and gs_h = 1, as the
    // quantizer writes them when no row is valid.
    for (int j = blockIdx.x * kGemmThreads + threadIdx.x; j < MEGAMOE_L1_AMAX_PARTS; j += gridDim.x * kGemmThreads)
      p1.amax_out[j] = 0.0f;
    if (!kCal) {
      const int64_t qblocks = a.M_cap * (p1.N / 16);
      for (int64_t j = (int64_t)blockIdx.x * kGemmThreads + threadIdx.x; j < qblocks;
           j += (int64_t)gridDim.x * kGemmThreads) {
        *reinterpret_cast<u32x2*>(a.hq_codes + j * 8) = u32x2{0u, 0u};
        a.hq_scales[j] = 0;
      }
      if (blockIdx.x == 0 && threadIdx.x == 0) *a.h_gs = 1.0f;
    }
    return;
  }
  uint32_t t_next = 0;
  if (threadIdx.x == 0) t_next = add_dev(ticket, 1u);  // the first claim, while the tables load
  SmallLds<kSNb> L;
  L.pref = reinterpret_cast<int*>(s_dyn);
  L.poff = L.pref + E + 1;
  L.cnt = L.poff + E;
  float* inv1 = reinterpret_cast<float*>(L.cnt + E);
  L.tiny = reinterpret_cast<int*>(inv1 + E);
  float* inv2 = reinterpret_cast<float*>(L.tiny + E);
  L.ntiny = &s_ntiny;
  L.scl = s_dyn + ffn_table_bytes(E);
  L.red = s_red;
  L.afrag = s_afrag;
  if (kCal) small_tables<CH>(p1, L, inv1, *p1.a_gs, inv2, *p2.a_gs, p2.w_gs);
  else small_tables<CH>(p1, L, inv1, *p1.a_gs);

  // Item counts (every workgroup derives the same from the same tables).
  const int mtiles = s_ntiny + L.pref[E];
  const int gm1 = (p1.N + small_group_units<true>() - 1) / small_group_units<true>();
  const int gm2 = (p2.N + small_group_units<false>() - 1) / small_group_units<false>();
  const int64_t n1 = (int64_t)mtiles * gm1 < kSmallGrid ? (int64_t)mtiles * gm1 : kSmallGrid;
  const int64_t n2 = (int64_t)mtiles * gm2 < kSmallGrid ? (int64_t)mtiles * gm2 : kSmallGrid;
  const int64_t qblocks = a.M_cap * (p1.N / 16);
  int64_t nq = 0;
  if (!kCal) {
    nq = (qblocks + kFfnQuantBlocks - 1) / kFfnQuantBlocks;
    if (nq > kFfnMaxQuantParts) nq = kFfnMaxQuantParts;
  }
  // this XCD's share of each kind of item
  const int nx = a.nxcd;
  const int64_t b1 = n1 * xcd / nx, c1 = n1 * (xcd + 1) / nx - b1;
  const int64_t bq = nq * xcd / nx, cq = nq * (xcd + 1) / nx - bq;
  const int64_t b2 = n2 * xcd / nx, c2 = n2 * (xcd + 1) / nx - b2;
  const int64_t total = c1 + cq + c2;

  // amax slots no L1 part writes: zero (read only after the launch)
  for (int j = blockIdx.x * kGemmThreads + threadIdx.x; j < MEGAMOE_L1_AMAX_PARTS; j += gridDim.x * kGemmThreads)
    if (j < kLargeGrid || j >= kLargeGrid + n1) p1.amax_out[j] = 0.0f;

  SmallSync l2sync;
  if (kCal) {
    l2sync.ready = sync + kSyncHeader;
    l2sync.gm1 = gm1;
    l2sync.err = err;
  }
  bool inv2_ready = kCal;
  uint32_t amax_bits = 0;
  int parity = 0;  // s_red buffer of the next group end (continues across items)
  for (;;) {
    if (threadIdx.x == 0) s_ticket = t_next;
    __syncthreads();
    const int64_t tx = s_ticket;
    __syncthreads();
    if (tx >= total) break;
    // the global item: L1 part t < n1, quantization part t - n1 < nq, L2 part t - n1 - nq
    const int64_t t = tx < c1 ? b1 + tx : tx < c1 + cq ? n1 + bq + (tx - c1) : n1 + nq + b2 + (tx - c1 - cq);
    if (t < n1) {
      small_pass<true, kSNb, CH, kStaged, kCal, true, kPacked>(p1, L, inv1, t, n1, amax_bits, parity, SmallSync{});
      // Publish: this wave's h stores have completed (vmcnt counts stores), then the counts.
      amax_bits = wave_max_u32(amax_bits);
      if (lane == 0) s_amax[wave] = amax_bits;
      amax_bits = 0;
      publish_fence();
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t m = s_amax[0];
        for (int w = 1; w < kSWaves; ++w) m = m > s_amax[w] ? m : s_amax[w];
        st_dev(p1.amax_out + kLargeGrid + t, bf16_bits_to_f32(m));
        if (kCal) {
          // per expert, the L1 groups of this part (both phases)
          for (int ph = 0; ph < 2; ++ph) {
            const int nm = ph == 0 ? s_ntiny : L.pref[E];
            int64_t gb, ge;
            phase_part(t, n1, (int64_t)nm * gm1, gb, ge);
            while (gb < ge) {
              const int mt = (int)(gb / gm1);
              const int64_t hi = (int64_t)(mt + 1) * gm1 < ge ? (int64_t)(mt + 1) * gm1 : ge;
              const int ex = ph == 0 ? L.tiny[mt] : find_expert(L.pref, E, 1, mt);
              add_dev(sync + kSyncHeader + ex * kSyncStride, (uint32_t)(hi - gb));
              gb = hi;
            }
          }
        } else {
          publish_fence();  // the amax slot before the count
          add_dev(sync + kSyncL1, 1u);
        }
      }
    } else if (!kCal && t < n1 + nq) {
      // Quantization part: wait for every L1 part, reduce the amax slots, quantize a share of h.
      const int64_t s = t - n1;
      if (threadIdx.x == 0) wait_count(sync + kSyncL1, (uint32_t)n1, err);
      __syncthreads();
      uint32_t am = 0;
      for (int j = threadIdx.x; j < n1; j += kGemmThreads) {
        const uint32_t v = ld_dev(reinterpret_cast<const uint32_t*>(p1.amax_out + kLargeGrid + j));
        am = am > v ? am : v;  // non-negative floats: uint order is float order
      }
      am = wave_max_u32(am);
      if (lane == 0) s_amax[wave] = am;
      __syncthreads();
      am = s_amax[0];
      for (int w = 1; w < kSWaves; ++w) am = am > s_amax[w] ? am : s_amax[w];
      const float gs = global_scale_of(__uint_as_float(am));
      if (s == 0 && threadIdx.x == 0) st_dev(a.h_gs, gs);
      int64_t bb, be;
      phase_part(s, nq, qblocks, bb, be);
      const int64_t bpr = p1.N / 16;
      const uint8_t* hsrc = reinterpret_cast<const uint8_t*>(p1.out);
      for (int64_t blk = bb + threadIdx.x; blk < be; blk += kGemmThreads) {
        uint64_t* cd = reinterpret_cast<uint64_t*>(a.hq_codes + blk * 8);
        uint8_t* sd = a.hq_scales + blk;
        if (a.row_valid[blk / bpr] < 0) {
          st_dev(cd, (uint64_t)0);
          st_dev(sd, (uint8_t)0);
          continue;
        }
        const u32x4 v0 = ld_dev_x4(hsrc + blk * 32), v1 = ld_dev_x4(hsrc + blk * 32 + 16);
        uint32_t o[2];
        const uint32_t sc = quant16(v0, v1, gs, o);
        st_dev(cd, (uint64_t)o[0] | ((uint64_t)o[1] << 32));
        st_dev(sd, (uint8_t)sc);
      }
      publish_fence();
      __syncthreads();
      if (threadIdx.x == 0) add_dev(sync + kSyncQ, 1u);
    } else {
      if (!inv2_ready) {  // the first L2 part of this workgroup: h and its global scale are final
        if (threadIdx.x == 0) wait_count(sync + kSyncQ, (uint32_t)nq, err);
        __syncthreads();
        const float gs_h = __uint_as_float(ld_dev(reinterpret_cast<const uint32_t*>(a.h_gs)));
        for (int j = threadIdx.x; j < E; j += kGemmThreads)
          inv2[j] = L.cnt[j] > 0 ? (float)(1.0 / ((double)gs_h * (double)p2.w_gs[j])) : 0.0f;
        __syncthreads();
        inv2_ready = true;
      }
      small_pass<false, kSNb, CH, kStaged, false, true, kPacked>(p2, L, inv2, t - n1 - nq, n2, amax_bits, parity, l2sync);
    }
    if (threadIdx.x == 0) t_next = add_dev(ticket, 1u);
  }

  // Leave; the last workgroup out sets the counters back to zero (everyone else is done with them).
  if (threadIdx.x == 0) s_ticket = add_dev(sync + kSyncExit, 1u) == gridDim.x - 1;
  __syncthreads();
  if (s_ticket) {
    for (int j = threadIdx.x; j < E; j += kGemmThreads) st_dev(sync + kSyncHeader + j * kSyncStride, 0u);
    if (threadIdx.x < 8) st_dev(sync + 32 * threadIdx.x, 0u);
    if (threadIdx.x == 0) {
      st_dev(sync + kSyncExit, 0u);
      st_dev(sync + kSyncL1, 0u);
      st_dev(sync + kSyncQ, 0u);
    }
  }
}

// ============================================================================================
// Large class: 256x256 tiles (128x512 for an expert's last rows when they are at most 128),
// stages of raw NVFP4 streamed straight into an LDS ring.
//
// Global -> LDS: gfx950's global_load_lds_dwordx4 writes each lane's 16 bytes into LDS without a
// register round trip (lane i of an instruction lands at base + 16*i).  Stage ks+kAhead is
// requested while stage ks is computed; a stage is consumed after an explicit s_waitcnt vmcnt
// (this wave's loads) and one s_barrier (everyone's).  The slot being refilled was last read two
// stages earlier, so that single barrier per stage orders both directions.  (__syncthreads()
// would also wait for every load still in flight.)  Measured on the 8192-token prefill, 128-K
// stages with 4 slots were faster than 64-K stages with 8 slots and six stages in flight.
//
// LDS holds raw codes and scales (0.5625 B/element) and each wave decodes the fragments it needs
// right before its MFMAs.  Decoding into fp16 tiles in LDS instead would move ~3.5x more LDS
// bytes per MFMA (measured slower); per-wave decoding costs 6 VALU instructions per 32-cycle
// v_mfma_f32_32x32x16_f16, which the VALU issues while the matrix core runs (the 32x32x16 shape
// sustains ~97% of the fp16 peak on gfx950, the 16x16x32 shape only ~55%).
//
// Stage layout (per operand): codes row-major, kLRowBytes per tile row R, with the 16-byte chunk
// c (elements 32c..32c+31 of the stage) stored in slot c ^ lswz(R) so that the 16-byte fragment
// reads of 16 consecutive rows hit distinct banks; a DMA instruction covers 1024 /
// kLRowBytes rows with kLChunks lanes per row (row-contiguous global bytes).  Scales: the stage's 8
// block scales of row R at R * 8 (lane half h reads the 4 bytes at R * 8 + 4h).
// Lane (p = lane % 32, h = lane / 32) of a 32-row fragment owns elements [h * kLKs/2, +kLKs/2) of
// its row and feeds [h * kLKs/2 + 8s, +8) to MFMA step s as the MFMA's k = 8h..8h+7.  A and B use
// the same map, so each dot product runs over every element once.
//
// Two tile shapes with the same per-wave block: 8 waves, each 64 token rows x 128 weight rows
// (2 x 4 MFMA blocks of 32x32, 128 fp32 accumulators), two per SIMD (they hide each other's LDS
// waits and barrier skew).  Full tiles are 256x256 with the waves 4 (M) x 2 (N); tail tiles are
// 128x512 with the waves 2 x 4 and serve an expert's last m-tile when it holds at most 128 token
// rows, which halves the padded rows there (on the 8192-token Zipf prefill the MFMA work of the
// class drops to 92%).  Both shapes cost the same per tile, so one persistent list holds them.
// L1: tile weight rows 0..BN/2-1 are gate rows nt*BN/2.., the next BN/2 the matching up rows, so a
// wave holds gate and up of the same 64 h columns and applies SiLU(gate)*up in registers.
// L2: tile weight rows are output rows nt*BN..+BN.
// The epilogue stages the bf16 tile in LDS and writes it with 16-byte row-contiguous stores, or
// (L1 with a given global scale for h) quantizes each 16-column block of a staged row to NVFP4.
// ============================================================================================
constexpr int kLWaves = 8, kLThreads = kLWaves * kWave;
constexpr int kLKs = 128;                                        // stage depth (K elements)
constexpr int kLRowBytes = kLKs / 2;                             // code bytes of one row per stage
constexpr int kLChunks = kLRowBytes / 16;                        // 16-byte chunks per row
// 16-byte chunk slot swizzle of tile row R: the fragment reads of 16 consecutive rows (16 lanes x
// 16 B, one 256-byte LDS cycle) and of 8 consecutive rows both hit distinct slots.
__device__ __forceinline__ constexpr int lswz(int R) { return ((R >> 1) ^ (R >> 3)) & 3; }
static_assert(kLChunks == 4, "lswz permutes 4 chunks per row");
constexpr int kLScaleRow = kLKs / 16;                            // scale bytes of one row per stage
constexpr int kLSteps = kLKs / 16;                               // 32x32x16 MFMA steps per stage
constexpr int kLMI = 2;                                          // 32-row MFMA blocks per wave

template <int BM, int BN, int Slots, int Ahead>
struct LShape {
  static constexpr int kBm = BM, kBn = BN;
  static constexpr int kWM = BM / 64, kWN = BN / 128;            // waves along M and N
  static constexpr int kSlots = Slots, kAhead = Ahead;           // ring slots, stages in flight
  static constexpr int kARows = BM / kLWaves, kBRows = BN / kLWaves;  // DMA rows per wave
  static constexpr int kACodeDma = kARows * kLRowBytes / 1024;   // 16-byte DMA per wave
  static constexpr int kBCodeDma = kBRows * kLRowBytes / 1024;
  static constexpr int kBScaleDma = kBRows * kLScaleRow / 256;   // 4-byte DMA per wave
  // A scales: one 4-byte DMA per wave covers 32 rows; with BM < 256 two waves load the same rows
  // (same bytes to the same place), which keeps every wave's load count equal.
  static constexpr int kAScaleRows = 32;
  static constexpr int kDmaPerWave = kACodeDma + kBCodeDma + 1 + kBScaleDma;
  static constexpr int kACodeBytes = BM * kLRowBytes, kBCodeBytes = BN * kLRowBytes;
  static constexpr int kAOpBytes = kACodeBytes + BM * kLScaleRow;
  static constexpr int kStageBytes = kAOpBytes + BN * (kLRowBytes + kLScaleRow);
  static constexpr int kRingBytes = Slots * kStageBytes;
  static constexpr int kPitchL1 = BN + 16, kPitchL2 = 2 * BN + 16;  // bf16 staging pitches
  static_assert(kWM * kWN == kLWaves, "8 waves of 64 x 128");
  static_assert(kACodeDma >= 1 && kBCodeDma >= 1 && kBScaleDma >= 1 && BM % kAScaleRows == 0, "DMA split");
  static_assert(kBRows * kLScaleRow % 256 == 0 && kARows <= kAScaleRows, "scale DMA split");
  static_assert(kAhead <= kSlots - 2, "refilled slot must have been read two stages earlier");
};
using LFull = LShape<kBlockMLarge, 256, 4, 2>;
using LTail = LShape<128, 512, 3, 1>;
constexpr int kLLdsBytes = LFull::kRingBytes > LTail::kRingBytes ? LFull::kRingBytes : LTail::kRingBytes;
static_assert(LFull::kBm * LFull::kPitchL2 <= kLLdsBytes && LTail::kBm * LTail::kPitchL2 <= kLLdsBytes,
              "staging fits");

// Wait until at most `stages_after` (<= S::kAhead) later stages' loads are outstanding for this wave.
template <class S, int K = S::kAhead>
__device__ __forceinline__ void wait_stage(int stages_after) {
  if constexpr (K == 0) {
    wait_vmcnt<0>();
  } else {
    if (stages_after >= K) wait_vmcnt<K * S::kDmaPerWave>();
    else wait_stage<S, K - 1>(stages_after);
  }
}

// One output tile of shape S: expert e, m-tile rows [row0, row0 + min(rows_left, BM)), n-tile nt.
template <bool kL1, bool kQ, class S>
__device__ __forceinline__ void large_tile(const GemmArgs& p, uint8_t* smem, int e, int row0, int rows_left, int nt,
                                           float gs_a, uint32_t& amax_bits) {
  constexpr int BM = S::kBm, BN = S::kBn;
  const int K = p.K, Kh = K / 2, Ks = K / 16;
  const int Nw = kL1 ? 2 * p.N : p.N;
  const int nks = K / kLKs;
  // wave index as a scalar: the LDS destinations of the DMA (M0) are then computed in SGPRs
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = lane_id();
  const int wm = wave / S::kWN, wn = wave % S::kWN;
  const int p32 = lane & 31, h2 = lane >> 5;

  // first tile weight row of this wave's 32-column fragment f
  auto brow_of = [&](int f) {
    return kL1 ? (f < 2 ? wn * 64 + 32 * f : BN / 2 + wn * 64 + 32 * (f - 2)) : wn * 128 + 32 * f;
  };
  // ---- DMA sources of this lane ----------------------------------------------------------------
  // codes: instruction j covers tile rows base + j*rows_per + lane/kLChunks; lane%kLChunks picks
  // the LDS slot and the global chunk (lane%kLChunks) ^ lswz(row) goes there; scales:
  // instruction j covers rows base + 32j + lane/2, lane%2 picking the 4-byte half (LDS scale
  // layout: 8 bytes per row).
  auto a_row_of = [&](int R) -> int64_t {
    const int Rv = R < rows_left ? R : 0;  // rows past the expert read row 0; never stored
    const int64_t r = row0 + Rv;
    return kL1 ? (int64_t)p.row_token[r] : r;
  };
  auto b_row_of = [&](int R) -> int64_t {
    if (kL1) return (int64_t)e * Nw + (R < BN / 2 ? nt * (BN / 2) + R : p.N + nt * (BN / 2) + R - BN / 2);
    return (int64_t)e * Nw + nt * BN + R;
  };
  constexpr int rows_per = 1024 / kLRowBytes;
  const uint8_t* a_code_src[S::kACodeDma];
  const uint8_t* b_code_src[S::kBCodeDma];
#pragma unroll
  for (int j = 0; j < S::kACodeDma; ++j) {
    const int R = S::kARows * wave + rows_per * j + lane / kLChunks;
    const int chunk = (lane % kLChunks) ^ lswz(R);
    a_code_src[j] = p.a_codes + a_row_of(R) * Kh + 16 * chunk;
  }
#pragma unroll
  for (int j = 0; j < S::kBCodeDma; ++j) {
    const int R = S::kBRows * wave + rows_per * j + lane / kLChunks;
    const int chunk = (lane % kLChunks) ^ lswz(R);
    b_code_src[j] = p.w_codes + b_row_of(R) * Kh + 16 * chunk;
  }
  static_assert(kLScaleRow == 8, "scale DMA assumes 128-K stages");
  const int a_scale_row0 = S::kAScaleRows * (wave % (BM / S::kAScaleRows));
  const uint8_t* a_scale_src = p.a_scales + a_row_of(a_scale_row0 + lane / 2) * Ks + 4 * (lane & 1);
  const uint8_t* b_scale_src[S::kBScaleDma];
#pragma unroll
  for (int j = 0; j < S::kBScaleDma; ++j) {
    const int R = S::kBRows * wave + 32 * j + lane / 2;
    b_scale_src[j] = p.w_scales + b_row_of(R) * Ks + 4 * (lane & 1);
  }

  f32x16 acc[kLMI][4];
#pragma unroll
  for (int i = 0; i < kLMI; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.f;

  // S::kDmaPerWave DMA instructions per wave: this wave's rows of both operands.
  auto issue_stage = [&](int ks, int slot) {
    const uint32_t lb = lds_addr(smem + slot * S::kStageBytes);
    const uint32_t lbb = lb + S::kAOpBytes;
    const int64_t off = (int64_t)ks * kLRowBytes, soff = (int64_t)ks * kLScaleRow;
#pragma unroll
    for (int j = 0; j < S::kACodeDma; ++j)
      dma16(a_code_src[j] + off, lb + (S::kARows * wave + rows_per * j) * kLRowBytes);
#pragma unroll
    for (int j = 0; j < S::kBCodeDma; ++j)
      dma16(b_code_src[j] + off, lbb + (S::kBRows * wave + rows_per * j) * kLRowBytes);
    dma4(a_scale_src + soff, lb + S::kACodeBytes + a_scale_row0 * kLScaleRow);
#pragma unroll
    for (int j = 0; j < S::kBScaleDma; ++j)
      dma4(b_scale_src[j] + soff, lbb + S::kBCodeBytes + (S::kBRows * wave + 32 * j) * kLScaleRow);
  };
  auto compute_stage = [&](int slot) {
    const uint8_t* base = smem + slot * S::kStageBytes;
    const uint8_t* a_codes = base;
    const uint8_t* a_scales = base + S::kACodeBytes;
    const uint8_t* b_codes = base + S::kAOpBytes;
    const uint8_t* b_scales = b_codes + S::kBCodeBytes;
    constexpr int CPL = kLChunks / 2;  // chunks per lane half
    // rows 32i + p and brow_of(f) + p have the swizzle of p: offsets are multiples of 32
    const int swz = lswz(p32);
    // scale bytes of this lane half: 4 per row (128-K stages)
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
      asc[i][1] = e4m3x2_to_f16(asw[i], true);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      bsc[f][0] = e4m3x2_to_f16(bsw[f], false);
      bsc[f][1] = e4m3x2_to_f16(bsw[f], true);
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

  for (int ks = 0; ks < S::kAhead && ks < nks; ++ks) issue_stage(ks, ks);
  for (int ks = 0; ks < nks; ++ks) {
    // Request stage ks+kAhead into the slot last read by stage ks-2 (every wave has passed the
    // barrier of stage ks-1 since), then wait until this wave's stage-ks loads have landed.
    if (ks + S::kAhead < nks) issue_stage(ks + S::kAhead, (ks + S::kAhead) % S::kSlots);
    const int after = nks - 1 - ks;
    wait_stage<S>(after < S::kAhead ? after : S::kAhead);
    __builtin_amdgcn_s_barrier();  // everyone's stage-ks loads have landed
    compute_stage(ks % S::kSlots);
  }
  __syncthreads();  // all waves are done reading the ring before it is reused for staging

  // ---- epilogue: scale, (SiLU*up), bf16, stage in LDS, coalesced stores ------------------------
  // accumulator r of block (i, f) is row 32i + 8(r/4) + 4h + r%4, column 32f + p of the wave tile
  const float inv = (float)(1.0 / ((double)gs_a * (double)p.w_gs[e]));
  constexpr int pitch = kL1 ? S::kPitchL1 : S::kPitchL2;
#pragma unroll
  for (int i = 0; i < kLMI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * (32 * kLMI) + 32 * i + 8 * (r >> 2) + 4 * h2 + (r & 3);
      const bool ok = row < rows_left;
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
  if constexpr (kL1 && kQ) {
    // NVFP4 h: one thread per 16-column block of a staged row (quantized with the given scale)
    constexpr int cols = BN / 2, nb = cols / 16;
    const int nrows = rows_left < BM ? rows_left : BM;
    const float gs_q = *p.q_gs;
    const int col0 = nt * cols;
    for (int idx = tid; idx < nrows * nb; idx += kLThreads) {
      const int r = idx / nb, c = idx - r * nb;
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(smem + r * pitch + 32 * c);
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(smem + r * pitch + 32 * c + 16);
      uint32_t q[2];
      const uint32_t sc = quant16(v0, v1, gs_q, q);
      const int64_t orow = row0 + r;
      const int col = col0 + 16 * c;
      *reinterpret_cast<u32x2*>(p.q_codes + orow * (p.N / 2) + col / 2) = u32x2{q[0], q[1]};
      p.q_scales[orow * (p.N / 16) + col / 16] = (uint8_t)sc;
    }
  } else {
    constexpr int cols = kL1 ? BN / 2 : BN;
    constexpr int chunks = cols * 2 / 16;  // 16-byte chunks per row
    const int nrows = rows_left < BM ? rows_left : BM;
    uint16_t* __restrict__ out = reinterpret_cast<uint16_t*>(p.out);
    const int col0 = nt * cols;
    // Non-temporal: the tile is read again only by the next kernel, and keeping it out of the
    // cache keeps the weight and A rows other tiles re-read (measured: L2 -2.5%, L1 -1%).
    for (int idx = tid; idx < nrows * chunks; idx += kLThreads) {
      const int r = idx / chunks, c = idx - r * chunks;
      const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * pitch + 16 * c);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + (int64_t)(row0 + r) * p.N + col0 + 8 * c));
    }
  }
  __syncthreads();  // staging reads done before the next tile's DMA refills the ring
}

template <bool kL1, bool kQ>
__global__ __launch_bounds__(kLThreads, 1) void gemm_large_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLLdsBytes];
  __shared__ int s_tpref[kMaxExperts + 1];  // exclusive prefix of tiles per expert
  __shared__ int s_mt[kMaxExperts];         // 2 * (large m-tiles) + (last one is a tail tile)
  __shared__ uint32_t s_amax[kLWaves];
  const int E = p.E;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  // n-tiles per m-tile: full tiles cover 256 weight rows, tail tiles 512 (L1: half gate, half up)
  const int ntn_full = kL1 ? p.N / 128 : p.N / 256;
  const bool tails = kL1 ? p.N % 256 == 0 : p.N % 512 == 0;
  const int ntn_tail = kL1 ? p.N / 256 : p.N / 512;
  {
    const int32_t* __restrict__ pref = p.sched + sched_pref_large(E);
    for (int j = tid; j < E; j += blockDim.x) {
      const int nm = pref[j + 1] - pref[j];
      const int last = p.counts[j] - kBlockMLarge * (nm - 1);
      const int tail = tails && nm > 0 && last <= LTail::kBm ? 1 : 0;
      s_mt[j] = 2 * nm + tail;
      s_tpref[j] = (nm - tail) * ntn_full + tail * ntn_tail;  // tiles of expert j (scanned below)
    }
    __syncthreads();
    if (tid < kWave) {  // wave 0: exclusive prefix over the experts
      int carry = 0;
      for (int c = 0; c < E; c += kWave) {
        const int e = c + lane;
        const int v = e < E ? s_tpref[e] : 0;
        int incl = v;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int t = __shfl_up(incl, o, kWave);
          if (lane >= o) incl += t;
        }
        if (e < E) s_tpref[e] = carry + incl - v;
        carry += __shfl(incl, kWave - 1, kWave);
      }
      if (lane == 0) s_tpref[E] = carry;
    }
    __syncthreads();
  }
  const float gs_a = *p.a_gs;
  uint32_t amax_bits = 0;

  const XcdTiles tl(s_tpref[E]);
  for (int t = tl.t; t < tl.end; t += tl.stride) {
    const int e = find_expert(s_tpref, E, 1, t);
    const int local = t - s_tpref[e];
    const int nm = s_mt[e] >> 1, tail = s_mt[e] & 1;
    const int nfull = (nm - tail) * ntn_full;
    // Full tiles of an expert go in bands of kBand m-tiles, n-tile major within a band: the
    // consecutive tiles an XCD runs at once share a few m-tiles' A rows and a few n-tiles' weight
    // rows (instead of one m-tile and all of the expert's weights), so fewer weight bytes are
    // fetched again for every m-tile.
    constexpr int kBand = 4;
    int mt, ntile;
    if (local < nfull) {
      const int band = local / (kBand * ntn_full);
      const int rem = (nm - tail) - band * kBand;
      const int h = rem < kBand ? rem : kBand;  // m-tiles in this band
      const int r = local - band * kBand * ntn_full;
      ntile = r / h;
      mt = band * kBand + (r - ntile * h);
    } else {
      mt = nm - 1;
      ntile = local - nfull;
    }
    const int row0 = p.padded_offsets[e] + kBlockMLarge * mt;
    const int rows_left = p.counts[e] - kBlockMLarge * mt;
    if (local < nfull) large_tile<kL1, kQ, LFull>(p, smem, e, row0, rows_left, ntile, gs_a, amax_bits);
    else large_tile<kL1, kQ, LTail>(p, smem, e, row0, rows_left, ntile, gs_a, amax_bits);
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
// kQ: L1 writing NVFP4 h (a.q_codes set); a separate instantiation, so the plain kernels carry
// none of its code.
template <bool kL1, bool kQ>
static hipError_t launch_gemm(GemmArgs a, GemmClasses c, hipStream_t stream) {
  a.clear_other = !(c.large && c.small);
  a.small_covers_large = c.small && !c.large;  // a row bound that was too low costs time only
  if (c.large) {
    hipLaunchKernelGGL((gemm_large_kernel<kL1, kQ>), dim3(kLargeGrid), dim3(kLThreads), 0, stream, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (c.small) {
    // Staged weight scales need whole 16-byte scale pieces per chunk (K a multiple of 256: a
    // staged row of K/16 bytes is K/256 whole pieces), at least 2 chunks of K for every wave (so
    // the loader never copies into the buffer of a group still being computed, see above) and 3
    // buffers beside the tables.  L2 sizes them for its wide groups; where those do not fit, the
    // staged scales (worth more) are kept and the kernel runs narrow groups only.
    constexpr int nb = small_nb<kL1>(), nbw = kL1 ? nb : kSNbWide;
    const int ch = a.K % 256 == 0 ? 256 : 128;
    const size_t tables = small_table_bytes(a.E);
    auto fits = [&](int w) { return tables + 3 * small_scale_buf_bytes(w, a.K) <= small_dyn_max_lds(w); };
    const bool can_stage = MEGAMOE_SMALL_STAGED && ch == 256 && a.K / ch >= 2 * kSWaves;
    const dim3 grid(kSmallGrid), block(kGemmThreads);
    // the packed codes are read by the staged configurations (a.w_packed is checked at the boundary)
    const bool packed = a.w_packed != nullptr;
    if (can_stage && fits(nbw)) {
      const size_t dyn = tables + 3 * small_scale_buf_bytes(nbw, a.K);
      if (packed) hipLaunchKernelGGL((gemm_small_kernel<kL1, 256, true, kQ, nbw, true>), grid, block, dyn, stream, a);
      else hipLaunchKernelGGL((gemm_small_kernel<kL1, 256, true, kQ, nbw>), grid, block, dyn, stream, a);
    } else if (can_stage && fits(nb)) {
      const size_t dyn = tables + 3 * small_scale_buf_bytes(nb, a.K);
      if (packed) hipLaunchKernelGGL((gemm_small_kernel<kL1, 256, true, kQ, nb, true>), grid, block, dyn, stream, a);
      else hipLaunchKernelGGL((gemm_small_kernel<kL1, 256, true, kQ, nb>), grid, block, dyn, stream, a);
    } else if (ch == 256) {  // the tables (at most 20.5 KB) fit beside the wide kernel's static LDS
      hipLaunchKernelGGL((gemm_small_kernel<kL1, 256, false, kQ, nbw>), grid, block, tables, stream, a);
    } else {
      hipLaunchKernelGGL((gemm_small_kernel<kL1, 128, false, kQ, nbw>), grid, block, tables, stream, a);
    }
    return hipGetLastError();
  }
  return hipSuccess;
}

// The fused small-class launch: CH and staging as launch_gemm would choose them for both GEMMs
// (one CH for both, so that both passes split the m-tiles into tiny and regular alike).
// XCDs of the current device: gfx950 has 32 CUs per XCD (a partitioned GPU shows fewer).
static int device_xcds() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 1;
  int n = dev < 64 ? cached[dev].load(std::memory_order_relaxed) : 0;
  if (n == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    n = cus / 32 < 1 ? 1 : cus / 32 > kXcds ? kXcds : cus / 32;
    if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_ffn_small(const FfnArgs& a0, hipStream_t stream) {
  FfnArgs a = a0;
  a.nxcd = device_xcds();
  a.l1.small_covers_large = 1;
  a.l2.small_covers_large = 1;
  const bool cal = a.l1.q_codes != nullptr;
  const int k1 = a.l1.K, k2 = a.l2.K;
  const int ch = k1 % 256 == 0 && k2 % 256 == 0 ? 256 : 128;
  const size_t tables = ffn_table_bytes(a.l1.E);
  const size_t b1 = small_scale_buf_bytes(small_nb<true>(), k1), b2 = small_scale_buf_bytes(small_nb<false>(), k2);
  const size_t bufs = 3 * (b1 > b2 ? b1 : b2);
  const bool staged = MEGAMOE_SMALL_STAGED && ch == 256 && k1 / ch >= 2 * kSWaves && k2 / ch >= 2 * kSWaves &&
                      tables + bufs <= small_dyn_max_lds(small_nb<true>());
  const size_t dyn = tables + (staged ? bufs : 0);
  const dim3 grid(kSmallGrid), block(kGemmThreads);
  // the packed codes of both GEMMs (checked at the boundary) are read by the staged configurations
  const bool packed = a.l1.w_packed != nullptr && a.l2.w_packed != nullptr;
  if (staged && packed) {
    if (cal) hipLaunchKernelGGL((ffn_small_kernel<256, true, true, true>), grid, block, dyn, stream, a);
    else hipLaunchKernelGGL((ffn_small_kernel<256, true, false, true>), grid, block, dyn, stream, a);
    return hipGetLastError();
  }
  if (cal) {
    if (staged) hipLaunchKernelGGL((ffn_small_kernel<256, true, true>), grid, block, dyn, stream, a);
    else if (ch == 256) hipLaunchKernelGGL((ffn_small_kernel<256, false, true>), grid, block, dyn, stream, a);
    else hipLaunchKernelGGL((ffn_small_kernel<128, false, true>), grid, block, dyn, stream, a);
  } else {
    if (staged) hipLaunchKernelGGL((ffn_small_kernel<256, true, false>), grid, block, dyn, stream, a);
    else if (ch == 256) hipLaunchKernelGGL((ffn_small_kernel<256, false, false>), grid, block, dyn, stream, a);
    else hipLaunchKernelGGL((ffn_small_kernel<128, false, false>), grid, block, dyn, stream, a);
  }
  return hipGetLastError();
}

// Packed weight codes for the 16-row kernels.  In the row-major layout a load instruction of the
// 16-row kernels reads 64 bytes from each of 16 weight rows; in the packed layout it reads 1 KB
// contiguous, which lets those loads be non-temporal (every weight byte is read once per call)
// without fetching a 128-byte line twice.  For 16-row block rb (weight rows 16 rb .. 16 rb + 15),
// 256-element chunk c and load instruction q (0, 1), lane L = 16 g + r holds the 16 code bytes
// 32 g + 16 q .. of chunk c of row 16 rb + r -- the bytes that lane loads from the row-major
// codes -- at byte ((rb * (K / 256) + c) * 2 + q) * 1024 + 16 L.  The same bytes, permuted: the
// products do not change.
__global__ __launch_bounds__(256) void pack_codes16_kernel(const u32x4* __restrict__ src, int64_t rows,
                                                           int64_t pieces_per_row, u32x4* __restrict__ dst) {
  const int64_t n = rows * pieces_per_row;  // 16-byte pieces
  const int64_t per_block = 16 * pieces_per_row;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t rb = i / per_block;
    const int64_t in_block = i - rb * per_block;
    const int64_t c = in_block / 128;  // 2 KB = 128 pieces per chunk of a block
    const int w = (int)(in_block - c * 128);
    const int q = w / kWave, L = w % kWave;
    const int r = L % 16, g = L / 16;
    dst[i] = src[(rb * 16 + r) * pieces_per_row + c * 8 + 2 * g + q];
  }
}

hipError_t launch_pack_codes16(const uint8_t* codes, int64_t rows, int64_t K, uint8_t* packed, hipStream_t stream) {
  const int64_t pieces = rows * (K / 32);
  int64_t grid = (pieces + 255) / 256;
  if (grid > 8192) grid = 8192;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(pack_codes16_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(codes), rows, K / 32, reinterpret_cast<u32x4*>(packed));
  return hipGetLastError();
}

hipError_t launch_gemm_l1(const GemmArgs& a, GemmClasses c, hipStream_t stream) {
  return a.q_codes ? launch_gemm<true, true>(a, c, stream) : launch_gemm<true, false>(a, c, stream);
}

hipError_t launch_gemm_l2(const GemmArgs& a, GemmClasses c, hipStream_t stream) {
  return launch_gemm<false, false>(a, c, stream);
}

}  // namespace megamoe
