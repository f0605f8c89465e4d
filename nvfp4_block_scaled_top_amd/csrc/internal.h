// Host-side declarations shared between the C-ABI layer (api.cpp) and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/megamoe.h"

namespace megamoe {

constexpr int kMaxExperts = MEGAMOE_MAX_EXPERTS;

// ---- routing ---------------------------------------------------------------------------------
constexpr int kRouteChunk = 1024;  // assignments per routing workgroup (one per thread)

// Layout of the int32 tile table written by the routing step and read by the GEMMs:
//   [0] E  [1] total small-class m-tiles  [2] total large-class m-tiles  [3] 0
//   [4, 4+E)           block_m of each expert (0 when it has no tokens)
//   [4+E, 5+2E)        exclusive prefix of small-class m-tiles per expert
//   [5+2E, 6+3E)       exclusive prefix of large-class m-tiles per expert
constexpr int kSchedHeader = 4;
inline int64_t sched_len(int32_t E) { return kSchedHeader + 3 * (int64_t)E + 2; }
__host__ __device__ inline int sched_block_m(int E) { (void)E; return kSchedHeader; }
__host__ __device__ inline int sched_pref_small(int E) { return kSchedHeader + E; }
__host__ __device__ inline int sched_pref_large(int E) { return kSchedHeader + 2 * E + 1; }

// Tile heights.  Small class: one 16-row MFMA block, weights streamed straight to registers with
// the reduction dimension split across the waves of a workgroup.  Large class: LDS-tiled.
constexpr int kBlockMSmall = 16;
constexpr int kBlockMLarge = 256;
// Experts with at most this many tokens use the small class when block_m is chosen per expert.
constexpr int kSmallClassMaxTokens = 16;

hipError_t launch_route(const int32_t* topk_ids, int32_t T, int32_t k, int32_t e0, int32_t E, int32_t P,
                        int32_t block_m_override, int32_t* counts, int32_t* eoff, int32_t* poff,
                        int32_t* row_token, int64_t M_cap, int32_t* token_rows, int32_t* sched,
                        int32_t* ws, hipStream_t stream);

// Device address of this GPU's static routing scratch (MEGAMOE_ROUTE_NOALLOC_SCRATCH_BYTES bytes),
// looked up once per device; it takes the place of the workspace in moe_route_permute_noalloc.
hipError_t route_noalloc_scratch(int32_t** addr);

// ---- router ----------------------------------------------------------------------------------
hipError_t launch_router(const float* logits, int32_t T, int32_t Eg, int32_t k, int32_t* ids, float* weights,
                         hipStream_t stream);

// Routing and the quantization of x in one launch (decode sizes: T*k <= 1024, T*H <= 2^16).
bool route_quant_fusable(int32_t T, int32_t k, int64_t H);
hipError_t launch_route_quant_small(const int32_t* topk_ids, int32_t T, int32_t k, int32_t e0, int32_t E, int32_t P,
                                    int32_t block_m_override, int32_t* counts, int32_t* eoff, int32_t* poff,
                                    int32_t* row_token, int64_t M_cap, int32_t* token_rows, int32_t* sched,
                                    const uint16_t* x, int64_t H, uint8_t* codes, uint8_t* scales, float* gs,
                                    const float* gs_in, hipStream_t stream);

// ---- quantizer -------------------------------------------------------------------------------
int quant_amax_parts(int64_t rows, int64_t cols);
hipError_t launch_quant(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* row_valid,
                        const float* amax_in, int32_t amax_in_count, uint8_t* codes, uint8_t* scales, float* gs, float* ws,
                        hipStream_t stream);

hipError_t launch_quant_gs(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* row_valid, const float* gs,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream);

// ---- grouped GEMMs ---------------------------------------------------------------------------
struct GemmArgs {
  // A operand: NVFP4 activations.  For L1, rows are gathered through row_token from a [T, K]
  // tensor; for L2 the permuted row index addresses the [M_cap, K] tensor directly.
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_gs;
  const int32_t* row_token;  // L1 only (NULL for L2)
  const int32_t* padded_offsets;
  const int32_t* counts;
  const int32_t* sched;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* w_gs;
  int32_t E, K, N;   // N = output columns: I for L1 (weights have 2I rows), H for L2
  void* out;         // bf16 [M_cap, N]
  float* amax_out;   // L1: per-workgroup max |h| slots [MEGAMOE_L1_AMAX_PARTS]; NULL for L2
  int clear_other;   // L1: the other tile class is not launched; this kernel zeroes its slots
  // The 256-row kernel is not launched: the 16-row kernel also takes experts the routing step gave
  // 256-row tiles (in 16-row m-tiles), so a caller's row bound below a real count is still correct.
  int small_covers_large = 0;
  // L1 only, optional: write h as NVFP4 with this global scale (codes [M_cap, N/2], scales
  // [M_cap, N/16]) instead of bf16 h into `out`.
  const float* q_gs = nullptr;
  uint8_t* q_codes = nullptr;
  uint8_t* q_scales = nullptr;
  // Optional: the weight codes also in the packed layout of nvfp4_pack_weight_codes, read by the
  // 16-row kernels instead of w_codes (the 256-row kernels read w_codes).
  const uint8_t* w_packed = nullptr;
};
// Which tile classes a call may contain, from the routing override and the caller's row bound.
struct GemmClasses {
  bool small, large;
};
hipError_t launch_gemm_l1(const GemmArgs& a, GemmClasses c, hipStream_t stream);
hipError_t launch_gemm_l2(const GemmArgs& a, GemmClasses c, hipStream_t stream);
// Weight codes [rows, K/2] (rows % 16 == 0, K % 256 == 0) into the packed layout of the 16-row
// kernels (nvfp4_pack_weight_codes).
hipError_t launch_pack_codes16(const uint8_t* codes, int64_t rows, int64_t K, uint8_t* packed, hipStream_t stream);
// L1, the requantization of h and L2 of the small class in one launch (moe_grouped_ffn_fused).
// Sync words: per-XCD tickets, three counters and the error word in the first 384, then one
// 32-word line per expert.
constexpr int kFfnSyncHeader = 384, kFfnSyncStride = 32;
struct FfnArgs {
  GemmArgs l1;  // q_codes/q_scales/q_gs set: calibrated scale of h (NVFP4 h from the L1 epilogue);
                // else out = bf16 h, requantized inside the launch
  GemmArgs l2;  // a_codes/a_scales: NVFP4 h; a_gs: its global scale (written here when not given)
  uint32_t* sync;             // MEGAMOE_FFN_SYNC words, zero before the launch (left zero)
  const int32_t* row_valid;   // row_token: rows without an assignment get zero h codes
  int64_t M_cap;
  uint8_t* hq_codes;          // NVFP4 h written by the requantization parts (no calibrated scale)
  uint8_t* hq_scales;
  float* h_gs;                // global scale of h written by the first requantization part
  int nxcd;                   // XCDs of the device (each has its own ticket counter)
};
hipError_t launch_ffn_small(const FfnArgs& a, hipStream_t stream);
// n floats at p set to v on the stream (graph-safe: a kernel, no memset node).
hipError_t launch_fill_f32(float* p, int n, float v, hipStream_t stream);

// ---- dense layers (one group of M rows) -------------------------------------------------------
// int32 workspace layout: counts [1], padded offsets [2], tile table [sched_len(1)], then the
// identity row map [M] (gate+up only).
constexpr int kDenseCounts = 0, kDensePoff = 1, kDenseSched = 4, kDenseHeader = 16;
static_assert(kDenseSched + 4 + 3 * 1 + 2 <= kDenseHeader, "dense tables fit the header");
hipError_t launch_dense_setup(int32_t M, int32_t* ws, bool with_rows, hipStream_t stream);

// ---- combine ---------------------------------------------------------------------------------
hipError_t launch_combine(const uint16_t* y, const int32_t* token_rows, const float* w, int32_t T,
                          int32_t k, int32_t H, const uint16_t* y_shared, uint16_t* out, hipStream_t stream);

}  // namespace megamoe
