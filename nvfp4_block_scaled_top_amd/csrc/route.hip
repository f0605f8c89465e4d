// Routing step: local filter, per-expert counts, offsets, stable permutation and the tile table.
//
// The runner receives top-k ids and variable token counts per expert, with each expert's rows
// padded to 128 (nvfp4-megamoe-kernel CURRENT_BUG.md@2e65594, "Test Plan" Phase 1), and the
// grouped GEMM needs expert_offsets / padded_expert_offsets and must skip zero-token experts
// ("Test Plan" Phase 2).  The per-expert tile height follows the tokens per expert, small at
// decode and large at prefill ("Key References").
//
// Up to 1024 assignments (decode) one workgroup does everything (route_small_kernel).  Above
// that, three kernels, no atomics on global memory, so the permutation is deterministic:
//   1. count:   one workgroup per 1024 assignments builds that chunk's expert histogram (LDS
//               atomics; counts do not depend on order) and resets row_token to -1;
//   2. scan:    one workgroup turns the per-chunk histograms into per-chunk bases (a column
//               prefix over chunks), writes counts and both offset arrays, and the tile table;
//   3. scatter: each chunk ranks its assignments among equal experts with wave ballots (a
//               lane's rank = earlier lanes with the same expert) plus the counts of earlier
//               waves, so rows inside an expert follow ascending (token, slot) order.
#include <atomic>
#include <mutex>

#include "device_common.h"
#include "internal.h"
#include "quant_device.h"

namespace megamoe {

__global__ __launch_bounds__(kRouteChunk) void route_count_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                                  int32_t e0, int32_t E, int32_t nchunks,
                                                                  int32_t* __restrict__ ws,
                                                                  int32_t* __restrict__ row_token, int64_t M_cap) {
  extern __shared__ int32_t cnt[];  // [E]
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < M_cap;
       r += (int64_t)gridDim.x * blockDim.x)
    row_token[r] = -1;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * kRouteChunk + threadIdx.x;
  if ((int)blockIdx.x < nchunks && i < n) {
    const int64_t e = (int64_t)ids[i] - e0;
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if ((int)blockIdx.x < nchunks)
    for (int e = threadIdx.x; e < E; e += blockDim.x) ws[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Inclusive scan of four ints per thread over a 1024-thread block: shuffle scans inside each wave,
// then the totals of the earlier waves added from LDS (one barrier).
struct Scan4 {
  int v[4];
};

__device__ __forceinline__ Scan4 block_incl_scan4(Scan4 s, Scan4* wtot /* [kRouteChunk / kWave] */) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = __shfl_up(s.v[j], o, kWave);
      if (lane >= o) s.v[j] += u;
    }
  }
  if (lane == kWave - 1) wtot[w] = s;
  __syncthreads();
  for (int q = 0; q < w; ++q) {
#pragma unroll
    for (int j = 0; j < 4; ++j) s.v[j] += wtot[q].v[j];
  }
  return s;
}

// Given each expert's total (thread e holds expert e's count; threads >= E hold 0), write counts,
// both offset arrays and the tile table.  Called by all 1024 threads of the block.
// If s_poff is given, padded_offsets[0..E) are also left there (LDS) for the caller.
__device__ void finish_tables(int total, int32_t E, int32_t P, int32_t bm_override, Scan4* wtot,
                              int32_t* __restrict__ counts, int32_t* __restrict__ eoff,
                              int32_t* __restrict__ poff, int32_t* __restrict__ sched, int* s_poff) {
  const int e = threadIdx.x;
  if (e < E) counts[e] = total;
  int bm = 0, small_tiles = 0, large_tiles = 0;
  int padded = 0;
  if (e < E && total > 0) {
    const bool small = bm_override ? (bm_override == kBlockMSmall) : (total <= kSmallClassMaxTokens);
    bm = small ? kBlockMSmall : kBlockMLarge;
    const int tiles = (total + bm - 1) / bm;
    if (small) small_tiles = tiles; else large_tiles = tiles;
    padded = (int)(((int64_t)total + P - 1) / P * P);
  }
  const Scan4 inc = block_incl_scan4(Scan4{{total, padded, small_tiles, large_tiles}}, wtot);
  const int inc_cnt = inc.v[0], inc_pad = inc.v[1], inc_small = inc.v[2], inc_large = inc.v[3];
  if (s_poff != nullptr && e < E) s_poff[e] = inc_pad - padded;
  if (e < E) {
    eoff[e + 1] = inc_cnt;
    poff[e + 1] = inc_pad;
    sched[sched_block_m(E) + e] = bm;
    sched[sched_pref_small(E) + e + 1] = inc_small;
    sched[sched_pref_large(E) + e + 1] = inc_large;
  }
  if (e == E - 1) {
    sched[1] = inc_small;
    sched[2] = inc_large;
  }
  if (e == 0) {
    eoff[0] = 0;
    poff[0] = 0;
    sched[0] = E;
    sched[3] = 0;
    sched[sched_pref_small(E)] = 0;
    sched[sched_pref_large(E)] = 0;
  }
}

__global__ __launch_bounds__(kRouteChunk) void route_scan_kernel(int32_t* __restrict__ ws, int32_t nchunks, int32_t E,
                                                          int32_t P, int32_t bm_override,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ eoff,
                                                          int32_t* __restrict__ poff, int32_t* __restrict__ sched) {
  __shared__ Scan4 wtot[kRouteChunk / kWave];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    // Column prefix over the chunks, 16 loads in flight per batch.
    for (int c0 = 0; c0 < nchunks; c0 += 16) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = c0 + j < nchunks ? ws[(int64_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (c0 + j < nchunks) ws[(int64_t)(c0 + j) * E + e] = total;
        total += v[j];
      }
    }
  }
  finish_tables(total, E, P, bm_override, wtot, counts, eoff, poff, sched, nullptr);
}

// Rank of this lane's expert among the lanes of its wave holding the same expert (values 0..E;
// E is the "not local" sentinel), and the number of such lanes.
__device__ __forceinline__ void wave_rank(int e, int E, int& rank, int& count) {
  uint64_t same = __ballot(1);
  for (int b = 0; (1 << b) <= E; ++b) {
    const int bit = (e >> b) & 1;
    const uint64_t m1 = __ballot(bit);
    same &= bit ? m1 : ~m1;
  }
  const int lane = lane_id();
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  rank = __popcll(same & below);
  count = __popcll(same);
}

__global__ __launch_bounds__(kRouteChunk) void route_scatter_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                                    int32_t k, int32_t e0, int32_t E,
                                                                    const int32_t* __restrict__ ws,
                                                                    const int32_t* __restrict__ poff,
                                                                    int32_t* __restrict__ row_token,
                                                                    int32_t* __restrict__ token_rows) {
  constexpr int kWaves = kRouteChunk / kWave;
  extern __shared__ int32_t wcnt[];  // [kWaves][E]
  for (int j = threadIdx.x; j < kWaves * E; j += blockDim.x) wcnt[j] = 0;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * kRouteChunk + threadIdx.x;
  int e = E;  // sentinel: not local (or past the end)
  if (i < n) {
    const int64_t v = (int64_t)ids[i] - e0;
    if (v >= 0 && v < E) e = (int)v;
  }
  int rank, cnt;
  wave_rank(e, E, rank, cnt);
  const int wave = threadIdx.x / kWave;
  if (e < E && rank == 0) wcnt[wave * E + e] = cnt;
  __syncthreads();
  if (i < n) {
    int row = -1;
    if (e < E) {
      int base = ws[(int64_t)blockIdx.x * E + e];
      for (int w = 0; w < wave; ++w) base += wcnt[w * E + e];
      row = poff[e] + base + rank;
      row_token[row] = (int32_t)(i / k);
    }
    token_rows[i] = row;
  }
}


// Whole routing step in one workgroup when T*k <= kRouteChunk (decode): count, scan and scatter
// with barriers in between instead of three launches.
// The whole routing of up to 1024 assignments by one 1024-thread workgroup.  LDS: wcnt
// [kWaves][E], wtot [kWaves], s_poff [E].
__device__ __forceinline__ void route_small_body(const int32_t* __restrict__ ids, int32_t n, int32_t k, int32_t e0,
                                                 int32_t E, int32_t P, int32_t bm_override,
                                                 int32_t* __restrict__ counts, int32_t* __restrict__ eoff,
                                                 int32_t* __restrict__ poff, int32_t* __restrict__ row_token,
                                                 int64_t M_cap, int32_t* __restrict__ token_rows,
                                                 int32_t* __restrict__ sched, int32_t* wcnt, Scan4* wtot, int* s_poff) {
  constexpr int kWaves = kRouteChunk / kWave;
  for (int j = threadIdx.x; j < kWaves * E; j += blockDim.x) wcnt[j] = 0;
  for (int64_t r = threadIdx.x; r < M_cap; r += blockDim.x) row_token[r] = -1;
  __syncthreads();
  const int i = threadIdx.x;
  int e = E;
  if (i < n) {
    const int64_t v = (int64_t)ids[i] - e0;
    if (v >= 0 && v < E) e = (int)v;
  }
  int rank, cnt;
  wave_rank(e, E, rank, cnt);
  const int wave = threadIdx.x / kWave;
  if (e < E && rank == 0) wcnt[wave * E + e] = cnt;
  __syncthreads();
  int total = 0;
  if ((int)threadIdx.x < E)
    for (int w = 0; w < kWaves; ++w) total += wcnt[w * E + threadIdx.x];
  finish_tables(total, E, P, bm_override, wtot, counts, eoff, poff, sched, s_poff);
  __syncthreads();  // s_poff and the -1 fill of row_token are complete
  if (i < n) {
    int row = -1;
    if (e < E) {
      int base = 0;
      for (int w = 0; w < wave; ++w) base += wcnt[w * E + e];
      row = s_poff[e] + base + rank;
      row_token[row] = i / k;
    }
    token_rows[i] = row;
  }
}

__global__ __launch_bounds__(kRouteChunk) void route_small_kernel(const int32_t* __restrict__ ids, int32_t n, int32_t k,
                                                                  int32_t e0, int32_t E, int32_t P, int32_t bm_override,
                                                                  int32_t* __restrict__ counts, int32_t* __restrict__ eoff,
                                                                  int32_t* __restrict__ poff, int32_t* __restrict__ row_token,
                                                                  int64_t M_cap, int32_t* __restrict__ token_rows,
                                                                  int32_t* __restrict__ sched) {
  extern __shared__ int32_t wcnt[];  // [kWaves][E]
  __shared__ Scan4 wtot[kRouteChunk / kWave];
  __shared__ int s_poff[kMaxExperts];
  route_small_body(ids, n, k, e0, E, P, bm_override, counts, eoff, poff, row_token, M_cap, token_rows, sched, wcnt,
                   wtot, s_poff);
}

// Decode: routing (workgroup 0) and the quantization of x (workgroups 1..) in one launch; they
// are independent, so one kernel replaces two launches and the two run side by side.  gs_in:
// NULL = global scale from the amax of x (written to gs_out), else the caller's scale.
static_assert(kQuantSmallThreads == kRouteChunk, "both parts use 1024-thread workgroups");
__global__ __launch_bounds__(kRouteChunk) void route_quant_small_kernel(
    const int32_t* __restrict__ ids, int32_t n, int32_t k, int32_t e0, int32_t E, int32_t P, int32_t bm_override,
    int32_t* __restrict__ counts, int32_t* __restrict__ eoff, int32_t* __restrict__ poff,
    int32_t* __restrict__ row_token, int64_t M_cap, int32_t* __restrict__ token_rows, int32_t* __restrict__ sched,
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ gs_out, const float* __restrict__ gs_in) {
  extern __shared__ int32_t wcnt[];  // [kWaves][E]
  __shared__ Scan4 wtot[kRouteChunk / kWave];
  __shared__ int s_poff[kMaxExperts];
  __shared__ uint32_t red[kQuantSmallThreads / kWave];
  if (blockIdx.x == 0)
    route_small_body(ids, n, k, e0, E, P, bm_override, counts, eoff, poff, row_token, M_cap, token_rows, sched, wcnt,
                     wtot, s_poff);
  else if (gs_in)
    quant_gs_small_body(x, rows, cols, *gs_in, codes, scales, (int)blockIdx.x - 1);
  else
    quant_small_body(x, rows, cols, nullptr, codes, scales, gs_out, (int)blockIdx.x - 1, red);
}

bool route_quant_fusable(int32_t T, int32_t k, int64_t H) {
  return (int64_t)T * k <= kRouteChunk && (int64_t)T * H <= kQuantSmallElems;
}

hipError_t launch_route_quant_small(const int32_t* topk_ids, int32_t T, int32_t k, int32_t e0, int32_t E, int32_t P,
                                    int32_t block_m_override, int32_t* counts, int32_t* eoff, int32_t* poff,
                                    int32_t* row_token, int64_t M_cap, int32_t* token_rows, int32_t* sched,
                                    const uint16_t* x, int64_t H, uint8_t* codes, uint8_t* scales, float* gs,
                                    const float* gs_in, hipStream_t stream) {
  const size_t wcnt_bytes = (size_t)(kRouteChunk / kWave) * E * sizeof(int32_t);
  const int64_t nblk = (int64_t)T * (H / 16);
  const int qgrid = (int)((nblk + kQuantSmallBlocks - 1) / kQuantSmallBlocks);
  hipLaunchKernelGGL(route_quant_small_kernel, dim3(1 + (qgrid > 0 ? qgrid : 1)), dim3(kRouteChunk), wcnt_bytes, stream,
                     topk_ids, T * k, k, e0, E, P, block_m_override, counts, eoff, poff, row_token, M_cap, token_rows,
                     sched, x, (int64_t)T, H, codes, scales, gs, gs_in);
  return hipGetLastError();
}

hipError_t launch_route(const int32_t* topk_ids, int32_t T, int32_t k, int32_t e0, int32_t E, int32_t P,
                        int32_t block_m_override, int32_t* counts, int32_t* eoff, int32_t* poff,
                        int32_t* row_token, int64_t M_cap, int32_t* token_rows, int32_t* sched,
                        int32_t* ws, hipStream_t stream) {
  const int64_t n = (int64_t)T * k;
  const size_t wcnt_bytes = (size_t)(kRouteChunk / kWave) * E * sizeof(int32_t);
  if (n <= kRouteChunk) {
    hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(kRouteChunk), wcnt_bytes, stream, topk_ids, (int32_t)n, k, e0,
                       E, P, block_m_override, counts, eoff, poff, row_token, M_cap, token_rows, sched);
    return hipGetLastError();
  }
  const int32_t nchunks = (int32_t)((n + kRouteChunk - 1) / kRouteChunk);
  hipLaunchKernelGGL(route_count_kernel, dim3(nchunks), dim3(kRouteChunk), (size_t)E * sizeof(int32_t), stream,
                     topk_ids, n, e0, E, nchunks, ws, row_token, M_cap);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kRouteChunk), 0, stream, ws, nchunks, E, P, block_m_override,
                     counts, eoff, poff, sched);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nchunks), dim3(kRouteChunk), wcnt_bytes, stream, topk_ids, n, k, e0, E,
                     ws, poff, row_token, token_rows);
  return hipGetLastError();
}

// ---- scratch for the no-allocation entry point ----------------------------------------------------
// moe_route_permute_noalloc serves callers that cannot allocate device memory: the per-chunk
// histograms that moe_route_permute keeps in the caller's workspace live here instead, in one static
// array per GPU (held until the process ends).  In host code `scratch` names a host-side stand-in,
// not device memory, so its device address is looked up once per device (with that device current)
// and only that address is used: it is what the kernels receive, like the workspace pointer.  Nothing
// in it needs to start at zero: route_count writes every histogram entry before route_scan reads it.
// Every call on a GPU shares that GPU's array, so calls that overlap in time on one GPU race.
static __device__ __align__(256) int32_t scratch[MEGAMOE_ROUTE_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<int32_t*> g_scratch_addr[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t route_noalloc_scratch(int32_t** addr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  int32_t* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* a = nullptr;
      err = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
      if (err != hipSuccess) return err;
      if (a == nullptr) return hipErrorInvalidSymbol;
      p = static_cast<int32_t*>(a);
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return hipSuccess;
}

}  // namespace megamoe
