// Dense NVFP4 linear layers on the grouped-GEMM kernels: one expert whose rows are all M input
// rows (the single-group case of the expert GEMM).  A tiny kernel writes that group's tables
// (counts, padded offsets and the tile table the GEMMs read, in the routing step's layout) into
// the caller's workspace, plus the identity row map the gate+up kernel gathers through.
#include "device_common.h"
#include "internal.h"

namespace megamoe {

__global__ __launch_bounds__(256) void dense_setup_kernel(int32_t M, int32_t* __restrict__ ws, int64_t nrows) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    const bool small = M <= kSmallClassMaxTokens;
    const int bm = M > 0 ? (small ? kBlockMSmall : kBlockMLarge) : 0;
    const int tiles = M > 0 ? (M + bm - 1) / bm : 0;
    int32_t* counts = ws + kDenseCounts;
    int32_t* poff = ws + kDensePoff;
    int32_t* sched = ws + kDenseSched;
    counts[0] = M;
    poff[0] = 0;
    poff[1] = M;
    sched[0] = 1;
    sched[1] = small ? tiles : 0;
    sched[2] = small ? 0 : tiles;
    sched[3] = 0;
    sched[sched_block_m(1)] = bm;
    sched[sched_pref_small(1)] = 0;
    sched[sched_pref_small(1) + 1] = small ? tiles : 0;
    sched[sched_pref_large(1)] = 0;
    sched[sched_pref_large(1) + 1] = small ? 0 : tiles;
  }
  int32_t* rows = ws + kDenseHeader;
  for (int64_t j = i; j < nrows; j += (int64_t)gridDim.x * blockDim.x) rows[j] = (int32_t)j;
}

hipError_t launch_dense_setup(int32_t M, int32_t* ws, bool with_rows, hipStream_t stream) {
  const int64_t nrows = with_rows ? M : 0;
  int64_t grid = (nrows + 255) / 256;
  if (grid < 1) grid = 1;
  if (grid > 1024) grid = 1024;
  hipLaunchKernelGGL(dense_setup_kernel, dim3((unsigned)grid), dim3(256), 0, stream, M, ws, nrows);
  return hipGetLastError();
}

}  // namespace megamoe
