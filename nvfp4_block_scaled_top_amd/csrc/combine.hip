// Routing-weighted combine of the expert outputs back into token order.
//
// Each (token, expert) output row is weighted by its top-k routing weight exactly once, here,
// and the k contributions of a token are summed in slot order in fp32 (the runner takes
// topk_weights from the router: nvfp4-megamoe-kernel CURRENT_BUG.md@2e65594, "Test Plan"
// Phase 1).  A gather per token (not a scatter with atomics) keeps the result deterministic.
// Memory-bound: one thread per 8 output columns (16-byte loads and stores).  A shared expert's
// output (y_shared, weight 1, one row per token) is added after the routed sum, before rounding.
#include "device_common.h"
#include "internal.h"

namespace megamoe {

// Slots are taken 8 at a time: their rows and weights are loaded first, then the 8 output rows
// together (two dependent round trips per 8 slots instead of two per slot), then added in slot order.
// The expert output rows are read once, as non-temporal loads (the 8192-token prefill's combine:
// 155 -> 134 us).
constexpr int kCombineSlots = 8;

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y, const int32_t* __restrict__ token_rows,
                                                      const float* __restrict__ w, int32_t T, int32_t k, int32_t H,
                                                      const uint16_t* __restrict__ y_shared,
                                                      uint16_t* __restrict__ out) {
  const int64_t per = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * per) return;
  const int64_t t = idx / per, c8 = idx - t * per;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += kCombineSlots) {
    int32_t r[kCombineSlots];
    float wt[kCombineSlots];
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u) {
      const int j = j0 + u;
      r[u] = j < k ? token_rows[t * k + j] : -1;
      wt[u] = j < k ? w[t * k + j] : 0.0f;
    }
    u32x4 v[kCombineSlots];
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u)
      if (r[u] >= 0) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y + (int64_t)r[u] * H + c8 * 8));
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u) {
      if (r[u] < 0) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(wt[u], bf16_bits_to_f32(v[u][q] & 0xFFFFu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(wt[u], bf16_bits_to_f32(v[u][q] >> 16), acc[2 * q + 1]);
      }
    }
  }
  if (y_shared != nullptr) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(y_shared + t * H + c8 * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += bf16_bits_to_f32(v[q] & 0xFFFFu);
      acc[2 * q + 1] += bf16_bits_to_f32(v[q] >> 16);
    }
  }
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = f32_to_bf16_bits(acc[2 * q]) | (f32_to_bf16_bits(acc[2 * q + 1]) << 16);
  *reinterpret_cast<u32x4*>(out + t * H + c8 * 8) = o;
}

hipError_t launch_combine(const uint16_t* y, const int32_t* token_rows, const float* w, int32_t T, int32_t k,
                          int32_t H, const uint16_t* y_shared, uint16_t* out, hipStream_t stream) {
  const int64_t n = (int64_t)T * (H / 8);
  if (n == 0) return hipSuccess;
  const int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)grid), dim3(256), 0, stream, y, token_rows, w, T, k, H, y_shared,
                     out);
  return hipGetLastError();
}

}  // namespace megamoe
