// Router: logits -> top-k expert ids and weights (the step that feeds topk_ids and topk_weights
// to the routed experts, CURRENT_BUG.md@2e65594, "Test Plan" Phase 1).
//
// Softmax over all global experts, the k largest probabilities in descending order with equal
// values going to the lower expert index, not renormalised.  The softmax is float64 over the
// float32 logits (max-subtracted); a weight is the float64 probability rounded to float32.
// Ranking by the float32 logits is the same as ranking by those probabilities: distinct float32
// logits differ by far more than a float64 exp can blur, and equal logits give equal
// probabilities, so the top-k decision is exact and needs no exp.
//
// One wave per token: each lane holds Eg/64 logits, a wave max and a float64 wave sum give the
// softmax denominator, and k rounds of a wave argmax over the (value, -index) order pick the
// experts; round r takes the best candidate strictly after round r-1's winner in that order, so no
// per-expert state is kept.  Lane r keeps winner r and the k weights are computed in parallel.
#include "device_common.h"
#include "internal.h"

namespace megamoe {

constexpr int kRouterWaves = 4;
constexpr int kRouterPerLane = MEGAMOE_ROUTER_MAX_EXPERTS / kWave;  // logits per lane

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__global__ __launch_bounds__(kRouterWaves* kWave) void router_topk_kernel(const float* __restrict__ logits, int T,
                                                                           int Eg, int k, int32_t* __restrict__ ids,
                                                                           float* __restrict__ weights) {
  const int lane = lane_id();
  const int t = blockIdx.x * kRouterWaves + threadIdx.x / kWave;
  if (t >= T) return;  // whole waves only
  const float* __restrict__ row = logits + (int64_t)t * Eg;
  float v[kRouterPerLane];
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int i = 0; i < kRouterPerLane; ++i) {
    const int j = lane + kWave * i;
    v[i] = j < Eg ? row[j] : -__builtin_huge_valf();
    m = fmaxf(m, v[i]);
  }
  m = wave_max_f32(m);
  const double md = (double)m;
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kRouterPerLane; ++i)
    if (lane + kWave * i < Eg) s += exp((double)v[i] - md);
  s = wave_sum_f64(s);

  float pv = __builtin_huge_valf();  // previous winner (value, index)
  int pj = -1;
  float wv = 0.0f;  // lane r keeps winner r
  int wj = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -__builtin_huge_valf();
    int bj = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kRouterPerLane; ++i) {
      const int j = lane + kWave * i;
      const bool after = v[i] < pv || (v[i] == pv && j > pj);
      if (j < Eg && after && (v[i] > bv || (v[i] == bv && j < bj))) {
        bv = v[i];
        bj = j;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oj = __shfl_xor(bj, o, kWave);
      if (ov > bv || (ov == bv && oj < bj)) {
        bv = ov;
        bj = oj;
      }
    }
    pv = bv;
    pj = bj;
    if (lane == r) {
      wv = bv;
      wj = bj;
    }
  }
  if (lane < k) {  // the k weights in parallel, one lane each
    ids[(int64_t)t * k + lane] = wj;
    weights[(int64_t)t * k + lane] = (float)(exp((double)wv - md) / s);
  }
}

hipError_t launch_router(const float* logits, int32_t T, int32_t Eg, int32_t k, int32_t* ids, float* weights,
                         hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int grid = (T + kRouterWaves - 1) / kRouterWaves;
  hipLaunchKernelGGL(router_topk_kernel, dim3(grid), dim3(kRouterWaves * kWave), 0, stream, logits, T, Eg, k, ids,
                     weights);
  return hipGetLastError();
}

}  // namespace megamoe
