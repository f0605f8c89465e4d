// NVFP4 quantization of activations with a global scale derived from amax.
//
// The FP4 quantizer multiplies the input by a global scale before it forms the E4M3 block
// scales; a global scale taken from a checkpoint (1/input_scale = 3977.6) overflows E4M3 for
// activations with amax 2-8 (nvfp4-megamoe-kernel CURRENT_BUG.md@2fc81cc, "Root Cause" and
// "Key evidence").  Here gs = fl32(2688 / amax) with 2688 = 448 (E4M3 max) * 6 (E2M1 max), so
// no block scale can exceed 448.
//
// Exactness.  Results are bit-exact with the real-number definition:
//  * block scale = E4M3 round-to-nearest-even of block_amax * gs / 6.  block_amax * gs is exact
//    in double (8 + 24 significant bits); the quotient by 6 is rounded once in double, and it
//    cannot land on or cross an E4M3 rounding midpoint unless the exact value is that midpoint
//    (a non-zero gap |p - 6*mid| is at least 2^-33 relative, far above double's 2^-53), so
//    rounding the double to the E4M3 grid with ties-to-even is exact;
//  * element code = nearest E2M1 point of x * gs / s: compare x * gs with each midpoint m * s
//    (exact in fp32: <= 7 significant bits).  fmaf(|x|, gs, -m*s) rounds the exact difference
//    once, which never changes its sign, so each comparison is exact; ties go to the even code.
//
// Two kernels: an amax pass writing per-workgroup partial maxima (skipped when the caller passes
// its own partial maxima in amax_in), then the quantization pass, whose every workgroup reduces
// the partials itself (no atomics, nothing to reset between calls).  Tensors of up to 2^16
// elements (decode activations) take a single launch (quant_small_kernel).
#include "device_common.h"
#include "internal.h"
#include "quant_device.h"

namespace megamoe {

constexpr int kQuantThreads = 256;
constexpr int kQuantMaxParts = 1024;

int quant_amax_parts(int64_t rows, int64_t cols) {
  const int64_t vecs = rows * cols / 8;
  int64_t b = (vecs + kQuantThreads * 4 - 1) / (kQuantThreads * 4);
  if (b < 1) b = 1;
  if (b > kQuantMaxParts) b = kQuantMaxParts;
  return (int)b;
}

// Block-level max of a non-negative uint (256 threads).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) red[w] = v;
  __syncthreads();
  uint32_t r = red[0];
  for (int j = 1; j < kQuantThreads / kWave; ++j) r = r > red[j] ? r : red[j];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kQuantThreads) void quant_amax_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                   int64_t cols, const int32_t* __restrict__ row_valid,
                                                                   float* __restrict__ parts) {
  __shared__ uint32_t red[kQuantThreads / kWave];
  const int64_t nvec = rows * cols / 8;
  uint32_t m = 0;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += (int64_t)gridDim.x * blockDim.x) {
    if (row_valid != nullptr && row_valid[(v * 8) / cols] < 0) continue;
    const u32x4 d = *reinterpret_cast<const u32x4*>(x + v * 8);
    const uint32_t t = bf16_abs_max8(d);
    m = m > t ? m : t;
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) parts[blockIdx.x] = bf16_bits_to_f32(m);
}

__global__ __launch_bounds__(kQuantThreads) void quant_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                              const int32_t* __restrict__ row_valid,
                                                              const float* __restrict__ amax_src, int nparts,
                                                              uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                              float* __restrict__ gs_out) {
  __shared__ uint32_t red[kQuantThreads / kWave];
  uint32_t am = 0;
  for (int j = threadIdx.x; j < nparts; j += blockDim.x) {
    const uint32_t b = __float_as_uint(amax_src[j]);  // non-negative: uint order is float order
    am = am > b ? am : b;
  }
  am = block_max_u32(am, red);
  const float gs = global_scale_of(__uint_as_float(am));
  if (blockIdx.x == 0 && threadIdx.x == 0) *gs_out = gs;

  const int64_t bpr = cols / 16;
  const int64_t nblk = rows * bpr;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * blockDim.x) {
    if (row_valid != nullptr && row_valid[b / bpr] < 0) {
      *reinterpret_cast<u32x2*>(codes + b * 8) = u32x2{0u, 0u};
      scales[b] = 0;
      continue;
    }
    quant_block(x, b, gs, codes, scales);
  }
}

// The quantization pass for tensors of up to kQuadMaxBlocks blocks (e.g. decode's h, whose global
// scale comes from the L1 amax slots): one block per quad of threads, as in the single-launch form,
// so that the per-element tests of a few thousand blocks spread over four times the threads.
// kGsIn: the caller's global scale; otherwise every workgroup reduces the amax partials.
constexpr int64_t kQuadMaxBlocks = 1 << 16;
template <bool kGsIn>
__global__ __launch_bounds__(kQuantThreads) void quant_quad_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                   int64_t cols, const int32_t* __restrict__ row_valid,
                                                                   const float* __restrict__ amax_src, int nparts,
                                                                   const float* __restrict__ gs_in,
                                                                   uint8_t* __restrict__ codes,
                                                                   uint8_t* __restrict__ scales,
                                                                   float* __restrict__ gs_out) {
  float gs;
  if (kGsIn) {
    gs = *gs_in;
  } else {
    __shared__ uint32_t red[kQuantThreads / kWave];
    uint32_t am = 0;
    for (int j = threadIdx.x; j < nparts; j += blockDim.x) {
      const uint32_t b = __float_as_uint(amax_src[j]);  // non-negative: uint order is float order
      am = am > b ? am : b;
    }
    am = block_max_u32(am, red);
    gs = global_scale_of(__uint_as_float(am));
    if (blockIdx.x == 0 && threadIdx.x == 0) *gs_out = gs;
  }
  const int64_t bpr = cols / 16, nblk = rows * bpr;
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x / kQuantQuad);
  // the four threads of a quad hold the same b in every iteration
  for (int64_t b = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kQuantQuad; b < nblk; b += stride)
    quant_block_quarter(x, b, gs, row_valid == nullptr || row_valid[b / bpr] >= 0, codes, scales);
}

static unsigned quant_quad_grid(int64_t nblk) {
  const int64_t g = (nblk * kQuantQuad + kQuantThreads - 1) / kQuantThreads;
  return (unsigned)(g < 1 ? 1 : g > 2048 ? 2048 : g);
}

__global__ __launch_bounds__(kQuantSmallThreads) void quant_small_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                         int64_t cols,
                                                                         const int32_t* __restrict__ row_valid,
                                                                         uint8_t* __restrict__ codes,
                                                                         uint8_t* __restrict__ scales,
                                                                         float* __restrict__ gs_out) {
  __shared__ uint32_t red[kQuantSmallThreads / kWave];
  quant_small_body(x, rows, cols, row_valid, codes, scales, gs_out, (int)blockIdx.x, red);
}

// Calibrated variant: the global scale comes from the caller (e.g. from a warm-up pass), so there
// is no amax pass; blocks whose amax * gs / 6 exceeds 448 get the largest E4M3 scale and their
// elements saturate at +-6.
__global__ __launch_bounds__(kQuantThreads) void quant_gs_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                 int64_t cols, const int32_t* __restrict__ row_valid,
                                                                 const float* __restrict__ gs_in,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales) {
  const float gs = *gs_in;
  const int64_t bpr = cols / 16;
  const int64_t nblk = rows * bpr;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * blockDim.x) {
    if (row_valid != nullptr && row_valid[b / bpr] < 0) {
      *reinterpret_cast<u32x2*>(codes + b * 8) = u32x2{0u, 0u};
      scales[b] = 0;
      continue;
    }
    quant_block(x, b, gs, codes, scales);
  }
}

hipError_t launch_quant_gs(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* row_valid, const float* gs,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t nblk = rows * (cols / 16);
  if (nblk == 0) return hipSuccess;
  if (nblk <= kQuadMaxBlocks) {
    hipLaunchKernelGGL(quant_quad_kernel<true>, dim3(quant_quad_grid(nblk)), dim3(kQuantThreads), 0, stream, x, rows,
                       cols, row_valid, nullptr, 0, gs, codes, scales, nullptr);
    return hipGetLastError();
  }
  int64_t grid = (nblk + kQuantThreads - 1) / kQuantThreads;
  if (grid > 2048) grid = 2048;
  hipLaunchKernelGGL(quant_gs_kernel, dim3((unsigned)grid), dim3(kQuantThreads), 0, stream, x, rows, cols, row_valid,
                     gs, codes, scales);
  return hipGetLastError();
}

// n floats of p set to v (e.g. the L1 amax slots of an empty layer) (a kernel rather than a memset node, so that captured graphs replay it).
__global__ __launch_bounds__(256) void fill_f32_kernel(float* p, int n, float v) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = v;
}

hipError_t launch_fill_f32(float* p, int n, float v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int grid = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

hipError_t launch_quant(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* row_valid,
                        const float* amax_in, int32_t amax_in_count, uint8_t* codes, uint8_t* scales, float* gs,
                        float* ws, hipStream_t stream) {
  const float* amax_src = amax_in;
  int nparts = amax_in_count;
  if (amax_in == nullptr && rows * cols <= kQuantSmallElems) {
    const int64_t nblk = rows * (cols / 16);
    const int grid = (int)((nblk + kQuantSmallBlocks - 1) / kQuantSmallBlocks);
    hipLaunchKernelGGL(quant_small_kernel, dim3(grid > 0 ? grid : 1), dim3(kQuantSmallThreads), 0, stream, x, rows,
                       cols, row_valid, codes, scales, gs);
    return hipGetLastError();
  }
  if (amax_in == nullptr) {
    nparts = quant_amax_parts(rows, cols);
    hipLaunchKernelGGL(quant_amax_kernel, dim3(nparts), dim3(kQuantThreads), 0, stream, x, rows, cols, row_valid, ws);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    amax_src = ws;
  }
  const int64_t nblk = rows * (cols / 16);
  if (nblk <= kQuadMaxBlocks) {
    hipLaunchKernelGGL(quant_quad_kernel<false>, dim3(quant_quad_grid(nblk)), dim3(kQuantThreads), 0, stream, x, rows,
                       cols, row_valid, amax_src, nparts, nullptr, codes, scales, gs);
    return hipGetLastError();
  }
  int64_t grid = (nblk + kQuantThreads - 1) / kQuantThreads;
  if (grid > 2048) grid = 2048;  // grid-stride beyond: every workgroup re-reduces the partial maxima
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(quant_kernel, dim3((unsigned)grid), dim3(kQuantThreads), 0, stream, x, rows, cols, row_valid,
                     amax_src, nparts, codes, scales, gs);
  return hipGetLastError();
}

}  // namespace megamoe
