// Device helpers shared by the gfx950 kernels of libmegamoe: vector types, NVFP4 decode to
// fp16, wave reductions and bf16 rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace megamoe {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------------------------
// NVFP4 decode.  An element's value before the global scale is e2m1(code) * e4m3(scale).  Every
// such product is exactly representable as a NORMAL fp16 number (magnitudes 2^-10 .. 2688), so
// decoding to fp16 and multiplying in fp16 loses nothing, and fp16 MFMA with fp32 accumulation
// sees the exact operands.
//
// v_cvt_scalef32_pk_f16_fp4 converts the two E2M1 codes of one byte (low nibble -> element 0)
// and multiplies by 2^exponent(scale) only (an MX-style power of two), so it is used with scale
// 1.0 and the E4M3 block scale is applied with a packed fp16 multiply.
// v_cvt_scalef32_pk_f16_fp8 converts two OCP E4M3 bytes to fp16 exactly (scale 1.0).
// ---------------------------------------------------------------------------------------------

// E4M3 scale bytes 0/1 (hi=false) or 2/3 (hi=true) of w -> fp16 pair.
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

// Broadcast one fp16 lane of a pair.
__device__ __forceinline__ f16x2 bcast_lo(f16x2 v) { return f16x2{v[0], v[0]}; }
__device__ __forceinline__ f16x2 bcast_hi(f16x2 v) { return f16x2{v[1], v[1]}; }

// Decode 8 E2M1 codes (one 32-bit word, element 2i in the low nibble of byte i) scaled by s2
// (the block scale in both halves) into 8 fp16 values, returned as a 16-byte vector in element
// order.
__device__ __forceinline__ f16x8 decode8(uint32_t w, f16x2 s2) {
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// ---------------------------------------------------------------------------------------------
// bf16 helpers (bf16 is carried as raw uint16_t storage).
// ---------------------------------------------------------------------------------------------

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// ---------------------------------------------------------------------------------------------
// Wave-level reductions (64 lanes).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t t = __shfl_xor(v, o, kWave);
    v = v > t ? v : t;
  }
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

}  // namespace megamoe
