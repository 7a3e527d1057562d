// Shared device helpers for the gfx950 kernels of librsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// 32x32x16 matrix-core products.  Operand layout (wave64): lane l supplies
// row (A) / column (B) l%32 and the 8 consecutive k values 8*(l/32)..+7.
// Result: lane l holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4, r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 result held in accumulator register r by a lane of half h.
__device__ __forceinline__ constexpr int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Exact power of two 2^e for e in the normal range.
__device__ __forceinline__ float pow2i(int e) {
  return __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
}

// Exponent of the largest finite |x| of a row: floor(log2(x)) for x > 0 normal.
__device__ __forceinline__ int ilog2f(float x) {
  return static_cast<int>((__float_as_uint(x) >> 23) & 0xff) - 127;
}

// Workgroups are dispatched to the 8 XCDs round-robin by id.  Remap ids so
// that XCD x works through one contiguous range of the logical tile order:
// neighbouring tiles (which read overlapping key blocks) then share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd, r = total % kXcd;
  const int xcd = bid % kXcd, local = bid / kXcd;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace rsa
