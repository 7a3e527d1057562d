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


typedef __attribute__((address_space(3))) void lvoid;

// Word 3 of a raw buffer resource (stride 0, 32-bit data format): loads past
// the record count return zeros.
constexpr int kRsrcWord3 = 0x00020000;

// XOR swizzle of the 16-byte chunks of an LDS tile row holding `cpr` chunks:
// 16 consecutive rows read at one logical chunk hit 16 distinct bank groups.
// Bank group of (row r, physical chunk p) is (r * CPR + p) mod 16; XOR-ing the
// logical chunk with the row bits above the rows sharing 256 bytes makes the
// 16 rows of one read distinct.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "swizzle defined for rows of 4, 8 or 16 chunks");
  if constexpr (CPR == 16) return r & 15;
  else if constexpr (CPR == 8) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would drain every outstanding direct-to-LDS prefetch.  The caller waits for
// exactly the loads it needs (wait_vm); this wave's LDS reads are drained
// first, so the slot they read may be refilled after the barrier.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), no vmcnt / expcnt wait
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most `n` of this wave's vector-memory loads are in flight
// (s_waitcnt with only the vmcnt field set; lgkmcnt 15 and expcnt 7 mean no
// wait).  The builtin, unlike inline asm, is seen by the compiler's own wait
// insertion, which then knows which direct-to-LDS loads have landed.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace rsa
