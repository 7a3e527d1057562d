// PARK block scoring (gfx950).
//
// PARK (Accurate Block Retrieval for Sparse Attention in Video Diffusion
// Transformers), Abstract: retrieval starts from the mean of each key block;
// PARK keeps every query, normalises its attention over the key blocks on its
// own, and averages those distributions within each query block.
//
//   pool:  Kbar[h,J] = mean of the b_J keys of block J, times scale*log2(e)
//          (fp64 sums, rounded once to fp32), and max |Kbar[h,J,:]|.
//   split: per head one power-of-two factor t_h brings max |Kbar| into
//          [2^13, 2^14); Kbar*t_h = hi + lo with hi, lo fp16.  hi+lo holds
//          22 significant bits, so the logits below are fp32-faithful.
//   score: one four-wave workgroup per (head, query block of 128 tokens, or
//          pair of 64-token blocks).  Each query row is scaled
//          by its own power of two and held as fp16 in registers (exact for
//          bf16 input; fp32 input is split into two fp16 terms); the split
//          pooled keys stream through an LDS ring.  The logits run on the
//          32x32x16 fp16 matrix cores.  Pass 1 forms each query's max and
//          normaliser over all key blocks; pass 2 recomputes the logits,
//          forms the per-query softmax and sums it over the query block in a
//          fixed order.  No atomics: the result is bitwise reproducible.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rsa {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kScoreThreads = 256;
constexpr int kScoreWaves = kScoreThreads / kWave;
constexpr int kSplitGroups = 16;

template <typename T>
__device__ __forceinline__ void load8(const T* src, float (&x)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* src, float (&x)[8]) {
  const u32x4 raw = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(raw[e] << 16);
    x[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* src, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(src);
  const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[4 + e] = b[e];
  }
}

// The same with a non-temporal load, for the pooling pass's read-once
// stream over K (the scorer's query loads keep the default policy, which
// measured faster there).
template <typename T>
__device__ __forceinline__ void load8_nt(const T* src, float (&x)[8]);

template <>
__device__ __forceinline__ void load8_nt<uint16_t>(const uint16_t* src, float (&x)[8]) {
  const u32x4 raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(raw[e] << 16);
    x[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load8_nt<float>(const float* src, float (&x)[8]) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + 4));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[4 + e] = b[e];
  }
}

// ---------------------------------------------------------------- pool
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(
    const T* __restrict__ k, const uint8_t* __restrict__ head_active, float* __restrict__ kt,
    float* __restrict__ bmax, int N, int NB, int B, double mul) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerPass = kPoolThreads / kLanesPerRow;
  __shared__ double part[kRowsPerPass][D];
  __shared__ float red[kPoolThreads / kWave];
  const int h = blockIdx.y, J = blockIdx.x;
  if (head_active != nullptr && head_active[h] == 0) return;
  const int tid = threadIdx.x;
  const int rg = tid / kLanesPerRow, c8 = tid % kLanesPerRow;
  const int lo = J * B, bJ = min(B, N - lo);
  const T* src = k + (static_cast<size_t>(h) * N + lo) * D + c8 * 8;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = rg; r < bJ; r += kRowsPerPass) {
    float x[8];
    load8_nt<T>(src + static_cast<size_t>(r) * D, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += static_cast<double>(x[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][c8 * 8 + e] = acc[e];
  __syncthreads();
  float a = 0.f;
  if (tid < D) {
    double s = 0.0;
    for (int g = 0; g < kRowsPerPass; ++g) s += part[g][tid];
    const float val = static_cast<float>(s / bJ * mul);
    kt[(static_cast<size_t>(h) * NB + J) * D + tid] = val;
    a = fabsf(val);
  }
  a = wave_max(a);
  if ((tid & 63) == 0) red[tid >> 6] = a;
  __syncthreads();
  if (tid == 0) {
    float m = red[0];
    for (int w = 1; w < kPoolThreads / kWave; ++w) m = fmaxf(m, red[w]);
    bmax[static_cast<size_t>(h) * NB + J] = m;
  }
}

// Power of two bringing `amax` into [2^13, 2^14) (1 for zero / non-finite).
__device__ __forceinline__ int scale_shift(float amax) {
  if (!(amax > 0.f) || !(amax < INFINITY)) return 0;
  const int s = 13 - ilog2f(amax);
  return s < -126 ? -126 : (s > 126 ? 126 : s);
}

// ---------------------------------------------------------------- split
template <int D>
__global__ __launch_bounds__(256) void split_kernel(
    const float* __restrict__ kt, const float* __restrict__ bmax,
    const uint8_t* __restrict__ head_active, _Float16* __restrict__ khi,
    _Float16* __restrict__ klo, float* __restrict__ inv_t, int NB, int NBp) {
  __shared__ float red[4];
  const int h = blockIdx.y;
  if (head_active != nullptr && head_active[h] == 0) return;
  const int tid = threadIdx.x;
  float m = 0.f;
  for (int j = tid; j < NB; j += 256) m = fmaxf(m, bmax[static_cast<size_t>(h) * NB + j]);
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int sh = scale_shift(m);
  const float t = pow2i(sh);
  if (blockIdx.x == 0 && tid == 0) inv_t[h] = pow2i(-sh);
  const int rows_per = (NBp + gridDim.x - 1) / gridDim.x;
  const int r0 = blockIdx.x * rows_per, r1 = min(NBp, r0 + rows_per);
  for (int e = r0 * D + tid; e < r1 * D; e += 256) {
    const int j = e / D;
    const size_t o = static_cast<size_t>(h) * NBp * D + e;
    if (j < NB) {
      const float x = kt[static_cast<size_t>(h) * NB * D + e] * t;
      const _Float16 hi = static_cast<_Float16>(x);
      khi[o] = hi;
      klo[o] = static_cast<_Float16>(x - static_cast<float>(hi));
    } else {
      khi[o] = static_cast<_Float16>(0.f);
      klo[o] = static_cast<_Float16>(0.f);
    }
  }
}

// ---------------------------------------------------------------- score
// Exchange with the lane whose index (within its 32-lane half) differs in the
// bits of `mask` (ds_swizzle bit mode: and 0x1f, or 0, xor mask).
template <int mask>
__device__ __forceinline__ float swap_lanes(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (mask << 10) | 0x1f));
}

// Reduce-scatter of 16 values over 32 lanes (16 exchanges instead of 80):
// returns, to lane `col`, the sum over the 32 lanes of v[col >> 1].
__device__ __forceinline__ float reduce_scatter_32(const float (&v)[16], int col) {
  float a[8];
  const bool b4 = col & 16, b3 = col & 8, b2 = col & 4, b1 = col & 2;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float keep = b4 ? v[j + 8] : v[j], send = b4 ? v[j] : v[j + 8];
    a[j] = keep + swap_lanes<16>(send);
  }
  float b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float keep = b3 ? a[j + 4] : a[j], send = b3 ? a[j] : a[j + 4];
    b[j] = keep + swap_lanes<8>(send);
  }
  float c[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float keep = b2 ? b[j + 2] : b[j], send = b2 ? b[j] : b[j + 2];
    c[j] = keep + swap_lanes<4>(send);
  }
  const float keep = b1 ? c[1] : c[0], send = b1 ? c[0] : c[1];
  const float d = keep + swap_lanes<2>(send);
  return d + swap_lanes<1>(d);
}

// One workgroup per (head, query block), one wave per 32 query rows.  Each
// wave keeps its rows in registers, scaled by the row's own power of two and
// held as fp16 (exact for bf16 input; fp32 input adds a second fp16 term).
// The split pooled keys stream in chunks of 32 key blocks (hi and lo tiles)
// into a ring of NBUF LDS slots with buffer loads, shared by all waves; with
// two slots (32 KB) four workgroups share a CU, with three slots (48 KB)
// three, and the register budget is capped to match.
// Both passes form one walk of 2 x NBp/32 chunk steps, so the prefetch runs
// on across the pass boundary:
//   pass 1 (chunk steps 0..nc-1): logits S^T = Kbar Q^T (hi and lo terms in
//     two accumulation chains), per-query running max and normaliser; the
//     two lane halves hold different key blocks of the same query and merge
//     once at the end of the pass;
//   pass 2 (steps nc..2nc-1): the logits again, untransposed this time
//     (S = Q Kbar^T: the same registers and LDS reads with the operands
//     swapped), so a lane holds one key block for 16 of the wave's queries
//     and the softmax summed over queries is 16 in-lane additions and one
//     exchange between the lane halves; each query's scale, maximum and
//     weight 1/(b_I * normaliser) enter as per-register constants (the
//     weight folded into the exponent).  The waves' partial sums of a chunk
//     meet in an LDS pair (indexed by chunk parity) and are added in wave
//     order after the next step's barrier.
// Store to LDS outside the compiler's wait tracking.  Its own wait insertion
// cannot tell this store from a write into the ring slots the direct-to-LDS
// loads fill, so it would drain them first; the target never overlaps a slot
// and the next barrier_lds() waits for the store (lgkmcnt).
__device__ __forceinline__ void lds_store_f32(float* p, float v) {
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lvoid*)p));
  asm volatile("ds_write_b32 %0, %1" ::"v"(a), "v"(v) : "memory");
}

// kColMask: key "blocks" are clusters, some possibly empty (colsize 0); an
// empty cluster takes no part in any query's softmax and scores 0.
// BQ < B: the workgroup's B rows are B / BQ consecutive query blocks of BQ
// tokens (waves of block P*B/BQ + w / (BQ/32)), each with its own weight and
// score row, so 64-token blocks still run four waves per workgroup.
template <typename T, int D, int B, int NBUF, bool kColMask = false, int BQ = B>
__global__ __launch_bounds__(2 * B, NBUF == 2 ? 4 : NBUF == 3 ? 3 : 2) void score_kernel(
    const T* __restrict__ q, const _Float16* __restrict__ khi, const _Float16* __restrict__ klo,
    const float* __restrict__ inv_t, const uint8_t* __restrict__ head_active,
    const int* __restrict__ colsize, float* __restrict__ scores, int N, int NB, int NBp) {
  constexpr bool kSplitQ = sizeof(T) == 4;
  constexpr int kWaves = B / 32, kThreads = kWaves * kWave;
  constexpr int kKS = D / 16;                              // k-steps over head_dim
  constexpr int kTile = 32 * D;                            // fp16 elements of a hi (or lo) tile
  constexpr int kCpr = D / 8;                              // 16-byte chunks per row
  constexpr int kLoads = kTile * 2 / 16 / kThreads;        // loads per lane per tile
  constexpr int kPer = 2 * kLoads;                         // loads per lane per step
  static_assert(kLoads >= 1 && kTile * 2 % (16 * kThreads) == 0, "tile not divisible");
  static_assert(NBUF >= 2 && NBUF <= 4, "ring of 2 to 4 LDS slots");
  __shared__ __attribute__((aligned(1024))) _Float16 slot0[2 * kTile];
  __shared__ __attribute__((aligned(1024))) _Float16 slot1[2 * kTile];
  __shared__ __attribute__((aligned(1024))) _Float16 slot2[NBUF > 2 ? 2 * kTile : 8];
  __shared__ __attribute__((aligned(1024))) _Float16 slot3[NBUF > 3 ? 2 * kTile : 8];
  __shared__ float part[2][kWaves][32];
  __shared__ float qconst[kWaves][2][32];  // per query of a wave: scale, -max - log2(weight)

  constexpr int kBlk = B / BQ, kWpb = BQ / 32;  // query blocks per workgroup, waves per block
  static_assert(BQ % 32 == 0 && B % BQ == 0, "whole waves per query block");
  const int units = (NB + kBlk - 1) / kBlk;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int h = tile / units, P = tile - h * units;
  if (head_active != nullptr && head_active[h] == 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, col = lane & 31;
  const int sub = wave / kWpb, I = P * kBlk + sub;  // this wave's query block (I >= NB: none)
  const int q0 = I * BQ, bI = I < NB ? min(BQ, N - q0) : 0;
  const int wrow = (wave % kWpb) * 32;  // first row of this wave inside its block
  const bool qvalid = wrow + col < bI;

  // ---- this lane's query values (row wave*32+col, columns 16s+8hl..+7)
  f16x8 qh[kKS], ql[kSplitQ ? kKS : 1];
  float sc;
  {
    float x[kKS][8];
    // rows past the last token read row q0 and are zeroed
    const T* src = q + (static_cast<size_t>(h) * N + (qvalid ? q0 + wrow + col : 0)) * D + 8 * hl;
    const float keep = qvalid ? 1.f : 0.f;
    float a = 0.f;
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
      load8<T>(src + 16 * s, x[s]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[s][e] *= keep;
        a = fmaxf(a, fabsf(x[s][e]));
      }
    }
    a = fmaxf(a, __shfl_xor(a, 32));  // the other half of the row
    const int sh = scale_shift(a);
    const float sf = pow2i(sh);
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xs = x[s][e] * sf;
        qh[s][e] = static_cast<_Float16>(xs);
        if constexpr (kSplitQ) ql[s][e] = static_cast<_Float16>(xs - static_cast<float>(qh[s][e]));
      }
    }
    sc = pow2i(-sh) * inv_t[h];
  }

  // ---- chunk loads: pooled-key rows 32c..32c+31, hi then lo
  const int nc = NBp / 32;
  const int U = 2 * nc;  // steps: pass 1 then pass 2
  const _Float16* kh_head = khi + static_cast<size_t>(h) * NBp * D;
  const _Float16* kl_head = klo + static_cast<size_t>(h) * NBp * D;
  uint32_t off[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int pc = (wave * kLoads + i) * 64 + lane;
    const int r = pc / kCpr;
    off[i] = static_cast<uint32_t>(r * D + ((pc % kCpr) ^ swz<kCpr>(r)) * 8) * 2u;
  }
  auto issue = [&](int u, _Float16* dst) __attribute__((always_inline)) {
    const int c = u < nc ? u : u - nc;
    const size_t base = static_cast<size_t>(32 * c) * D;
    const __amdgpu_buffer_rsrc_t rh =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(kh_head + base), 0, kTile * 2, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rl =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(kl_head + base), 0, kTile * 2, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int blk = wave * kLoads + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lvoid*)(dst + blk * 512), 16, static_cast<int>(off[i]), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lvoid*)(dst + kTile + blk * 512), 16, static_cast<int>(off[i]), 0,
                                               0, 0);
    }
  };

  // ---- logits of one chunk, raw units (rows past NB: -inf)
  // kTr: S^T (lane = query, registers = key blocks) for pass 1, else S
  // (lane = key block, registers = queries) for pass 2
  auto logits = [&](int c, const _Float16* cur, auto kTr) __attribute__((always_inline)) {
    const char* th = reinterpret_cast<const char*>(cur);
    const char* tl = reinterpret_cast<const char*>(cur + kTile);
    // hi and lo terms in one accumulation chain (several waves per SIMD
    // interleave their chains; two chains would cost 16 adds per chunk)
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
      const int o = col * (2 * D) + (((2 * s + hl) ^ swz<kCpr>(col)) * 16);
      const f16x8 ah = *reinterpret_cast<const f16x8*>(th + o);
      const f16x8 al = *reinterpret_cast<const f16x8*>(tl + o);
      if constexpr (decltype(kTr)::value) {
        acc = mfma32(ah, qh[s], acc);
        acc = mfma32(al, qh[s], acc);
        if constexpr (kSplitQ) acc = mfma32(ah, ql[s], acc);
      } else {
        acc = mfma32(qh[s], ah, acc);
        acc = mfma32(qh[s], al, acc);
        if constexpr (kSplitQ) acc = mfma32(ql[s], ah, acc);
      }
    }
    return acc;
  };

  float mraw = -INFINITY, z = 0.f;  // pass 1, this half's key blocks
  float qs[16], qm[16];              // pass 2: per register (query) constants
  // score row written by this lane in finish(): block P*kBlk + hl (lanes of
  // wave 0, one lane half per block)
  static_assert(kBlk <= 2, "one lane half of wave 0 per query block");
  const int Iw = P * kBlk + hl;
  float* srow = scores + (static_cast<size_t>(h) * NB + min(Iw, NB - 1)) * NB;
  // column 32c + col of this lane holds keys (cluster mode)
  auto live_col = [&](int c) __attribute__((always_inline)) {
    const int j = 32 * c + col;
    return j < NB && colsize[static_cast<size_t>(h) * NB + j] > 0;
  };
  // all waves' partial sums of chunk c are in part[c & 1]; each block's
  // waves are added in wave order
  auto finish = [&](int c) __attribute__((always_inline)) {
    if (wave == 0 && hl < kBlk && Iw < NB && 32 * c + col < NB) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < kWpb; ++w) t += part[c & 1][hl * kWpb + w][col];
      srow[32 * c + col] = t;
    }
  };
  auto body = [&](int u, const _Float16* cur) __attribute__((always_inline)) {
    if (u < nc) {
      f32x16 acc = logits(u, cur, std::true_type{});
      if constexpr (kColMask) {
        // lane col's bit says whether column 32u + col is a live cluster
        const uint32_t live = static_cast<uint32_t>(__ballot(live_col(u)));
        // register r holds column acc_row(r, 0) + 4 hl: its test is uniform in
        // each lane half, so it is a lane mask built in scalar registers
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = acc_row(r, 0);
          const uint64_t m = (((live >> c) & 1u) ? 0ull : 0xffffffffull) |
                             (((live >> (c + 4)) & 1u) ? 0ull : 0xffffffff00000000ull);
          if (__builtin_amdgcn_inverse_ballot_w64(m)) acc[r] = -INFINITY;
        }
      } else if (32 * u + 32 > NB) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 32 * u + acc_row(r, 0);
          const uint64_t m = (c >= NB ? 0xffffffffull : 0ull) | (c + 4 >= NB ? 0xffffffff00000000ull : 0ull);
          if (__builtin_amdgcn_inverse_ballot_w64(m)) acc[r] = -INFINITY;
        }
      }
      float cm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) cm = fmaxf(cm, acc[r]);
      if (cm > mraw) {
        z *= exp2f((mraw - cm) * sc);
        mraw = cm;
      }
      if (mraw > -INFINITY) {
        const float mb = -mraw * sc;
        float zs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 16; ++r) zs[r & 3] += __builtin_amdgcn_exp2f(fmaf(acc[r], sc, mb));
        z += (zs[0] + zs[1]) + (zs[2] + zs[3]);
      }
      if (u == nc - 1) {
        // merge the two halves' statistics of each query; hand every lane the
        // constants of the 16 queries its registers hold in pass 2
        const float ml = mraw > -INFINITY ? mraw * sc : -INFINITY;
        const float mo = __shfl_xor(ml, 32), zo = __shfl_xor(z, 32);
        const float m = fmaxf(ml, mo);
        const float zt = (ml > -INFINITY ? z * exp2f(ml - m) : 0.f) + (mo > -INFINITY ? zo * exp2f(mo - m) : 0.f);
        // p / (b_I zt) = 2^(s*sc - m - log2(b_I zt)); rows past the end get
        // +inf, so their terms are exactly 0
        const float mw = qvalid ? m + log2f(static_cast<float>(bI) * zt) : INFINITY;
        if (hl == 0) {
          lds_store_f32(&qconst[wave][0][col], sc);
          lds_store_f32(&qconst[wave][1][col], mw);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's stores (lgkmcnt(0))
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          qs[r] = qconst[wave][0][acc_row(r, hl)];
          qm[r] = -qconst[wave][1][acc_row(r, hl)];
        }
      }
      return;
    }
    const int c = u - nc;
    if (c > 0) finish(c - 1);
    const f32x16 acc = logits(c, cur, std::false_type{});
    // key block 32c + col of this lane; the registers hold 16 queries
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) ps[r & 3] += __builtin_amdgcn_exp2f(fmaf(acc[r], qs[r], qm[r]));
    float t = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    t += __shfl_xor(t, 32);  // the other 16 queries
    if constexpr (kColMask) {
      if (!live_col(c)) t = 0.f;
    }
    if (hl == 0) lds_store_f32(&part[c & 1][wave][col], t);
  };

  // ---- the walk: ring slot u % NBUF, NBUF-1 chunks in flight
  auto ring = [&](int i) { return i == 0 ? slot0 : i == 1 ? slot1 : i == 2 ? slot2 : slot3; };
  auto steady = [&](int u, const _Float16* cur, _Float16* nxt) __attribute__((always_inline)) {
    wait_vm<(NBUF - 2) * kPer>();
    barrier_lds();
    issue(u + NBUF - 1, nxt);
    body(u, cur);
  };
  int u = 0;
  if (U >= 2 * NBUF - 1) {
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) issue(i, ring(i));
    do {
      steady(u, slot0, ring(NBUF - 1));
      steady(u + 1, slot1, slot0);
      if constexpr (NBUF > 2) steady(u + 2, slot2, slot1);
      if constexpr (NBUF > 3) steady(u + 3, slot3, slot2);
      u += NBUF;
    } while (u + 2 * NBUF - 2 < U);
  } else {
    for (int i = 0; i < NBUF - 1 && i < U; ++i) issue(i, ring(i));
  }
  for (; u < U; ++u) {
    wait_vm<0>();
    barrier_lds();
    if (u + NBUF - 1 < U) issue(u + NBUF - 1, ring((u + NBUF - 1) % NBUF));
    body(u, ring(u % NBUF));
  }
  __syncthreads();
  finish(nc - 1);
}

template <typename T, int D>
hipError_t launch_scoring_t(const Problem& p, const void* q, const void* k,
                            const uint8_t* head_active, float* scores, const ScoreWs& ws,
                            hipStream_t stream) {
  const int NBp = (p.nb + kScoreRowPad - 1) / kScoreRowPad * kScoreRowPad;
  const double mul = static_cast<double>(p.scale) * 1.4426950408889634;
  hipLaunchKernelGGL((pool_kernel<T, D>), dim3(p.nb, p.heads), dim3(kPoolThreads), 0, stream,
                     static_cast<const T*>(k), head_active, ws.kt, ws.bmax, p.tokens, p.nb,
                     p.block, mul);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((split_kernel<D>), dim3(kSplitGroups, p.heads), dim3(256), 0, stream,
                     ws.kt, ws.bmax, head_active, ws.khi, ws.klo, ws.inv_t, p.nb, NBp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = p.heads * p.nb;
  // bf16 queries: a ring of two slots (32 KB, one chunk in flight), four
  // workgroups per CU (four waves per SIMD at 128 registers); fp32 queries
  // need more registers
  constexpr int kNbuf = std::is_same_v<T, uint16_t> ? 2 : 4;
  if (p.block == 128)
    hipLaunchKernelGGL((score_kernel<T, D, 128, kNbuf>), dim3(grid), dim3(256), 0, stream,
                       static_cast<const T*>(q), ws.khi, ws.klo, ws.inv_t, head_active, nullptr, scores,
                       p.tokens, p.nb, NBp);
  else  // 64-token blocks: two per four-wave workgroup
    hipLaunchKernelGGL((score_kernel<T, D, 128, kNbuf, false, 64>), dim3(p.heads * ((p.nb + 1) / 2)), dim3(256),
                       0, stream, static_cast<const T*>(q), ws.khi, ws.klo, ws.inv_t, head_active, nullptr,
                       scores, p.tokens, p.nb, NBp);
  return hipGetLastError();
}

// Cluster centroids as pooled keys: kt = c * mul (one rounding), zero rows
// and max 0 for empty clusters; one wave per (cluster, head).
template <int D>
__global__ __launch_bounds__(kWave) void cent_prep_kernel(const float* __restrict__ cent,
                                                          const int* __restrict__ sizes, float* __restrict__ kt,
                                                          float* __restrict__ bmax, int NB, double mul) {
  const int j = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const size_t row = static_cast<size_t>(h) * NB + j;
  const bool live = sizes[row] > 0;
  float a = 0.f;
  for (int d = lane; d < D; d += kWave) {
    const float x = live ? static_cast<float>(static_cast<double>(cent[row * D + d]) * mul) : 0.f;
    kt[row * D + d] = x;
    a = fmaxf(a, fabsf(x));
  }
  a = wave_max(a);
  if (lane == 0) bmax[row] = a;
}

template <typename T, int D>
hipError_t launch_cluster_scoring_t(const Problem& p, const void* q, const float* cent, const int* sizes,
                                    float* scores, const ScoreWs& ws, hipStream_t stream) {
  const int NBp = (p.nb + kScoreRowPad - 1) / kScoreRowPad * kScoreRowPad;
  const double mul = static_cast<double>(p.scale) * 1.4426950408889634;
  hipLaunchKernelGGL((cent_prep_kernel<D>), dim3(p.nb, p.heads), dim3(kWave), 0, stream, cent, sizes, ws.kt,
                     ws.bmax, p.nb, mul);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((split_kernel<D>), dim3(kSplitGroups, p.heads), dim3(256), 0, stream,
                     ws.kt, ws.bmax, nullptr, ws.khi, ws.klo, ws.inv_t, p.nb, NBp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = p.heads * p.nb;
  // bf16 queries: two slots, four workgroups per CU, as for key blocks
  constexpr int kNbuf = std::is_same_v<T, uint16_t> ? 2 : 4;
  if (p.block == 128)
    hipLaunchKernelGGL((score_kernel<T, D, 128, kNbuf, true>), dim3(grid), dim3(256), 0, stream,
                       static_cast<const T*>(q), ws.khi, ws.klo, ws.inv_t, nullptr, sizes, scores, p.tokens,
                       p.nb, NBp);
  else  // 64-token blocks: two per four-wave workgroup
    hipLaunchKernelGGL((score_kernel<T, D, 128, kNbuf, true, 64>), dim3(p.heads * ((p.nb + 1) / 2)), dim3(256),
                       0, stream, static_cast<const T*>(q), ws.khi, ws.klo, ws.inv_t, nullptr, sizes, scores,
                       p.tokens, p.nb, NBp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_means(const Problem& p, const void* x, double mul, float* out, float* bmax,
                              hipStream_t stream) {
  if (p.dtype == 0) {
    if (p.head_dim == 128)
      hipLaunchKernelGGL((pool_kernel<uint16_t, 128>), dim3(p.nb, p.heads), dim3(kPoolThreads), 0, stream,
                         static_cast<const uint16_t*>(x), nullptr, out, bmax, p.tokens, p.nb, p.block, mul);
    else
      hipLaunchKernelGGL((pool_kernel<uint16_t, 64>), dim3(p.nb, p.heads), dim3(kPoolThreads), 0, stream,
                         static_cast<const uint16_t*>(x), nullptr, out, bmax, p.tokens, p.nb, p.block, mul);
  } else {
    if (p.head_dim == 128)
      hipLaunchKernelGGL((pool_kernel<float, 128>), dim3(p.nb, p.heads), dim3(kPoolThreads), 0, stream,
                         static_cast<const float*>(x), nullptr, out, bmax, p.tokens, p.nb, p.block, mul);
    else
      hipLaunchKernelGGL((pool_kernel<float, 64>), dim3(p.nb, p.heads), dim3(kPoolThreads), 0, stream,
                         static_cast<const float*>(x), nullptr, out, bmax, p.tokens, p.nb, p.block, mul);
  }
  return hipGetLastError();
}

size_t score_ws_layout(const Problem& p, ScoreWs* ws, void* base) {
  const size_t NBp = (p.nb + kScoreRowPad - 1) / kScoreRowPad * kScoreRowPad;
  auto align = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t kt = align(sizeof(float) * p.heads * p.nb * p.head_dim);
  const size_t bm = align(sizeof(float) * p.heads * p.nb);
  const size_t sp = align(sizeof(_Float16) * p.heads * NBp * p.head_dim);
  const size_t it = align(sizeof(float) * p.heads);
  if (ws != nullptr) {
    char* b = static_cast<char*>(base);
    ws->kt = reinterpret_cast<float*>(b);
    ws->bmax = reinterpret_cast<float*>(b + kt);
    ws->khi = reinterpret_cast<_Float16*>(b + kt + bm);
    ws->klo = reinterpret_cast<_Float16*>(b + kt + bm + sp);
    ws->inv_t = reinterpret_cast<float*>(b + kt + bm + 2 * sp);
  }
  return kt + bm + 2 * sp + it;
}

hipError_t launch_scoring(const Problem& p, const void* q, const void* k,
                          const uint8_t* head_active, float* scores, const ScoreWs& ws,
                          hipStream_t stream) {
  if (p.dtype == 0) {
    return p.head_dim == 128 ? launch_scoring_t<uint16_t, 128>(p, q, k, head_active, scores, ws, stream)
                             : launch_scoring_t<uint16_t, 64>(p, q, k, head_active, scores, ws, stream);
  }
  return p.head_dim == 128 ? launch_scoring_t<float, 128>(p, q, k, head_active, scores, ws, stream)
                           : launch_scoring_t<float, 64>(p, q, k, head_active, scores, ws, stream);
}

hipError_t launch_cluster_scoring(const Problem& p, const void* q, const float* cent, const int* sizes,
                                  float* scores, const ScoreWs& ws, hipStream_t stream) {
  if (p.dtype == 0)
    return p.head_dim == 128 ? launch_cluster_scoring_t<uint16_t, 128>(p, q, cent, sizes, scores, ws, stream)
                             : launch_cluster_scoring_t<uint16_t, 64>(p, q, cent, sizes, scores, ws, stream);
  return p.head_dim == 128 ? launch_cluster_scoring_t<float, 128>(p, q, cent, sizes, scores, ws, stream)
                           : launch_cluster_scoring_t<float, 64>(p, q, cent, sizes, scores, ws, stream);
}

}  // namespace rsa
