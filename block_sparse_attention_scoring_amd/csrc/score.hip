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
//   score: one workgroup per (head, query block).  Each query row is scaled
//          by its own power of two and held as fp16 in LDS (exact for bf16
//          input; fp32 input is split into two fp16 terms).  The logits
//          S^T = Kbar Q^T run on the 32x32x16 fp16 matrix cores.  Pass 1
//          forms each query's max and normaliser over all key blocks; pass 2
//          recomputes the logits, forms the per-query softmax and sums it
//          over the query block in a fixed order.  No atomics: the result is
//          bitwise reproducible.
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
    load8<T>(src + static_cast<size_t>(r) * D, x);
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

template <typename T, int D, int B>
struct ScoreShape {
  static constexpr bool kSplitQ = sizeof(T) == 4;  // fp32 queries: two fp16 terms
  static constexpr int kSub = B / 32;              // 32-row query sub-tiles
  static constexpr int kKS = D / 16;               // k-steps over head_dim
  static constexpr int kQStride = D + 8;           // LDS pitch (fp16), 16 B pad
  static constexpr int kLanesPerRow = D / 8;
  static constexpr int kRowsPerPass = kScoreThreads / kLanesPerRow;
};

template <typename T, int D, int B>
__global__ __launch_bounds__(kScoreThreads, 2) void score_kernel(
    const T* __restrict__ q, const _Float16* __restrict__ khi, const _Float16* __restrict__ klo,
    const float* __restrict__ inv_t, const uint8_t* __restrict__ head_active,
    float* __restrict__ scores, int N, int NB, int NBp) {
  using S = ScoreShape<T, D, B>;
  __shared__ __attribute__((aligned(16))) _Float16 Qh[B * S::kQStride];
  __shared__ __attribute__((aligned(16))) _Float16 Ql[S::kSplitQ ? B * S::kQStride : 8];
  __shared__ float row_inv[B];
  __shared__ float part_m[kScoreWaves * 2][B];
  __shared__ float part_z[kScoreWaves * 2][B];
  __shared__ float row_m[B];
  __shared__ float row_w[B];

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int h = tile / NB, I = tile - h * NB;
  if (head_active != nullptr && head_active[h] == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int q0 = I * B, bI = min(B, N - q0);

  // ---- queries -> per-row power-of-two scale -> fp16 in LDS
  {
    const int rg = tid / S::kLanesPerRow, c8 = tid % S::kLanesPerRow;
    for (int r = rg; r < B; r += S::kRowsPerPass) {
      float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (r < bI) load8<T>(q + (static_cast<size_t>(h) * N + q0 + r) * D + c8 * 8, x);
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(x[e]));
#pragma unroll
      for (int o = 1; o < S::kLanesPerRow; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
      const int sh = scale_shift(a);
      const float s = pow2i(sh);
      f16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xs = x[e] * s;
        hi[e] = static_cast<_Float16>(xs);
        lo[e] = static_cast<_Float16>(xs - static_cast<float>(hi[e]));
      }
      *reinterpret_cast<f16x8*>(&Qh[r * S::kQStride + c8 * 8]) = hi;
      if constexpr (S::kSplitQ) *reinterpret_cast<f16x8*>(&Ql[r * S::kQStride + c8 * 8]) = lo;
      if (c8 == 0) row_inv[r] = pow2i(-sh);
    }
  }
  __syncthreads();

  const float it_h = inv_t[h];
  float sc[S::kSub];
#pragma unroll
  for (int st = 0; st < S::kSub; ++st) sc[st] = row_inv[32 * st + col] * it_h;

  const int n_chunks = NBp / 32;
  const _Float16* kh_head = khi + static_cast<size_t>(h) * NBp * D;
  const _Float16* kl_head = klo + static_cast<size_t>(h) * NBp * D;

  // logits of chunk c (32 key blocks) for query sub-tile st, raw units; the
  // hi and lo terms run as two independent accumulation chains
  auto logits = [&](const f16x8 (&ahi)[S::kKS], const f16x8 (&alo)[S::kKS], int st) {
    f32x16 acc_hi = f32x16{}, acc_lo = f32x16{};
#pragma unroll
    for (int s = 0; s < S::kKS; ++s) {
      const f16x8 b = *reinterpret_cast<const f16x8*>(&Qh[(32 * st + col) * S::kQStride + 16 * s + 8 * hl]);
      acc_hi = mfma32(ahi[s], b, acc_hi);
      acc_lo = mfma32(alo[s], b, acc_lo);
      if constexpr (S::kSplitQ) {
        const f16x8 bl = *reinterpret_cast<const f16x8*>(&Ql[(32 * st + col) * S::kQStride + 16 * s + 8 * hl]);
        acc_lo = mfma32(ahi[s], bl, acc_lo);
      }
    }
    return acc_hi + acc_lo;
  };
  auto load_a = [&](int c, f16x8 (&ahi)[S::kKS], f16x8 (&alo)[S::kKS]) {
    const size_t row = static_cast<size_t>(32 * c + col) * D + 8 * hl;
#pragma unroll
    for (int s = 0; s < S::kKS; ++s) {
      ahi[s] = *reinterpret_cast<const f16x8*>(kh_head + row + 16 * s);
      alo[s] = *reinterpret_cast<const f16x8*>(kl_head + row + 16 * s);
    }
  };

  // ---- pass 1: per-query max and normaliser over all key blocks
  float mraw[S::kSub], z[S::kSub];
#pragma unroll
  for (int st = 0; st < S::kSub; ++st) {
    mraw[st] = -INFINITY;
    z[st] = 0.f;
  }
  for (int c = wave; c < n_chunks; c += kScoreWaves) {
    f16x8 ahi[S::kKS], alo[S::kKS];
    load_a(c, ahi, alo);
    const bool tail = 32 * c + 32 > NB;
#pragma unroll
    for (int st = 0; st < S::kSub; ++st) {
      __builtin_amdgcn_sched_barrier(0);  // one sub-tile's registers live at a time
      f32x16 acc = logits(ahi, alo, st);
      if (tail) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * c + acc_row(r, hl) >= NB) acc[r] = -INFINITY;
      }
      float cm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) cm = fmaxf(cm, acc[r]);
      if (cm > mraw[st]) {
        z[st] *= exp2f((mraw[st] - cm) * sc[st]);
        mraw[st] = cm;
      }
      if (mraw[st] > -INFINITY) {
        const float mb = -mraw[st] * sc[st];
        float zs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) zs += __builtin_amdgcn_exp2f(fmaf(acc[r], sc[st], mb));
        z[st] += zs;
      }
    }
  }
#pragma unroll
  for (int st = 0; st < S::kSub; ++st) {
    part_m[wave * 2 + hl][32 * st + col] = mraw[st] > -INFINITY ? mraw[st] * sc[st] : -INFINITY;
    part_z[wave * 2 + hl][32 * st + col] = z[st];
  }
  __syncthreads();
  if (tid < B) {
    float m = -INFINITY;
#pragma unroll
    for (int g = 0; g < kScoreWaves * 2; ++g) m = fmaxf(m, part_m[g][tid]);
    float zt = 0.f;
#pragma unroll
    for (int g = 0; g < kScoreWaves * 2; ++g)
      if (part_m[g][tid] > -INFINITY) zt += part_z[g][tid] * exp2f(part_m[g][tid] - m);
    row_m[tid] = m;
    row_w[tid] = tid < bI ? 1.f / (static_cast<float>(bI) * zt) : 0.f;
  }
  __syncthreads();

  float rm[S::kSub], rw[S::kSub];
#pragma unroll
  for (int st = 0; st < S::kSub; ++st) {
    rm[st] = -row_m[32 * st + col];
    rw[st] = row_w[32 * st + col];
  }

  // ---- pass 2: softmax of every query, summed over the query block
  float* srow = scores + (static_cast<size_t>(h) * NB + I) * NB;
  for (int c = wave; c < n_chunks; c += kScoreWaves) {
    f16x8 ahi[S::kKS], alo[S::kKS];
    load_a(c, ahi, alo);
    const bool tail = 32 * c + 32 > NB;
    float colsum[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) colsum[r] = 0.f;
#pragma unroll
    for (int st = 0; st < S::kSub; ++st) {
      __builtin_amdgcn_sched_barrier(0);  // one sub-tile's registers live at a time
      f32x16 acc = logits(ahi, alo, st);
      if (tail) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * c + acc_row(r, hl) >= NB) acc[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) colsum[r] += __builtin_amdgcn_exp2f(fmaf(acc[r], sc[st], rm[st])) * rw[st];
    }
    // Sum over the 32 query rows held by the 32 lanes of this half, as a
    // reduce-scatter: at the exchange over lane bit b a lane keeps the half of
    // its values that matches its bit and adds the partner's copy of them.
    // Lane `col` ends with the total of accumulator register col >> 1.
    const float total = reduce_scatter_32(colsum, col);
    if ((col & 1) == 0) {
      const int J = 32 * c + acc_row(col >> 1, hl);
      if (J < NB) srow[J] = total;
    }
  }
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
  if (p.block == 128)
    hipLaunchKernelGGL((score_kernel<T, D, 128>), dim3(grid), dim3(kScoreThreads), 0, stream,
                       static_cast<const T*>(q), ws.khi, ws.klo, ws.inv_t, head_active, scores,
                       p.tokens, p.nb, NBp);
  else
    hipLaunchKernelGGL((score_kernel<T, D, 64>), dim3(grid), dim3(kScoreThreads), 0, stream,
                       static_cast<const T*>(q), ws.khi, ws.klo, ws.inv_t, head_active, scores,
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

}  // namespace rsa
