// Retrieval accuracy on gfx950: dense block mass and the query-pooled scorer.
//
// PARK (Accurate Block Retrieval for Sparse Attention in Video Diffusion
// Transformers), Abstract: the method retrieves the key blocks that matter to
// each query block more accurately than a scorer that averages the queries
// before the softmax.  These kernels give the yardstick and the comparison:
//
//   mass[h, I, J]  = mean over the queries i of block I of the dense softmax
//                    (over all N keys) of scale * <q_i, k_t>, summed over the
//                    tokens t of key block J (every row sums to 1);
//   pooled[h, I, J] = softmax over J of scale * <qbar_I, kbar_J>, the block
//                    means of the queries and keys (the averaging PARK's
//                    abstract names as the defect).
#include "common.h"
#include "kernels.h"

namespace rsa {
namespace {

// Sum over the 64 lanes of a wave (fixed butterfly order).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Dense block mass, bf16 inputs.  One workgroup per (head, query block), one
// wave per 32 query rows, S^T = K Q^T on the matrix cores (as in the
// attention kernel: a lane owns one query, the two lane halves hold
// different keys of it).  Pass 1 walks all keys in 32-key sub-tiles and
// keeps each query's exact running maximum and fp64 normaliser; pass 2
// recomputes the same S^T, turns it into normalised probabilities and sums
// them per key block over the keys and the block's real queries.  K
// sub-tiles stream into two LDS slots with buffer loads (rows past the last
// token read as zeros and are masked).  At the end of key block J every wave
// leaves its total in an LDS pair indexed by J's parity; one thread adds the
// waves' totals in wave order after the next barrier.
template <int D, int B>
__global__ __launch_bounds__(2 * B, 2) void dense_mass_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, float* __restrict__ mass,
    int H, int N, int NB, float scale_log2) {
  constexpr int KS = 32, kWaves = B / 32, kThreads = kWaves * kWave;
  constexpr int kTile = KS * D, kCprK = D / 8, kKSD = D / 16, kSub = B / KS;
  constexpr int kLoads = kTile * 2 / 16 / kThreads;
  static_assert(kLoads >= 1 && kTile * 2 % (16 * kThreads) == 0, "tile not divisible");
  __shared__ __attribute__((aligned(1024))) uint16_t slot0[kTile];
  __shared__ __attribute__((aligned(1024))) uint16_t slot1[kTile];
  __shared__ float red[2][kWaves];

  // head-synchronous schedule, as in the attention kernel
  const int per_xcd = (NB + 7) / 8;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int h = slot / per_xcd, I = xcd * per_xcd + slot % per_xcd;
  if (h >= H || I >= NB) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, col = lane & 31;
  const size_t head_off = static_cast<size_t>(h) * N * D;
  const int qrow = I * B + wave * 32 + col;
  const bool qvalid = qrow < N;
  const int bI = min(B, N - I * B);

  bf16x8 qf[kKSD];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(q + head_off + static_cast<size_t>(qvalid ? qrow : 0) * D);
#pragma unroll
    for (int s = 0; s < kKSD; ++s) {
      u32x4 raw = qvalid ? src[2 * s + hl] : u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  uint32_t koff[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int pc = (wave * kLoads + i) * 64 + lane;
    const int kr = pc / kCprK;
    koff[i] = static_cast<uint32_t>(kr * D + ((pc % kCprK) ^ swz<kCprK>(kr)) * 8) * 2u;
  }
  const uint16_t* kh = k + head_off;
  auto issue = [&](int u, uint16_t* dst) {
    const int kbase = u * KS;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kh + static_cast<size_t>(kbase) * D), 0, max(N - kbase, 0) * D * 2, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lvoid*)(dst + (wave * kLoads + i) * 512), 16,
                                               static_cast<int>(koff[i]), 0, 0, 0);
  };
  // S^T of sub-tile u (keys past the last token: -inf)
  auto scores = [&](int u, const uint16_t* cur) {
    const char* kt = reinterpret_cast<const char*>(cur);
    f32x16 s{};
#pragma unroll
    for (int st = 0; st < kKSD; ++st) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + col * (2 * D) + (((2 * st + hl) ^ swz<kCprK>(col)) * 16));
      s = mfma32(a, qf[st], s);
    }
    const int valid = N - u * KS;
    if (valid < KS) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (acc_row(r, hl) >= valid) s[r] = -INFINITY;
    }
    return s;
  };
  const int T = (N + KS - 1) / KS;  // key sub-tiles
  // Walk all sub-tiles: two slots, sub-tile u+1 loads while u is used.
  auto walk = [&](auto&& body) {
    barrier_lds();  // nobody still reads a slot of the previous walk
    issue(0, slot0);
    for (int u = 0; u < T; u += 2) {
      wait_vm<0>();
      barrier_lds();
      if (u + 1 < T) issue(u + 1, slot1);
      body(u, slot0);
      if (u + 1 < T) {
        wait_vm<0>();
        barrier_lds();
        if (u + 2 < T) issue(u + 2, slot0);
        body(u + 1, slot1);
      }
    }
  };

  // pass 1: running maximum (shared by the two halves) and fp64 normaliser
  float m_run = -INFINITY;
  double l_run = 0.0;
  walk([&](int u, const uint16_t* cur) {
    const f32x16 s = scores(u, cur);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    const float m_new = fmaxf(m_run, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2);
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) part[r & 3] += __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -m_new));
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run = l_run * static_cast<double>(alpha) + static_cast<double>((part[0] + part[1]) + (part[2] + part[3]));
    m_run = m_new;
  });
  const double l_tot = l_run + __shfl_xor(l_run, 32);
  const float lse2 = static_cast<float>(static_cast<double>(m_run) + log2(l_tot));

  // pass 2: normalised probabilities summed per key block
  float* row = mass + (static_cast<size_t>(h) * NB + I) * NB;
  auto finish = [&](int J) {  // all waves' totals of block J are in red[J & 1]
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += red[J & 1][w];
    row[J] = t / static_cast<float>(bI);
  };
  float acc = 0.f;
  walk([&](int u, const uint16_t* cur) {
    // block u/kSub - 1 was completed before this step's barrier
    if (tid == 0 && u > 0 && u % kSub == 0) finish(u / kSub - 1);
    const f32x16 s = scores(u, cur);
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) part[r & 3] += __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -lse2));
    acc += (part[0] + part[1]) + (part[2] + part[3]);
    if ((u + 1) % kSub == 0 || u == T - 1) {
      const float t = wave_sum(qvalid ? acc : 0.f);
      if (lane == 0) red[(u / kSub) & 1][wave] = t;
      acc = 0.f;
    }
  });
  __syncthreads();
  if (tid == 0) finish(NB - 1);
}

// Dense block mass, fp32 inputs: one thread per query row, keys read from
// global memory, fp64 normaliser; per key block the workgroup adds its
// threads' sums in a fixed tree.
template <int D, int B>
__global__ __launch_bounds__(B) void dense_mass_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, float* __restrict__ mass,
    int N, int NB, float scale_log2) {
  __shared__ double part[B];
  const int h = blockIdx.y, I = blockIdx.x, tid = threadIdx.x;
  const int qrow = I * B + tid;
  const bool qvalid = qrow < N;
  const int bI = min(B, N - I * B);
  const size_t head_off = static_cast<size_t>(h) * N * D;
  float qv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) qv[d] = qvalid ? q[head_off + static_cast<size_t>(qrow) * D + d] : 0.f;
  auto logit = [&](int t) {
    const float* kr = k + head_off + static_cast<size_t>(t) * D;
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) acc = fmaf(qv[d], kr[d], acc);
    return acc * scale_log2;
  };
  float m = -INFINITY;
  for (int t = 0; t < N; ++t) m = fmaxf(m, logit(t));
  double l = 0.0;
  for (int t = 0; t < N; ++t) l += static_cast<double>(exp2f(logit(t) - m));
  const double lse2 = static_cast<double>(m) + log2(l);
  for (int J = 0; J < NB; ++J) {
    double acc = 0.0;
    const int hi = min(N, (J + 1) * B);
    for (int t = J * B; t < hi; ++t) acc += exp2(static_cast<double>(logit(t)) - lse2);
    part[tid] = qvalid ? acc : 0.0;
    __syncthreads();
    for (int w = B / 2; w >= 1; w >>= 1) {
      if (tid < w) part[tid] += part[tid + w];
      __syncthreads();
    }
    if (tid == 0) mass[(static_cast<size_t>(h) * NB + I) * NB + J] = static_cast<float>(part[0] / bI);
    __syncthreads();
  }
}

// Query-pooled scores: one workgroup per (query block, head).  qbar: block
// means of q; kbar: block means of k times scale*log2 e (both fp32); logits
// and softmax in fp64, fixed reduction order.
template <int D>
__global__ __launch_bounds__(256) void pooled_score_kernel(const float* __restrict__ qbar,
                                                           const float* __restrict__ kbar,
                                                           float* __restrict__ scores, int NB) {
  extern __shared__ double lg[];  // NB logits
  __shared__ double qs[D];
  __shared__ double red[4];
  const int I = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if (tid < D) qs[tid] = qbar[(static_cast<size_t>(h) * NB + I) * D + tid];
  __syncthreads();
  double mx = -INFINITY;
  for (int J = tid; J < NB; J += 256) {
    const float* kr = kbar + (static_cast<size_t>(h) * NB + J) * D;
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += qs[d] * static_cast<double>(kr[d]);
    lg[J] = acc;
    mx = fmax(mx, acc);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  __syncthreads();
  double z = 0.0;
  for (int J = tid; J < NB; J += 256) z += exp2(lg[J] - mx);
  z = wave_sum_f64(z);
  if (lane == 0) red[wave] = z;
  __syncthreads();
  z = (red[0] + red[1]) + (red[2] + red[3]);
  float* row = scores + (static_cast<size_t>(h) * NB + I) * NB;
  for (int J = tid; J < NB; J += 256) row[J] = static_cast<float>(exp2(lg[J] - mx) / z);
}

template <int D, int B>
hipError_t launch_dense_mass_t(const Problem& p, const void* q, const void* k, float* mass,
                               hipStream_t stream) {
  const float sl2 = p.scale * kLog2e;
  if (p.dtype == 0) {
    const int grid = 8 * ((p.nb + 7) / 8) * p.heads;
    hipLaunchKernelGGL((dense_mass_bf16_kernel<D, B>), dim3(grid), dim3(2 * B), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), mass,
                       p.heads, p.tokens, p.nb, sl2);
  } else {
    hipLaunchKernelGGL((dense_mass_f32_kernel<D, B>), dim3(p.nb, p.heads), dim3(B), 0, stream,
                       static_cast<const float*>(q), static_cast<const float*>(k), mass, p.tokens,
                       p.nb, sl2);
  }
  return hipGetLastError();
}

struct PooledWs {
  float *qbar, *kbar, *bmax;
  size_t total;
};

PooledWs pooled_ws_layout(const Problem& p, void* base) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t means = al(sizeof(float) * p.heads * static_cast<size_t>(p.nb) * p.head_dim);
  const size_t bm = al(sizeof(float) * p.heads * static_cast<size_t>(p.nb));
  char* b = static_cast<char*>(base);
  PooledWs w;
  w.qbar = reinterpret_cast<float*>(b);
  w.kbar = reinterpret_cast<float*>(b + means);
  w.bmax = reinterpret_cast<float*>(b + 2 * means);
  w.total = 2 * means + bm;
  return w;
}

}  // namespace

hipError_t launch_dense_mass(const Problem& p, const void* q, const void* k, float* mass,
                             hipStream_t stream) {
  if (p.head_dim == 128 && p.block == 128) return launch_dense_mass_t<128, 128>(p, q, k, mass, stream);
  if (p.head_dim == 128 && p.block == 64) return launch_dense_mass_t<128, 64>(p, q, k, mass, stream);
  if (p.head_dim == 64 && p.block == 128) return launch_dense_mass_t<64, 128>(p, q, k, mass, stream);
  return launch_dense_mass_t<64, 64>(p, q, k, mass, stream);
}

size_t pooled_ws_bytes(const Problem& p) { return pooled_ws_layout(p, nullptr).total; }

hipError_t launch_pooled_scores(const Problem& p, const void* q, const void* k, float* scores,
                                void* ws, hipStream_t stream) {
  const PooledWs w = pooled_ws_layout(p, ws);
  hipError_t e = launch_block_means(p, q, 1.0, w.qbar, w.bmax, stream);
  if (e != hipSuccess) return e;
  e = launch_block_means(p, k, static_cast<double>(p.scale) * 1.4426950408889634, w.kbar, w.bmax, stream);
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(double) * p.nb;
  if (p.head_dim == 128)
    hipLaunchKernelGGL((pooled_score_kernel<128>), dim3(p.nb, p.heads), dim3(256), lds, stream, w.qbar,
                       w.kbar, scores, p.nb);
  else
    hipLaunchKernelGGL((pooled_score_kernel<64>), dim3(p.nb, p.heads), dim3(256), lds, stream, w.qbar,
                       w.kbar, scores, p.nb);
  return hipGetLastError();
}

}  // namespace rsa
