// Top-p block selection (gfx950).
//
// HASTE (Training-Free Video Diffusion Acceleration via Head-Wise Adaptive
// Sparse Attention), Abstract: the mask comes from online top-p selection,
// with a threshold per head (also HEART: Exploiting Head Heterogeneity in
// Sparse Attention for Video Diffusion, Abstract).
//
// One workgroup per (head, query block) row.  The row's scores are packed
// into 64-bit keys (inverted order-preserving score bits, key-block index),
// so one ascending bitonic sort in LDS orders the blocks by score descending
// and, for equal scores, by index ascending.  The sorted scores are summed in
// fp64 with a block-wide scan; the first rank whose running mass reaches
// p[h] fixes k*; the kept blocks are flagged and compacted in ascending
// index order with an integer scan.  Nothing here depends on thread timing.
#include "common.h"
#include "kernels.h"

namespace rsa {
namespace {

constexpr int kSelThreads = 256;

__device__ __forceinline__ uint32_t order_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending in f
}

template <typename V>
__device__ V block_exclusive_scan(V x, V* wave_tot, V& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  V incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const V y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  V before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / kWave; ++w) {
    if (w < wave) before += wave_tot[w];
    all += wave_tot[w];
  }
  __syncthreads();
  total = all;
  return before + incl - x;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ scores, const float* __restrict__ top_p, int max_blocks,
    const uint8_t* __restrict__ head_active, uint8_t* __restrict__ mask,
    int32_t* __restrict__ counts, int32_t* __restrict__ idx, int NB, int MP) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);           // [MP]
  float* sval = reinterpret_cast<float*>(keys + MP);             // [MP]
  uint8_t* flag = reinterpret_cast<uint8_t*>(sval + MP);         // [MP]
  __shared__ double dtot[kSelThreads / kWave];
  __shared__ int itot[kSelThreads / kWave];
  __shared__ int first_hit;

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int h = tile / NB, I = tile - h * NB;
  if (head_active != nullptr && head_active[h] == 0) return;
  const int tid = threadIdx.x;
  const float* srow = scores + (static_cast<size_t>(h) * NB + I) * NB;

  for (int j = tid; j < MP; j += kSelThreads) {
    if (j < NB) {
      const float s = srow[j];
      sval[j] = s;
      keys[j] = (static_cast<uint64_t>(~order_bits(s)) << 32) | static_cast<uint32_t>(j);
    } else {
      keys[j] = ~0ull;
    }
    flag[j] = 0;
  }
  if (tid == 0) first_hit = 0x7fffffff;
  __syncthreads();

  // ascending bitonic sort of MP keys
  for (int size = 2; size <= MP; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < MP / 2; t += kSelThreads) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const uint64_t a = keys[i], b = keys[j];
        if ((a > b) == up) {
          keys[i] = b;
          keys[j] = a;
        }
      }
      __syncthreads();
    }
  }

  // fp64 running mass over the sorted order: each thread owns E consecutive ranks
  const int E = MP / kSelThreads;
  const int r0 = tid * E;
  double local = 0.0;
  for (int e = 0; e < E; ++e) {
    const int r = r0 + e;
    if (r < NB) local += static_cast<double>(sval[static_cast<uint32_t>(keys[r])]);
  }
  double total;
  double run = block_exclusive_scan<double>(local, dtot, total);
  const double p = static_cast<double>(top_p[h]);
  int kstar;
  if (p >= 1.0) {
    kstar = NB;
  } else {
    for (int e = 0; e < E; ++e) {
      const int r = r0 + e;
      if (r >= NB) break;
      run += static_cast<double>(sval[static_cast<uint32_t>(keys[r])]);
      if (run >= p) {
        atomicMin(&first_hit, r);
        break;
      }
    }
    __syncthreads();
    kstar = first_hit == 0x7fffffff ? NB : first_hit + 1;
  }
  if (max_blocks > 0 && kstar > max_blocks) kstar = max_blocks;

  for (int r = tid; r < kstar; r += kSelThreads) flag[static_cast<uint32_t>(keys[r])] = 1;
  __syncthreads();

  uint8_t* mrow = mask + (static_cast<size_t>(h) * NB + I) * NB;
  for (int j = tid; j < NB; j += kSelThreads) mrow[j] = flag[j];

  // ascending compaction: thread owns E consecutive block indices
  int cnt = 0;
  for (int e = 0; e < E; ++e) cnt += (r0 + e < NB) ? flag[r0 + e] : 0;
  int all;
  int pos = block_exclusive_scan<int>(cnt, itot, all);
  int32_t* irow = idx + (static_cast<size_t>(h) * NB + I) * NB;
  for (int e = 0; e < E; ++e) {
    const int j = r0 + e;
    if (j < NB && flag[j]) irow[pos++] = j;
  }
  if (tid == 0) counts[static_cast<size_t>(h) * NB + I] = kstar;
}

// density[h] = sum_I counts[h, I] / NB^2, exact integer sum
__global__ __launch_bounds__(256) void density_kernel(const int32_t* __restrict__ counts,
                                                      float* __restrict__ density, int NB) {
  __shared__ long long part[4];
  const int h = blockIdx.x, tid = threadIdx.x;
  long long s = 0;
  for (int i = tid; i < NB; i += 256) s += counts[static_cast<size_t>(h) * NB + i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if ((tid & 63) == 0) part[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    const long long t = part[0] + part[1] + part[2] + part[3];
    density[h] = static_cast<float>(static_cast<double>(t) / (static_cast<double>(NB) * NB));
  }
}

}  // namespace

hipError_t launch_select(const Problem& p, const float* scores, const float* top_p,
                         int max_blocks, const uint8_t* head_active, uint8_t* mask,
                         int32_t* counts, int32_t* idx, float* density, hipStream_t stream) {
  int MP = kSelThreads;
  while (MP < p.nb) MP <<= 1;
  const size_t lds = static_cast<size_t>(MP) * (sizeof(uint64_t) + sizeof(float) + 1);
  hipLaunchKernelGGL(select_kernel, dim3(p.heads * p.nb), dim3(kSelThreads), lds, stream, scores,
                     top_p, max_blocks, head_active, mask, counts, idx, p.nb, MP);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || density == nullptr) return e;
  hipLaunchKernelGGL(density_kernel, dim3(p.heads), dim3(256), 0, stream, counts, density, p.nb);
  return hipGetLastError();
}

}  // namespace rsa
