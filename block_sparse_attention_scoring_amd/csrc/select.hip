// Top-p block selection (gfx950).
//
// HASTE (Training-Free Video Diffusion Acceleration via Head-Wise Adaptive
// Sparse Attention), Abstract: the mask comes from online top-p selection,
// with a threshold per head (also HEART: Exploiting Head Heterogeneity in
// Sparse Attention for Video Diffusion, Abstract).
//
// One wave per (head, query block) row, four rows per workgroup, no LDS and
// no barriers.  The row's scores become 64-bit keys (inverted
// order-preserving score bits, key-block index), so an ascending sort orders
// the blocks by score descending and, for equal scores, by index ascending.
// Each lane holds E consecutive keys of the padded row (MP = 64 E >= NB) in
// registers; the bitonic network runs its strides below E inside the lane
// and the others between lanes (shuffles).  The running mass is the fp64 sum
// of the sorted scores in rank order; it is formed in-lane plus a wave scan,
// and re-summed in rank order whenever a prefix lies within that scan's
// rounding bound of p[h], so the decision is the rank-order one.  The first
// rank whose running mass reaches p[h] fixes k*, and the key at rank k* - 1 is the threshold: block
// j is kept when its key is not above it, which the lanes test on the
// unsorted row (E consecutive indices each) to write the mask and, with a
// wave scan of the counts, the ascending list.  Nothing depends on timing.
#include "common.h"
#include "kernels.h"

// The sort network asks for full unrolling at every row width; for the
// widest rows the compiler may keep some loops (its size limit), which is
// correct, only slower, so that remark is not reported.
#pragma clang diagnostic ignored "-Wpass-failed"

namespace rsa {
namespace {

constexpr int kSelWaves = 4;  // rows per workgroup

__device__ __forceinline__ uint32_t order_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending in f
}
// inverse of ~order_bits: the score a key carries in its high word
__device__ __forceinline__ float key_score(uint64_t key) {
  const uint32_t o = ~static_cast<uint32_t>(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

template <typename V>
__device__ __forceinline__ V wave_exclusive_scan(V x, V& total) {
  const int lane = threadIdx.x & 63;
  V incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const V y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  total = __shfl(incl, 63);
  return incl - x;
}

template <int E>
__global__ __launch_bounds__(kSelWaves * kWave) void select_kernel(
    const float* __restrict__ scores, const float* __restrict__ top_p, int max_blocks,
    const uint8_t* __restrict__ head_active, uint8_t* __restrict__ mask,
    int32_t* __restrict__ counts, int32_t* __restrict__ idx, int H, int NB) {
  constexpr int MP = E * kWave;
  const int lane = threadIdx.x & 63;
  const int row_id = blockIdx.x * kSelWaves + static_cast<int>(threadIdx.x >> 6);
  if (row_id >= H * NB) return;  // whole waves leave together
  const int h = row_id / NB;
  if (head_active != nullptr && head_active[h] == 0) return;
  const size_t row = static_cast<size_t>(row_id);
  const float* srow = scores + row * NB;

  // key of block j with score s (block index in the low word)
  auto key_of = [](float s, int j) {
    return (static_cast<uint64_t>(~order_bits(s)) << 32) | static_cast<uint32_t>(j);
  };
  // the row: lane holds indices lane*E .. lane*E + E - 1; its scores stay in
  // registers for the mask and list at the end (padding past NB sorts last)
  uint64_t v[E];
  float sv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane * E + e;
    sv[e] = j < NB ? srow[j] : 0.f;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane * E + e;
    v[e] = j < NB ? key_of(sv[e], j) : ~0ull;
  }
  // ascending bitonic sort of the MP keys (counted loops, fully unrolled:
  // every size and stride is a compile-time constant)
  constexpr int kLogMP = __builtin_ctz(MP);
#pragma unroll
  for (int ls = 1; ls <= kLogMP; ++ls) {
    const int size = 1 << ls;
#pragma unroll
    for (int ts = 1; ts <= ls; ++ts) {
      const int stride = size >> ts;
      if (stride < E) continue;
      const int dl = stride / E;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint64_t a = v[e], b = __shfl_xor(a, dl);
        const int i = lane * E + e;
        const bool lower = (i & stride) == 0, up = (i & size) == 0;
        v[e] = (lower == up) ? (a < b ? a : b) : (a < b ? b : a);
      }
    }
#pragma unroll
    for (int st = E / 2; st >= 1; st >>= 1) {  // strides inside the lane (compile-time indices)
      if (st < size) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e & st) == 0) {
            const uint64_t a = v[e], b = v[e + st];
            const bool up = ((lane * E + e) & size) == 0;
            if ((a > b) == up) {
              v[e] = b;
              v[e + st] = a;
            }
          }
        }
      }
    }
  }

  // k*: first rank whose running mass reaches p (ranks lane*E .. +E-1).
  // The running mass is defined as the fp64 sum of the sorted fp32 scores
  // taken one after another in rank order.  The fast path sums in-lane and
  // scans across lanes, a different association; its prefixes differ from
  // the rank-order ones by at most (2E + 6 + NB) fp64 roundings of the mass
  // of absolute values, under 2^-40 of it for NB <= 4096.  When no prefix
  // lies within twice that of p the two orders take the same decision;
  // otherwise the row is summed again in rank order (one lane after another).
  const double p = static_cast<double>(top_p[h]);
  int kstar = NB;
  if (p < 1.0) {
    double local = 0.0, labs = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (lane * E + e < NB) {
        const double x = static_cast<double>(key_score(v[e]));
        local += x;
        labs += fabs(x);
      }
    double total, tabs;
    double run = wave_exclusive_scan<double>(local, total);
    wave_exclusive_scan<double>(labs, tabs);
    int hit = 0x7fffffff;
    double gap = INFINITY;  // distance of the nearest prefix to p
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int r = lane * E + e;
      if (r < NB) {
        run += static_cast<double>(key_score(v[e]));
        gap = fmin(gap, fabs(run - p));
        if (run >= p && hit == 0x7fffffff) hit = r;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      hit = min(hit, __shfl_xor(hit, o));
      gap = fmin(gap, __shfl_xor(gap, o));
    }
    if (gap <= ldexp(tabs, -39)) {
      // near the threshold: the rank-order sum, lane by lane (rare)
      double carry = 0.0;
      hit = 0x7fffffff;
      for (int L = 0; L < kWave && L * E < NB && hit == 0x7fffffff; ++L) {
        double acc = carry;
        int h2 = 0x7fffffff;
        if (lane == L) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const int r = L * E + e;
            if (r < NB) {
              acc += static_cast<double>(key_score(v[e]));
              if (acc >= p && h2 == 0x7fffffff) h2 = r;
            }
          }
        }
        carry = __shfl(acc, L);
        hit = __shfl(h2, L);
      }
    }
    if (hit != 0x7fffffff) kstar = hit + 1;
  }
  if (max_blocks > 0 && kstar > max_blocks) kstar = max_blocks;
  // the key of rank kstar - 1: every key not above it is kept
  const int rk = kstar - 1;
  uint64_t thr = 0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (e == rk % E) thr = v[e];
  thr = __shfl(thr, rk / E);

  // mask and ascending list from the unsorted row (keys rebuilt from the
  // scores held in registers; keys are unique, so exactly k* pass)
  uint8_t* mrow = mask + row * NB;
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane * E + e;
    if (j < NB) {
      const bool keep = key_of(sv[e], j) <= thr;
      mrow[j] = keep ? 1 : 0;
      cnt += keep;
    }
  }
  int all;
  int pos = wave_exclusive_scan<int>(cnt, all);
  int32_t* irow = idx + row * NB;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane * E + e;
    if (j < NB && key_of(sv[e], j) <= thr) irow[pos++] = j;
  }
  if (lane == 0) counts[row] = kstar;
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
  int MP = kWave;
  while (MP < p.nb) MP <<= 1;
  const int rows = p.heads * p.nb;
  const dim3 grid((rows + kSelWaves - 1) / kSelWaves);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kSelWaves * kWave), 0, stream, scores, top_p, max_blocks, head_active,
                       mask, counts, idx, p.heads, p.nb);
  };
  switch (MP / kWave) {
    case 1: go(select_kernel<1>); break;
    case 2: go(select_kernel<2>); break;
    case 4: go(select_kernel<4>); break;
    case 8: go(select_kernel<8>); break;
    case 16: go(select_kernel<16>); break;
    case 32: go(select_kernel<32>); break;
    default: go(select_kernel<64>); break;  // NB <= 4096
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || density == nullptr) return e;
  hipLaunchKernelGGL(density_kernel, dim3(p.heads), dim3(256), 0, stream, counts, density, p.nb);
  return hipGetLastError();
}

}  // namespace rsa
