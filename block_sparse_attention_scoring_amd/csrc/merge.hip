// Joining two attentions over disjoint key sets (RECAP: Reciprocal Sparse
// Attention and Hierarchical Caching for Efficient Video Diffusion, Abstract:
// a cached refinement over the interactions sparse attention omits corrects
// each fresh sparse output, weighted by the fresh sparse statistics).
//
// Each part is a softmax normalised over its own keys, and exp(lse) is its
// total of exponentiated logits, so the softmax over the union gives part a
// the weight exp(lse_a) / (exp(lse_a) + exp(lse_b)).  A streaming kernel:
// every byte is touched once, so it is bound by HBM bandwidth.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace rsa {
namespace {

__device__ __forceinline__ float to_f32(__bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T>
__device__ __forceinline__ T from_f32(float x) { return static_cast<T>(x); }  // bf16: round to nearest even

// In place on (out, lse): kCpr lanes share a row, 16 bytes each; a 256-thread
// workgroup covers 256 / kCpr rows.  The lanes of a row lie in one wave, so
// every lane has read lse[r] before lane 0 of the row overwrites it.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(T* __restrict__ out, float* __restrict__ lse,
                                                    const T* __restrict__ part,
                                                    const float* __restrict__ part_lse,
                                                    long long rows) {
  constexpr int kEl = 16 / static_cast<int>(sizeof(T));
  constexpr int kCpr = D / kEl;
  static_assert(kCpr <= kWave && kWave % kCpr == 0, "a row must sit inside one wave");
  constexpr int kRows = 256 / kCpr;
  const long long r = static_cast<long long>(blockIdx.x) * kRows + threadIdx.x / kCpr;
  const int c = threadIdx.x % kCpr;
  if (r >= rows) return;
  const float la = lse[r], lb = part_lse[r];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, l = -INFINITY;
  if (m > -INFINITY) {
    const float ea = expf(la - m), eb = expf(lb - m);  // the larger of the two is 1
    const float z = ea + eb;
    wa = ea / z;
    wb = eb / z;
    l = m + logf(z);
  }
  typedef T vec __attribute__((ext_vector_type(kEl)));
  vec* po = reinterpret_cast<vec*>(out + r * D) + c;
  const vec a = *po;
  const vec b = reinterpret_cast<const vec*>(part + r * D)[c];
  vec o;
#pragma unroll
  for (int e = 0; e < kEl; ++e) o[e] = from_f32<T>(wa * to_f32(a[e]) + wb * to_f32(b[e]));
  *po = o;
  if (c == 0) lse[r] = l;
}

template <typename T, int D>
hipError_t launch_t(const Problem& p, void* out, float* lse, const void* part, const float* part_lse,
                    hipStream_t stream) {
  constexpr int kRows = 256 / (D * static_cast<int>(sizeof(T)) / 16);
  const long long rows = static_cast<long long>(p.heads) * p.tokens;
  const long long grid = (rows + kRows - 1) / kRows;
  hipLaunchKernelGGL((merge_kernel<T, D>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                     static_cast<T*>(out), lse, static_cast<const T*>(part), part_lse, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const Problem& p, void* out, float* lse, const void* part,
                        const float* part_lse, hipStream_t stream) {
  if (p.dtype == 0)
    return p.head_dim == 128 ? launch_t<__bf16, 128>(p, out, lse, part, part_lse, stream)
                             : launch_t<__bf16, 64>(p, out, lse, part, part_lse, stream);
  return p.head_dim == 128 ? launch_t<float, 128>(p, out, lse, part, part_lse, stream)
                           : launch_t<float, 64>(p, out, lse, part, part_lse, stream);
}

}  // namespace rsa
