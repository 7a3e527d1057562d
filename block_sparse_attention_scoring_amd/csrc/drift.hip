// Per-head query-key drift and refresh flags (gfx950).
//
// HEART (Exploiting Head Heterogeneity in Sparse Attention for Video
// Diffusion), Abstract (Temporal Mask Reuse): a head keeps its cached mask
// until a cheap measure of how far its queries and keys have moved rises above
// a threshold tau, and only then is the mask recomputed; HASTE, Abstract, uses
// the same kind of measure to decide when mask prediction can be skipped.  The signal is the relative Frobenius change
// of the head's stacked (Q, K) since its last refresh:
//
//   d_h = sqrt(|Q - Qref|^2 + |K - Kref|^2) / sqrt(|Qref|^2 + |Kref|^2).
//
// Three launches, all bandwidth-bound streams over the four tensors:
//   partial: kDriftGroups workgroups per head each reduce a contiguous slice
//            (fp32 within one 16-byte vector, fp64 across vectors, fixed
//            wave and workgroup trees);
//   final:   one wave per head adds its partials in index order, decides
//            d_h > threshold in fp64 and writes drift (fp32) and the flag;
//   copy:    (optional) refreshed heads overwrite their snapshot with Q, K.
#include "common.h"
#include "kernels.h"

namespace rsa {
namespace {

constexpr int kDriftThreads = 256;

// 16-byte vector of T, as floats.  Non-temporal loads: each byte is read
// once, and the streams pass the caches by (7 % faster on the 720p shape).
template <typename T>
struct Vec16;

template <>
struct Vec16<uint16_t> {
  static constexpr int kN = 8;
  __device__ static void load(const uint16_t* p, float (&x)[8]) {
    const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(r[e] << 16);
      x[2 * e + 1] = __uint_as_float(r[e] & 0xffff0000u);
    }
  }
};

template <>
struct Vec16<float> {
  static constexpr int kN = 4;
  __device__ static void load(const float* p, float (&x)[4]) {
    const f32x4 r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = r[e];
  }
};

template <typename T>
__global__ __launch_bounds__(kDriftThreads) void drift_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ qr,
    const T* __restrict__ kr, double* __restrict__ partial, size_t per_head) {
  constexpr int kN = Vec16<T>::kN;
  __shared__ double red[2][kDriftThreads / kWave];
  const int h = blockIdx.y, g = blockIdx.x;
  const size_t nvec = per_head / kN;
  const size_t per_group = (nvec + kDriftGroups - 1) / kDriftGroups;
  const size_t v0 = g * per_group, v1 = min(nvec, v0 + per_group);
  const size_t base = static_cast<size_t>(h) * per_head;
  double num = 0.0, den = 0.0;
  for (size_t vi = v0 + threadIdx.x; vi < v1; vi += kDriftThreads) {
    const size_t o = base + vi * kN;
    float a[kN], b[kN], c[kN], d[kN];
    Vec16<T>::load(q + o, a);
    Vec16<T>::load(qr + o, b);
    Vec16<T>::load(k + o, c);
    Vec16<T>::load(kr + o, d);
    float n = 0.f, r = 0.f;
#pragma unroll
    for (int e = 0; e < kN; ++e) {
      const float dq = a[e] - b[e], dk = c[e] - d[e];
      n = fmaf(dq, dq, fmaf(dk, dk, n));
      r = fmaf(b[e], b[e], fmaf(d[e], d[e], r));
    }
    num += static_cast<double>(n);
    den += static_cast<double>(r);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    num += __shfl_xor(num, o);
    den += __shfl_xor(den, o);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = num;
    red[1][threadIdx.x >> 6] = den;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double n = 0.0, r = 0.0;
    for (int w = 0; w < kDriftThreads / kWave; ++w) {
      n += red[0][w];
      r += red[1][w];
    }
    partial[(static_cast<size_t>(h) * kDriftGroups + g) * 2] = n;
    partial[(static_cast<size_t>(h) * kDriftGroups + g) * 2 + 1] = r;
  }
}

__global__ __launch_bounds__(kWave) void drift_final_kernel(const double* __restrict__ partial,
                                                           float threshold, float* __restrict__ drift,
                                                           uint8_t* __restrict__ refresh) {
  const int h = blockIdx.x, lane = threadIdx.x;
  double n = 0.0, r = 0.0;
  if (lane < kDriftGroups) {
    n = partial[(static_cast<size_t>(h) * kDriftGroups + lane) * 2];
    r = partial[(static_cast<size_t>(h) * kDriftGroups + lane) * 2 + 1];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    n += __shfl_xor(n, o);
    r += __shfl_xor(r, o);
  }
  if (lane == 0) {
    double d;
    if (r > 0.0)
      d = sqrt(n) / sqrt(r);
    else
      d = n == 0.0 ? 0.0 : static_cast<double>(INFINITY);
    drift[h] = static_cast<float>(d);
    refresh[h] = d > static_cast<double>(threshold) ? 1 : 0;
  }
}

template <typename T>
__global__ __launch_bounds__(kDriftThreads) void drift_copy_kernel(
    const T* __restrict__ q, const T* __restrict__ k, T* __restrict__ qr, T* __restrict__ kr,
    const uint8_t* __restrict__ refresh, size_t per_head) {
  const int h = blockIdx.y;
  if (refresh[h] == 0) return;
  const size_t nvec = per_head * sizeof(T) / 16;
  const size_t base = static_cast<size_t>(h) * per_head * sizeof(T) / 16;
  const u32x4* qs = reinterpret_cast<const u32x4*>(q) + base;
  const u32x4* ks = reinterpret_cast<const u32x4*>(k) + base;
  u32x4* qd = reinterpret_cast<u32x4*>(qr) + base;
  u32x4* kd = reinterpret_cast<u32x4*>(kr) + base;
  for (size_t i = blockIdx.x * static_cast<size_t>(kDriftThreads) + threadIdx.x; i < nvec;
       i += static_cast<size_t>(gridDim.x) * kDriftThreads) {
    qd[i] = qs[i];
    kd[i] = ks[i];
  }
}

template <typename T>
hipError_t launch_drift_t(const Problem& p, const void* q, const void* k, void* q_ref,
                          void* k_ref, float threshold, int update_ref, float* drift,
                          uint8_t* refresh, void* ws, hipStream_t stream) {
  const size_t per_head = static_cast<size_t>(p.tokens) * p.head_dim;
  double* partial = static_cast<double*>(ws);
  hipLaunchKernelGGL((drift_partial_kernel<T>), dim3(kDriftGroups, p.heads), dim3(kDriftThreads), 0,
                     stream, static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<const T*>(q_ref), static_cast<const T*>(k_ref), partial, per_head);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(drift_final_kernel, dim3(p.heads), dim3(kWave), 0, stream, partial, threshold,
                     drift, refresh);
  e = hipGetLastError();
  if (e != hipSuccess || !update_ref) return e;
  hipLaunchKernelGGL((drift_copy_kernel<T>), dim3(kDriftGroups, p.heads), dim3(kDriftThreads), 0,
                     stream, static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<T*>(q_ref), static_cast<T*>(k_ref), refresh, per_head);
  return hipGetLastError();
}

}  // namespace

size_t drift_ws_bytes(const Problem& p) {
  return sizeof(double) * 2 * kDriftGroups * static_cast<size_t>(p.heads);
}

hipError_t launch_drift(const Problem& p, const void* q, const void* k, void* q_ref, void* k_ref,
                        float threshold, int update_ref, float* drift, uint8_t* refresh, void* ws,
                        hipStream_t stream) {
  if (p.dtype == 0)
    return launch_drift_t<uint16_t>(p, q, k, q_ref, k_ref, threshold, update_ref, drift, refresh, ws, stream);
  return launch_drift_t<float>(p, q, k, q_ref, k_ref, threshold, update_ref, drift, refresh, ws, stream);
}

}  // namespace rsa
