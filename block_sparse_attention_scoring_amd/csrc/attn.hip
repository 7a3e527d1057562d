// Block-sparse attention over a compacted key-block list (gfx950).
//
// PARK (Accurate Block Retrieval for Sparse Attention in Video Diffusion
// Transformers), Abstract: attention is computed only inside the retrieved
// key blocks.  Query i of block I sees the tokens of the key blocks listed
// for (h, I); the softmax is normalised over exactly those tokens.
//
// bf16 kernel, one workgroup per (head, query block), one wave per 32 query
// rows.  Everything is computed transposed so that a lane owns one query:
//   S^T = K Q^T   (32x32x16 bf16 MFMA, A = K from LDS, B = Q held in VGPRs)
//   O^T = V^T P^T (A = V^T from LDS, B = P straight from the S^T registers)
// The row statistics of the online softmax are then per-lane values (two
// lanes share a query and exchange once per key block).  The S^T result
// layout puts keys {4h..4h+3, 8+4h..8+4h+3} of every 16 in lane half h, so
// V^T is written to LDS with the middle two groups of four keys of every 16
// swapped; P then feeds the second product without any lane exchange.
// The online softmax runs in fp32 in the log2 domain, and rescales the
// output only when the running maximum grows by more than 2^8 (exact: the
// final normalisation uses the same reference maximum).
#include "common.h"
#include "kernels.h"

namespace rsa {
namespace {

template <int D, int B>
struct AttnShape {
  static constexpr int kWaves = B / 32;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kKT = B / 32;    // 32-key tiles of a key block
  static constexpr int kDT = D / 32;    // 32-wide head_dim tiles
  static constexpr int kKSD = D / 16;   // MFMA k-steps over head_dim
  static constexpr int kKSB = B / 16;   // MFMA k-steps over keys
  static constexpr int kKStride = D + 8;  // LDS row pitch of K (bf16), 16 B pad
  static constexpr int kVStride = B + 8;  // LDS row pitch of V^T (bf16)
  static constexpr int kKChunks = B * D / 8 / kThreads;        // 16-byte K loads per thread
  static constexpr int kVGroups = (B / 4) * (D / 8) / kThreads;  // 4-key x 8-d V groups per thread
};

__device__ __forceinline__ int vt_pos(int key) {
  // position of `key` inside its 16-key group of V^T: swap groups 1 and 2
  const int g4 = (key >> 2) & 3;
  const int sw = ((g4 & 1) << 1) | (g4 >> 1);
  return (key & ~15) | (sw << 2) | (key & 3);
}

template <int D, int B>
__global__ __launch_bounds__(2 * B, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int* __restrict__ counts,
    const int* __restrict__ block_idx, uint16_t* __restrict__ out,
    float* __restrict__ lse, int N, int NB, float scale_log2) {
  using S = AttnShape<D, B>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[B * S::kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * S::kVStride];

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int h = tile / NB, I = tile - h * NB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const size_t head_off = static_cast<size_t>(h) * N * D;
  const int qrow = I * B + wave * 32 + col;

  bf16x8 qf[S::kKSD];
  {
    const bool ok = qrow < N;
    const u32x4* src = reinterpret_cast<const u32x4*>(q + head_off + static_cast<size_t>(ok ? qrow : 0) * D);
#pragma unroll
    for (int s = 0; s < S::kKSD; ++s) {
      u32x4 raw = ok ? src[2 * s + hl] : u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 oacc[S::kDT];
#pragma unroll
  for (int t = 0; t < S::kDT; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY;  // reference maximum, log2 units
  float l_run = 0.f;        // this lane's share of the row sum

  const int cnt = counts[h * NB + I];
  const int* list = block_idx + (static_cast<size_t>(h) * NB + I) * NB;
  const uint16_t* kh = k + head_off;
  const uint16_t* vh = v + head_off;

  for (int it = 0; it < cnt; ++it) {
    const int J = list[it];
    const int kbase = J * B;
    const int bJ = min(B, N - kbase);

    u32x4 kr[S::kKChunks];
#pragma unroll
    for (int i = 0; i < S::kKChunks; ++i) {
      const int c = tid + i * S::kThreads;
      const int row = c / (D / 8), c8 = c % (D / 8);
      kr[i] = row < bJ ? *reinterpret_cast<const u32x4*>(kh + static_cast<size_t>(kbase + row) * D + c8 * 8)
                       : u32x4{0, 0, 0, 0};
    }
    u32x4 vr[S::kVGroups][4];
#pragma unroll
    for (int i = 0; i < S::kVGroups; ++i) {
      const int gi = tid + i * S::kThreads;
      const int c8 = gi % (D / 8), g = gi / (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;
        vr[i][r] = row < bJ ? *reinterpret_cast<const u32x4*>(vh + static_cast<size_t>(kbase + row) * D + c8 * 8)
                            : u32x4{0, 0, 0, 0};
      }
    }
    __syncthreads();  // previous block's LDS reads are done
#pragma unroll
    for (int i = 0; i < S::kKChunks; ++i) {
      const int c = tid + i * S::kThreads;
      const int row = c / (D / 8), c8 = c % (D / 8);
      *reinterpret_cast<u32x4*>(&Ks[row * S::kKStride + c8 * 8]) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < S::kVGroups; ++i) {
      const int gi = tid + i * S::kThreads;
      const int c8 = gi % (D / 8), g = gi / (D / 8);
      const int pos = vt_pos(4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a0 = vr[i][0][e], a1 = vr[i][1][e], a2 = vr[i][2][e], a3 = vr[i][3][e];
        u32x2 lo, hi;
        lo[0] = (a0 & 0xffffu) | (a1 << 16);
        lo[1] = (a2 & 0xffffu) | (a3 << 16);
        hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
        hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        const int d = c8 * 8 + 2 * e;
        *reinterpret_cast<u32x2*>(&Vt[d * S::kVStride + pos]) = lo;
        *reinterpret_cast<u32x2*>(&Vt[(d + 1) * S::kVStride + pos]) = hi;
      }
    }
    __syncthreads();

    f32x16 sacc[S::kKT];
#pragma unroll
    for (int t = 0; t < S::kKT; ++t) {
      sacc[t] = f32x16{};
#pragma unroll
      for (int s = 0; s < S::kKSD; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(32 * t + col) * S::kKStride + 16 * s + 8 * hl]);
        sacc[t] = mfma32(a, qf[s], sacc[t]);
      }
    }
    if (bJ < B) {
#pragma unroll
      for (int t = 0; t < S::kKT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * t + acc_row(r, hl) >= bJ) sacc[t][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < S::kKT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_blk = mx * scale_log2;
    const bool need = m_blk > m_run + 8.f;
    if (__any(need)) {
      const float m_new = need ? m_blk : m_run;
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < S::kDT; ++t) oacc[t] *= alpha;
      m_run = m_new;
    }
    bf16x8 pb[S::kKSB];
#pragma unroll
    for (int t = 0; t < S::kKT; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[t][r], scale_log2, -m_run));
        l_run += p;
        pb[2 * t + (r >> 3)][r & 7] = static_cast<__bf16>(p);
      }
    }
#pragma unroll
    for (int dt = 0; dt < S::kDT; ++dt) {
#pragma unroll
      for (int u = 0; u < S::kKSB; ++u) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Vt[(32 * dt + col) * S::kVStride + 16 * u + 8 * hl]);
        oacc[dt] = mfma32(a, pb[u], oacc[dt]);
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* dst = out + head_off + static_cast<size_t>(qrow) * D;
#pragma unroll
    for (int dt = 0; dt < S::kDT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = static_cast<__bf16>(oacc[dt][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(dst + 32 * dt + 8 * g + 4 * hl) = o;
      }
    }
    if (lse != nullptr && hl == 0)
      lse[static_cast<size_t>(h) * N + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// fp32 inputs: plain fp32 arithmetic, one thread per query row, K and V
// staged in LDS 32 keys at a time and read as broadcasts.  Same online
// softmax (exact rescaling at every chunk).
template <int D, int B>
__global__ __launch_bounds__(B) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int* __restrict__ counts, const int* __restrict__ block_idx,
    float* __restrict__ out, float* __restrict__ lse, int N, int NB, float scale_log2) {
  constexpr int kChunk = 32;
  __shared__ float Ks[kChunk * D];
  __shared__ float Vs[kChunk * D];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int h = tile / NB, I = tile - h * NB;
  const int tid = threadIdx.x;
  const int qrow = I * B + tid;
  const size_t head_off = static_cast<size_t>(h) * N * D;
  float qv[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = qrow < N ? q[head_off + static_cast<size_t>(qrow) * D + d] * scale_log2 : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int cnt = counts[h * NB + I];
  const int* list = block_idx + (static_cast<size_t>(h) * NB + I) * NB;
  for (int it = 0; it < cnt; ++it) {
    const int kbase = list[it] * B;
    const int bJ = min(B, N - kbase);
    for (int kc = 0; kc < bJ; kc += kChunk) {
      const int nk = min(kChunk, bJ - kc);
      __syncthreads();
      for (int e = tid; e < kChunk * D; e += B) {
        const int row = e / D;
        const size_t g = head_off + static_cast<size_t>(kbase + kc) * D + e;
        Ks[e] = row < nk ? k[g] : 0.f;
        Vs[e] = row < nk ? v[g] : 0.f;
      }
      __syncthreads();
      for (int j0 = 0; j0 < nk; j0 += 8) {
        float s[8];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float acc = 0.f;
#pragma unroll 16
          for (int d = 0; d < D; ++d) acc = fmaf(qv[d], Ks[(j0 + j) * D + d], acc);
          s[j] = j0 + j < nk ? acc : -INFINITY;
          mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m, mx);
        const float alpha = exp2f(m - m_new);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = exp2f(s[j] - m_new);
          l += p;
#pragma unroll 16
          for (int d = 0; d < D; ++d) o[d] = fmaf(p, Vs[(j0 + j) * D + d], o[d]);
        }
        m = m_new;
      }
    }
  }
  if (qrow < N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) out[head_off + static_cast<size_t>(qrow) * D + d] = o[d] * inv;
    if (lse != nullptr) lse[static_cast<size_t>(h) * N + qrow] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, int B>
hipError_t launch_attn_t(const Problem& p, const void* q, const void* k, const void* v,
                         const int* counts, const int* idx, void* out, float* lse,
                         hipStream_t stream) {
  const int grid = p.heads * p.nb;
  const float sl2 = p.scale * kLog2e;
  if (p.dtype == 0) {
    using S = AttnShape<D, B>;
    hipLaunchKernelGGL((attn_bf16_kernel<D, B>), dim3(grid), dim3(S::kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), counts, idx, static_cast<uint16_t*>(out),
                       lse, p.tokens, p.nb, sl2);
  } else {
    hipLaunchKernelGGL((attn_f32_kernel<D, B>), dim3(grid), dim3(B), 0, stream,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), counts, idx, static_cast<float*>(out),
                       lse, p.tokens, p.nb, sl2);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const Problem& p, const void* q, const void* k, const void* v,
                            const int* counts, const int* idx, void* out, float* lse,
                            hipStream_t stream) {
  if (p.head_dim == 128 && p.block == 128) return launch_attn_t<128, 128>(p, q, k, v, counts, idx, out, lse, stream);
  if (p.head_dim == 128 && p.block == 64) return launch_attn_t<128, 64>(p, q, k, v, counts, idx, out, lse, stream);
  if (p.head_dim == 64 && p.block == 128) return launch_attn_t<64, 128>(p, q, k, v, counts, idx, out, lse, stream);
  return launch_attn_t<64, 64>(p, q, k, v, counts, idx, out, lse, stream);
}

}  // namespace rsa
