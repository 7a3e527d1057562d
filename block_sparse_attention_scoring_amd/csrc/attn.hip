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

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// Position of `key` inside its 16-key group of V^T: the S^T result layout
// gives lane half h keys {4h..4h+3, 8+4h..8+4h+3}, so groups 1 and 2 of
// four keys are swapped.
__host__ __device__ __forceinline__ int vt_pos(int key) {
  const int g4 = (key >> 2) & 3;
  const int sw = ((g4 & 1) << 1) | (g4 >> 1);
  return (key & ~15) | (sw << 2) | (key & 3);
}

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

// Work of one workgroup: B/32 waves (32 query rows each) against key
// sub-tiles of KS keys; NBUF LDS buffers per operand.
template <int D, int B, int KS, int NBUF>
struct AttnShape {
  static constexpr int kWaves = B / 32;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kKT = KS / 32;   // 32-key tiles of a sub-tile
  static constexpr int kDT = D / 32;    // 32-wide head_dim tiles
  static constexpr int kKSD = D / 16;   // MFMA k-steps over head_dim
  static constexpr int kKSK = KS / 16;  // MFMA k-steps over the sub-tile's keys
  static constexpr int kTile = KS * D;  // elements of a K or V^T sub-tile
  static constexpr int kCprK = D / 8;   // 16-byte chunks per K row
  static constexpr int kCprV = KS / 8;  // 16-byte chunks per V^T row
  static constexpr int kLoads = kTile * 2 / 16 / kThreads;  // 16-byte loads per lane per operand
  static constexpr int kSub = B / KS;   // sub-tiles per key block
  static_assert(kLoads >= 1 && kTile * 2 % (16 * kThreads) == 0, "tile not divisible");
};

// V [H, N, D] -> V^T [H, D, NB*B] with vt_pos order inside every 16 keys and
// zeros past the last token: the operand layout of O^T = V^T P^T.
template <int D, int B>
__global__ __launch_bounds__(256) void vt_kernel(const uint16_t* __restrict__ v,
                                                 uint16_t* __restrict__ vt, int N, int NB) {
  __shared__ uint16_t tile[B][D + 2];
  const int J = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int kbase = J * B, bJ = min(B, N - kbase);
  const size_t np = static_cast<size_t>(NB) * B;
  for (int c = tid; c < B * D / 8; c += 256) {
    const int r = c / (D / 8), c8 = c % (D / 8);
    u32x4 x = r < bJ ? *reinterpret_cast<const u32x4*>(v + (static_cast<size_t>(h) * N + kbase + r) * D + c8 * 8)
                     : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[r][c8 * 8 + 2 * e] = static_cast<uint16_t>(x[e] & 0xffffu);
      tile[r][c8 * 8 + 2 * e + 1] = static_cast<uint16_t>(x[e] >> 16);
    }
  }
  __syncthreads();
  for (int c = tid; c < D * B / 8; c += 256) {
    const int d = c / (B / 8), p8 = c % (B / 8);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[vt_pos(8 * p8 + 2 * e)][d];
      const uint32_t hi = tile[vt_pos(8 * p8 + 2 * e + 1)][d];
      o[e] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(vt + (static_cast<size_t>(h) * D + d) * np + kbase + 8 * p8) = o;
  }
}

// One workgroup per (head, query block): B/32 waves, 32 query rows each,
// walking its key blocks in sub-tiles of KS keys.  K and V^T sub-tiles
// stream global -> LDS directly (16-byte loads whose LDS destinations are
// consecutive per wave; each lane picks the global chunk that belongs at its
// slot of the swizzled layout).  NBUF = 2: the next sub-tile loads while the
// current one is used.  Two or more workgroups share a CU, so one's softmax
// (VALU) overlaps another's matrix products on every SIMD.
template <int D, int B, int KS, int NBUF>
__global__ __launch_bounds__(2 * B, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, const int* __restrict__ counts,
    const int* __restrict__ block_idx, uint16_t* __restrict__ out,
    float* __restrict__ lse, int H, int N, int NB, float scale_log2) {
  using S = AttnShape<D, B, KS, NBUF>;
  static_assert(NBUF == 2, "two LDS slots");
  // Slot arrays: K sub-tile at [0, kTile), V^T sub-tile after it.  Separate
  // arrays, addressed with compile-time slot numbers, let the compiler see
  // that the slot being filled is not the one being read, so it does not
  // drain the prefetch before the matrix products.
  __shared__ __attribute__((aligned(1024))) uint16_t slot0[2 * S::kTile];
  __shared__ __attribute__((aligned(1024))) uint16_t slot1[2 * S::kTile];

  // Head-synchronous schedule: workgroup ids go round-robin over the 8 XCDs;
  // XCD x takes the x-th contiguous eighth of the query blocks of one head
  // after another, so all XCDs share one head's K/V at a time.
  const int per_xcd = (NB + 7) / 8;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int h = slot / per_xcd, I = xcd * per_xcd + slot % per_xcd;
  if (h >= H || I >= NB) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const size_t head_off = static_cast<size_t>(h) * N * D;
  const size_t np = static_cast<size_t>(NB) * B;
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

  const int cnt = counts[h * NB + I];
  const int total = cnt * S::kSub;  // sub-tiles to visit
  const int* list = block_idx + (static_cast<size_t>(h) * NB + I) * NB;
  const uint16_t* kh = k + head_off;
  const uint16_t* vth = vt + static_cast<size_t>(h) * D * np;

  // first key and number of real keys of sub-tile u
  auto sub_base = [&](int u) { return list[u / S::kSub] * B + (u % S::kSub) * KS; };

  auto issue = [&](int u, uint16_t* dst) {
    const int kbase = sub_base(u);
    const int last = max(0, min(KS, N - kbase) - 1);
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) {
      const int blk = wave * S::kLoads + i;  // 1 KB block of the sub-tile
      const int pc = blk * 64 + lane;        // physical 16-byte chunk
      {
        const int r = pc / S::kCprK, c = (pc % S::kCprK) ^ swz<S::kCprK>(r);
        const uint16_t* src = kh + static_cast<size_t>(min(kbase + min(r, last), N - 1)) * D + c * 8;
        __builtin_amdgcn_global_load_lds((const gvoid*)src, (lvoid*)(dst + blk * 512), 16, 0, 0);
      }
      {
        const int r = pc / S::kCprV, c = (pc % S::kCprV) ^ swz<S::kCprV>(r);
        const uint16_t* src = vth + static_cast<size_t>(r) * np + kbase + c * 8;
        __builtin_amdgcn_global_load_lds((const gvoid*)src, (lvoid*)(dst + S::kTile + blk * 512), 16, 0, 0);
      }
    }
  };

  f32x16 oacc[S::kDT];
#pragma unroll
  for (int t = 0; t < S::kDT; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY;  // reference maximum, log2 units
  float l_part[4] = {0.f, 0.f, 0.f, 0.f};

  // sub-tile u is computed from `cur` while sub-tile u+1 loads into `nxt`
  auto step = [&](int u, const uint16_t* cur, uint16_t* nxt) {
    if (u + 1 < total) issue(u + 1, nxt);
    const int valid = N - sub_base(u);  // real keys of this sub-tile (>= KS on all but the tail)
    const char* kt = reinterpret_cast<const char*>(cur);
    const char* vs = reinterpret_cast<const char*>(cur + S::kTile);
    f32x16 sacc[S::kKT];
#pragma unroll
    for (int t = 0; t < S::kKT; ++t) {
      const int r = 32 * t + col;
      bf16x8 a[S::kKSD];
#pragma unroll
      for (int s = 0; s < S::kKSD; ++s)
        a[s] = *reinterpret_cast<const bf16x8*>(kt + r * (2 * D) + (((2 * s + hl) ^ swz<S::kCprK>(r)) * 16));
      sacc[t] = f32x16{};
#pragma unroll
      for (int s = 0; s < S::kKSD; ++s) sacc[t] = mfma32(a[s], qf[s], sacc[t]);
    }
    if (valid < KS) {
#pragma unroll
      for (int t = 0; t < S::kKT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * t + acc_row(r, hl) >= valid) sacc[t][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < S::kKT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_blk = mx * scale_log2;
    const bool need = m_blk > m_run + 8.f;
    const float m_use = need ? m_blk : m_run;
    const float alpha = need ? exp2f(m_run - m_use) : 1.f;
    m_run = m_use;
#pragma unroll
    for (int e = 0; e < 4; ++e) l_part[e] *= alpha;
    if (__any(need)) {
#pragma unroll
      for (int t = 0; t < S::kDT; ++t) oacc[t] *= alpha;
    }
    bf16x8 pb[S::kKSK];
#pragma unroll
    for (int t = 0; t < S::kKT; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[t][r], scale_log2, -m_use));
        l_part[r & 3] += p;
        pb[2 * t + (r >> 3)][r & 7] = static_cast<__bf16>(p);
      }
    }
#pragma unroll
    for (int dt = 0; dt < S::kDT; ++dt) {
      const int r = 32 * dt + col;
      bf16x8 a[S::kKSK];
#pragma unroll
      for (int w = 0; w < S::kKSK; ++w)
        a[w] = *reinterpret_cast<const bf16x8*>(vs + r * (2 * KS) + (((2 * w + hl) ^ swz<S::kCprV>(r)) * 16));
#pragma unroll
      for (int w = 0; w < S::kKSK; ++w) oacc[dt] = mfma32(a[w], pb[w], oacc[dt]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // sub-tile u+1 landed; every wave is done with sub-tile u
  };

  if (total > 0) {
    issue(0, slot0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  for (int u = 0; u < total; u += 2) {
    step(u, slot0, slot1);
    if (u + 1 < total) step(u + 1, slot1, slot0);
  }

  const float l_run = (l_part[0] + l_part[1]) + (l_part[2] + l_part[3]);
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
                         const int* counts, const int* idx, void* out, float* lse, void* ws,
                         hipStream_t stream) {
  const float sl2 = p.scale * kLog2e;
  if (p.dtype == 0) {
    // two LDS slots per workgroup: 64-key sub-tiles for 128-row blocks (64 KB,
    // two workgroups per CU), 32-key sub-tiles for 64-row blocks (32 KB, four)
    constexpr int kKs = B == 128 ? 64 : 32, kNbuf = 2;
    using S = AttnShape<D, B, kKs, kNbuf>;
    uint16_t* vt = static_cast<uint16_t*>(ws);
    hipLaunchKernelGGL((vt_kernel<D, B>), dim3(p.nb, p.heads), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(v), vt, p.tokens, p.nb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int grid = 8 * ((p.nb + 7) / 8) * p.heads;
    hipLaunchKernelGGL((attn_bf16_kernel<D, B, kKs, kNbuf>), dim3(grid), dim3(S::kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), vt, counts,
                       idx, static_cast<uint16_t*>(out), lse, p.heads, p.tokens, p.nb, sl2);
  } else {
    hipLaunchKernelGGL((attn_f32_kernel<D, B>), dim3(p.heads * p.nb), dim3(B), 0, stream,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), counts, idx, static_cast<float*>(out),
                       lse, p.tokens, p.nb, sl2);
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_ws_bytes(const Problem& p) {
  if (p.dtype != 0) return 0;
  return (sizeof(uint16_t) * p.heads * p.head_dim * static_cast<size_t>(p.nb) * p.block + 255) / 256 * 256;
}

hipError_t launch_attention(const Problem& p, const void* q, const void* k, const void* v,
                            const int* counts, const int* idx, void* out, float* lse, void* ws,
                            hipStream_t stream) {
  if (p.head_dim == 128 && p.block == 128) return launch_attn_t<128, 128>(p, q, k, v, counts, idx, out, lse, ws, stream);
  if (p.head_dim == 128 && p.block == 64) return launch_attn_t<128, 64>(p, q, k, v, counts, idx, out, lse, ws, stream);
  if (p.head_dim == 64 && p.block == 128) return launch_attn_t<64, 128>(p, q, k, v, counts, idx, out, lse, ws, stream);
  return launch_attn_t<64, 64>(p, q, k, v, counts, idx, out, lse, ws, stream);
}

}  // namespace rsa
