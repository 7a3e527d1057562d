// Query-aware key clustering (gfx950).
//
// PARK (Accurate Block Retrieval for Sparse Attention in Video Diffusion
// Transformers), Abstract: keys are transformed with information from the
// current queries before clustering, so that keys the queries score alike are
// grouped, and the clusters' mean representations drive block retrieval.
//
// The metric is the one the current queries induce: G = Q^T Q / N, and the
// squared distance of a key k to a centroid c is (k - c)^T G (k - c), the
// mean over the queries of the squared gap between their scores of k and c.
//
//   gram:   per chunk of tokens a partial Q^T Q (bf16: 32x32x16 matrix-core
//           products of exact bf16 values, fp32 sums), then the chunks added
//           in a fixed order in fp64 and divided by N.
//   k-means iteration (Lloyd):
//     wprep   W_j = 2 G c_j and b_j = c_j^T G c_j for every centroid; W_j
//             times its own power of two split into two fp16 terms (22
//             significant bits) for the matrix cores;
//     assign  the nearest centroid maximises 2 k.G c_j - c_j^T G c_j: one
//             workgroup per 128 keys, the keys in registers, centroid chunks of
//             32 streamed through LDS, a running maximum per key (ties: the
//             lower cluster index);
//     sort    a stable counting sort of the keys by cluster (per-chunk
//             histograms and in-chunk ranks, a scan over chunks and clusters,
//             a scatter), deterministic, no floating-point atomics;
//     means   each non-empty cluster's centroid = mean of its keys in sorted
//             order (fp64 sums over fixed segments of the order, segments
//             added in order, one rounding); an empty cluster keeps its own.
#include "common.h"
#include "kernels.h"

namespace rsa {
namespace {

constexpr int kGramChunk = 2048;  // tokens per partial Gram matrix
constexpr int kGramStage = 128;   // tokens staged in LDS at a time
constexpr int kHistChunk = 256;   // tokens per histogram chunk
constexpr int kAssignRows = 128;  // keys per assignment workgroup
constexpr int kSeg = 256;         // sorted positions per mean segment

// ---------------------------------------------------------------- gram
// Partial Q^T Q of one chunk of kGramChunk tokens, bf16 input.  The chunk is
// staged kGramStage tokens at a time in LDS transposed (dim-major), so that
// both operands of a 32x32x16 product (8 consecutive tokens of one dim per
// lane) are single 16-byte reads.  Each thread stages an 8-token x 8-dim
// block: eight 16-byte loads (one per token), a transpose in registers (byte
// selects), eight 16-byte LDS writes (one per dim).  Wave w owns output tiles
// w*kPerWave.. of the (D/32)^2 tiles of G.
template <int D>
__global__ __launch_bounds__(256) void gram_bf16_kernel(const uint16_t* __restrict__ q,
                                                        float* __restrict__ part, int N, int nchunk) {
  constexpr int kT = D / 32;                // tiles per side
  constexpr int kPerWave = kT * kT / 4;     // tiles per wave
  constexpr int kStride = kGramStage + 8;   // LDS row pitch in tokens (bank spread; 16-byte rows stay aligned)
  static_assert(kStride * 2 % 16 == 0 && kGramChunk % kGramStage == 0, "aligned rows, whole stages");
  __shared__ __attribute__((aligned(16))) uint16_t qt[D * kStride];
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, hl = lane >> 5, col = lane & 31;
  const int t0 = c * kGramChunk, t1 = min(N, t0 + kGramChunk);
  const uint16_t* qh = q + static_cast<size_t>(h) * N * D;
  f32x16 acc[kPerWave];
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) acc[i] = f32x16{};
  for (int s0 = t0; s0 < t1; s0 += kGramStage) {
    __syncthreads();
    for (int e = tid; e < (kGramStage / 8) * (D / 8); e += 256) {
      const int g = e / (D / 8), d8 = (e % (D / 8)) * 8;  // tokens s0 + 8g.., dims d8..
      u32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = s0 + 8 * g + u;
        x[u] = t < t1 ? *reinterpret_cast<const u32x4*>(qh + static_cast<size_t>(t) * D + d8) : u32x4{0, 0, 0, 0};
      }
      // word w of x[u] holds dims d8 + 2w (low half) and d8 + 2w + 1 (high
      // half) of token u; word m of row y[dd] holds tokens 2m (low) and
      // 2m + 1 (high) of dim d8 + dd
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x4 lo, hi;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          lo[m] = __builtin_amdgcn_perm(x[2 * m + 1][w], x[2 * m][w], 0x05040100u);  // low halves
          hi[m] = __builtin_amdgcn_perm(x[2 * m + 1][w], x[2 * m][w], 0x07060302u);  // high halves
        }
        *reinterpret_cast<u32x4*>(&qt[(d8 + 2 * w) * kStride + 8 * g]) = lo;
        *reinterpret_cast<u32x4*>(&qt[(d8 + 2 * w + 1) * kStride + 8 * g]) = hi;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kGramStage / 16; ++ks) {
      const int tk = ks * 16 + 8 * hl;
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int tile = wave * kPerWave + i, ti = tile / kT, tj = tile % kT;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&qt[(32 * ti + col) * kStride + tk]);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(&qt[(32 * tj + col) * kStride + tk]);
        acc[i] = mfma32(a, b, acc[i]);
      }
    }
  }
  float* dst = part + (static_cast<size_t>(h) * nchunk + c) * D * D;
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int tile = wave * kPerWave + i, ti = tile / kT, tj = tile % kT;
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[(32 * ti + acc_row(r, hl)) * D + 32 * tj + col] = acc[i][r];
  }
}

// fp32 input: one thread per entry of G, fp64 sum over all tokens (the
// correctness path of fp32 problems, which are small).
template <int D>
__global__ __launch_bounds__(256) void gram_f32_kernel(const float* __restrict__ q, float* __restrict__ gram,
                                                       int N) {
  const int h = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  const int a = e / D, b = e % D;
  const float* qh = q + static_cast<size_t>(h) * N * D;
  double s = 0.0;
  for (int t = 0; t < N; ++t) s += static_cast<double>(qh[static_cast<size_t>(t) * D + a]) * qh[static_cast<size_t>(t) * D + b];
  gram[static_cast<size_t>(h) * D * D + e] = static_cast<float>(s / N);
}

// G = (sum of the chunks' partials, in chunk order, fp64) / N.
template <int D>
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* __restrict__ part, float* __restrict__ gram,
                                                          int N, int nchunk) {
  const int h = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  const float* p = part + static_cast<size_t>(h) * nchunk * D * D + e;
  double s = 0.0;
  for (int c = 0; c < nchunk; ++c) s += p[static_cast<size_t>(c) * D * D];
  gram[static_cast<size_t>(h) * D * D + e] = static_cast<float>(s / N);
}

// ---------------------------------------------------------------- wprep
// For 32 centroids per workgroup: W_j = 2 G c_j (fp32) and b_j = c_j . (G c_j);
// W_j times its own power of two t_j (max |W_j t_j| in [2^13, 2^14)) split
// into fp16 hi + lo, 22 significant bits, and 1 / t_j.  Rows past NB get zero
// W and b = +inf, so they never win the assignment.  bt holds per chunk of
// 32 centroids the 32 b_j and then the 32 1 / t_j (one 256-byte run, which
// the assignment loads with the chunk's tiles).
template <int D>
__global__ __launch_bounds__(256) void wprep_kernel(const float* __restrict__ gram, const float* __restrict__ cent,
                                                    _Float16* __restrict__ whi, _Float16* __restrict__ wlo,
                                                    float* __restrict__ w32, float* __restrict__ bvec,
                                                    float* __restrict__ bt, int NB, int NBp) {
  __shared__ float cs[32][D];
  __shared__ float ws[32][D + 1];
  __shared__ float tsc[32];
  const int j0 = blockIdx.x * 32, h = blockIdx.y, tid = threadIdx.x;
  const float* g = gram + static_cast<size_t>(h) * D * D;  // read by rows: neighbouring threads, neighbouring d
  for (int e = tid; e < 32 * D; e += 256) {
    const int j = e / D, d = e % D;
    cs[j][d] = j0 + j < NB ? cent[(static_cast<size_t>(h) * NB + j0 + j) * D + d] : 0.f;
  }
  __syncthreads();
  {
    // thread (grp, d) takes dim d of centroids grp, grp + kG, ...: each G
    // element is read once per group and used for all its centroids
    constexpr int kG = 256 / D, kJ = 32 / kG;
    static_assert(256 % D == 0 && 32 % kG == 0, "threads per dim group");
    const int d = tid % D, grp = tid / D;
    float acc[kJ];
#pragma unroll
    for (int m = 0; m < kJ; ++m) acc[m] = 0.f;
#pragma unroll 4
    for (int x = 0; x < D; ++x) {
      const float gv = g[x * D + d];  // G symmetric: G[d][x] = G[x][d]
#pragma unroll
      for (int m = 0; m < kJ; ++m) acc[m] = fmaf(gv, cs[grp + kG * m][x], acc[m]);
    }
#pragma unroll
    for (int m = 0; m < kJ; ++m) {
      const int j = grp + kG * m;
      ws[j][d] = acc[m];
      w32[(static_cast<size_t>(h) * NBp + j0 + j) * D + d] = 2.f * acc[m];
    }
  }
  __syncthreads();
  if (tid < 32) {
    float b = 0.f, m = 0.f;
    for (int d = 0; d < D; ++d) {
      b = fmaf(cs[tid][d], ws[tid][d], b);
      m = fmaxf(m, fabsf(2.f * ws[tid][d]));
    }
    const int sh = (m > 0.f && m < INFINITY) ? 13 - ilog2f(m) : 0;
    const int shc = sh < -126 ? -126 : (sh > 126 ? 126 : sh);
    tsc[tid] = pow2i(shc);
    const size_t o = static_cast<size_t>(h) * NBp + j0 + tid;
    bvec[o] = j0 + tid < NB ? b : INFINITY;
    float* btc = bt + (static_cast<size_t>(h) * (NBp / 32) + blockIdx.x) * 64;
    btc[tid] = j0 + tid < NB ? b : INFINITY;
    btc[32 + tid] = pow2i(-shc);
  }
  __syncthreads();
  for (int e = tid; e < 32 * D; e += 256) {
    const int j = e / D, d = e % D;
    const float x = 2.f * ws[j][d] * tsc[j];
    const _Float16 hi = static_cast<_Float16>(x);
    const size_t o = (static_cast<size_t>(h) * NBp + j0 + j) * D + d;
    whi[o] = hi;
    wlo[o] = static_cast<_Float16>(x - static_cast<float>(hi));
  }
}

// ---------------------------------------------------------------- assign
// One workgroup per 128 keys (4 waves of 32).  Each lane holds its key's
// dims 16s + 8hl..+7 in registers as fp16, scaled by the key's own power of
// two s_k (exact for bf16 keys).  Centroid chunks of 32 (W_j t_j hi and lo
// tiles, swizzled, and the chunk's b_j and 1 / t_j) stream into a ring of two
// LDS slots with buffer loads straight into LDS (one chunk in flight, four
// workgroups per CU).  S^T = W K^T puts the 16 clusters 32c + acc_row(r, hl)
// of this lane's key in its registers, both terms in one accumulation chain,
// so 2 k.G c_j = acc / (t_j s_k) to about fp32 accuracy (the unscaling is
// exact) and the running maximum of 2 k.G c_j - b_j stays in-lane; the
// halves merge last.
template <int D>
__global__ __launch_bounds__(256, 4) void assign_bf16_kernel(const uint16_t* __restrict__ k,
                                                             const _Float16* __restrict__ whi,
                                                             const _Float16* __restrict__ wlo,
                                                             const float* __restrict__ bt,
                                                             int* __restrict__ labels, int N, int NBp) {
  constexpr int kKS = D / 16, kCpr = D / 8;
  constexpr int kTile = 32 * D;                  // fp16 elements of a hi (or lo) tile
  constexpr int kLoads = kTile * 2 / 16 / 256;   // 16-byte loads per lane per tile
  static_assert(kLoads >= 1 && kTile * 2 % (16 * 256) == 0, "tile not divisible");
  constexpr int kSlot = 2 * kTile + 128;         // hi, lo, then 64 floats of (b, 1/t)
  __shared__ __attribute__((aligned(1024))) _Float16 slot0[kSlot];
  __shared__ __attribute__((aligned(1024))) _Float16 slot1[kSlot];
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, col = lane & 31;
  const int t = blockIdx.x * kAssignRows + wave * 32 + col;
  f16x8 kf[kKS];
  float kinv;
  {
    const bool ok = t < N;
    const u32x4* src = reinterpret_cast<const u32x4*>(k + (static_cast<size_t>(h) * N + (ok ? t : 0)) * D);
    float x[kKS][8];
    float a = 0.f;
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
      const u32x4 raw = ok ? src[2 * s + hl] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[s][2 * e] = __uint_as_float(raw[e] << 16);
        x[s][2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(x[s][e]));
    }
    a = fmaxf(a, __shfl_xor(a, 32));  // the other half of the key
    const int sh0 = (a > 0.f && a < INFINITY) ? 13 - ilog2f(a) : 0;
    const int sh = sh0 < -126 ? -126 : (sh0 > 126 ? 126 : sh0);
    const float sf = pow2i(sh);
#pragma unroll
    for (int s = 0; s < kKS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[s][e] = static_cast<_Float16>(x[s][e] * sf);
    kinv = pow2i(-sh);
  }
  const int nc = NBp / 32;
  const _Float16* wh = whi + static_cast<size_t>(h) * NBp * D;
  const _Float16* wl = wlo + static_cast<size_t>(h) * NBp * D;
  const float* bth = bt + static_cast<size_t>(h) * nc * 64;
  // each lane's byte offset inside a tile: the chunk that belongs at its
  // slot of the swizzled layout
  uint32_t off[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int pc = (wave * kLoads + i) * 64 + lane;
    const int r = pc / kCpr;
    off[i] = static_cast<uint32_t>(r * D + ((pc % kCpr) ^ swz<kCpr>(r)) * 8) * 2u;
  }
  auto issue = [&](int c, _Float16* dst) __attribute__((always_inline)) {
    const size_t base = static_cast<size_t>(32 * c) * D;
    const __amdgpu_buffer_rsrc_t rh =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(wh + base), 0, kTile * 2, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rl =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(wl + base), 0, kTile * 2, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int blk = wave * kLoads + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lvoid*)(dst + blk * 512), 16, static_cast<int>(off[i]), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lvoid*)(dst + kTile + blk * 512), 16, static_cast<int>(off[i]), 0,
                                               0, 0);
    }
    if (wave == 0) {  // the chunk's 32 b_j then 32 1 / t_j, one dword per lane
      const __amdgpu_buffer_rsrc_t rb =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(bth + 64 * c), 0, 256, kRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lvoid*)(dst + 2 * kTile), 4, 4 * lane, 0, 0, 0);
    }
  };
  float best = -INFINITY;
  int bj = 0;
  auto body = [&](int c, const _Float16* cur) __attribute__((always_inline)) {
    const char* th = reinterpret_cast<const char*>(cur);
    const char* tl = reinterpret_cast<const char*>(cur + kTile);
    const float* bs = reinterpret_cast<const float*>(cur + 2 * kTile);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
      const int o = col * (2 * D) + ((2 * s + hl) ^ swz<kCpr>(col)) * 16;
      acc = mfma32(*reinterpret_cast<const f16x8*>(th + o), kf[s], acc);
      acc = mfma32(*reinterpret_cast<const f16x8*>(tl + o), kf[s], acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jr = acc_row(r, hl);
      const float v = acc[r] * bs[32 + jr] * kinv - bs[jr];  // the two products by powers of two are exact
      if (v > best) {  // rows ascend with r: the first maximum is the lowest index
        best = v;
        bj = 32 * c + jr;
      }
    }
  };
  // chunk c lives in slot c % 2; before chunk c is read, every wave has
  // finished chunk c - 1, whose slot is then refilled with chunk c + 1
  issue(0, slot0);
  int c = 0;
  for (; c + 1 < nc; c += 2) {
    wait_vm<0>();
    barrier_lds();
    issue(c + 1, slot1);
    body(c, slot0);
    wait_vm<0>();
    barrier_lds();
    if (c + 2 < nc) issue(c + 2, slot0);
    body(c + 1, slot1);
  }
  if (c < nc) {
    wait_vm<0>();
    barrier_lds();
    body(c, slot0);
  }
  const float ob = __shfl_xor(best, 32);
  const int oj = __shfl_xor(bj, 32);
  if (ob > best || (ob == best && oj < bj)) bj = oj;
  if (hl == 0 && t < N) labels[static_cast<size_t>(h) * N + t] = bj;
}

// fp32 keys: one thread per key, fp64 dot products with the fp32 W.
template <int D>
__global__ __launch_bounds__(256) void assign_f32_kernel(const float* __restrict__ k, const float* __restrict__ w32,
                                                         const float* __restrict__ bvec, int* __restrict__ labels,
                                                         int N, int NB, int NBp) {
  const int h = blockIdx.y, t = blockIdx.x * 256 + threadIdx.x;
  if (t >= N) return;
  const float* kr = k + (static_cast<size_t>(h) * N + t) * D;
  double best = -INFINITY;
  int bj = 0;
  for (int j = 0; j < NB; ++j) {
    const float* w = w32 + (static_cast<size_t>(h) * NBp + j) * D;
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += static_cast<double>(kr[d]) * w[d];
    const double v = s - bvec[static_cast<size_t>(h) * NBp + j];
    if (v > best) {
      best = v;
      bj = j;
    }
  }
  labels[static_cast<size_t>(h) * N + t] = bj;
}

// ---------------------------------------------------------------- sort
// Per chunk of 256 keys: the count of every cluster in the chunk and each
// key's rank among the chunk's earlier keys of its cluster.
__global__ __launch_bounds__(kHistChunk) void hist_kernel(const int* __restrict__ labels, int* __restrict__ hist,
                                                          int* __restrict__ rank, int N, int NB, int nch) {
  __shared__ int lab[kHistChunk];
  __shared__ int cnt[kMaxClusters];
  const int ch = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int t = ch * kHistChunk + tid;
  const int my = t < N ? labels[static_cast<size_t>(h) * N + t] : -1;
  lab[tid] = my;
  for (int j = tid; j < NB; j += kHistChunk) cnt[j] = 0;
  __syncthreads();
  if (my >= 0) {
    int r = 0;
    for (int i = 0; i < tid; ++i) r += lab[i] == my;
    rank[static_cast<size_t>(h) * N + t] = r;
    atomicAdd(&cnt[my], 1);  // integer counts: the same for every order
  }
  __syncthreads();
  int* dst = hist + (static_cast<size_t>(h) * nch + ch) * NB;
  for (int j = tid; j < NB; j += kHistChunk) dst[j] = cnt[j];
}

// One thread per (cluster, head): the chunk histograms become each chunk's
// first rank in the cluster (exclusive over chunks, in place); the total is
// the cluster's size.
__global__ __launch_bounds__(64) void chunk_scan_kernel(int* __restrict__ hist, int* __restrict__ sizes, int NB,
                                                        int nch) {
  const int h = blockIdx.y, j = blockIdx.x * 64 + threadIdx.x;
  if (j >= NB) return;
  int* p = hist + static_cast<size_t>(h) * nch * NB + j;
  int run = 0;
  // batches of loads first, then their stores: the loads of a batch are in
  // flight together instead of each waiting behind the previous store
  constexpr int kB = 16;
  for (int c0 = 0; c0 < nch; c0 += kB) {
    int v[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) v[u] = c0 + u < nch ? p[static_cast<size_t>(c0 + u) * NB] : 0;
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      if (c0 + u < nch) p[static_cast<size_t>(c0 + u) * NB] = run;
      run += v[u];
    }
  }
  sizes[static_cast<size_t>(h) * NB + j] = run;
}

// Per head: each cluster's first position in the sorted order (exclusive
// sum of the sizes over clusters).
__global__ __launch_bounds__(256) void scan_kernel(const int* __restrict__ sizes, int* __restrict__ offs, int NB) {
  __shared__ int sz[kMaxClusters];
  __shared__ int part[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  for (int j = tid; j < NB; j += 256) sz[j] = sizes[static_cast<size_t>(h) * NB + j];
  __syncthreads();
  constexpr int kPer = kMaxClusters / 256;  // clusters per thread in the scan
  int local = 0;
  for (int e = 0; e < kPer; ++e) {
    const int j = tid * kPer + e;
    if (j < NB) local += sz[j];
  }
  part[tid] = local;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int v = part[i];
      part[i] = run;
      run += v;
    }
  }
  __syncthreads();
  int run = part[tid];
  for (int e = 0; e < kPer; ++e) {
    const int j = tid * kPer + e;
    if (j < NB) {
      offs[static_cast<size_t>(h) * NB + j] = run;
      run += sz[j];
    }
  }
}

// order[first(cluster) + first rank of this chunk + rank in chunk] = key.
__global__ __launch_bounds__(kHistChunk) void scatter_kernel(const int* __restrict__ labels,
                                                             const int* __restrict__ hist,
                                                             const int* __restrict__ rank,
                                                             const int* __restrict__ offs, int* __restrict__ order,
                                                             int N, int NB, int nch) {
  const int ch = blockIdx.x, h = blockIdx.y;
  const int t = ch * kHistChunk + threadIdx.x;
  if (t >= N) return;
  const size_t ht = static_cast<size_t>(h) * N + t;
  const int j = labels[ht];
  const int pos = offs[static_cast<size_t>(h) * NB + j] + hist[(static_cast<size_t>(h) * nch + ch) * NB + j] + rank[ht];
  order[static_cast<size_t>(h) * N + pos] = t;
}

// ---------------------------------------------------------------- means
// Cluster means over the sorted order, cut into segments of kSeg positions
// so that a large cluster does not rest on one workgroup.  One workgroup per
// (segment, head), one thread per dim, the segment's keys in sorted order,
// fp64 sums: a cluster that lies inside the segment gets its mean at once;
// the first and the last run of the segment (which may continue into the
// neighbours) leave their sums in part[h, seg, 0 / 1] for seg_combine_kernel.
template <typename T, int D>
__global__ __launch_bounds__(D) void seg_sum_kernel(const T* __restrict__ k, const int* __restrict__ order,
                                                    const int* __restrict__ labels, const int* __restrict__ sizes,
                                                    const int* __restrict__ offs, double* __restrict__ part,
                                                    float* __restrict__ cent, int N, int NB, int nseg) {
  __shared__ int tok[kSeg];
  __shared__ int lab[kSeg];
  const int sg = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int p0 = sg * kSeg, len = min(kSeg, N - p0);
  for (int i = d; i < len; i += D) {
    const int t = order[static_cast<size_t>(h) * N + p0 + i];
    tok[i] = t;
    lab[i] = labels[static_cast<size_t>(h) * N + t];
  }
  __syncthreads();
  const T* kh = k + static_cast<size_t>(h) * N * D + d;
  double acc = 0.0;
  int first = 1;
  constexpr int kBatch = 16;  // loads in flight per thread
  for (int i0 = 0; i0 < len; i0 += kBatch) {
    float xb[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = min(i0 + u, len - 1);
      if constexpr (sizeof(T) == 2)
        xb[u] = __uint_as_float(static_cast<uint32_t>(kh[static_cast<size_t>(tok[i]) * D]) << 16);
      else
        xb[u] = kh[static_cast<size_t>(tok[i]) * D];
    }
    for (int u = 0; u < kBatch && i0 + u < len; ++u) {
      const int i = i0 + u;
      acc += static_cast<double>(xb[u]);
      const int j = lab[i];
      if (i + 1 == len || lab[i + 1] != j) {  // end of a run
        const size_t row = static_cast<size_t>(h) * NB + j;
        const int off = offs[row], n = sizes[row];
        if (off >= p0 && off + n <= p0 + len) {
          cent[row * D + d] = static_cast<float>(acc / n);
        } else {
          double* ps = part + (static_cast<size_t>(h) * nseg + sg) * 2 * D + d;
          if (first) ps[0] = acc;
          if (i + 1 == len) ps[D] = acc;
        }
        acc = 0.0;
        first = 0;
      }
    }
  }
}

// Clusters spanning several segments: their last-run sum in the first
// segment, whole middle segments, the first-run sum in the last segment,
// added in segment order.
template <int D>
__global__ __launch_bounds__(D) void seg_combine_kernel(const double* __restrict__ part,
                                                        const int* __restrict__ sizes, const int* __restrict__ offs,
                                                        float* __restrict__ cent, int NB, int nseg) {
  const int j = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const size_t row = static_cast<size_t>(h) * NB + j;
  const int n = sizes[row], off = offs[row];
  if (n == 0) return;
  const int s0 = off / kSeg, s1 = (off + n - 1) / kSeg;
  if (s0 == s1) return;  // done by seg_sum_kernel
  const double* ph = part + static_cast<size_t>(h) * nseg * 2 * D + d;
  double acc = ph[(static_cast<size_t>(s0) * 2 + 1) * D];
  for (int sg = s0 + 1; sg < s1; ++sg) acc += ph[static_cast<size_t>(sg) * 2 * D];
  acc += ph[static_cast<size_t>(s1) * 2 * D];
  cent[row * D + d] = static_cast<float>(acc / n);
}

struct KmeansWs {
  _Float16 *whi, *wlo;
  float *w32, *bvec, *bmax, *bt;
  int *hist, *rank, *offs;
  double* part;
  size_t total;
};

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

KmeansWs kmeans_ws_layout(const Problem& p, void* base) {
  const size_t NBp = (p.nb + 31) / 32 * 32;
  const size_t nch = (p.tokens + kHistChunk - 1) / kHistChunk;
  const size_t H = p.heads, D = p.head_dim;
  const size_t nseg = (p.tokens + kSeg - 1) / kSeg;
  const size_t sizes[] = {al256(2 * H * NBp * D), al256(2 * H * NBp * D), al256(4 * H * NBp * D),
                          al256(4 * H * NBp), al256(4 * H * p.nb), al256(4 * H * nch * p.nb),
                          al256(4 * H * static_cast<size_t>(p.tokens)), al256(4 * H * p.nb),
                          al256(8 * H * nseg * 2 * D), al256(8 * H * NBp)};
  KmeansWs w{};
  char* b = static_cast<char*>(base);
  size_t off = 0;
  void** ptrs[] = {(void**)&w.whi, (void**)&w.wlo, (void**)&w.w32, (void**)&w.bvec, (void**)&w.bmax,
                   (void**)&w.hist, (void**)&w.rank, (void**)&w.offs, (void**)&w.part, (void**)&w.bt};
  for (int i = 0; i < 10; ++i) {
    if (b != nullptr) *ptrs[i] = b + off;
    off += sizes[i];
  }
  w.total = off;
  return w;
}

size_t gram_chunks(const Problem& p) { return (p.tokens + kGramChunk - 1) / kGramChunk; }

template <int D>
hipError_t launch_kmeans_t(const Problem& p, const void* k, const float* gram, int iters, int init, float* cent,
                           int* labels, int* sizes, int* order, void* ws, hipStream_t stream) {
  const KmeansWs w = kmeans_ws_layout(p, ws);
  const int NB = p.nb, NBp = (p.nb + 31) / 32 * 32, N = p.tokens, H = p.heads;
  const int nch = (N + kHistChunk - 1) / kHistChunk;
  const int nseg = (N + kSeg - 1) / kSeg;
  hipError_t e;
  if (init) {
    e = launch_block_means(p, k, 1.0, cent, w.bmax, stream);
    if (e != hipSuccess) return e;
  }
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL((wprep_kernel<D>), dim3(NBp / 32, H), dim3(256), 0, stream, gram, cent, w.whi, w.wlo,
                       w.w32, w.bvec, w.bt, NB, NBp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.dtype == 0)
      hipLaunchKernelGGL((assign_bf16_kernel<D>), dim3((N + kAssignRows - 1) / kAssignRows, H), dim3(256), 0,
                         stream, static_cast<const uint16_t*>(k), w.whi, w.wlo, w.bt, labels, N, NBp);
    else
      hipLaunchKernelGGL((assign_f32_kernel<D>), dim3((N + 255) / 256, H), dim3(256), 0, stream,
                         static_cast<const float*>(k), w.w32, w.bvec, labels, N, NB, NBp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(hist_kernel, dim3(nch, H), dim3(kHistChunk), 0, stream, labels, w.hist, w.rank, N, NB, nch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_scan_kernel, dim3((NB + 63) / 64, H), dim3(64), 0, stream, w.hist, sizes, NB, nch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(scan_kernel, dim3(H), dim3(256), 0, stream, sizes, w.offs, NB);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(scatter_kernel, dim3(nch, H), dim3(kHistChunk), 0, stream, labels, w.hist, w.rank, w.offs,
                       order, N, NB, nch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.dtype == 0)
      hipLaunchKernelGGL((seg_sum_kernel<uint16_t, D>), dim3(nseg, H), dim3(D), 0, stream,
                         static_cast<const uint16_t*>(k), order, labels, sizes, w.offs, w.part, cent, N, NB, nseg);
    else
      hipLaunchKernelGGL((seg_sum_kernel<float, D>), dim3(nseg, H), dim3(D), 0, stream, static_cast<const float*>(k),
                         order, labels, sizes, w.offs, w.part, cent, N, NB, nseg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((seg_combine_kernel<D>), dim3(NB, H), dim3(D), 0, stream, w.part, sizes, w.offs, cent, NB,
                       nseg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D>
hipError_t launch_gram_t(const Problem& p, const void* q, float* gram, void* ws, hipStream_t stream) {
  if (p.dtype != 0) {
    hipLaunchKernelGGL((gram_f32_kernel<D>), dim3((D * D + 255) / 256, p.heads), dim3(256), 0, stream,
                       static_cast<const float*>(q), gram, p.tokens);
    return hipGetLastError();
  }
  const int nchunk = static_cast<int>(gram_chunks(p));
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL((gram_bf16_kernel<D>), dim3(nchunk, p.heads), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), part, p.tokens, nchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gram_reduce_kernel<D>), dim3((D * D + 255) / 256, p.heads), dim3(256), 0, stream, part, gram,
                     p.tokens, nchunk);
  return hipGetLastError();
}

}  // namespace

size_t gram_ws_bytes(const Problem& p) {
  return p.dtype == 0 ? al256(sizeof(float) * p.heads * gram_chunks(p) * p.head_dim * p.head_dim) : 0;
}

hipError_t launch_gram(const Problem& p, const void* q, float* gram, void* ws, hipStream_t stream) {
  return p.head_dim == 128 ? launch_gram_t<128>(p, q, gram, ws, stream) : launch_gram_t<64>(p, q, gram, ws, stream);
}

size_t kmeans_ws_bytes(const Problem& p) { return kmeans_ws_layout(p, nullptr).total; }

hipError_t launch_kmeans(const Problem& p, const void* k, const float* gram, int iters, int init, float* cent,
                         int* labels, int* sizes, int* order, void* ws, hipStream_t stream) {
  return p.head_dim == 128
             ? launch_kmeans_t<128>(p, k, gram, iters, init, cent, labels, sizes, order, ws, stream)
             : launch_kmeans_t<64>(p, k, gram, iters, init, cent, labels, sizes, order, ws, stream);
}

}  // namespace rsa
