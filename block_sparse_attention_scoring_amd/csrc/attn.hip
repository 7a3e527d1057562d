// Block-sparse attention over compacted key-block lists (gfx950).
//
// PARK (Accurate Block Retrieval for Sparse Attention in Video Diffusion
// Transformers), Abstract: attention is computed only inside the retrieved
// key blocks.  Query i of block I sees the tokens of the key blocks listed
// for (h, I); the softmax is normalised over exactly those tokens (a block
// listed twice counts once, the order of a list does not matter).  A first
// kernel rewrites every list in canonical form (ascending, no repeats, no
// invalid entries); the attention kernels walk the canonical lists.
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
#include <algorithm>
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace rsa {
namespace {

// Key sub-tile width of the 128-row bf16 kernel and the LDS ring depth of
// its single-block mode (kept overridable at build time for tuning sweeps).
#ifndef RSA_ATTN_KS
#define RSA_ATTN_KS 32
#endif
#ifndef RSA_ATTN_NBUF
#define RSA_ATTN_NBUF 3
#endif

// Position of `key` inside its 16-key group of V^T: the S^T result layout
// gives lane half h keys {4h..4h+3, 8+4h..8+4h+3}, so groups 1 and 2 of
// four keys are swapped.
__host__ __device__ __forceinline__ int vt_pos(int key) {
  const int g4 = (key >> 2) & 3;
  const int sw = ((g4 & 1) << 1) | (g4 >> 1);
  return (key & ~15) | (sw << 2) | (key & 3);
}


constexpr int kMaxNB = 4096;  // largest number of blocks per sequence

// Canonical lists.  One workgroup per (query block I, head h): marks the
// listed blocks in an LDS byte map and compacts the map in ascending order
// into clist[h, I, 0..ccount[h, I]).  The count is clamped to [0, NB] and
// indices outside [0, NB) are dropped.  With `complement` set, the blocks
// the row does not list are compacted instead.  Heads with head_active[h]
// == 0 are skipped (head_active NULL: every head).
__global__ __launch_bounds__(256) void canon_kernel(const int* __restrict__ counts,
                                                    const int* __restrict__ block_idx,
                                                    const uint8_t* __restrict__ head_active,
                                                    int complement, int* __restrict__ ccount,
                                                    int* __restrict__ clist, int NB) {
  __shared__ uint8_t mark[kMaxNB];
  __shared__ int wsum[4];
  const int I = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  if (head_active != nullptr && head_active[h] == 0) return;
  const int lane = tid & 63, wave = tid >> 6;
  const size_t row = static_cast<size_t>(h) * NB + I;
  for (int e = tid; e < NB; e += 256) mark[e] = 0;
  __syncthreads();
  const int c = min(max(counts[row], 0), NB);
  for (int t = tid; t < c; t += 256) {
    const int j = block_idx[row * NB + t];
    if (static_cast<unsigned>(j) < static_cast<unsigned>(NB)) mark[j] = 1;  // repeats write the same byte
  }
  __syncthreads();
  int* out = clist + row * NB;
  int base = 0;
  for (int r0 = 0; r0 < NB; r0 += 256) {
    const int e = r0 + tid;
    const bool f = e < NB && (mark[e] != 0) != (complement != 0);
    const uint64_t bal = __ballot(f);
    const int pre = __builtin_popcountll(bal & ((1ull << lane) - 1));
    if (lane == 0) wsum[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int off = base, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      off += w < wave ? wsum[w] : 0;
      tot += wsum[w];
    }
    if (f) out[off + pre] = e;
    base += tot;
    __syncthreads();
  }
  if (tid == 0) ccount[row] = base;
}

// ---------------------------------------------------------------- pairing
// 64-token blocks run in pairs, one 128-row workgroup walking the union of
// two blocks' key sets, and a wave idles on the key blocks only its partner
// selected.  So a pair costs the size of the symmetric difference of its two
// sets on top of their own work, and the pairs are chosen to keep that
// small: each block may pair with the kPairWin blocks on either side (in the
// (frame, height, width) token order this reaches the same place in the
// neighbouring frame for a 21 x 30 x 52 latent: 24.4 blocks per frame),
// inside segments of kPairSeg blocks.  The matching is the greedy one
// (lightest edge first, ties by the lower block and then the shorter
// distance), computed in rounds: every unmatched block proposes its
// lightest edge to an unmatched block, and mutual proposals are matched.
// After kPairRounds rounds the blocks left without a partner are paired in
// ascending order; only the last segment can leave one block alone.  The
// pairs change which blocks share a workgroup, not what any query sees:
// each block still walks its own set in ascending order.
constexpr int kPairWin = 32;     // candidate partners on each side
constexpr int kPairSeg = 128;    // blocks matched together (one workgroup, one per thread)
constexpr int kPairRounds = 8;   // rounds before the rest is paired in order
static_assert(kPairSeg == 128 && kPairWin == 32, "key packing: weight (13 bits), block (7), distance (5)");

// One workgroup per (row, head): the row's set (as canon_kernel reads it,
// complement applied) as NW = ceil(NB / 64) words of bits.
__global__ __launch_bounds__(256) void pair_bits_kernel(const int* __restrict__ counts,
                                                        const int* __restrict__ block_idx,
                                                        const uint8_t* __restrict__ head_active,
                                                        int complement, uint64_t* __restrict__ bits, int NB) {
  __shared__ uint8_t mark[kMaxNB];
  const int I = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  if (head_active != nullptr && head_active[h] == 0) return;
  const int lane = tid & 63, wave = tid >> 6;
  const size_t row = static_cast<size_t>(h) * NB + I;
  for (int e = tid; e < NB; e += 256) mark[e] = 0;
  __syncthreads();
  const int c = min(max(counts[row], 0), NB);
  for (int t = tid; t < c; t += 256) {
    const int j = block_idx[row * NB + t];
    if (static_cast<unsigned>(j) < static_cast<unsigned>(NB)) mark[j] = 1;
  }
  __syncthreads();
  const int nw = (NB + 63) / 64;
  for (int w = wave; w < nw; w += 4) {
    const int e = 64 * w + lane;
    const uint64_t b = __ballot(e < NB && (mark[e] != 0) != (complement != 0));
    if (lane == 0) bits[row * nw + w] = b;
  }
}

// One wave per (row i, head): lane t < kPairWin writes the symmetric
// difference of rows i and i + 1 + t (0xffff when that row is past the end
// or in the next segment).
__global__ __launch_bounds__(64) void pair_weight_kernel(const uint64_t* __restrict__ bits,
                                                         const uint8_t* __restrict__ head_active,
                                                         uint16_t* __restrict__ wtab, int NB) {
  const int i = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  if (head_active != nullptr && head_active[h] == 0) return;
  if (t >= kPairWin) return;
  const int j = i + 1 + t, nw = (NB + 63) / 64;
  int w = 0xffff;
  if (j < NB && j / kPairSeg == i / kPairSeg) {
    const uint64_t* a = bits + (static_cast<size_t>(h) * NB + i) * nw;
    const uint64_t* b = bits + (static_cast<size_t>(h) * NB + j) * nw;
    w = 0;
    for (int k = 0; k < nw; ++k) w += __builtin_popcountll(a[k] ^ b[k]);
  }
  wtab[(static_cast<size_t>(h) * NB + i) * kPairWin + t] = static_cast<uint16_t>(w);
}

// Exclusive rank of `f` over the workgroup's kPairSeg threads, and the total.
__device__ __forceinline__ int rank_seg(bool f, int* wsum, int* total) {
  constexpr int kW = kPairSeg / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t bal = __ballot(f);
  if (lane == 0) wsum[wave] = __builtin_popcountll(bal);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    off += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return off + __builtin_popcountll(bal & ((1ull << lane) - 1));
}

// One workgroup per (segment, head), thread r holding block s0 + r of the
// segment.  Edge keys: weight << 12 | lower block << 5 | distance - 1,
// unique per edge, so the lightest edge of the rest is always mutual and
// every round matches at least one pair.  Output: unit P of the head holds
// blocks pairs[P].x < pairs[P].y (y = -1: a block alone), units in order of
// their first block, (NB + 1) / 2 of them.
__global__ __launch_bounds__(kPairSeg) void pair_match_kernel(const uint16_t* __restrict__ wtab,
                                                              const uint8_t* __restrict__ head_active,
                                                              int2* __restrict__ pairs, int NB) {
  constexpr int kWords = kPairSeg / 32 + 3;  // taken bits: 32 guard bits, the segment, 64 guard bits
  constexpr int kW = kPairSeg / 64;
  __shared__ uint16_t wf_s[kPairSeg][kPairWin];  // forward weights of each block
  __shared__ int st[kPairSeg];                   // partner (index in the segment), -1 unmatched, -2 none
  __shared__ uint32_t best[kPairSeg];            // proposal of each block
  __shared__ uint32_t taken[kWords];             // bit 32 + k: block k is matched or absent
  __shared__ int idx[kPairSeg];                  // leftover of each rank
  __shared__ int wsum[kW];
  __shared__ int anyw[kW];
  const int s0 = blockIdx.x * kPairSeg, h = blockIdx.y, r = threadIdx.x, lane = r & 63, wave = r >> 6;
  if (head_active != nullptr && head_active[h] == 0) return;
  const int units = (NB + 1) / 2, n = min(kPairSeg, NB - s0);
  const bool live = r < n;
  constexpr uint32_t kNone = 0xffffffffu;
  // this block's edge weights, two per register: forward to block r + 1 + t,
  // backward from block r - 1 - t (0xffff: no edge); then its edge keys
  uint32_t fw[kPairWin / 2];
  uint32_t fk[kPairWin], bk[kPairWin];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(wtab + (static_cast<size_t>(h) * NB + s0 + (live ? r : 0)) *
                                                                 kPairWin);
#pragma unroll
    for (int c = 0; c < kPairWin / 8; ++c) {
      const u32x4 x = live ? src[c] : u32x4{kNone, kNone, kNone, kNone};
#pragma unroll
      for (int e = 0; e < 4; ++e) fw[4 * c + e] = x[e];
    }
#pragma unroll
    for (int t = 0; t < kPairWin; t += 2)
      *reinterpret_cast<uint32_t*>(&wf_s[r][t]) = fw[t / 2];
  }
  st[r] = live ? -1 : -2;
  best[r] = kNone;
  if (r == 0) taken[0] = kNone;              // the 32 blocks before the segment
  if (r < 2) taken[kWords - 2 + r] = kNone;  // the 64 after it
  // lane 0 of each wave publishes which of its blocks are taken
  auto publish = [&](bool tk) {
    const uint64_t m = __ballot(tk);
    if (lane == 0) {
      taken[1 + 2 * wave] = static_cast<uint32_t>(m);
      taken[2 + 2 * wave] = static_cast<uint32_t>(m >> 32);
    }
  };
  publish(!live);
  __syncthreads();
  auto key = [&](uint32_t w, int a, int t) {
    return w == 0xffffu ? kNone : (w << 12) | (static_cast<uint32_t>(a) << 5) | static_cast<uint32_t>(t);
  };
#pragma unroll
  for (int t = 0; t < kPairWin; ++t) {
    fk[t] = key((fw[t / 2] >> ((t & 1) * 16)) & 0xffffu, r, t);
    bk[t] = key(live && r - 1 - t >= 0 ? wf_s[r - 1 - t][t] : 0xffffu, r - 1 - t, t);
  }
  for (int round = 0; round < kPairRounds; ++round) {
    // proposals, recomputed when the block proposed to has been taken
    if (st[r] == -1) {
      uint32_t b = best[r];
      bool stale = b == kNone;
      if (!stale) {
        const int a = (b >> 5) & (kPairSeg - 1);
        stale = st[a == r ? a + 1 + static_cast<int>(b & 31) : a] != -1;
      }
      if (stale) {
        const int pf = r + 33, pb = r;  // bit positions of blocks r + 1 and r - 32
        const uint64_t wfv = (static_cast<uint64_t>(taken[pf / 32 + 1]) << 32) | taken[pf / 32];
        const uint64_t wbv = (static_cast<uint64_t>(taken[pb / 32 + 1]) << 32) | taken[pb / 32];
        const uint32_t tf = static_cast<uint32_t>(wfv >> (pf & 31));  // bit t: block r + 1 + t
        const uint32_t tb = static_cast<uint32_t>(wbv >> (pb & 31));  // bit 31 - t: block r - 1 - t
        b = kNone;
#pragma unroll
        for (int t = 0; t < kPairWin; ++t) {
          b = min(b, ((tf >> t) & 1u) ? kNone : fk[t]);
          b = min(b, ((tb >> (31 - t)) & 1u) ? kNone : bk[t]);
        }
        best[r] = b;
      }
    }
    __syncthreads();
    bool matched = false;
    if (st[r] == -1 && best[r] != kNone) {
      const uint32_t b = best[r];
      const int a = (b >> 5) & (kPairSeg - 1), o = a == r ? a + 1 + static_cast<int>(b & 31) : a;
      if (best[o] == b) {
        st[r] = o;
        matched = true;
      }
    }
    publish(st[r] != -1);
    const uint64_t mm = __ballot(matched);
    if (lane == 0) anyw[wave] = mm != 0;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) any |= anyw[w];
    if (any == 0) break;
  }
  // the rest in ascending order: ranks 2m and 2m + 1 pair up
  int nleft;
  const bool left = st[r] == -1;
  const int rk = rank_seg(left, wsum, &nleft);
  if (left) idx[rk] = r;
  __syncthreads();
  if (left) st[r] = (rk & 1) ? idx[rk - 1] : rk + 1 < nleft ? idx[rk + 1] : -2;
  __syncthreads();
  int nunits;
  const bool lead = live && (st[r] > r || st[r] == -2);
  const int P = s0 / 2 + rank_seg(lead, wsum, &nunits);
  if (lead && P < units)
    pairs[static_cast<size_t>(h) * units + P] = make_int2(s0 + r, st[r] >= 0 ? s0 + st[r] : -1);
}

// Pair lists for 64-token blocks.  One workgroup per (unit P, head h): the
// lists of the unit's blocks a = pairs[P].x and b = pairs[P].y (pair_match_kernel;
// b = -1: a alone), read as sets like canon_kernel reads them, are marked in
// two LDS byte maps; the union is compacted in ascending order, each entry
// J | (bits << 16) where bit 0 / bit 1 says that block a / b lists J.  With
// `complement` set each row's blocks not listed are taken instead.  Heads
// with head_active[h] == 0 are skipped.
__global__ __launch_bounds__(256) void pair_canon_kernel(const int* __restrict__ counts,
                                                         const int* __restrict__ block_idx,
                                                         const uint8_t* __restrict__ head_active,
                                                         const int2* __restrict__ pairs,
                                                         int complement, int* __restrict__ ccount,
                                                         int* __restrict__ clist, int NB) {
  __shared__ uint8_t mark0[kMaxNB];
  __shared__ uint8_t mark1[kMaxNB];
  __shared__ int wsum[4];
  const int P = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  if (head_active != nullptr && head_active[h] == 0) return;
  const int lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < NB; e += 256) {
    mark0[e] = 0;
    mark1[e] = 0;
  }
  __syncthreads();
  const int2 pr = pairs[static_cast<size_t>(h) * ((NB + 1) / 2) + P];
  const int nrows = pr.y >= 0 ? 2 : 1;
  for (int q = 0; q < nrows; ++q) {
    const size_t row = static_cast<size_t>(h) * NB + (q == 0 ? pr.x : pr.y);
    uint8_t* mk = q == 0 ? mark0 : mark1;
    const int c = min(max(counts[row], 0), NB);
    for (int t = tid; t < c; t += 256) {
      const int j = block_idx[row * NB + t];
      if (static_cast<unsigned>(j) < static_cast<unsigned>(NB)) mk[j] = 1;
    }
  }
  __syncthreads();
  const int rows_bits = nrows == 2 ? 3 : 1;
  int* out = clist + (static_cast<size_t>(h) * NB + P) * NB;
  int base = 0;
  for (int r0 = 0; r0 < NB; r0 += 256) {
    const int e = r0 + tid;
    int bits = 0;
    if (e < NB) {
      bits = mark0[e] | (mark1[e] << 1);
      if (complement) bits = rows_bits & ~bits;
    }
    const bool f = bits != 0;
    const uint64_t bal = __ballot(f);
    const int pre = __builtin_popcountll(bal & ((1ull << lane) - 1));
    if (lane == 0) wsum[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int off = base, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      off += w < wave ? wsum[w] : 0;
      tot += wsum[w];
    }
    if (f) out[off + pre] = e | (bits << 16);
    base += tot;
    __syncthreads();
  }
  if (tid == 0) ccount[static_cast<size_t>(h) * NB + P] = base;
}

// Heads taken together by the dispatch order: ng groups of nearly equal size
// (the first H mod ng groups hold one head more), so a group's K and V^T
// stay in the 256 MB Infinity Cache together and hold at most kMaxOrder
// units.
constexpr int kMaxOrder = 4096;                       // units per group, at most
constexpr double kGroupBytes = 160.0 * 1024 * 1024;  // K + V^T bytes per group, about

struct HeadGroups {
  int ng, per_xcd;  // groups; units per XCD per group (the largest group)
};

HeadGroups head_groups(const Problem& p, int units) {
  const double head_bytes = 2.0 * p.tokens * p.head_dim * (p.dtype == 0 ? 2.0 : 4.0);
  int ng = static_cast<int>(std::ceil(p.heads * head_bytes / kGroupBytes));
  ng = std::min(std::max(ng, 1), p.heads);
  while (ng < p.heads && (p.heads + ng - 1) / ng * units > kMaxOrder) ++ng;
  const int gmax = (p.heads + ng - 1) / ng;
  return {ng, (gmax * units + 7) / 8};
}

// Dispatch order over the 8 XCDs, one workgroup per head group.  The
// group's units (query blocks, or pairs of them, of all its heads) are ranked
// by list length (ccount, clamped to [0, maxlen], maxlen <= kMaxNB; inactive
// heads count 0), longest first (counting sort; equal lengths in any order),
// and dealt in a snake over the XCDs: ranks 0-7 to XCDs 0..7, ranks 8-15 to
// XCDs 7..0, and so on.  Every XCD gets an eighth of the group's work,
// longest walks first, so the XCDs finish together and the grid's tail holds
// only short walks; the groups follow one another, so the XCDs share one
// group's K/V at a time.  perm[g, x, r] = (h - first head of g) * units +
// unit for the r-th workgroup XCD x runs in group g, or -1.
__global__ __launch_bounds__(256) void order_kernel(const int* __restrict__ ccount,
                                                    const uint8_t* __restrict__ head_active,
                                                    int* __restrict__ perm, int H, int NB, int units, int ng,
                                                    int per_xcd, int maxlen) {
  constexpr int kPer = (kMaxNB + 1 + 255) / 256;  // lengths 0..maxlen
  __shared__ int start[kMaxNB + 1];  // per length: first rank, then next free rank
  __shared__ int sorted[kMaxOrder];  // unit of each rank
  __shared__ int part[256];
  const int g = blockIdx.x, tid = threadIdx.x;
  const int base = H / ng, rem = H % ng;
  const int h0 = g * base + min(g, rem), n = (base + (g < rem ? 1 : 0)) * units;
  auto length = [&](int e) {
    const int h = h0 + e / units;
    if (head_active != nullptr && head_active[h] == 0) return 0;
    return min(max(ccount[static_cast<size_t>(h) * NB + e % units], 0), maxlen);
  };
  for (int i = tid; i <= maxlen; i += 256) start[i] = 0;
  __syncthreads();
  for (int e = tid; e < n; e += 256) atomicAdd(&start[length(e)], 1);
  __syncthreads();
  // exclusive scan over lengths maxlen, ..., 0 (longest first): thread t
  // takes positions [t*kPer, (t+1)*kPer) of that descending order
  int local = 0;
  for (int k = 0; k < kPer; ++k) {
    const int len = maxlen - (tid * kPer + k);
    if (len >= 0) local += start[len];
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
  for (int k = 0; k < kPer; ++k) {
    const int len = maxlen - (tid * kPer + k);
    if (len >= 0) {
      const int c = start[len];
      start[len] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int e = tid; e < n; e += 256) sorted[atomicAdd(&start[length(e)], 1)] = e;
  __syncthreads();
  int* pg = perm + static_cast<size_t>(g) * 8 * per_xcd;
  for (int pos = tid; pos < 8 * per_xcd; pos += 256) {
    const int x = pos / per_xcd, row = pos % per_xcd;
    const int r = row * 8 + ((row & 1) ? 7 - x : x);
    pg[pos] = r < n ? sorted[r] : -1;
  }
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
                                                 const uint8_t* __restrict__ head_active,
                                                 uint16_t* __restrict__ vt, int N, int NB) {
  __shared__ uint16_t tile[B][D + 2];
  const int J = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  if (head_active != nullptr && head_active[h] == 0) return;
  const int kbase = J * B, bJ = min(B, N - kbase);
  const size_t np = static_cast<size_t>(NB) * B;
  for (int c = tid; c < B * D / 8; c += 256) {
    const int r = c / (D / 8), c8 = c % (D / 8);
    // (non-temporal: V is read once)
    u32x4 x = r < bJ ? __builtin_nontemporal_load(
                           reinterpret_cast<const u32x4*>(v + (static_cast<size_t>(h) * N + kbase + r) * D + c8 * 8))
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
// stream from HBM straight into a ring of NBUF LDS slots (buffer loads,
// 16 bytes per lane, each lane fetching the chunk that belongs at its slot of
// the swizzled layout).  Each wave software-pipelines its own work: the
// matrix products for sub-tile j run next to the exponentials of sub-tile
// j-1.  Several workgroups share a CU, so the waves on every SIMD also
// overlap each other's vector and matrix work: with a ring of three slots
// (48 KB of LDS at D = 128) three workgroups fit, and the register budget
// is capped to match (168 VGPRs, three waves per SIMD); with four slots
// (64 KB) two fit, at up to 256 VGPRs.
//
// kTable: the row lists 32-key sub-tiles instead of key blocks (clusters as
// key blocks): entry e is a sub-tile at key e & ~31 of the padded cluster
// layout holding (e & 31) + 1 real keys; K has Nk rows and V^T Nv columns per
// head.  Every sub-tile may be partial, so each step applies its mask.
//
// BQ < B (pair mode, BQ = B/2 = 64): the workgroup serves the two query
// blocks of BQ tokens of a unit (pair_match_kernel; waves 0-1 and 2-3) over
// the union of their lists (pair_canon_kernel); each wave skips the
// sub-tiles its own block did not select.  Each SIMD's waves still come
// from different workgroups.
template <int D, int B, int KS, int NBUF, bool kTable = false, int BQ = B>
__global__ __launch_bounds__(2 * B, NBUF == 3 ? 3 : 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, const int* __restrict__ ccount,
    const int* __restrict__ clist, const uint8_t* __restrict__ head_active, const int* __restrict__ perm,
    const int2* __restrict__ pairs, const uint16_t* part, const float* part_lse, uint16_t* out, float* lse, int H,
    int N, int NB,
    float scale_log2, int Nk, int Nv, int lstride, int ng, int per_xcd) {
  using S = AttnShape<D, B, KS, NBUF>;
  static_assert(NBUF >= 3 && NBUF <= 4, "ring of 3 or 4 LDS slots");
  static_assert(!kTable || KS == 32, "table entries are 32-key sub-tiles");
  constexpr bool kPair = BQ != B;
  static_assert(!kPair || (2 * BQ == B && !kTable && BQ % KS == 0), "pair mode: two blocks of B/2 tokens");
  constexpr int kSubQ = BQ / KS;  // sub-tiles per listed key block
  // Ring slots: K sub-tile at [0, kTile), V^T sub-tile after it.  Separate
  // arrays, addressed with compile-time slot numbers, let the compiler see
  // that the slot being filled is not the one being read, so it does not
  // drain the prefetches before the matrix products.
  __shared__ __attribute__((aligned(1024))) uint16_t slot0[2 * S::kTile];
  __shared__ __attribute__((aligned(1024))) uint16_t slot1[2 * S::kTile];
  __shared__ __attribute__((aligned(1024))) uint16_t slot2[NBUF > 2 ? 2 * S::kTile : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t slot3[NBUF > 3 ? 2 * S::kTile : 8];

  // Group-synchronous schedule: workgroup ids go round-robin over the 8
  // XCDs; XCD x takes the x-th eighth of one head group's units after
  // another (order_kernel: balanced by list length, longest walks first), so
  // all XCDs share one group's K/V at a time.
  const int units = kPair ? (NB + 1) / 2 : NB;  // query blocks, or pairs of them
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int g = slot / per_xcd;
  if (g >= ng) return;
  const int e = perm[static_cast<size_t>(g) * 8 * per_xcd + xcd * per_xcd + slot % per_xcd];
  if (e < 0) return;
  const int h = g * (H / ng) + min(g, H % ng) + e / units, I = e % units;
  if (h >= H || I >= units) return;
  if (head_active != nullptr && head_active[h] == 0) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS addresses stay scalar
  const int hl = lane >> 5, col = lane & 31;
  const size_t head_off = static_cast<size_t>(h) * N * D;
  const size_t np = static_cast<size_t>(Nv);
  // pair mode: waves 0-1 hold block pairs[I].x, waves 2-3 block pairs[I].y
  // (none: y = -1, taken as block NB, whose rows all lie past the end)
  int qblk = I;
  if constexpr (kPair) {
    const int2 pr = pairs[static_cast<size_t>(h) * units + I];
    qblk = (wave >> 1) == 0 ? pr.x : pr.y >= 0 ? pr.y : NB;
  }
  const int qrow = kPair ? qblk * BQ + (wave & 1) * 32 + col : I * B + wave * 32 + col;
  const int mbit = kPair ? 1 << (wave >> 1) : 0;  // this wave's bit in a pair entry

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

  const int cnt = ccount[h * NB + I];
  const int total = kTable ? cnt : cnt * kSubQ;  // sub-tiles to visit
  const int* list = clist + (static_cast<size_t>(h) * NB + I) * lstride;
  const uint16_t* kh = k + static_cast<size_t>(h) * Nk * D;
  const uint16_t* vth = vt + static_cast<size_t>(h) * D * np;

  // first key of sub-tile u
  auto sub_base = [&](int u) {
    if constexpr (kTable) return list[u] & ~31;
    else return (list[u / kSubQ] & 0xffff) * BQ + (u % kSubQ) * KS;
  };
  // whether this wave's query block selected sub-tile u (pair mode)
  auto member = [&](int u) { return !kPair || ((list[u / kSubQ] >> 16) & mbit) != 0; };

  // Tiles are fetched with buffer loads straight into LDS.  Each lane's byte
  // offset inside a sub-tile is fixed for the whole loop, so only scalar
  // registers change per sub-tile.  K: one buffer per sub-tile starting at
  // its first key and ending at the last token, so rows past the end read as
  // zeros (their scores are masked).  V^T: one buffer for the head's padded
  // V^T, the sub-tile's first key added as the scalar offset.
  uint32_t koff[S::kLoads], voff[S::kLoads];
#pragma unroll
  for (int i = 0; i < S::kLoads; ++i) {
    const int pc = (wave * S::kLoads + i) * 64 + lane;
    const int kr = pc / S::kCprK;
    koff[i] = static_cast<uint32_t>(kr * D + ((pc % S::kCprK) ^ swz<S::kCprK>(kr)) * 8) * 2u;
    const int vr = pc / S::kCprV;
    voff[i] = (static_cast<uint32_t>(vr) * static_cast<uint32_t>(np) +
               static_cast<uint32_t>(((pc % S::kCprV) ^ swz<S::kCprV>(vr)) * 8)) * 2u;
  }
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vth), 0, static_cast<int>(D * np * 2), kRsrcWord3);
  auto issue = [&](int u, uint16_t* dst) {
    const int kbase = sub_base(u);
    const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kh + static_cast<size_t>(kbase) * D), 0, max(Nk - kbase, 0) * D * 2, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) {
      const int blk = wave * S::kLoads + i;  // 1 KB block of the sub-tile
      // (offsets passed as int: clang's host pass drops the kernel's launch
      // stub when these arguments are unsigned array elements)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lvoid*)(dst + blk * 512), 16,
                                               static_cast<int>(koff[i]), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (lvoid*)(dst + S::kTile + blk * 512), 16,
                                               static_cast<int>(voff[i]), kbase * 2, 0, 0);
    }
  };

  f32x16 oacc[S::kDT];
#pragma unroll
  for (int t = 0; t < S::kDT; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY;  // reference maximum, log2 units
  float l_part[4] = {0.f, 0.f, 0.f, 0.f};

  // Per-lane byte offsets of the operand reads inside a slot, one per
  // k-step: the swizzle repeats every 16 rows, so rows 32t + col share col's
  // swizzle and a read is slot + 32-row block + this offset.
  // The empty asm keeps each offset whole, so the constant part of an
  // address goes into the LDS read's immediate offset instead of a vector add.
  uint32_t klane[S::kKSD], vlane[S::kKSK];
#pragma unroll
  for (int s = 0; s < S::kKSD; ++s) {
    klane[s] = static_cast<uint32_t>(col * (2 * D) + (((2 * s + hl) ^ swz<S::kCprK>(col)) * 16));
    asm volatile("" : "+v"(klane[s]));
  }
#pragma unroll
  for (int w = 0; w < S::kKSK; ++w) {
    vlane[w] = static_cast<uint32_t>(col * (2 * KS) + (((2 * w + hl) ^ swz<S::kCprV>(col)) * 16));
    asm volatile("" : "+v"(vlane[w]));
  }

  // S^T of one sub-tile (keys x this wave's queries) from the K slot `cur`
  auto qk = [&](const uint16_t* cur, f32x16* sacc) {
    const char* kt = reinterpret_cast<const char*>(cur);
#pragma unroll
    for (int t = 0; t < S::kKT; ++t) sacc[t] = f32x16{};
#pragma unroll
    for (int s = 0; s < S::kKSD; ++s) {
      bf16x8 a[S::kKT];
#pragma unroll
      for (int t = 0; t < S::kKT; ++t)
        a[t] = *reinterpret_cast<const bf16x8*>(kt + t * (32 * 2 * D) + klane[s]);
#pragma unroll
      for (int t = 0; t < S::kKT; ++t) sacc[t] = mfma32(a[t], qf[s], sacc[t]);
    }
  };
  // keys at or past the last token (tail sub-tile only) get score -inf; in
  // table mode the keys past the sub-tile's count
  auto mask_tail = [&](int u, f32x16* sacc) {
    const int valid = kTable ? (list[u] & 31) + 1 : N - sub_base(u);
    if (valid < KS) {
      // register r of tile t holds key 32t + acc_row(r, 0) + 4 hl: whether it
      // lies past the end is uniform in each lane half, so the condition is a
      // lane mask built in scalar registers (no per-lane value kept live)
#pragma unroll
      for (int t = 0; t < S::kKT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 32 * t + acc_row(r, 0);
          const uint64_t m = (c >= valid ? 0xffffffffull : 0ull) | (c + 4 >= valid ? 0xffffffff00000000ull : 0ull);
          if (__builtin_amdgcn_inverse_ballot_w64(m)) sacc[t][r] = -INFINITY;
        }
    }
  };
  // maximum of this query's scores in the sub-tile, log2 units; the two
  // lane halves hold different keys of the same query and swap once
  auto rowmax = [&](const f32x16* sacc) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < S::kKT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    // scores are never NaN: a plain v_max, without the quieting moves the
    // compiler adds to a max of values taken from another lane
    float m2;
    asm("v_max_f32 %0, %1, %2" : "=v"(m2) : "v"(__uint_as_float(sw[0])), "v"(__uint_as_float(sw[1])));
    return m2 * scale_log2;
  };
  // lazy rescale: move the reference maximum only when the sub-tile's
  // maximum exceeds it by more than 2^8
  auto rescale = [&](float m_blk) {
    const bool need = m_blk > m_run + 8.f;
    if (__any(need)) {  // rare: skip the factor's exponential otherwise
      const float m_use = need ? m_blk : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
      m_run = m_use;
#pragma unroll
      for (int e = 0; e < 4; ++e) l_part[e] *= alpha;
#pragma unroll
      for (int t = 0; t < S::kDT; ++t) oacc[t] *= alpha;
    }
  };
  // P = 2^(S*scale - m) in bf16, row sums in fp32, then O^T += V^T P^T with
  // V^T from the slot `cur`
  auto pv = [&](const f32x16* sacc, const uint16_t* cur) {
    const char* vs = reinterpret_cast<const char*>(cur + S::kTile);
    bf16x8 pb[S::kKSK];
#pragma unroll
    for (int t = 0; t < S::kKT; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[t][r], scale_log2, -m_run));
        l_part[r & 3] += p;
        pb[2 * t + (r >> 3)][r & 7] = static_cast<__bf16>(p);
      }
    }
#pragma unroll
    for (int dt = 0; dt < S::kDT; ++dt) {
      bf16x8 a[S::kKSK];
#pragma unroll
      for (int w = 0; w < S::kKSK; ++w)
        a[w] = *reinterpret_cast<const bf16x8*>(vs + dt * (32 * 2 * KS) + vlane[w]);
#pragma unroll
      for (int w = 0; w < S::kKSK; ++w) oacc[dt] = mfma32(a[w], pb[w], oacc[dt]);
    }
  };
  // pv in two parts for pair mode: P and its row sums (pexp), then the
  // products (pvm)
  auto pexp = [&](const f32x16* sacc, bf16x8* pb) {
#pragma unroll
    for (int t = 0; t < S::kKT; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[t][r], scale_log2, -m_run));
        l_part[r & 3] += p;
        pb[2 * t + (r >> 3)][r & 7] = static_cast<__bf16>(p);
      }
    }
  };
  auto pvm = [&](const bf16x8* pb, const uint16_t* cur) {
    const char* vs = reinterpret_cast<const char*>(cur + S::kTile);
#pragma unroll
    for (int dt = 0; dt < S::kDT; ++dt) {
      bf16x8 a[S::kKSK];
#pragma unroll
      for (int w = 0; w < S::kKSK; ++w)
        a[w] = *reinterpret_cast<const bf16x8*>(vs + dt * (32 * 2 * KS) + vlane[w]);
#pragma unroll
      for (int w = 0; w < S::kKSK; ++w) oacc[dt] = mfma32(a[w], pb[w], oacc[dt]);
    }
  };
  auto ring = [&](int i) { return i == 0 ? slot0 : i == 1 ? slot1 : i == 2 ? slot2 : slot3; };

  // Sub-tile u lives in ring slot u % NBUF.  Software pipeline over the
  // sub-tiles whose keys are all real: step j computes S^T of sub-tile j
  // (matrix cores) next to the exponentials of sub-tile j-1 (VALU), then
  // O += P V of sub-tile j-1.  Slots j-1 and j are read, the slot of j-2 is
  // refilled with sub-tile j+NBUF-2, and NBUF-3 sub-tiles may still be in
  // flight when step j waits for sub-tile j.
  constexpr int kPer = 2 * S::kLoads;  // buffer loads per lane per sub-tile
  f32x16 sprev[S::kKT];
  float mprev = -INFINITY;
  // leading sub-tiles with no key past the last token: the canonical list is
  // ascending, so only its last entry can be the ragged block NB-1
  int total_full = total;
  if (!kTable && total > 0) {
    const int last = list[cnt - 1] & 0xffff;
    if (last == NB - 1) total_full = total - kSubQ + min(kSubQ, (N - last * BQ) / KS);
  }
  int next = min(NBUF - 2, total);  // first sub-tile not yet requested
  for (int i = 0; i < NBUF - 2 && i < total; ++i) issue(i, ring(i));
  int j = 0;
  bool pending = false;  // sprev holds sub-tile j-1, not yet in O (if pvalid)
  bool pvalid = true;
  if (total_full >= NBUF + 1 && total >= 2 * NBUF - 2) {
    wait_vm<(NBUF - 3) * kPer>();
    barrier_lds();
    issue(NBUF - 2, ring(NBUF - 2));
    pvalid = member(0);  // sprev holds a sub-tile this wave selected
    if (pvalid) {
      qk(slot0, sprev);
      if constexpr (kTable) mask_tail(0, sprev);
      mprev = rowmax(sprev);
    }
    j = 1;
    pending = true;
    auto step = [&](const uint16_t* kslot, const uint16_t* vslot, uint16_t* fill, int jj) {
      if constexpr (!kPair) {
        rescale(mprev);
        wait_vm<(NBUF - 3) * kPer>();
        barrier_lds();
        issue(jj + NBUF - 2, fill);
        f32x16 scur[S::kKT];
        qk(kslot, scur);
        pv(sprev, vslot);
#pragma unroll
        for (int t = 0; t < S::kKT; ++t) sprev[t] = scur[t];
        if constexpr (kTable) mask_tail(jj, sprev);
        mprev = rowmax(sprev);
      } else {
        // the single-block step with each half skipped where this wave's
        // block did not select the sub-tile (wave-uniform branches).  The
        // exponentials of sub-tile j-1 come first, so its scores are dead
        // before S^T of sub-tile j is written into the same registers: the
        // step fits the three-workgroup register budget without spills.
        const bool mc = member(jj);
        if (pvalid) rescale(mprev);
        wait_vm<(NBUF - 3) * kPer>();
        barrier_lds();
        issue(jj + NBUF - 2, fill);
        bf16x8 pb[S::kKSK];
        if (pvalid) pexp(sprev, pb);
        if (mc) qk(kslot, sprev);
        if (pvalid) pvm(pb, vslot);
        if (mc) mprev = rowmax(sprev);
        pvalid = mc;
      }
    };
    // groups of NBUF steps starting at j = 1 mod NBUF: compile-time slots
    while (j + NBUF - 1 < total_full && j + 2 * NBUF - 3 < total) {
      step(ring(1 % NBUF), slot0, ring((NBUF - 1) % NBUF), j);
      step(ring(2 % NBUF), ring(1 % NBUF), slot0, j + 1);
      if constexpr (NBUF > 2) step(ring(3 % NBUF), ring(2 % NBUF), ring(1 % NBUF), j + 2);
      if constexpr (NBUF > 3) step(slot0, ring(3 % NBUF), ring(2 % NBUF), j + 3);
      j += NBUF;
    }
    next = j + NBUF - 2;
  }
  if (pending && pvalid) {  // finish sub-tile j-1
    rescale(mprev);
    pv(sprev, ring((j - 1) % NBUF));
  }
  // the rest, one sub-tile per step with full waits (ragged tail included)
  for (; j < total; ++j) {
    wait_vm<0>();
    barrier_lds();
    for (; next < total && next <= j + NBUF - 1; ++next) issue(next, ring(next % NBUF));
    if (member(j)) {
      f32x16 sc[S::kKT];
      qk(ring(j % NBUF), sc);
      mask_tail(j, sc);
      rescale(rowmax(sc));
      pv(sc, ring(j % NBUF));
    }
  }

  const float l_run = (l_part[0] + l_part[1]) + (l_part[2] + l_part[3]);
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < N) {
    const size_t row = static_cast<size_t>(h) * N + qrow;
    float ls = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;  // natural log
    // out = wa * O_unnormalised + wb * cached part
    float wa = l_tot > 0.f ? 1.f / l_tot : 0.f, wb = 0.f;
    if (part != nullptr) {
      // join with a cached attention over the complementary keys: the
      // softmax over the union weighs each part by its exp(lse)
      const float lb = part_lse[row];
      const float m = fmaxf(ls, lb);
      if (m > -INFINITY) {
        const float ea = expf(ls - m), eb = expf(lb - m);  // the larger of the two is 1
        const float z = ea + eb;
        wa *= ea / z;
        wb = eb / z;
        ls = m + logf(z);
      } else {
        wa = 0.f;
      }
    }
    uint16_t* dst = out + row * D;
    const uint16_t* src = part != nullptr ? part + row * D : nullptr;
#pragma unroll
    for (int dt = 0; dt < S::kDT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 32 * dt + 8 * g + 4 * hl;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = oacc[dt][4 * g + e] * wa;
        if (src != nullptr) {
          const bf16x4 b = *reinterpret_cast<const bf16x4*>(src + c);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = fmaf(wb, static_cast<float>(b[e]), x[e]);
        }
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = static_cast<__bf16>(x[e]);
        *reinterpret_cast<bf16x4*>(dst + c) = o;
      }
    }
    if (lse != nullptr && hl == 0) lse[row] = ls;
  }
}

// fp32 inputs: plain fp32 arithmetic over the canonical list, K and V staged
// in LDS 32 keys at a time and read as broadcasts.  Each query row has two
// lanes, l and l ^ 32 of a wave, each holding half of head_dim (query and
// output in registers, loops fully unrolled, so nothing goes to scratch); a
// score is the two halves' partial dot products added across the lane pair.
// Same online softmax (exact rescaling at every 8 keys).
// kTable: as in attn_bf16_kernel; k and v are the padded cluster layout,
// row-major, Nk rows per head.
template <int D, int B, bool kTable = false>
__global__ __launch_bounds__(2 * B) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int* __restrict__ ccount, const int* __restrict__ clist,
    const uint8_t* __restrict__ head_active, const float* part, const float* part_lse, float* out, float* lse,
    int N, int NB, float scale_log2, int Nk, int lstride) {
  constexpr int kChunk = 32;
  constexpr int DH = D / 2;  // dims per lane
  __shared__ float Ks[kChunk * D];
  __shared__ float Vs[kChunk * D];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int h = tile / NB, I = tile - h * NB;
  if (head_active != nullptr && head_active[h] == 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int half = lane >> 5, d0 = half * DH;
  const int qrow = I * B + (tid >> 6) * 32 + (lane & 31);
  const size_t head_off = static_cast<size_t>(h) * N * D;
  float qv[DH], o[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    qv[d] = qrow < N ? q[head_off + static_cast<size_t>(qrow) * D + d0 + d] * scale_log2 : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int cnt = ccount[h * NB + I];
  const int* list = clist + (static_cast<size_t>(h) * NB + I) * lstride;
  const size_t kv_off = static_cast<size_t>(h) * Nk * D;
  for (int it = 0; it < cnt; ++it) {
    const int kbase = kTable ? list[it] & ~31 : list[it] * B;
    const int bJ = kTable ? (list[it] & 31) + 1 : min(B, N - kbase);
    for (int kc = 0; kc < bJ; kc += kChunk) {
      const int nk = min(kChunk, bJ - kc);
      __syncthreads();
      for (int e = tid; e < kChunk * D; e += 2 * B) {
        const int row = e / D;
        const size_t g = kv_off + static_cast<size_t>(kbase + kc) * D + e;
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
#pragma unroll
          for (int d = 0; d < DH; ++d) acc = fmaf(qv[d], Ks[(j0 + j) * D + d0 + d], acc);
          acc += __shfl_xor(acc, 32);  // the other half of head_dim
          s[j] = j0 + j < nk ? acc : -INFINITY;
          mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m, mx);
        const float alpha = exp2f(m - m_new);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < DH; ++d) o[d] *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = exp2f(s[j] - m_new);
          l += p;
#pragma unroll
          for (int d = 0; d < DH; ++d) o[d] = fmaf(p, Vs[(j0 + j) * D + d0 + d], o[d]);
        }
        m = m_new;
      }
    }
  }
  if (qrow < N) {
    const size_t row = static_cast<size_t>(h) * N + qrow;
    float ls = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    float wa = l > 0.f ? 1.f / l : 0.f, wb = 0.f;
    if (part != nullptr) {  // join with the cached complementary part (as attn_bf16_kernel)
      const float lb = part_lse[row];
      const float mm = fmaxf(ls, lb);
      if (mm > -INFINITY) {
        const float ea = expf(ls - mm), eb = expf(lb - mm);
        const float z = ea + eb;
        wa *= ea / z;
        wb = eb / z;
        ls = mm + logf(z);
      } else {
        wa = 0.f;
      }
    }
#pragma unroll
    for (int d = 0; d < DH; ++d) {
      const float c = part != nullptr ? wb * part[row * D + d0 + d] : 0.f;
      out[row * D + d0 + d] = fmaf(o[d], wa, c);
    }
    if (lse != nullptr && half == 0) lse[row] = ls;
  }
}

// Attention workspace: [V^T (bf16 only)][canonical counts][canonical lists],
// each part 256-byte aligned.
struct AttnWs {
  size_t ccount_off, clist_off, perm_off, pairs_off, bits_off, wtab_off, total;
};

AttnWs attn_ws_layout(const Problem& p) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = static_cast<size_t>(p.heads) * p.nb;
  AttnWs w;
  w.ccount_off = p.dtype == 0 ? al(sizeof(uint16_t) * p.heads * p.head_dim * static_cast<size_t>(p.nb) * p.block) : 0;
  w.clist_off = w.ccount_off + al(sizeof(int) * rows);
  w.perm_off = w.clist_off + al(sizeof(int) * rows * p.nb);
  // dispatch order (bf16 path): per head group 8 eighths of its units
  const HeadGroups hg = head_groups(p, p.block == 64 ? (p.nb + 1) / 2 : p.nb);
  w.pairs_off = w.perm_off + (p.dtype == 0 ? al(sizeof(int) * 8 * static_cast<size_t>(hg.ng) * hg.per_xcd) : 0);
  // pairing of 64-token blocks (bf16): the pairs, the rows' bit sets, the edge weights
  const bool pairs = p.dtype == 0 && p.block == 64;
  const size_t nw = (static_cast<size_t>(p.nb) + 63) / 64;
  w.bits_off = w.pairs_off + (pairs ? al(sizeof(int2) * p.heads * ((static_cast<size_t>(p.nb) + 1) / 2)) : 0);
  w.wtab_off = w.bits_off + (pairs ? al(sizeof(uint64_t) * rows * nw) : 0);
  w.total = w.wtab_off + (pairs ? al(sizeof(uint16_t) * rows * kPairWin) : 0);
  return w;
}

template <int D, int B>
hipError_t launch_attn_t(const Problem& p, const void* q, const void* k, const void* v,
                         const int* counts, const int* idx, const uint8_t* head_active,
                         int complement, const void* part, const float* part_lse, void* out, float* lse,
                         void* ws, hipStream_t stream) {
  const float sl2 = p.scale * kLog2e;
  const AttnWs w = attn_ws_layout(p);
  char* base = static_cast<char*>(ws);
  int* ccount = reinterpret_cast<int*>(base + w.ccount_off);
  int* clist = reinterpret_cast<int*>(base + w.clist_off);
  // 64-token blocks on the matrix cores: pairs of query blocks per workgroup
  constexpr bool kPairs = B == 64;
  int2* pairs = reinterpret_cast<int2*>(base + w.pairs_off);
  if (p.dtype == 0 && kPairs) {
    uint64_t* bits = reinterpret_cast<uint64_t*>(base + w.bits_off);
    uint16_t* wtab = reinterpret_cast<uint16_t*>(base + w.wtab_off);
    hipLaunchKernelGGL(pair_bits_kernel, dim3(p.nb, p.heads), dim3(256), 0, stream, counts, idx, head_active,
                       complement, bits, p.nb);
    hipLaunchKernelGGL(pair_weight_kernel, dim3(p.nb, p.heads), dim3(64), 0, stream, bits, head_active, wtab, p.nb);
    hipLaunchKernelGGL(pair_match_kernel, dim3((p.nb + kPairSeg - 1) / kPairSeg, p.heads), dim3(kPairSeg), 0, stream,
                       wtab, head_active, pairs, p.nb);
    hipLaunchKernelGGL(pair_canon_kernel, dim3((p.nb + 1) / 2, p.heads), dim3(256), 0, stream, counts, idx,
                       head_active, pairs, complement, ccount, clist, p.nb);
  } else
    hipLaunchKernelGGL(canon_kernel, dim3(p.nb, p.heads), dim3(256), 0, stream, counts, idx, head_active,
                       complement, ccount, clist, p.nb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.dtype == 0) {
    // A ring of three 32-key sub-tiles, three workgroups per CU (single
    // blocks and pairs alike).
    constexpr int kKs = RSA_ATTN_KS, kNbuf = RSA_ATTN_NBUF;
    constexpr int kRows = 128;  // query rows per workgroup (a block, or a pair of 64-token blocks)
    using S = AttnShape<D, kRows, kKs, kNbuf>;
    uint16_t* vt = reinterpret_cast<uint16_t*>(base);
    hipLaunchKernelGGL((vt_kernel<D, B>), dim3(p.nb, p.heads), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(v), head_active, vt, p.tokens, p.nb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int units = kPairs ? (p.nb + 1) / 2 : p.nb;
    const HeadGroups hg = head_groups(p, units);
    int* perm = reinterpret_cast<int*>(base + w.perm_off);
    hipLaunchKernelGGL(order_kernel, dim3(hg.ng), dim3(256), 0, stream, ccount, head_active, perm, p.heads, p.nb,
                       units, hg.ng, hg.per_xcd, p.nb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int grid = 8 * hg.per_xcd * hg.ng;
    hipLaunchKernelGGL((attn_bf16_kernel<D, kRows, kKs, kNbuf, false, B>), dim3(grid), dim3(S::kThreads), 0,
                       stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), vt, ccount,
                       clist, head_active, perm, kPairs ? pairs : nullptr, static_cast<const uint16_t*>(part),
                       part_lse, static_cast<uint16_t*>(out), lse, p.heads, p.tokens, p.nb, sl2, p.tokens, p.nb * B,
                       p.nb, hg.ng, hg.per_xcd);
  } else {
    hipLaunchKernelGGL((attn_f32_kernel<D, B>), dim3(p.heads * p.nb), dim3(2 * B), 0, stream,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), ccount, clist, head_active,
                       static_cast<const float*>(part), part_lse, static_cast<float*>(out), lse, p.tokens, p.nb,
                       sl2, p.tokens, p.nb);
  }
  return hipGetLastError();
}


// ------------------------------------------------------------ clusters as key blocks
// Keys of cluster j sit at [pstart_j, pstart_j + 32 * ceil(size_j / 32)) of a
// padded per-head layout, in the order rsa_kmeans sorted them (order), with
// zero keys and values in the padding; every 32-key sub-tile of the layout
// lies inside one cluster.

// Per head: pstart (exclusive sum of the padded sizes) and ostart (exclusive
// sum of the sizes: where the cluster starts in `order`), and the sizes as
// used (csize): each clamped to [0, N - ostart] so that the layout stays
// inside its buffers whatever the caller passes.
__global__ __launch_bounds__(256) void cl_scan_kernel(const int* __restrict__ sizes, int* __restrict__ pstart,
                                                      int* __restrict__ ostart, int* __restrict__ csize, int NB,
                                                      int N) {
  constexpr int kPer = kMaxNB / 256;
  __shared__ int2 part[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int* sz = sizes + static_cast<size_t>(h) * NB;
  // pass 1: unclamped key counts per thread's clusters (64-bit: any input)
  long long local = 0;
  for (int e = 0; e < kPer; ++e) {
    const int j = tid * kPer + e;
    if (j < NB) local += max(sz[j], 0);
  }
  __shared__ long long opart[256];
  opart[tid] = local;
  __syncthreads();
  if (tid == 0) {
    long long run = 0;
    for (int i = 0; i < 256; ++i) {
      const long long v = opart[i];
      opart[i] = run;
      run += v;
    }
  }
  __syncthreads();
  // pass 2: clamp against the keys left, then the padded starts
  long long orun = opart[tid];
  int plocal = 0;
  for (int e = 0; e < kPer; ++e) {
    const int j = tid * kPer + e;
    if (j < NB) {
      const long long left = orun < N ? N - orun : 0;
      const int n = static_cast<int>(min(static_cast<long long>(max(sz[j], 0)), left));
      plocal += (n + 31) & ~31;
      orun += max(sz[j], 0);
    }
  }
  part[tid] = make_int2(plocal, 0);
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int v = part[i].x;
      part[i].x = run;
      run += v;
    }
  }
  __syncthreads();
  int prun = part[tid].x;
  orun = opart[tid];
  for (int e = 0; e < kPer; ++e) {
    const int j = tid * kPer + e;
    if (j < NB) {
      const long long left = orun < N ? N - orun : 0;
      const int n = static_cast<int>(min(static_cast<long long>(max(sz[j], 0)), left));
      const size_t o = static_cast<size_t>(h) * NB + j;
      pstart[o] = prun;
      ostart[o] = static_cast<int>(min(orun, static_cast<long long>(N)));
      csize[o] = n;
      prun += (n + 31) & ~31;
      orun += max(sz[j], 0);
    }
  }
}

// One workgroup per (32-key sub-tile of the padded layout, head): K rows
// into the padded layout and V^T columns (vt_pos order inside every 16 keys,
// as the attention kernel reads them) through an LDS tile.  The sub-tile's
// cluster is the last j with pstart[j] <= its first key (an empty cluster
// shares its start with the next one); sub-tiles past the last cluster are
// left alone (no table entry names them).  Per sub-tile rather than per
// cluster, so the largest clusters do not set the time.
template <int D>
__global__ __launch_bounds__(256) void cl_gather_bf16_kernel(const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             const int* __restrict__ sizes,
                                                             const int* __restrict__ order,
                                                             const int* __restrict__ pstart,
                                                             const int* __restrict__ ostart,
                                                             uint16_t* __restrict__ kp, uint16_t* __restrict__ vtp,
                                                             int N, int NB, int Np) {
  __shared__ uint16_t tile[32][D + 2];
  const int t = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int key0 = 32 * t;
  const int* ps_h = pstart + static_cast<size_t>(h) * NB;
  // last j with ps_h[j] <= key0 (ps_h is non-decreasing, ps_h[0] = 0)
  int lo = 0, hi = NB - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ps_h[mid] <= key0) lo = mid;
    else hi = mid - 1;
  }
  const size_t row = static_cast<size_t>(h) * NB + lo;
  const int n = sizes[row];
  const int s0 = key0 - ps_h[lo];  // first key of the sub-tile inside the cluster
  if (n <= 0 || s0 >= ((n + 31) & ~31)) return;
  const int* ord = order + static_cast<size_t>(h) * N + ostart[row];
  for (int c = tid; c < 32 * D / 8; c += 256) {
    const int r = c / (D / 8), c8 = c % (D / 8);
    const int tok = s0 + r < n ? ord[s0 + r] : -1;
    u32x4 kx = u32x4{0, 0, 0, 0}, vx = u32x4{0, 0, 0, 0};
    if (static_cast<unsigned>(tok) < static_cast<unsigned>(N)) {  // padding, or an invalid id: zeros
      const size_t g = (static_cast<size_t>(h) * N + tok) * D + c8 * 8;
      kx = *reinterpret_cast<const u32x4*>(k + g);
      vx = *reinterpret_cast<const u32x4*>(v + g);
    }
    *reinterpret_cast<u32x4*>(kp + (static_cast<size_t>(h) * Np + key0 + r) * D + c8 * 8) = kx;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[r][c8 * 8 + 2 * e] = static_cast<uint16_t>(vx[e] & 0xffffu);
      tile[r][c8 * 8 + 2 * e + 1] = static_cast<uint16_t>(vx[e] >> 16);
    }
  }
  __syncthreads();
  for (int c = tid; c < D * 4; c += 256) {
    const int d = c / 4, p8 = c % 4;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo16 = tile[vt_pos(8 * p8 + 2 * e)][d];
      const uint32_t hi16 = tile[vt_pos(8 * p8 + 2 * e + 1)][d];
      o[e] = lo16 | (hi16 << 16);
    }
    *reinterpret_cast<u32x4*>(vtp + (static_cast<size_t>(h) * D + d) * Np + key0 + 8 * p8) = o;
  }
}

// fp32: K and V rows into the padded layout, row-major.
template <int D>
__global__ __launch_bounds__(256) void cl_gather_f32_kernel(const float* __restrict__ k, const float* __restrict__ v,
                                                            const int* __restrict__ sizes,
                                                            const int* __restrict__ order,
                                                            const int* __restrict__ pstart,
                                                            const int* __restrict__ ostart, float* __restrict__ kp,
                                                            float* __restrict__ vp, int N, int NB, int Np) {
  const int j = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const size_t row = static_cast<size_t>(h) * NB + j;
  const int n = sizes[row];
  if (n <= 0) return;
  const int ps = pstart[row], npad = (n + 31) & ~31;
  const int* ord = order + static_cast<size_t>(h) * N + ostart[row];
  for (int c = tid; c < npad * D / 4; c += 256) {
    const int r = c / (D / 4), c4 = (c % (D / 4)) * 4;
    const int tok = r < n ? ord[r] : -1;
    f32x4 kx = f32x4{0.f, 0.f, 0.f, 0.f}, vx = f32x4{0.f, 0.f, 0.f, 0.f};
    if (static_cast<unsigned>(tok) < static_cast<unsigned>(N)) {
      const size_t g = (static_cast<size_t>(h) * N + tok) * D + c4;
      kx = *reinterpret_cast<const f32x4*>(k + g);
      vx = *reinterpret_cast<const f32x4*>(v + g);
    }
    const size_t o = (static_cast<size_t>(h) * Np + ps + r) * D + c4;
    *reinterpret_cast<f32x4*>(kp + o) = kx;
    *reinterpret_cast<f32x4*>(vp + o) = vx;
  }
}

// Inclusive prefix sum over the 256 threads of a workgroup (wave scans, then
// the four wave totals); `wsum` is LDS scratch of 4 ints.
__device__ __forceinline__ int block_scan_256(int x, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? wsum[w] : 0;
    all += wsum[w];
  }
  __syncthreads();
  *total = all;
  return x + before;
}

// Sub-tile table of one row (query block I, head h): the row's listed
// clusters as a set (as canon_kernel reads lists), ascending, empty ones
// dropped; cluster j contributes ceil(size_j / 32) entries
// pstart_j + 32 s + (real keys of sub-tile s) - 1.
__global__ __launch_bounds__(256) void cl_table_kernel(const int* __restrict__ counts,
                                                       const int* __restrict__ block_idx,
                                                       const int* __restrict__ sizes,
                                                       const int* __restrict__ pstart, int* __restrict__ tcount,
                                                       int* __restrict__ table, int NB, int stride) {
  __shared__ uint8_t mark[kMaxNB];
  __shared__ int wsum[4];
  const int I = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const size_t row = static_cast<size_t>(h) * NB + I;
  for (int e = tid; e < NB; e += 256) mark[e] = 0;
  __syncthreads();
  const int c = min(max(counts[row], 0), NB);
  for (int t = tid; t < c; t += 256) {
    const int j = block_idx[row * NB + t];
    if (static_cast<unsigned>(j) < static_cast<unsigned>(NB)) mark[j] = 1;
  }
  __syncthreads();
  int* out = table + row * stride;
  int base = 0;
  for (int r0 = 0; r0 < NB; r0 += 256) {
    const int j = r0 + tid;
    const int n = j < NB && mark[j] ? sizes[static_cast<size_t>(h) * NB + j] : 0;
    const int w = n > 0 ? (n + 31) >> 5 : 0;
    int tot;
    const int incl = block_scan_256(w, wsum, &tot);
    if (w > 0) {
      const int ps = pstart[static_cast<size_t>(h) * NB + j];
      int* dst = out + base + incl - w;
      for (int s = 0; s < w; ++s) dst[s] = ps + 32 * s + (min(32, n - 32 * s) - 1);
    }
    base += tot;
  }
  if (tid == 0) tcount[row] = base;
}

struct ClAttnWs {
  size_t kp_off, vp_off, pstart_off, ostart_off, csize_off, tcount_off, table_off, perm_off, total;
  int Np, stride;
};

ClAttnWs cl_attn_ws_layout(const Problem& p) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  ClAttnWs w;
  // every cluster padded to whole 32-key sub-tiles: at most 31 * NB extra keys
  w.Np = (p.tokens + 31 * p.nb + 31) / 32 * 32;
  w.stride = w.Np / 32;  // sub-tiles per row at most
  const size_t es = p.dtype == 0 ? 2 : 4;
  const size_t kv = al(es * p.heads * static_cast<size_t>(w.Np) * p.head_dim);
  const size_t rows = static_cast<size_t>(p.heads) * p.nb;
  w.kp_off = 0;
  w.vp_off = kv;
  w.pstart_off = 2 * kv;
  w.ostart_off = w.pstart_off + al(4 * rows);
  w.csize_off = w.ostart_off + al(4 * rows);
  w.tcount_off = w.csize_off + al(4 * rows);
  w.table_off = w.tcount_off + al(4 * rows);
  w.perm_off = w.table_off + al(4 * rows * w.stride);
  // dispatch order (bf16 path): per head group 8 eighths of its query blocks
  const HeadGroups hg = head_groups(p, p.nb);
  w.total = w.perm_off + (p.dtype == 0 ? al(4 * 8 * static_cast<size_t>(hg.ng) * hg.per_xcd) : 0);
  return w;
}

template <int D, int B>
hipError_t launch_cluster_attn_t(const Problem& p, const void* q, const void* k, const void* v, const int* sizes,
                                 const int* order, const int* counts, const int* idx, void* out, float* lse,
                                 void* ws, hipStream_t stream) {
  const float sl2 = p.scale * kLog2e;
  const ClAttnWs w = cl_attn_ws_layout(p);
  char* base = static_cast<char*>(ws);
  int* pstart = reinterpret_cast<int*>(base + w.pstart_off);
  int* ostart = reinterpret_cast<int*>(base + w.ostart_off);
  int* csize = reinterpret_cast<int*>(base + w.csize_off);
  int* tcount = reinterpret_cast<int*>(base + w.tcount_off);
  int* table = reinterpret_cast<int*>(base + w.table_off);
  hipLaunchKernelGGL(cl_scan_kernel, dim3(p.heads), dim3(256), 0, stream, sizes, pstart, ostart, csize, p.nb,
                     p.tokens);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.dtype == 0)
    hipLaunchKernelGGL((cl_gather_bf16_kernel<D>), dim3(w.stride, p.heads), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), csize, order, pstart,
                       ostart, reinterpret_cast<uint16_t*>(base + w.kp_off),
                       reinterpret_cast<uint16_t*>(base + w.vp_off), p.tokens, p.nb, w.Np);
  else
    hipLaunchKernelGGL((cl_gather_f32_kernel<D>), dim3(p.nb, p.heads), dim3(256), 0, stream,
                       static_cast<const float*>(k), static_cast<const float*>(v), csize, order, pstart, ostart,
                       reinterpret_cast<float*>(base + w.kp_off), reinterpret_cast<float*>(base + w.vp_off),
                       p.tokens, p.nb, w.Np);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(cl_table_kernel, dim3(p.nb, p.heads), dim3(256), 0, stream, counts, idx, csize, pstart,
                     tcount, table, p.nb, w.stride);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.dtype == 0) {
    // three slots, three workgroups per CU (the sub-tile masks are built in
    // scalar registers, so they fit the three-wave register budget)
    constexpr int kNbuf = 3;
    using S = AttnShape<D, B, 32, kNbuf>;
    const HeadGroups hg = head_groups(p, p.nb);
    int* perm = reinterpret_cast<int*>(base + w.perm_off);
    // balanced by sub-tile count (lengths past kMaxNB share the top rank)
    hipLaunchKernelGGL(order_kernel, dim3(hg.ng), dim3(256), 0, stream, tcount, nullptr, perm, p.heads, p.nb,
                       p.nb, hg.ng, hg.per_xcd, std::min(w.stride, kMaxNB));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int grid = 8 * hg.per_xcd * hg.ng;
    hipLaunchKernelGGL((attn_bf16_kernel<D, B, 32, kNbuf, true>), dim3(grid), dim3(S::kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(base + w.kp_off),
                       reinterpret_cast<const uint16_t*>(base + w.vp_off), tcount, table, nullptr, perm, nullptr,
                       nullptr, nullptr, static_cast<uint16_t*>(out), lse, p.heads, p.tokens, p.nb, sl2, w.Np, w.Np, w.stride,
                       hg.ng, hg.per_xcd);
  } else {
    hipLaunchKernelGGL((attn_f32_kernel<D, B, true>), dim3(p.heads * p.nb), dim3(2 * B), 0, stream,
                       static_cast<const float*>(q), reinterpret_cast<const float*>(base + w.kp_off),
                       reinterpret_cast<const float*>(base + w.vp_off), tcount, table, nullptr, nullptr, nullptr,
                       static_cast<float*>(out), lse, p.tokens, p.nb, sl2, w.Np, w.stride);
  }
  return hipGetLastError();
}
}  // namespace

size_t attn_ws_bytes(const Problem& p) { return attn_ws_layout(p).total; }

hipError_t launch_attention(const Problem& p, const void* q, const void* k, const void* v,
                            const int* counts, const int* idx, const uint8_t* head_active,
                            int complement, const void* part, const float* part_lse, void* out, float* lse,
                            void* ws, hipStream_t stream) {
  auto go = [&](auto fn) {
    return fn(p, q, k, v, counts, idx, head_active, complement, part, part_lse, out, lse, ws, stream);
  };
  if (p.head_dim == 128 && p.block == 128) return go(launch_attn_t<128, 128>);
  if (p.head_dim == 128 && p.block == 64) return go(launch_attn_t<128, 64>);
  if (p.head_dim == 64 && p.block == 128) return go(launch_attn_t<64, 128>);
  return go(launch_attn_t<64, 64>);
}

size_t cluster_attn_ws_bytes(const Problem& p) { return cl_attn_ws_layout(p).total; }

hipError_t launch_cluster_attention(const Problem& p, const void* q, const void* k, const void* v,
                                    const int* sizes, const int* order, const int* counts, const int* idx,
                                    void* out, float* lse, void* ws, hipStream_t stream) {
  auto go = [&](auto fn) { return fn(p, q, k, v, sizes, order, counts, idx, out, lse, ws, stream); };
  if (p.head_dim == 128 && p.block == 128) return go(launch_cluster_attn_t<128, 128>);
  if (p.head_dim == 128 && p.block == 64) return go(launch_cluster_attn_t<128, 64>);
  if (p.head_dim == 64 && p.block == 128) return go(launch_cluster_attn_t<64, 128>);
  return go(launch_cluster_attn_t<64, 64>);
}

}  // namespace rsa
