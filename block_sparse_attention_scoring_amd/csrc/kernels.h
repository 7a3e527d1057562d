// Internal interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rsa {

constexpr int kMaxClusters = 4096;  // largest number of blocks (and clusters) per sequence

// Validated problem, derived sizes included.
struct Problem {
  int heads, tokens, head_dim, block, nb;
  int dtype;    // 0 = bf16, 1 = fp32
  float scale;  // logit scale actually used
};

// Scoring workspace: pooled keys (fp32, already times scale*log2 e), per
// block max |.|, their 2-term fp16 split (rows padded to a multiple of 32
// with zeros) and the per-head power-of-two unscale factor.
struct ScoreWs {
  float* kt;
  float* bmax;
  _Float16* khi;
  _Float16* klo;
  float* inv_t;
};
constexpr int kScoreRowPad = 32;
size_t score_ws_layout(const Problem& p, ScoreWs* ws, void* base);

constexpr int kDriftGroups = 64;  // partial sums per head
size_t drift_ws_bytes(const Problem& p);

hipError_t launch_scoring(const Problem& p, const void* q, const void* k,
                          const uint8_t* head_active, float* scores, const ScoreWs& ws,
                          hipStream_t stream);
// The same scores with clusters as key blocks: centroids [H, NB, D] fp32 as
// the pooled keys, empty clusters (sizes 0) left out of every softmax.
hipError_t launch_cluster_scoring(const Problem& p, const void* q, const float* cent, const int* sizes,
                                  float* scores, const ScoreWs& ws, hipStream_t stream);
hipError_t launch_select(const Problem& p, const float* scores, const float* top_p,
                         int max_blocks, const uint8_t* head_active, uint8_t* mask,
                         int32_t* counts, int32_t* idx, float* density, hipStream_t stream);
hipError_t launch_drift(const Problem& p, const void* q, const void* k, void* q_ref,
                        void* k_ref, float threshold, int update_ref, float* drift,
                        uint8_t* refresh, void* ws, hipStream_t stream);
// Attention workspace: (bf16) V re-laid out for the matrix cores, then the
// canonical counts and lists.  With `complement` set the attention runs over
// the blocks each row does not list; heads with head_active[h] == 0 (when
// head_active is not NULL) are skipped and their outputs left untouched.
size_t attn_ws_bytes(const Problem& p);
// With part != NULL the result is joined with a cached attention over the
// complementary keys (part, part_lse: [heads, tokens, head_dim] and
// [heads, tokens]) in the epilogue; out may be part.
hipError_t launch_attention(const Problem& p, const void* q, const void* k, const void* v,
                            const int* counts, const int* idx, const uint8_t* head_active,
                            int complement, const void* part, const float* part_lse, void* out, float* lse,
                            void* ws, hipStream_t stream);
// Attention with clusters as key blocks (lists name clusters): K and V are
// gathered into a padded cluster layout, each row's clusters become a table
// of 32-key sub-tiles, and the attention kernels walk the tables.
size_t cluster_attn_ws_bytes(const Problem& p);
hipError_t launch_cluster_attention(const Problem& p, const void* q, const void* k, const void* v,
                                    const int* sizes, const int* order, const int* counts, const int* idx,
                                    void* out, float* lse, void* ws, hipStream_t stream);
// In place: (out, lse) <- attention over the union of the key sets behind
// (out, lse) and (part, part_lse), two disjoint parts.
hipError_t launch_merge(const Problem& p, void* out, float* lse, const void* part,
                        const float* part_lse, hipStream_t stream);

// Block means of x [H, N, D] times `mul`, written as fp32 [H, NB, D] (the
// scoring pool kernel; bmax gets each block's max |.|).
hipError_t launch_block_means(const Problem& p, const void* x, double mul, float* out, float* bmax,
                              hipStream_t stream);
// Retrieval accuracy: dense block mass (no workspace) and the query-pooled
// comparison scorer (workspace: pooled q and k, block maxima).
hipError_t launch_dense_mass(const Problem& p, const void* q, const void* k, float* mass,
                             hipStream_t stream);
size_t pooled_ws_bytes(const Problem& p);
hipError_t launch_pooled_scores(const Problem& p, const void* q, const void* k, float* scores,
                                void* ws, hipStream_t stream);

// Query-aware key clustering: G = Q^T Q / N per head (workspace: per-chunk
// partial sums, bf16 only), and `iters` Lloyd iterations in the metric of G
// (from the contiguous block means when `init` is set).
size_t gram_ws_bytes(const Problem& p);
hipError_t launch_gram(const Problem& p, const void* q, float* gram, void* ws, hipStream_t stream);
size_t kmeans_ws_bytes(const Problem& p);
hipError_t launch_kmeans(const Problem& p, const void* k, const float* gram, int iters, int init, float* cent,
                         int* labels, int* sizes, int* order, void* ws, hipStream_t stream);

}  // namespace rsa
