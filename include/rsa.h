/*
 * librsa - block-sparse attention scoring for video diffusion transformers,
 * hand-written HIP kernels for gfx950 (MI355X).
 *
 * Four calls make the hot path.  Each is defined by the pages it cites:
 *
 *   rsa_score_blocks      PARK's block scorer (PARK: Accurate Block Retrieval
 *                         for Sparse Attention in Video Diffusion Transformers,
 *                         Abstract): pool each key block to its mean, take a
 *                         softmax of every query over the pooled key blocks,
 *                         average those distributions within each query block.
 *   rsa_select_topp       online top-p block selection with a per-head
 *                         threshold (HASTE: Training-Free Video Diffusion
 *                         Acceleration via Head-Wise Adaptive Sparse
 *                         Attention, Abstract; HEART: Exploiting Head
 *                         Heterogeneity in Sparse Attention for Video
 *                         Diffusion, Abstract).
 *   rsa_mask_drift        Temporal Mask Reuse's per-head query-key drift
 *                         signal and refresh decision (HEART, Abstract; HASTE,
 *                         Abstract); with RAPID (Reusing Attention Sparsity
 *                         with Inter-step Adaptation for Efficient Video
 *                         Diffusion, Abstract) it lets cached scores and masks
 *                         be reused across denoising steps.
 *   rsa_block_sparse_attn attention computed only inside the retrieved key
 *                         blocks (PARK, Abstract).
 *
 * Two more calls measure block retrieval accuracy, PARK's stated goal
 * (Abstract): rsa_dense_block_mass gives each query block's exact dense
 * attention mass per key block, and rsa_score_blocks_pooled the comparison
 * scorer that averages the queries before the softmax.
 *
 * Three calls carry the cached correction of RECAP (Reciprocal Sparse
 * Attention and Hierarchical Caching for Efficient Video Diffusion, Abstract):
 * rsa_attn_omitted computes, at a mask refresh, the attention over the key
 * blocks each list leaves out, to be cached; rsa_attn_merge joins a fresh
 * sparse output with that cached part, weighted by their log-sum-exps; and
 * rsa_block_sparse_attn_corrected does both of the last in one pass.
 *
 * Common conventions
 * ------------------
 * Tensors q, k, v, out are [heads, tokens, head_dim], row-major, tokens in
 * (frame, height, width) raster order.  A block is a run of `block`
 * consecutive tokens; query blocks and key blocks share one partition of
 * NB = ceil(tokens / block) blocks and the last block may be shorter.
 *
 * Pointers are device pointers (HBM) unless a comment says "host".  The
 * caller owns every buffer, including the workspace; the library never
 * allocates, frees or keeps a device pointer and holds no global state, so
 * calls on different streams do not interfere.  Every call only enqueues
 * kernels on `stream` and returns without synchronising.
 *
 * Errors: arguments are validated on the host before anything is enqueued;
 * on any error nothing is launched and no output is touched.  The status is
 * the return value; nothing is printed, nothing aborts and no exception
 * crosses the ABI.  A launch failure reported by the HIP runtime returns
 * RSA_ERR_HIP; device faults surface at the caller's next synchronisation.
 *
 * Results are bitwise deterministic for identical inputs (fixed reduction
 * orders; no floating-point atomics).
 */
#ifndef RSA_H
#define RSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RSA_VERSION 10000 /* 1.0.0 */

/* Element type of q, k, v, the drift snapshots and the attention output. */
typedef enum { RSA_BF16 = 0, RSA_FP32 = 1 } rsa_dtype;

typedef enum {
  RSA_OK = 0,
  RSA_ERR_NULL = 1,      /* a required pointer is NULL */
  RSA_ERR_SHAPE = 2,     /* sizes out of range or inconsistent */
  RSA_ERR_DTYPE = 3,     /* unknown dtype */
  RSA_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned */
  RSA_ERR_WORKSPACE = 5, /* workspace missing, too small or not 256-byte aligned */
  RSA_ERR_HIP = 6,       /* the HIP runtime rejected a launch */
  RSA_ERR_ARG = 7        /* a scalar argument is out of range (e.g. NaN threshold) */
} rsa_status;

typedef enum {
  RSA_OP_SCORE = 0,
  RSA_OP_SELECT = 1,
  RSA_OP_DRIFT = 2,
  RSA_OP_ATTN = 3,
  RSA_OP_POOLED = 4, /* rsa_score_blocks_pooled */
  RSA_OP_GRAM = 5,   /* rsa_query_gram */
  RSA_OP_KMEANS = 6, /* rsa_kmeans */
  RSA_OP_CLUSTER_ATTN = 7 /* rsa_cluster_attn */
} rsa_op;

/*
 * Problem descriptor (host struct, read during the call only).
 *   heads >= 1; tokens == grid_f * grid_h * grid_w (each >= 1);
 *   head_dim in {64, 128}; block in {64, 128}; NB = ceil(tokens/block) <= 4096;
 *   dtype: rsa_dtype;
 *   softmax_scale: logit scale shared by scoring and attention; a value <= 0
 *   (or NaN) means 1/sqrt(head_dim); +inf is rejected (RSA_ERR_ARG).
 */
typedef struct {
  int32_t heads;
  int32_t tokens;
  int32_t head_dim;
  int32_t grid_f;
  int32_t grid_h;
  int32_t grid_w;
  int32_t block;
  int32_t dtype;
  float softmax_scale;
} rsa_problem;

/*
 * Bytes of workspace `op` needs for `p` (0 when none).  Returns 0 for an
 * invalid problem as well; the compute calls report that case themselves.
 */
size_t rsa_workspace_bytes(const rsa_problem* p, int32_t op);

/* Static string naming a status code ("RSA_OK", ...); "unknown" otherwise. */
const char* rsa_status_str(int32_t status);

/* RSA_VERSION of the built library. */
int32_t rsa_version(void);

/*
 * PARK block scores (PARK, Abstract; the Summary calls it keeping each
 * query's own information).
 *
 *   For head h, key block J with b_J tokens:  Kbar[h,J] = mean of its keys.
 *   For query i:  P[i,J] = softmax over J of  scale * <q_i, Kbar[h,J]>.
 *   For query block I with b_I queries:  scores[h,I,J] = mean over i in I of P[i,J].
 *
 * q, k: [heads, tokens, head_dim] of `dtype`, 16-byte aligned.
 * head_active: [heads] u8 or NULL (= all heads).  Heads with 0 are skipped and
 *   their rows of `scores` are left as they are (a cached mask's scores).
 * scores: [heads, NB, NB] fp32 output; every row sums to 1 up to rounding.
 * ws / ws_bytes: workspace of at least rsa_workspace_bytes(p, RSA_OP_SCORE)
 *   bytes, 256-byte aligned; its contents on entry do not matter.
 * Logits are formed to about fp32 accuracy (a 2-term fp16 split of the pooled
 * keys on the matrix cores), the softmax and the query-block means in fp32.
 */
rsa_status rsa_score_blocks(const rsa_problem* p, const void* q, const void* k,
                            const uint8_t* head_active, float* scores,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Top-p block selection (HASTE, Abstract: online top-p; HEART, Abstract:
 * one threshold per head under a global sparsity budget).
 *
 *   Row (h,I): key blocks ordered by score descending, equal scores by index
 *   ascending; running mass in fp64; keep the smallest prefix whose mass is
 *   >= top_p[h] (at least one block; top_p[h] >= 1 keeps all NB; no prefix
 *   reaching top_p[h], e.g. NaN, keeps all NB); then at most max_blocks
 *   blocks when max_blocks > 0.
 *
 * scores: [heads, NB, NB] fp32 (any non-negative values; rows need not sum to 1).
 * top_p: [heads] fp32 thresholds (device).
 * max_blocks: >= 0; 0 = no per-row cap.
 * head_active: [heads] u8 or NULL; rows of inactive heads are left untouched.
 * mask: [heads, NB, NB] u8 output, 1 = block kept.
 * counts: [heads, NB] int32 output, blocks kept per row.
 * block_idx: [heads, NB, NB] int32 output; row (h,I) lists its kept key
 *   blocks in ascending order in its first counts[h,I] entries; the other
 *   entries of the row are not written.
 * density: [heads] fp32 output or NULL: kept pairs / NB^2 per head, recomputed
 *   from all rows of `counts` (cached rows of inactive heads included).
 * ws / ws_bytes: unused (rsa_workspace_bytes returns 0); may be NULL / 0.
 */
rsa_status rsa_select_topp(const rsa_problem* p, const float* scores, const float* top_p,
                           int32_t max_blocks, const uint8_t* head_active,
                           uint8_t* mask, int32_t* counts, int32_t* block_idx,
                           float* density, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Per-head query-key drift and refresh flags (HEART, Abstract: a head's
 * cached mask is recomputed only once its drift is above tau; HASTE,
 * Abstract: the drift decides when mask prediction may be skipped).
 *
 *   drift[h] = sqrt(|Q_h - Qref_h|^2 + |K_h - Kref_h|^2) / sqrt(|Qref_h|^2 + |Kref_h|^2)
 *   refresh[h] = drift[h] > threshold  (strict; an all-zero snapshot gives
 *   drift 0 if nothing changed and +inf otherwise)
 *
 * Sums of squares are accumulated in fp64 in a fixed order; the comparison is
 * done in fp64 before drift is rounded to fp32.
 * q, k: current [heads, tokens, head_dim] of `dtype`.
 * q_ref, k_ref: snapshots, same shape and dtype.  When update_ref != 0 the
 *   snapshot of every refreshed head is overwritten with its current q, k
 *   (after the drift is measured), so the next call measures against the
 *   step at which that head's mask was recomputed.
 * threshold: finite or +inf; NaN is rejected (RSA_ERR_ARG).
 * drift: [heads] fp32 output; refresh: [heads] u8 output (pass it as
 *   head_active to rsa_score_blocks / rsa_select_topp).
 * ws / ws_bytes: at least rsa_workspace_bytes(p, RSA_OP_DRIFT), 256-byte aligned.
 */
rsa_status rsa_mask_drift(const rsa_problem* p, const void* q, const void* k,
                          void* q_ref, void* k_ref, float threshold, int32_t update_ref,
                          float* drift, uint8_t* refresh,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Block-sparse attention (PARK, Abstract: attention computed only inside the
 * retrieved blocks).  For query i of block I of head h, the visible keys are
 * the tokens of the key blocks block_idx[h,I,0..counts[h,I]); the softmax is
 * normalised over those keys only:
 *
 *   out[h,i,:] = sum_t softmax_t(scale * <q_i, k_t>) v_t,
 *   lse[h,i]   = log sum_t exp(scale * <q_i, k_t>)   (natural log).
 *
 * q, k, v: [heads, tokens, head_dim] of `dtype`, 16-byte aligned.
 * counts: [heads, NB] int32; block_idx: [heads, NB, NB] int32 (e.g. the
 *   output of rsa_select_topp, fresh or cached).  Row (h, I) lists the key
 *   blocks block_idx[h,I,0..counts[h,I]) in any order; a block listed twice
 *   counts once, counts are clamped to [0, NB] and entries outside [0, NB)
 *   are ignored.  A row with no valid entry gives out = 0 and lse = -inf.
 * out: [heads, tokens, head_dim] of `dtype` (bf16 rounded to nearest even).
 * lse: [heads, tokens] fp32 output or NULL.
 * bf16 inputs: bf16 matrix-core products with fp32 accumulation and an fp32
 *   online softmax; fp32 inputs: fp32 arithmetic throughout.
 * ws / ws_bytes: at least rsa_workspace_bytes(p, RSA_OP_ATTN) bytes, 256-byte
 *   aligned, each part rounded up to 256 bytes: (bf16 only) v re-laid out
 *   key-major for the matrix cores, heads * head_dim * NB * block * 2 bytes;
 *   then every row's list in canonical form (ascending, no repeats, no
 *   invalid entries; bf16 with block 64: per pair of query blocks the union
 *   of their lists, with membership bits): counts, heads * NB * 4 bytes, and
 *   lists, heads * NB * NB * 4 bytes; then (bf16 only) the workgroup
 *   dispatch order, 4 bytes per query block (per pair of 64-token blocks)
 *   plus padding to whole eighths of each head group; then (bf16 with block
 *   64 only) the pairing of query blocks: the pairs, heads * ceil(NB/2) * 8
 *   bytes, each row's set as bits, heads * NB * ceil(NB/64) * 8 bytes, and
 *   the overlap of each block with its 32 successors, heads * NB * 64 bytes.
 * Non-finite values in q, k or v give undefined results.
 */
rsa_status rsa_block_sparse_attn(const rsa_problem* p, const void* q, const void* k,
                                 const void* v, const int32_t* counts,
                                 const int32_t* block_idx, void* out, float* lse,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Dense block mass: the retrieval-accuracy yardstick (PARK, Abstract: block
 * retrieval accuracy).  For query block I of head h, with the softmax taken
 * over all N keys,
 *
 *   mass[h,I,J] = (1/b_I) sum_{i in I} sum_{t in J} softmax_t(scale * <q_i, k_t>),
 *
 * the mean over I's queries of the attention mass on key block J; every row
 * sums to 1.  q, k: [heads, tokens, head_dim] of `dtype`, 16-byte aligned.
 * mass: [heads, NB, NB] fp32, 16-byte aligned.  No workspace.  Costs two
 * dense Q K^T passes (bf16 matrix cores, fp32 exponentials, fp64 row
 * normalisers); meant for measurement, not for the sparse step.
 */
rsa_status rsa_dense_block_mass(const rsa_problem* p, const void* q, const void* k, float* mass,
                                hipStream_t stream);

/*
 * Query-pooled block scores: the scorer PARK's abstract argues against
 * (averaging a block's queries before the softmax loses their individual
 * preferences), kept as the comparison for retrieval accuracy:
 *
 *   pooled[h,I,J] = softmax_J(scale * <qbar_I, kbar_J>),
 *
 * qbar_I and kbar_J the block means (over the tokens each block holds).
 * Rows sum to 1.  q, k as in rsa_score_blocks; pooled: [heads, NB, NB] fp32.
 * ws / ws_bytes: at least rsa_workspace_bytes(p, RSA_OP_POOLED) bytes,
 * 256-byte aligned (pooled q and k, [heads, NB, head_dim] fp32 each, and a
 * block-maximum scratch).  Block means are fp64 sums rounded once to fp32;
 * logits and the softmax are fp64.
 */
rsa_status rsa_score_blocks_pooled(const rsa_problem* p, const void* q, const void* k,
                                   float* pooled, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Attention over the omitted key blocks (RECAP, Abstract: a dense refinement,
 * computed at refresh time and cached, for the interactions that sparse
 * attention leaves out).  For query i of block I of head h, the visible keys
 * are the tokens of every key block that row (h, I) does NOT list:
 *
 *   out[h,i,:] = sum_{t omitted} softmax_t(scale * <q_i, k_t>) v_t,
 *   lse[h,i]   = log sum_{t omitted} exp(scale * <q_i, k_t>).
 *
 * A row that lists every block has nothing omitted: out = 0, lse = -inf.
 * Lists are read as in rsa_block_sparse_attn (any order, repeats once,
 * counts clamped to [0, NB], invalid entries ignored).  Joined with the
 * sparse pass over the same list by rsa_attn_merge it gives dense attention.
 * head_active: [heads] u8 or NULL (all heads).  Heads with head_active[h] == 0
 * are skipped: their rows of out and lse keep what they held, so the outputs
 * can be a per-head cache refreshed with rsa_mask_drift's refresh flags.
 * q, k, v, out: as in rsa_block_sparse_attn; lse: [heads, tokens] fp32
 * output (required).  ws / ws_bytes: at least rsa_workspace_bytes(p,
 * RSA_OP_ATTN), laid out as for rsa_block_sparse_attn (the canonical lists
 * hold the omitted blocks).
 * Non-finite values in q, k or v give undefined results.
 */
rsa_status rsa_attn_omitted(const rsa_problem* p, const void* q, const void* k, const void* v,
                            const int32_t* counts, const int32_t* block_idx,
                            const uint8_t* head_active, void* out, float* lse, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * Join two attentions over disjoint key sets, in place (RECAP, Abstract: the
 * cached refinement corrects each fresh sparse output, and the fresh sparse
 * statistics set how much the ageing cached part counts).  Per row r of the
 * heads * tokens rows, with L = log(exp(lse[r]) + exp(part_lse[r])):
 *
 *   out[r,:] <- exp(lse[r] - L) out[r,:] + exp(part_lse[r] - L) part_out[r,:],
 *   lse[r]   <- L.
 *
 * A part with lse = -inf has weight 0; both -inf give out = 0, lse = -inf.
 * out, part_out: [heads, tokens, head_dim] of `dtype`, 16-byte aligned (bf16
 * results rounded to nearest even; fp32 arithmetic).  lse, part_lse:
 * [heads, tokens] fp32.  No workspace.  Typical use: out/lse from
 * rsa_block_sparse_attn on the current step, part_out/part_lse the cache
 * rsa_attn_omitted wrote when the head's mask was last refreshed.
 */
rsa_status rsa_attn_merge(const rsa_problem* p, void* out, float* lse, const void* part_out,
                          const float* part_lse, hipStream_t stream);

/*
 * Corrected block-sparse attention: rsa_block_sparse_attn over the current
 * lists joined, inside the same kernel, with a cached attention over the
 * complementary keys (RECAP, Abstract, as rsa_attn_merge):
 *
 *   out[r,:] = exp(lse_s[r] - L) O_s[r,:] + exp(part_lse[r] - L) part_out[r,:],
 *   lse[r]   = L = log(exp(lse_s[r]) + exp(part_lse[r])),
 *
 * O_s, lse_s the sparse attention of row r.  Equal to rsa_block_sparse_attn
 * followed by rsa_attn_merge, except that O_s enters in fp32 rather than
 * rounded to the output type first, and no separate pass reads and writes
 * the outputs again.  Arguments as in rsa_block_sparse_attn and
 * rsa_attn_merge; part_out ([heads, tokens, head_dim] of `dtype`, 16-byte
 * aligned) and part_lse ([heads, tokens] fp32) are read only; lse is
 * required.  out may be part_out and lse may be part_lse (in place: every
 * element is read before the same thread writes it).  ws / ws_bytes: as for
 * rsa_block_sparse_attn (RSA_OP_ATTN).
 * Non-finite values in q, k or v give undefined results.
 */
rsa_status rsa_block_sparse_attn_corrected(const rsa_problem* p, const void* q, const void* k, const void* v,
                                           const int32_t* counts, const int32_t* block_idx, const void* part_out,
                                           const float* part_lse, void* out, float* lse, void* ws,
                                           size_t ws_bytes, hipStream_t stream);

/*
 * Gram matrix of the current queries (PARK, Abstract: the keys are transformed
 * with information from the current queries before they are clustered):
 *
 *   gram[h] = (1/N) sum_i q_i q_i^T,   [heads, head_dim, head_dim] fp32.
 *
 * It defines the metric of rsa_kmeans: (k - c)^T gram (k - c) is the mean over
 * the current queries of the squared difference of their scores <q_i, k> and
 * <q_i, c>.  q: [heads, tokens, head_dim] of `dtype`, 16-byte aligned; gram
 * 16-byte aligned.  bf16: exact products on the matrix cores, fp32 sums per
 * chunk of 2048 tokens, chunks added in fp64 in a fixed order; fp32: fp64
 * sums.  ws / ws_bytes: at least rsa_workspace_bytes(p, RSA_OP_GRAM) bytes,
 * 256-byte aligned (the chunks' partial sums; 0 bytes for fp32).
 */
rsa_status rsa_query_gram(const rsa_problem* p, const void* q, float* gram, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * Lloyd k-means of each head's keys in the metric of `gram` (PARK, Abstract:
 * keys that receive similar query-key scores are grouped; the clusters are the
 * key blocks).  NB = ceil(tokens / block) clusters.  With init != 0 the
 * centroids first become the means of the contiguous key blocks; otherwise
 * `centroids` holds the starting centroids.  Each of the `iters` iterations
 * (1..1000) assigns every key to the centroid c_j minimising
 * (k - c_j)^T gram (k - c_j) (ties: the lowest j), then moves every non-empty
 * cluster's centroid to the mean of its keys; an empty cluster keeps its
 * centroid.  Outputs, all for the last iteration:
 *   centroids [heads, NB, head_dim] fp32 (in/out), 16-byte aligned;
 *   labels    [heads, tokens] int32: each key's cluster;
 *   sizes     [heads, NB] int32: keys per cluster (0 = empty);
 *   order     [heads, tokens] int32: the keys sorted by (cluster, token), so
 *             cluster j is order[h, off_j .. off_j + sizes[h, j]) with off_j
 *             the sum of the sizes before j.
 * The assignment runs on the matrix cores with 2 gram c_j times a power of two
 * split into two fp16 terms (22 significant bits) and each key as fp16 times
 * its own power of two (exact for bf16), so 2 k.gram c_j carries about fp32
 * accuracy (fp64 products for fp32 keys); the sort is a
 * stable counting sort and the means are fp64 sums rounded once, so results
 * are deterministic.  ws / ws_bytes: at least rsa_workspace_bytes(p,
 * RSA_OP_KMEANS) bytes, 256-byte aligned.
 */
rsa_status rsa_kmeans(const rsa_problem* p, const void* k, const float* gram, int32_t iters, int32_t init,
                      float* centroids, int32_t* labels, int32_t* sizes, int32_t* order, void* ws,
                      size_t ws_bytes, hipStream_t stream);

/*
 * PARK scores with the clusters of rsa_kmeans as key blocks (PARK, Abstract:
 * the clusters' mean representations serve block retrieval).  For query
 * block I (contiguous, as everywhere) and cluster J:
 *
 *   scores[h,I,J] = (1/b_I) sum_{i in I} softmax_J'(scale * <q_i, centroids[h,J']>)[J],
 *
 * the softmax taken over the non-empty clusters J' (sizes[h,J'] > 0); an empty
 * cluster scores 0.  Rows sum to 1, so rsa_select_topp applies unchanged and
 * never needs an empty cluster before every live one.  q as in
 * rsa_score_blocks; centroids [heads, NB, head_dim] fp32 and sizes [heads, NB]
 * int32 as rsa_kmeans writes them; scores [heads, NB, NB] fp32, 16-byte
 * aligned.  Arithmetic as rsa_score_blocks (centroid times scale*log2(e)
 * rounded once to fp32, two fp16 terms on the matrix cores).  ws / ws_bytes:
 * at least rsa_workspace_bytes(p, RSA_OP_SCORE) bytes, 256-byte aligned.
 */
rsa_status rsa_score_clusters(const rsa_problem* p, const void* q, const float* centroids, const int32_t* sizes,
                              float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Attention with the clusters of rsa_kmeans as key blocks (PARK, Abstract:
 * attention computed only inside the retrieved blocks).  Row (h, I) of
 * counts / block_idx lists clusters (e.g. rsa_select_topp on the scores of
 * rsa_score_clusters), read as a set as in rsa_block_sparse_attn; empty
 * clusters add nothing.  For query i of the contiguous query block I the
 * visible keys are the keys of the listed clusters:
 *
 *   out[h,i,:] = sum_{t : labels[h,t] listed} softmax_t(scale * <q_i, k_t>) v_t,
 *
 * and lse as in rsa_block_sparse_attn (a row with no key: out 0, lse -inf).
 * sizes, order: as rsa_kmeans writes them.  Other values give meaningless
 * results but stay inside the buffers: each size is clamped to [0, keys not
 * yet taken by earlier clusters] and token ids outside [0, tokens) read as
 * zero keys.  q, k, v, out, lse as in rsa_block_sparse_attn.  The call gathers k and v into cluster order (each
 * cluster padded with zeros to whole 32-key sub-tiles), turns each row's list
 * into a table of sub-tiles and runs the block-sparse attention kernel over
 * the tables (bf16: matrix cores as rsa_block_sparse_attn; fp32: fp32 FMA).
 * ws / ws_bytes: at least rsa_workspace_bytes(p, RSA_OP_CLUSTER_ATTN) bytes,
 * 256-byte aligned: padded k and v (bf16: v transposed), Np = tokens +
 * 31 * NB rounded up to 32 keys per head; cluster starts (padded and in
 * `order`) and the sizes as used; per-row sub-tile counts and tables of
 * Np / 32 entries; (bf16 only) the workgroup dispatch order, 4 bytes per
 * query block plus padding to whole eighths of each head group.
 * Non-finite values in q, k or v give undefined results.
 */
rsa_status rsa_cluster_attn(const rsa_problem* p, const void* q, const void* k, const void* v, const int32_t* sizes,
                            const int32_t* order, const int32_t* counts, const int32_t* block_idx, void* out,
                            float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * rsa_score_blocks without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same inputs, output, results (bit for
 * bit) and errors as rsa_score_blocks; the workspace is a static device array
 * of RSA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
 * the process ends.  The call allocates nothing: its first call on a device
 * looks up that device's copy of the array (hipGetSymbolAddress) and keeps the
 * address.
 * Errors: RSA_ERR_WORKSPACE when rsa_workspace_bytes(p, RSA_OP_SCORE) exceeds
 * RSA_NOALLOC_SCRATCH_BYTES (64 MiB: e.g. 40 heads x 591 blocks of 128 need
 * 25 MB), RSA_ERR_HIP when the array's address cannot be obtained; otherwise
 * as rsa_score_blocks.
 * All calls on one device share the array: calls that overlap in time on the
 * same device (other streams, other host threads) race and must not be made.
 */
#define RSA_NOALLOC_SCRATCH_BYTES (64u << 20)
rsa_status rsa_score_blocks_noalloc(const rsa_problem* p, const void* q, const void* k,
                                    const uint8_t* head_active, float* scores, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RSA_H */
