// C-ABI entry points of librsa: host-side validation, then kernel launches on
// the caller's stream.  Declarations and contracts are in include/rsa.h.
#include <cmath>

#include "rsa.h"
#include "kernels.h"

namespace {

constexpr int kMaxBlocks = rsa::kMaxClusters;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

rsa_status make_problem(const rsa_problem* in, rsa::Problem* out) {
  if (in == nullptr) return RSA_ERR_NULL;
  if (in->dtype != RSA_BF16 && in->dtype != RSA_FP32) return RSA_ERR_DTYPE;
  if (in->heads < 1 || in->tokens < 1 || in->grid_f < 1 || in->grid_h < 1 || in->grid_w < 1)
    return RSA_ERR_SHAPE;
  const long long grid = static_cast<long long>(in->grid_f) * in->grid_h * in->grid_w;
  if (grid != in->tokens) return RSA_ERR_SHAPE;
  if (in->head_dim != 64 && in->head_dim != 128) return RSA_ERR_SHAPE;
  if (in->block != 64 && in->block != 128) return RSA_ERR_SHAPE;
  const int nb = (in->tokens + in->block - 1) / in->block;
  if (nb > kMaxBlocks) return RSA_ERR_SHAPE;
  // element offsets of [heads, tokens, head_dim] and [heads, NB, NB] stay below 2^62
  const long long elems = static_cast<long long>(in->heads) * in->tokens * in->head_dim;
  if (elems > (1ll << 40)) return RSA_ERR_SHAPE;
  const float s = in->softmax_scale;
  if (std::isinf(s) && s > 0) return RSA_ERR_ARG;
  out->heads = in->heads;
  out->tokens = in->tokens;
  out->head_dim = in->head_dim;
  out->block = in->block;
  out->nb = nb;
  out->dtype = in->dtype;
  out->scale = (s > 0.f) ? s : 1.0f / std::sqrt(static_cast<float>(in->head_dim));
  return RSA_OK;
}

rsa_status hip_status(hipError_t e) { return e == hipSuccess ? RSA_OK : RSA_ERR_HIP; }

size_t ws_bytes_for(const rsa::Problem& p, int op) {
  switch (op) {
    case RSA_OP_SCORE: return rsa::score_ws_layout(p, nullptr, nullptr);
    case RSA_OP_DRIFT: return rsa::drift_ws_bytes(p);
    case RSA_OP_ATTN: return rsa::attn_ws_bytes(p);
    case RSA_OP_POOLED: return rsa::pooled_ws_bytes(p);
    case RSA_OP_GRAM: return rsa::gram_ws_bytes(p);
    case RSA_OP_KMEANS: return rsa::kmeans_ws_bytes(p);
    case RSA_OP_CLUSTER_ATTN: return rsa::cluster_attn_ws_bytes(p);
    default: return 0;
  }
}

rsa_status check_ws(const rsa::Problem& p, int op, const void* ws, size_t ws_bytes) {
  const size_t need = ws_bytes_for(p, op);
  if (need == 0) return RSA_OK;
  if (ws == nullptr || ws_bytes < need || !aligned256(ws)) return RSA_ERR_WORKSPACE;
  return RSA_OK;
}

}  // namespace

extern "C" {

size_t rsa_workspace_bytes(const rsa_problem* p, int32_t op) {
  rsa::Problem pr;
  if (make_problem(p, &pr) != RSA_OK) return 0;
  return ws_bytes_for(pr, op);
}

const char* rsa_status_str(int32_t s) {
  switch (s) {
    case RSA_OK: return "RSA_OK";
    case RSA_ERR_NULL: return "RSA_ERR_NULL";
    case RSA_ERR_SHAPE: return "RSA_ERR_SHAPE";
    case RSA_ERR_DTYPE: return "RSA_ERR_DTYPE";
    case RSA_ERR_ALIGN: return "RSA_ERR_ALIGN";
    case RSA_ERR_WORKSPACE: return "RSA_ERR_WORKSPACE";
    case RSA_ERR_HIP: return "RSA_ERR_HIP";
    case RSA_ERR_ARG: return "RSA_ERR_ARG";
    default: return "unknown";
  }
}

int32_t rsa_version(void) { return RSA_VERSION; }

rsa_status rsa_score_blocks(const rsa_problem* p, const void* q, const void* k,
                            const uint8_t* head_active, float* scores, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (q == nullptr || k == nullptr || scores == nullptr) return RSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(scores)) return RSA_ERR_ALIGN;
  st = check_ws(pr, RSA_OP_SCORE, ws, ws_bytes);
  if (st != RSA_OK) return st;
  rsa::ScoreWs w;
  rsa::score_ws_layout(pr, &w, ws);
  return hip_status(rsa::launch_scoring(pr, q, k, head_active, scores, w, stream));
}

rsa_status rsa_select_topp(const rsa_problem* p, const float* scores, const float* top_p,
                           int32_t max_blocks, const uint8_t* head_active, uint8_t* mask,
                           int32_t* counts, int32_t* block_idx, float* density, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (scores == nullptr || top_p == nullptr || mask == nullptr || counts == nullptr ||
      block_idx == nullptr)
    return RSA_ERR_NULL;
  if (max_blocks < 0) return RSA_ERR_ARG;
  if (!aligned16(scores) || !aligned16(block_idx) || !aligned16(counts)) return RSA_ERR_ALIGN;
  return hip_status(rsa::launch_select(pr, scores, top_p, max_blocks, head_active, mask, counts,
                                       block_idx, density, stream));
}

rsa_status rsa_mask_drift(const rsa_problem* p, const void* q, const void* k, void* q_ref,
                          void* k_ref, float threshold, int32_t update_ref, float* drift,
                          uint8_t* refresh, void* ws, size_t ws_bytes, hipStream_t stream) {
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (q == nullptr || k == nullptr || q_ref == nullptr || k_ref == nullptr || drift == nullptr ||
      refresh == nullptr)
    return RSA_ERR_NULL;
  if (std::isnan(threshold)) return RSA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_ref) || !aligned16(k_ref)) return RSA_ERR_ALIGN;
  st = check_ws(pr, RSA_OP_DRIFT, ws, ws_bytes);
  if (st != RSA_OK) return st;
  return hip_status(rsa::launch_drift(pr, q, k, q_ref, k_ref, threshold, update_ref, drift,
                                      refresh, ws, stream));
}

rsa_status rsa_block_sparse_attn(const rsa_problem* p, const void* q, const void* k, const void* v,
                                 const int32_t* counts, const int32_t* block_idx, void* out,
                                 float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || counts == nullptr || block_idx == nullptr ||
      out == nullptr)
    return RSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return RSA_ERR_ALIGN;
  st = check_ws(pr, RSA_OP_ATTN, ws, ws_bytes);
  if (st != RSA_OK) return st;
  return hip_status(rsa::launch_attention(pr, q, k, v, counts, block_idx, nullptr, 0, nullptr, nullptr, out, lse,
                                          ws, stream));
}

rsa_status rsa_dense_block_mass(const rsa_problem* p, const void* q, const void* k, float* mass,
                                hipStream_t stream) {
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (q == nullptr || k == nullptr || mass == nullptr) return RSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(mass)) return RSA_ERR_ALIGN;
  return hip_status(rsa::launch_dense_mass(pr, q, k, mass, stream));
}

rsa_status rsa_score_blocks_pooled(const rsa_problem* p, const void* q, const void* k,
                                   float* pooled, void* ws, size_t ws_bytes, hipStream_t stream) {
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (q == nullptr || k == nullptr || pooled == nullptr) return RSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(pooled)) return RSA_ERR_ALIGN;
  st = check_ws(pr, RSA_OP_POOLED, ws, ws_bytes);
  if (st != RSA_OK) return st;
  return hip_status(rsa::launch_pooled_scores(pr, q, k, pooled, ws, stream));
}

rsa_status rsa_attn_omitted(const rsa_problem* p, const void* q, const void* k, const void* v,
                            const int32_t* counts, const int32_t* block_idx,
                            const uint8_t* head_active, void* out, float* lse, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || counts == nullptr || block_idx == nullptr ||
      out == nullptr || lse == nullptr)
    return RSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return RSA_ERR_ALIGN;
  st = check_ws(pr, RSA_OP_ATTN, ws, ws_bytes);
  if (st != RSA_OK) return st;
  return hip_status(rsa::launch_attention(pr, q, k, v, counts, block_idx, head_active, 1, nullptr, nullptr, out,
                                          lse, ws, stream));
}

rsa_status rsa_block_sparse_attn_corrected(const rsa_problem* p, const void* q, const void* k, const void* v,
                                           const int32_t* counts, const int32_t* block_idx, const void* part_out,
                                           const float* part_lse, void* out, float* lse, void* ws,
                                           size_t ws_bytes, hipStream_t stream) {
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || counts == nullptr || block_idx == nullptr ||
      part_out == nullptr || part_lse == nullptr || out == nullptr || lse == nullptr)
    return RSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(part_out) || !aligned16(out))
    return RSA_ERR_ALIGN;
  st = check_ws(pr, RSA_OP_ATTN, ws, ws_bytes);
  if (st != RSA_OK) return st;
  return hip_status(rsa::launch_attention(pr, q, k, v, counts, block_idx, nullptr, 0, part_out, part_lse, out,
                                          lse, ws, stream));
}

rsa_status rsa_attn_merge(const rsa_problem* p, void* out, float* lse, const void* part_out,
                          const float* part_lse, hipStream_t stream) {
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (out == nullptr || lse == nullptr || part_out == nullptr || part_lse == nullptr)
    return RSA_ERR_NULL;
  if (!aligned16(out) || !aligned16(part_out)) return RSA_ERR_ALIGN;
  return hip_status(rsa::launch_merge(pr, out, lse, part_out, part_lse, stream));
}

rsa_status rsa_query_gram(const rsa_problem* p, const void* q, float* gram, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (q == nullptr || gram == nullptr) return RSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(gram)) return RSA_ERR_ALIGN;
  st = check_ws(pr, RSA_OP_GRAM, ws, ws_bytes);
  if (st != RSA_OK) return st;
  return hip_status(rsa::launch_gram(pr, q, gram, ws, stream));
}

rsa_status rsa_kmeans(const rsa_problem* p, const void* k, const float* gram, int32_t iters, int32_t init,
                      float* centroids, int32_t* labels, int32_t* sizes, int32_t* order, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (k == nullptr || gram == nullptr || centroids == nullptr || labels == nullptr || sizes == nullptr ||
      order == nullptr)
    return RSA_ERR_NULL;
  if (iters < 1 || iters > 1000) return RSA_ERR_ARG;
  if (!aligned16(k) || !aligned16(centroids)) return RSA_ERR_ALIGN;
  st = check_ws(pr, RSA_OP_KMEANS, ws, ws_bytes);
  if (st != RSA_OK) return st;
  return hip_status(rsa::launch_kmeans(pr, k, gram, iters, init != 0, centroids, labels, sizes, order, ws, stream));
}

rsa_status rsa_score_clusters(const rsa_problem* p, const void* q, const float* centroids, const int32_t* sizes,
                              float* scores, void* ws, size_t ws_bytes, hipStream_t stream) {
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (q == nullptr || centroids == nullptr || sizes == nullptr || scores == nullptr) return RSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(scores)) return RSA_ERR_ALIGN;
  st = check_ws(pr, RSA_OP_SCORE, ws, ws_bytes);
  if (st != RSA_OK) return st;
  rsa::ScoreWs w;
  rsa::score_ws_layout(pr, &w, ws);
  return hip_status(rsa::launch_cluster_scoring(pr, q, centroids, sizes, scores, w, stream));
}

rsa_status rsa_cluster_attn(const rsa_problem* p, const void* q, const void* k, const void* v, const int32_t* sizes,
                            const int32_t* order, const int32_t* counts, const int32_t* block_idx, void* out,
                            float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  rsa::Problem pr;
  rsa_status st = make_problem(p, &pr);
  if (st != RSA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || sizes == nullptr || order == nullptr || counts == nullptr ||
      block_idx == nullptr || out == nullptr)
    return RSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return RSA_ERR_ALIGN;
  st = check_ws(pr, RSA_OP_CLUSTER_ATTN, ws, ws_bytes);
  if (st != RSA_OK) return st;
  return hip_status(
      rsa::launch_cluster_attention(pr, q, k, v, sizes, order, counts, block_idx, out, lse, ws, stream));
}

}  // extern "C"
