// C ABI entry points: host-side validation, then the kernel launches.
// Nothing here allocates, synchronizes or reads device memory.
#include "dsa_indexer.h"

#include "common.h"

namespace {

thread_local int g_last_hip_error = 0;

}  // namespace

int dsa::record_hip_error(hipError_t e) {
  if (e == hipSuccess) return DSA_OK;
  g_last_hip_error = static_cast<int>(e);
  return DSA_ERR_HIP;
}

namespace {

bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
bool misaligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) != 0; }

int from_hip(hipError_t e) { return dsa::record_hip_error(e); }

constexpr int32_t kMaxBatch = 65535;  // grid y / x limit used by the launches
constexpr int32_t kMaxPages = dsa::kMaxRowPositions / dsa::kPage;
constexpr int64_t kMaxSlots = int64_t(1) << 26;  // batch * max_pages: at most 2^32 logits
// Attention: pool rows (page * 64 + row) are 32-bit codes below two reserved values.
constexpr int64_t kMaxAttPages = (int64_t(1) << 26) - 1;

}  // namespace

extern "C" {

int dsa_indexer_abi_version(void) { return DSA_INDEXER_ABI_VERSION; }

const char* dsa_indexer_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "batch, tokens, max_pages, num_pages, max_c4 or scale out of range";
    case DSA_ERR_ALIGN: return "a pointer misses its required alignment";
    case DSA_ERR_K: return "k out of range (top-k: [1, max_c4]; attention: [1, 2048])";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_HIP: return "HIP runtime error on launch";
    case DSA_ERR_SCRATCH: return "the sizes need more top-k workspace than the fixed scratch array holds";
    default: return "unknown status";
  }
}

int dsa_indexer_last_hip_error(void) { return g_last_hip_error; }

int dsa_indexer_score(const void* q, const float* w, const void* k_pool, int64_t num_pages,
                      const int32_t* page_table, const int32_t* seq_lens, int32_t batch,
                      int32_t max_pages, float* logits, int32_t* row_hwm, hipStream_t stream) {
  if (!q || !w || !k_pool || !page_table || !seq_lens || !logits) return DSA_ERR_NULL;
  if (batch < 1 || batch > kMaxBatch || max_pages < 1 || max_pages > kMaxPages || num_pages < 1 ||
      (int64_t)batch * max_pages > kMaxSlots)
    return DSA_ERR_SHAPE;
  if (misaligned16(q) || misaligned16(w) || misaligned16(k_pool) || misaligned16(logits) ||
      misaligned4(page_table) || misaligned4(seq_lens) || misaligned4(row_hwm))
    return DSA_ERR_ALIGN;
  return from_hip(dsa::launch_score(q, w, k_pool, nullptr, num_pages, page_table, seq_lens, batch, 1, max_pages,
                                    logits, row_hwm, nullptr, stream));
}

int dsa_indexer_score_hist(const void* q, const float* w, const void* k_pool, int64_t num_pages,
                           const int32_t* page_table, const int32_t* seq_lens, int32_t batch, int32_t max_pages,
                           float* logits, int32_t* row_hwm, uint32_t* hist, hipStream_t stream) {
  if (!q || !w || !k_pool || !page_table || !seq_lens || !logits || !hist) return DSA_ERR_NULL;
  if (batch < 1 || batch > kMaxBatch || max_pages < 1 || max_pages > kMaxPages || num_pages < 1 ||
      (int64_t)batch * max_pages > kMaxSlots)
    return DSA_ERR_SHAPE;
  if (misaligned16(q) || misaligned16(w) || misaligned16(k_pool) || misaligned16(logits) || misaligned16(hist) ||
      misaligned4(page_table) || misaligned4(seq_lens) || misaligned4(row_hwm))
    return DSA_ERR_ALIGN;
  return from_hip(dsa::launch_score(q, w, k_pool, nullptr, num_pages, page_table, seq_lens, batch, 1, max_pages,
                                    logits, row_hwm, hist, stream));
}

int dsa_indexer_score_fp8(const void* q, const float* w, const void* k_pool_fp8, const float* k_scale,
                          int64_t num_pages, const int32_t* page_table, const int32_t* seq_lens, int32_t batch,
                          int32_t max_pages, float* logits, int32_t* row_hwm, hipStream_t stream) {
  if (!q || !w || !k_pool_fp8 || !k_scale || !page_table || !seq_lens || !logits) return DSA_ERR_NULL;
  if (batch < 1 || batch > kMaxBatch || max_pages < 1 || max_pages > kMaxPages || num_pages < 1 ||
      (int64_t)batch * max_pages > kMaxSlots)
    return DSA_ERR_SHAPE;
  if (misaligned16(q) || misaligned16(w) || misaligned16(k_pool_fp8) || misaligned16(logits) ||
      misaligned4(k_scale) || misaligned4(page_table) || misaligned4(seq_lens) || misaligned4(row_hwm))
    return DSA_ERR_ALIGN;
  return from_hip(dsa::launch_score(q, w, k_pool_fp8, k_scale, num_pages, page_table, seq_lens, batch, 1,
                                    max_pages, logits, row_hwm, nullptr, stream));
}

int dsa_indexer_score_mtp(const void* q, const float* w, const void* k_pool, int64_t num_pages,
                          const int32_t* page_table, const int32_t* seq_lens, int32_t batch, int32_t tokens,
                          int32_t max_pages, float* logits, int32_t* row_hwm, hipStream_t stream) {
  if (!q || !w || !k_pool || !page_table || !seq_lens || !logits) return DSA_ERR_NULL;
  if (batch < 1 || batch > kMaxBatch || tokens < 1 || tokens > dsa::kMaxTokens || max_pages < 1 ||
      max_pages > kMaxPages || num_pages < 1 || (int64_t)batch * tokens * max_pages > kMaxSlots)
    return DSA_ERR_SHAPE;
  if (misaligned16(q) || misaligned16(w) || misaligned16(k_pool) || misaligned16(logits) ||
      misaligned4(page_table) || misaligned4(seq_lens) || misaligned4(row_hwm))
    return DSA_ERR_ALIGN;
  return from_hip(dsa::launch_score(q, w, k_pool, nullptr, num_pages, page_table, seq_lens, batch, tokens, max_pages,
                                    logits, row_hwm, nullptr, stream));
}

size_t dsa_indexer_topk_workspace_bytes(int32_t batch, int32_t max_c4, int32_t k) {
  (void)k;
  if (batch < 1 || batch > kMaxBatch || max_c4 < 1 || max_c4 > dsa::kMaxRowPositions) return 0;
  return dsa::topk_workspace_words(batch, max_c4) * sizeof(uint32_t);
}

int dsa_indexer_topk(const float* logits, const int32_t* seq_lens, int32_t batch, int32_t max_c4,
                     int32_t k, int32_t* out_idx, float* out_vals, void* workspace, size_t ws_bytes,
                     hipStream_t stream) {
  if (!logits || !seq_lens || !out_idx) return DSA_ERR_NULL;
  if (batch < 1 || batch > kMaxBatch || max_c4 < 1 || max_c4 > dsa::kMaxRowPositions) return DSA_ERR_SHAPE;
  if (k < 1 || k > max_c4) return DSA_ERR_K;
  const size_t need = dsa_indexer_topk_workspace_bytes(batch, max_c4, k);
  if (ws_bytes < need || (need > 0 && workspace == nullptr)) return DSA_ERR_WORKSPACE;
  if (misaligned4(logits) || misaligned4(seq_lens) || misaligned4(out_idx) || misaligned4(out_vals) ||
      misaligned16(workspace))
    return DSA_ERR_ALIGN;
  return from_hip(
      dsa::launch_topk(logits, seq_lens, batch, max_c4, k, out_idx, out_vals, workspace, nullptr, stream));
}

int dsa_indexer_topk_hist(const float* logits, const int32_t* seq_lens, int32_t batch, int32_t max_c4, int32_t k,
                          int32_t* out_idx, float* out_vals, uint32_t* hist, void* workspace, size_t ws_bytes,
                          hipStream_t stream) {
  if (!logits || !seq_lens || !out_idx || !hist) return DSA_ERR_NULL;
  if (batch < 1 || batch > kMaxBatch || max_c4 < 1 || max_c4 > dsa::kMaxRowPositions) return DSA_ERR_SHAPE;
  if (k < 1 || k > max_c4) return DSA_ERR_K;
  const size_t need = dsa_indexer_topk_workspace_bytes(batch, max_c4, k);
  if (ws_bytes < need || (need > 0 && workspace == nullptr)) return DSA_ERR_WORKSPACE;
  if (misaligned4(logits) || misaligned4(seq_lens) || misaligned4(out_idx) || misaligned4(out_vals) ||
      misaligned16(workspace) || misaligned16(hist))
    return DSA_ERR_ALIGN;
  return from_hip(
      dsa::launch_topk(logits, seq_lens, batch, max_c4, k, out_idx, out_vals, workspace, hist, stream));
}

size_t dsa_indexer_sparse_attention_workspace_bytes(int32_t batch, int32_t k) {
  if (batch < 1 || batch > kMaxBatch || k < 1 || k > dsa::kMaxAttK) return 0;
  return dsa::att_workspace_bytes(batch, k);
}

int dsa_indexer_sparse_attention(const void* q, const void* kv_pool, int64_t num_pages, const int32_t* page_table,
                                 int32_t batch, int32_t max_pages, const int32_t* idx, int32_t k, float scale,
                                 float* out, float* lse, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!q || !kv_pool || !page_table || !idx || !out || !lse) return DSA_ERR_NULL;
  if (batch < 1 || batch > kMaxBatch || max_pages < 1 || max_pages > kMaxPages || num_pages < 1 ||
      num_pages > kMaxAttPages)
    return DSA_ERR_SHAPE;
  if (k < 1 || k > dsa::kMaxAttK) return DSA_ERR_K;
  if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff()) return DSA_ERR_SHAPE;
  const size_t need = dsa_indexer_sparse_attention_workspace_bytes(batch, k);
  if (ws_bytes < need || (need > 0 && workspace == nullptr)) return DSA_ERR_WORKSPACE;
  if (misaligned16(q) || misaligned16(kv_pool) || misaligned16(out) || misaligned4(lse) ||
      misaligned4(page_table) || misaligned4(idx) || misaligned16(workspace))
    return DSA_ERR_ALIGN;
  return from_hip(dsa::launch_attention(q, kv_pool, num_pages, page_table, batch, max_pages, idx, k, scale, out,
                                        lse, workspace, stream));
}

}  // extern "C"
