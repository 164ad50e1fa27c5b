// C ABI of libsparse_mla: argument checks, workspace carving, launches and the
// IndexShare layer scheduler (hermosaai "GLM 5.2", "MLA + DSA with IndexShare":
// a full layer scores and selects, the following shared layers reuse its
// selection; llm-architectures-explained "GLM-5.2", "Every architecture field",
// row "layout": the full/shared sequence of the 78 layers).
#include <stdarg.h>
#include <stdio.h>

#include "sa_common.h"

namespace sa_host {

static thread_local char g_msg[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
}

int32_t check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return SA_ERR_HIP;
  }
  return SA_OK;
}

int indexer_algo(int32_t n_q, int32_t n_seq, int algo);
int32_t launch_indexer(const void* q_idx, const float* w, const void* k_idx, const int64_t* seq_start,
                       const int32_t* q_seq, const int32_t* q_pos, int32_t n_q, int32_t n_seq, float* scores,
                       int64_t ld, int algo, hipStream_t stream, uint32_t* clear, int64_t n_clear);
void topk_clear_range(void* ws, int32_t n_q, int64_t ld, uint32_t** p, int64_t* n);

size_t topk_workspace_size(int32_t n_q, int64_t ld, int32_t k);
int32_t launch_topk(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q, int32_t k, int32_t* idx,
                    void* ws, int algo, hipStream_t stream, bool cleared);
size_t mla_workspace_size(int32_t n_q, int32_t k);
int32_t launch_mla(const void* q_abs, const void* kv, const int64_t* seq_start, const int32_t* q_seq,
                   const int32_t* idx, int32_t n_q, int32_t k, const void* w_uv, float scale, void* out, float* lse,
                   void* ws, hipStream_t stream);

int32_t launch_cache_write(const void* kv_a, const void* gamma, const void* k_raw, const void* ln_w, const void* ln_b,
                           const int32_t* pos, const int64_t* dst, int32_t n, void* kv_cache, void* k_cache,
                           hipStream_t stream);

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

#define SA_REQUIRE(cond, code, ...) \
  do {                              \
    if (!(cond)) {                  \
      set_error(__VA_ARGS__);       \
      return (code);                \
    }                               \
  } while (0)

static int32_t check_indexer_args(const void* q_idx, const float* w, const void* k_idx, const int64_t* seq_start,
                                  const int32_t* q_seq, const int32_t* q_pos, int32_t n_q, int32_t n_seq,
                                  const float* scores, int64_t ld) {
  SA_REQUIRE(n_q >= 0 && n_seq >= 0, SA_ERR_INVALID_ARG, "indexer: negative count (n_q=%d, n_seq=%d)", n_q, n_seq);
  if (n_q == 0) return SA_OK;
  SA_REQUIRE(n_seq >= 1, SA_ERR_INVALID_ARG, "indexer: queries without sequences");
  SA_REQUIRE(q_idx && w && k_idx && seq_start && q_seq && q_pos && scores, SA_ERR_INVALID_ARG,
             "indexer: null pointer argument");
  SA_REQUIRE(aligned16(q_idx) && aligned16(k_idx), SA_ERR_INVALID_ARG, "indexer: q_idx/k_idx not 16-byte aligned");
  SA_REQUIRE(ld >= 1 && ld < ((int64_t)1 << 31), SA_ERR_INVALID_ARG, "indexer: ld=%lld out of range", (long long)ld);
  return SA_OK;
}

static int32_t check_topk_args(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q, int32_t k,
                               const int32_t* idx) {
  SA_REQUIRE(n_q >= 0, SA_ERR_INVALID_ARG, "topk: negative n_q");
  SA_REQUIRE(k >= 1 && k <= SA_MAX_TOPK, SA_ERR_INVALID_ARG, "topk: k=%d outside 1..%d", k, SA_MAX_TOPK);
  if (n_q == 0) return SA_OK;
  SA_REQUIRE(scores && q_pos && idx, SA_ERR_INVALID_ARG, "topk: null pointer argument");
  SA_REQUIRE(ld >= 1 && ld < ((int64_t)1 << 31), SA_ERR_INVALID_ARG, "topk: ld=%lld out of range", (long long)ld);
  return SA_OK;
}

static int32_t check_mla_args(const void* q_abs, const void* kv, const int64_t* seq_start, const int32_t* q_seq,
                              const int32_t* idx, int32_t n_q, int32_t k, const void* w_uv, float scale,
                              const void* out) {
  SA_REQUIRE(n_q >= 0, SA_ERR_INVALID_ARG, "mla: negative n_q");
  SA_REQUIRE(k >= 1 && k <= SA_MAX_TOPK, SA_ERR_INVALID_ARG, "mla: k=%d outside 1..%d", k, SA_MAX_TOPK);
  SA_REQUIRE(scale > 0.f && scale < 1e30f, SA_ERR_INVALID_ARG, "mla: scale must be positive and finite");
  if (n_q == 0) return SA_OK;
  SA_REQUIRE(q_abs && kv && seq_start && q_seq && idx && w_uv && out, SA_ERR_INVALID_ARG, "mla: null pointer argument");
  SA_REQUIRE(aligned16(q_abs) && aligned16(kv) && aligned16(w_uv), SA_ERR_INVALID_ARG,
             "mla: q_abs/kv/w_uv not 16-byte aligned");
  return SA_OK;
}

static int32_t record(sa_event_t ev, hipStream_t stream) {
  if (!ev) return SA_OK;
  if (hipEventRecord((hipEvent_t)ev, stream) != hipSuccess) {
    set_error("hipEventRecord failed");
    return SA_ERR_HIP;
  }
  return SA_OK;
}

}  // namespace sa_host

using namespace sa_host;

extern "C" {

int32_t sa_version(void) { return (0 << 16) | (1 << 8) | 0; }

const char* sa_status_string(int32_t status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported request";
    case SA_ERR_WORKSPACE: return "workspace missing or too small";
    case SA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sa_last_error_message(void) { return g_msg; }

int32_t sa_layer_is_full(int32_t layer) {
  if (layer < 0) return -1;
  return (layer < 3 || layer % 4 == 2) ? 1 : 0;
}

int32_t sa_indexer_score_algo(const void* q_idx, const float* w, const void* k_idx, const int64_t* seq_start,
                              const int32_t* q_seq, const int32_t* q_pos, int32_t n_q, int32_t n_seq, float* scores,
                              int64_t ld, int32_t algo, sa_stream_t stream) {
  int32_t rc = check_indexer_args(q_idx, w, k_idx, seq_start, q_seq, q_pos, n_q, n_seq, scores, ld);
  if (rc) return rc;
  SA_REQUIRE(algo >= 0 && algo <= 2, SA_ERR_INVALID_ARG, "indexer: unknown algo %d", algo);
  if (n_q == 0) return SA_OK;
  return launch_indexer(q_idx, w, k_idx, seq_start, q_seq, q_pos, n_q, n_seq, scores, ld, algo, (hipStream_t)stream,
                        nullptr, 0);
}

int32_t sa_indexer_score(const void* q_idx, const float* w, const void* k_idx, const int64_t* seq_start,
                         const int32_t* q_seq, const int32_t* q_pos, int32_t n_q, int32_t n_seq, float* scores,
                         int64_t ld, sa_stream_t stream) {
  return sa_indexer_score_algo(q_idx, w, k_idx, seq_start, q_seq, q_pos, n_q, n_seq, scores, ld, 0, stream);
}

size_t sa_topk_workspace_size(int32_t n_q, int64_t ld, int32_t k) {
  if (n_q <= 0 || ld <= 0) return 256;
  return topk_workspace_size(n_q, ld, k);
}

int32_t sa_topk_select_algo(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q, int32_t k,
                            int32_t* idx, void* ws, size_t ws_bytes, int32_t algo, sa_stream_t stream) {
  int32_t rc = check_topk_args(scores, ld, q_pos, n_q, k, idx);
  if (rc) return rc;
  SA_REQUIRE(algo >= 0 && algo <= 2, SA_ERR_INVALID_ARG, "topk: unknown algo %d", algo);
  if (n_q == 0) return SA_OK;
  const size_t need = topk_workspace_size(n_q, ld, k);
  SA_REQUIRE(ws && ws_bytes >= need, SA_ERR_WORKSPACE, "topk: workspace of %zu bytes, %zu needed", ws_bytes, need);
  SA_REQUIRE(((uintptr_t)ws & 255u) == 0, SA_ERR_INVALID_ARG, "topk: workspace not 256-byte aligned");
  return launch_topk(scores, ld, q_pos, n_q, k, idx, ws, algo, (hipStream_t)stream, false);
}

int32_t sa_topk_select(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q, int32_t k, int32_t* idx,
                       void* ws, size_t ws_bytes, sa_stream_t stream) {
  return sa_topk_select_algo(scores, ld, q_pos, n_q, k, idx, ws, ws_bytes, 0, stream);
}

size_t sa_mla_workspace_size(int32_t n_q, int32_t k) {
  if (n_q <= 0 || k <= 0) return 256;
  return mla_workspace_size(n_q, k > SA_MAX_TOPK ? SA_MAX_TOPK : k);
}

int32_t sa_mla_sparse_attn(const void* q_abs, const void* kv, const int64_t* seq_start, const int32_t* q_seq,
                           const int32_t* idx, int32_t n_q, int32_t k, const void* w_uv, float scale, void* out,
                           float* lse, void* ws, size_t ws_bytes, sa_stream_t stream) {
  int32_t rc = check_mla_args(q_abs, kv, seq_start, q_seq, idx, n_q, k, w_uv, scale, out);
  if (rc) return rc;
  if (n_q == 0) return SA_OK;
  const size_t need = mla_workspace_size(n_q, k);
  SA_REQUIRE(ws && ws_bytes >= need, SA_ERR_WORKSPACE, "mla: workspace of %zu bytes, %zu needed", ws_bytes, need);
  SA_REQUIRE(((uintptr_t)ws & 255u) == 0, SA_ERR_INVALID_ARG, "mla: workspace not 256-byte aligned");
  return launch_mla(q_abs, kv, seq_start, q_seq, idx, n_q, k, w_uv, scale, out, lse, ws, (hipStream_t)stream);
}

size_t sa_layer_stack_workspace_size(int32_t n_q, int64_t ld, int32_t k) {
  if (n_q <= 0 || ld <= 0 || k <= 0) return 256;
  return align256((size_t)n_q * (size_t)ld * 4) + align256(topk_workspace_size(n_q, ld, k)) +
         align256(mla_workspace_size(n_q, k > SA_MAX_TOPK ? SA_MAX_TOPK : k));
}

int32_t sa_layer_stack(const sa_layer_desc* layers, int32_t n_layers, const sa_batch_desc* batch, int32_t k,
                       float scale, void* ws, size_t ws_bytes, const sa_stage_events* events, sa_stream_t stream) {
  SA_REQUIRE(layers && batch, SA_ERR_INVALID_ARG, "layer_stack: null descriptor");
  SA_REQUIRE(n_layers >= 0, SA_ERR_INVALID_ARG, "layer_stack: negative n_layers");
  SA_REQUIRE(k >= 1 && k <= SA_MAX_TOPK, SA_ERR_INVALID_ARG, "layer_stack: k=%d outside 1..%d", k, SA_MAX_TOPK);
  const int32_t n_q = batch->n_q;
  const int64_t ld = batch->ld;
  SA_REQUIRE(n_q >= 0 && batch->n_seq >= 0, SA_ERR_INVALID_ARG, "layer_stack: negative count");
  if (n_layers == 0 || n_q == 0) return SA_OK;
  SA_REQUIRE(layers[0].is_full, SA_ERR_INVALID_ARG, "layer_stack: layer 0 must run its own indexer");
  const size_t need = sa_layer_stack_workspace_size(n_q, ld, k);
  SA_REQUIRE(ws && ws_bytes >= need, SA_ERR_WORKSPACE, "layer_stack: workspace of %zu bytes, %zu needed", ws_bytes,
             need);
  SA_REQUIRE(((uintptr_t)ws & 255u) == 0, SA_ERR_INVALID_ARG, "layer_stack: workspace not 256-byte aligned");
  // Check every layer before enqueuing anything.
  for (int l = 0; l < n_layers; ++l) {
    const sa_layer_desc& L = layers[l];
    int32_t rc;
    if (L.is_full) {
      rc = check_indexer_args(L.q_idx, L.w, L.k_idx, batch->seq_start, batch->q_seq, batch->q_pos, n_q,
                              batch->n_seq, (const float*)ws, ld);
      if (rc) return rc;
      SA_REQUIRE(L.idx, SA_ERR_INVALID_ARG, "layer_stack: full layer %d has no idx buffer", l);
    }
    rc = check_mla_args(L.q_abs, L.kv, batch->seq_start, batch->q_seq, (const int32_t*)1, n_q, k, L.w_uv, scale,
                        L.out);
    if (rc) {
      char tmp[512];
      snprintf(tmp, sizeof tmp, "layer %d: %s", l, sa_last_error_message());
      set_error("%s", tmp);
      return rc;
    }
  }
  uint8_t* p = (uint8_t*)ws;
  float* scores = (float*)p;
  p += align256((size_t)n_q * (size_t)ld * 4);
  void* topk_ws = p;
  p += align256(topk_workspace_size(n_q, ld, k));
  void* mla_ws = p;

  hipStream_t st = (hipStream_t)stream;
  const int32_t* cur_idx = nullptr;
  bool rec_idx = false, rec_topk = false, rec_attn = false;
  int32_t rc;
  // Decode batches score one query per workgroup column; batches with at
  // least 16 queries per sequence (chunked prefill) use the query-blocked
  // indexer.  The top-k then runs its own first-digit histogram pass over the
  // scores.  The decode indexer also clears the top-k's histograms and
  // counters on the side, which saves the top-k a launch of its own for that.
  const int ialgo = indexer_algo(n_q, batch->n_seq, 0);
  uint32_t* clear = nullptr;
  int64_t n_clear = 0;
  if (ialgo == 1) topk_clear_range(topk_ws, n_q, ld, &clear, &n_clear);
  for (int l = 0; l < n_layers; ++l) {
    const sa_layer_desc& L = layers[l];
    if (L.is_full) {
      const bool ev = events && !rec_idx && events->indexer_begin && events->indexer_end;
      if (ev && (rc = record(events->indexer_begin, st))) return rc;
      rc = launch_indexer(L.q_idx, L.w, L.k_idx, batch->seq_start, batch->q_seq, batch->q_pos, n_q, batch->n_seq, scores,
                          ld, ialgo, st, clear, n_clear);
      if (rc) return rc;
      if (ev && (rc = record(events->indexer_end, st))) return rc;
      rec_idx |= ev;
      const bool evt = events && !rec_topk && events->topk_begin && events->topk_end;
      if (evt && (rc = record(events->topk_begin, st))) return rc;
      rc = launch_topk(scores, ld, batch->q_pos, n_q, k, L.idx, topk_ws, 0, st, ialgo == 1);
      if (rc) return rc;
      if (evt && (rc = record(events->topk_end, st))) return rc;
      rec_topk |= evt;
      cur_idx = L.idx;
    }
    const bool eva = events && !rec_attn && events->attn_begin && events->attn_end;
    if (eva && (rc = record(events->attn_begin, st))) return rc;
    rc = launch_mla(L.q_abs, L.kv, batch->seq_start, batch->q_seq, cur_idx, n_q, k, L.w_uv, scale, L.out, nullptr,
                    mla_ws, st);
    if (rc) return rc;
    if (eva && (rc = record(events->attn_end, st))) return rc;
    rec_attn |= eva;
  }
  return SA_OK;
}

int32_t sa_cache_write(const void* kv_a, const void* gamma, const void* k_raw, const void* ln_w, const void* ln_b,
                       const int32_t* pos, const int64_t* dst, int32_t n, void* kv_cache, void* k_cache,
                       sa_stream_t stream) {
  SA_REQUIRE(n >= 0, SA_ERR_INVALID_ARG, "cache_write: negative n");
  if (n == 0) return SA_OK;
  SA_REQUIRE(kv_a && gamma && pos && dst && kv_cache, SA_ERR_INVALID_ARG, "cache_write: null pointer argument");
  SA_REQUIRE(aligned16(kv_a) && aligned16(gamma) && aligned16(kv_cache), SA_ERR_INVALID_ARG,
             "cache_write: kv_a/gamma/kv_cache not 16-byte aligned");
  if (k_raw) {
    SA_REQUIRE(ln_w && ln_b && k_cache, SA_ERR_INVALID_ARG, "cache_write: indexer key without ln_w/ln_b/k_cache");
    SA_REQUIRE((((uintptr_t)k_raw | (uintptr_t)ln_w | (uintptr_t)ln_b | (uintptr_t)k_cache) & 3u) == 0,
               SA_ERR_INVALID_ARG, "cache_write: indexer key pointers not 4-byte aligned");
  }
  return launch_cache_write(kv_a, gamma, k_raw, ln_w, ln_b, pos, dst, n, kv_cache, k_cache, (hipStream_t)stream);
}

}  // extern "C"
