// C ABI of libsparse_mla: argument checks, workspace carving, launches and the
// IndexShare layer scheduler (hermosaai "GLM 5.2", "MLA + DSA with IndexShare":
// a full layer scores and selects, the following shared layers reuse its
// selection; llm-architectures-explained "GLM-5.2", "Every architecture field",
// row "layout": the full/shared sequence of the 78 layers).
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "sa_common.h"

// Workspace of sa_layer_stack_noalloc: one array per GPU, held until the
// process ends.  Host code never uses this name as an address (on the host it
// is only a stand-in); it uses the per-device pointer from
// hipGetSymbolAddress instead.
static __device__ __align__(256) uint8_t scratch[SA_NOALLOC_SCRATCH_BYTES];

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
int32_t launch_indexer(const void* q_idx, const float* w, const void* k_idx, const float* k_scale,
                       const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq, const int32_t* q_pos,
                       int32_t n_q, int32_t n_seq, float* scores, int64_t ld, int algo, hipStream_t stream,
                       uint32_t* clear, int64_t n_clear);
void topk_clear_range(void* ws, int32_t n_q, int64_t ld, uint32_t** p, int64_t* n);

size_t topk_workspace_size(int32_t n_q, int64_t ld, int32_t k);
int32_t launch_topk(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q, int32_t k, int32_t* idx,
                    void* ws, int algo, hipStream_t stream, bool cleared);
size_t mla_workspace_size(int32_t n_q, int32_t k);
void mla_split(int32_t n_q, int32_t k, int* n_sp, int* kps);
int mla_partial_bits(int32_t n_q, int32_t k);
int32_t launch_mla(const void* q_abs, const void* kv, const float* kv_scale, const int64_t* seq_start,
                   const int32_t* q_seq, const int32_t* idx, int32_t n_q, int32_t k, const void* w_uv, float scale,
                   void* out, float* lse, void* ws, hipStream_t stream, bool shared_rows, int part_half = 0);
int32_t launch_quantize(const void* src, int64_t n_rows, int32_t d, const int64_t* dst_rows, void* codes, float* scales,
                        hipStream_t stream);
int32_t launch_fp8_decode(const void* codes, int64_t n, void* out, hipStream_t stream);

int32_t launch_cache_write(const void* kv_a, const void* gamma, const void* k_raw, const void* ln_w, const void* ln_b,
                           const int32_t* pos, const int64_t* dst, int32_t n, void* kv_cache, void* k_cache,
                           hipStream_t stream);

int32_t debug_batch(const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq, const int32_t* q_pos,
                    int32_t n_q, int32_t n_seq, int64_t ld, hipStream_t stream);
int32_t debug_idx(const int32_t* idx, int32_t n_q, int32_t k, const int32_t* q_pos, const int32_t* q_seq,
                  hipStream_t stream);
int32_t debug_scores(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q, hipStream_t stream);
int32_t debug_cache(const int32_t* pos, const int64_t* dst, int32_t n, hipStream_t stream);
int32_t launch_q_project(const void* c_q, const void* w_qb, const void* w_iq, const void* w_iw, const int32_t* pos,
                         int32_t n, void* q, void* q_idx, float* w, hipStream_t stream);
int32_t launch_q_absorb(const void* q, const void* w_uk_t, int32_t n, void* q_abs, hipStream_t stream);
int32_t debug_share(const int32_t* sel_of, int32_t n_sel, const int32_t* q_seq, const int32_t* sel_seq, int32_t n_q,
                    hipStream_t stream);
int32_t launch_share(const int32_t* sel_idx, int32_t n_sel, int32_t k, const int32_t* sel_of, const int32_t* q_pos,
                     int32_t n_q, int32_t* idx, hipStream_t stream);

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
                                  const int32_t* seq_len, const int32_t* q_seq, const int32_t* q_pos, int32_t n_q,
                                  int32_t n_seq, const float* scores, int64_t ld) {
  SA_REQUIRE(n_q >= 0 && n_seq >= 0, SA_ERR_INVALID_ARG, "indexer: negative count (n_q=%d, n_seq=%d)", n_q, n_seq);
  if (n_q == 0) return SA_OK;
  SA_REQUIRE(n_seq >= 1, SA_ERR_INVALID_ARG, "indexer: queries without sequences");
  SA_REQUIRE(q_idx && w && k_idx && seq_start && seq_len && q_seq && q_pos && scores, SA_ERR_INVALID_ARG,
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

int32_t sa_version(void) { return (0 << 16) | (2 << 8) | 0; }

const char* sa_status_string(int32_t status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported request";
    case SA_ERR_WORKSPACE: return "workspace missing or too small";
    case SA_ERR_HIP: return "HIP runtime error";
    case SA_ERR_DEBUG: return "debug check failed";
    default: return "unknown status";
  }
}

const char* sa_last_error_message(void) { return g_msg; }

int32_t sa_layer_is_full(int32_t layer) {
  if (layer < 0) return -1;
  return (layer < 3 || layer % 4 == 2) ? 1 : 0;
}

int32_t sa_indexer_score_algo(const void* q_idx, const float* w, const void* k_idx, const int64_t* seq_start,
                              const int32_t* seq_len, const int32_t* q_seq, const int32_t* q_pos, int32_t n_q,
                              int32_t n_seq, float* scores, int64_t ld, int32_t algo, sa_stream_t stream) {
  int32_t rc = check_indexer_args(q_idx, w, k_idx, seq_start, seq_len, q_seq, q_pos, n_q, n_seq, scores, ld);
  if (rc) return rc;
  SA_REQUIRE(algo >= 0 && algo <= 2, SA_ERR_INVALID_ARG, "indexer: unknown algo %d", algo);
  if (n_q == 0) return SA_OK;
  if ((rc = debug_batch(seq_start, seq_len, q_seq, q_pos, n_q, n_seq, ld, (hipStream_t)stream))) return rc;
  return launch_indexer(q_idx, w, k_idx, nullptr, seq_start, seq_len, q_seq, q_pos, n_q, n_seq, scores, ld, algo,
                        (hipStream_t)stream, nullptr, 0);
}

int32_t sa_indexer_score(const void* q_idx, const float* w, const void* k_idx, const int64_t* seq_start,
                         const int32_t* seq_len, const int32_t* q_seq, const int32_t* q_pos, int32_t n_q,
                         int32_t n_seq, float* scores, int64_t ld, sa_stream_t stream) {
  return sa_indexer_score_algo(q_idx, w, k_idx, seq_start, seq_len, q_seq, q_pos, n_q, n_seq, scores, ld, 0, stream);
}

int32_t sa_indexer_score_fp8_algo(const void* q_idx, const float* w, const void* k_codes, const float* k_scale,
                                  const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq,
                                  const int32_t* q_pos, int32_t n_q, int32_t n_seq, float* scores, int64_t ld,
                                  int32_t algo, sa_stream_t stream) {
  int32_t rc = check_indexer_args(q_idx, w, k_codes, seq_start, seq_len, q_seq, q_pos, n_q, n_seq, scores, ld);
  if (rc) return rc;
  SA_REQUIRE(algo >= 0 && algo <= 2, SA_ERR_INVALID_ARG, "indexer: unknown algo %d", algo);
  if (n_q == 0) return SA_OK;
  SA_REQUIRE(k_scale, SA_ERR_INVALID_ARG, "indexer: FP8 keys without k_scale");
  if ((rc = debug_batch(seq_start, seq_len, q_seq, q_pos, n_q, n_seq, ld, (hipStream_t)stream))) return rc;
  return launch_indexer(q_idx, w, k_codes, k_scale, seq_start, seq_len, q_seq, q_pos, n_q, n_seq, scores, ld, algo,
                        (hipStream_t)stream, nullptr, 0);
}

int32_t sa_indexer_score_fp8(const void* q_idx, const float* w, const void* k_codes, const float* k_scale,
                             const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq,
                             const int32_t* q_pos, int32_t n_q, int32_t n_seq, float* scores, int64_t ld,
                             sa_stream_t stream) {
  return sa_indexer_score_fp8_algo(q_idx, w, k_codes, k_scale, seq_start, seq_len, q_seq, q_pos, n_q, n_seq, scores,
                                   ld, 0, stream);
}

int32_t sa_quantize_rows_fp8(const void* src, int64_t n_rows, int32_t d, const int64_t* dst_rows, void* codes,
                             float* scales, sa_stream_t stream) {
  SA_REQUIRE(n_rows >= 0, SA_ERR_INVALID_ARG, "quantize: negative n_rows");
  SA_REQUIRE(d == SA_ROW || d == SA_INDEX_DIM, SA_ERR_UNSUPPORTED, "quantize: d=%d is neither %d nor %d", d, SA_ROW,
             SA_INDEX_DIM);
  if (n_rows == 0) return SA_OK;
  SA_REQUIRE(src && codes && scales, SA_ERR_INVALID_ARG, "quantize: null pointer argument");
  SA_REQUIRE(aligned16(src) && aligned16(codes), SA_ERR_INVALID_ARG, "quantize: src/codes not 16-byte aligned");
  return launch_quantize(src, n_rows, d, dst_rows, codes, scales, (hipStream_t)stream);
}

int32_t sa_fp8_decode(const void* codes, int64_t n, void* out, sa_stream_t stream) {
  SA_REQUIRE(n >= 0 && n % 16 == 0, SA_ERR_INVALID_ARG, "fp8_decode: n=%lld is not a multiple of 16", (long long)n);
  if (n == 0) return SA_OK;
  SA_REQUIRE(codes && out, SA_ERR_INVALID_ARG, "fp8_decode: null pointer argument");
  SA_REQUIRE(aligned16(codes) && aligned16(out), SA_ERR_INVALID_ARG, "fp8_decode: pointers not 16-byte aligned");
  return launch_fp8_decode(codes, n, out, (hipStream_t)stream);
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
  if ((rc = debug_scores(scores, ld, q_pos, n_q, (hipStream_t)stream))) return rc;
  return launch_topk(scores, ld, q_pos, n_q, k, idx, ws, algo, (hipStream_t)stream, false);
}

int32_t sa_topk_select(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q, int32_t k, int32_t* idx,
                       void* ws, size_t ws_bytes, sa_stream_t stream) {
  return sa_topk_select_algo(scores, ld, q_pos, n_q, k, idx, ws, ws_bytes, 0, stream);
}

int32_t sa_mla_split_info(int32_t n_q, int32_t k, int32_t* n_sp, int32_t* kps) {
  SA_REQUIRE(n_q >= 1 && k >= 1 && k <= SA_MAX_TOPK && n_sp && kps, SA_ERR_INVALID_ARG,
             "mla_split_info: n_q=%d, k=%d", n_q, k);
  int a, b;
  mla_split(n_q, k, &a, &b);
  *n_sp = a;
  *kps = b;
  return SA_OK;
}

int32_t sa_mla_partial_bits(int32_t n_q, int32_t k) {
  SA_REQUIRE(n_q >= 1 && k >= 1 && k <= SA_MAX_TOPK, SA_ERR_INVALID_ARG, "mla_partial_bits: n_q=%d, k=%d", n_q, k);
  return mla_partial_bits(n_q, k);
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
  if ((rc = debug_idx(idx, n_q, k, nullptr, q_seq, (hipStream_t)stream))) return rc;
  // (no sequence count here: the gathers stream, as for decode batches)
  return launch_mla(q_abs, kv, nullptr, seq_start, q_seq, idx, n_q, k, w_uv, scale, out, lse, ws,
                    (hipStream_t)stream, false);
}

int32_t sa_mla_sparse_attn_fp8(const void* q_abs, const void* kv_codes, const float* kv_scale, const int64_t* seq_start,
                               const int32_t* q_seq, const int32_t* idx, int32_t n_q, int32_t k, const void* w_uv,
                               float scale, void* out, float* lse, void* ws, size_t ws_bytes, sa_stream_t stream) {
  int32_t rc = check_mla_args(q_abs, kv_codes, seq_start, q_seq, idx, n_q, k, w_uv, scale, out);
  if (rc) return rc;
  if (n_q == 0) return SA_OK;
  SA_REQUIRE(kv_scale, SA_ERR_INVALID_ARG, "mla: FP8 rows without kv_scale");
  const size_t need = mla_workspace_size(n_q, k);
  SA_REQUIRE(ws && ws_bytes >= need, SA_ERR_WORKSPACE, "mla: workspace of %zu bytes, %zu needed", ws_bytes, need);
  SA_REQUIRE(((uintptr_t)ws & 255u) == 0, SA_ERR_INVALID_ARG, "mla: workspace not 256-byte aligned");
  if ((rc = debug_idx(idx, n_q, k, nullptr, q_seq, (hipStream_t)stream))) return rc;
  return launch_mla(q_abs, kv_codes, kv_scale, seq_start, q_seq, idx, n_q, k, w_uv, scale, out, lse, ws,
                    (hipStream_t)stream, false);
}

// Layout: scores [n_q, ld] fp32, the top-k workspace, the attention
// workspace, and the selecting queries' rows [n_q, k] int32 of a shared
// selection (used only when the batch has one; sized for n_sel <= n_q).
size_t sa_layer_stack_workspace_size(int32_t n_q, int64_t ld, int32_t k) {
  if (n_q <= 0 || ld <= 0 || k <= 0) return 256;
  const int32_t kk = k > SA_MAX_TOPK ? SA_MAX_TOPK : k;
  return align256((size_t)n_q * (size_t)ld * 4) + align256(topk_workspace_size(n_q, ld, k)) +
         align256(mla_workspace_size(n_q, kk)) + align256((size_t)n_q * kk * 4);
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
  // Every selected position is below ld; the attention gather addresses
  // positions below SA_MAX_SEQ_LEN (32-bit row offsets within a sequence).
  SA_REQUIRE(ld >= 1 && ld <= SA_MAX_SEQ_LEN, SA_ERR_UNSUPPORTED,
             "layer_stack: ld=%lld outside 1..%d (the longest sequence the attention gather addresses)",
             (long long)ld, SA_MAX_SEQ_LEN);
  SA_REQUIRE(layers[0].is_full, SA_ERR_INVALID_ARG, "layer_stack: layer 0 must run its own indexer");
  // With a shared selection the indexer and the top-k run for the n_sel
  // selecting queries; otherwise every query selects for itself.
  const int32_t n_sel = batch->n_sel;
  SA_REQUIRE(n_sel >= 0 && n_sel <= n_q, SA_ERR_INVALID_ARG, "layer_stack: n_sel=%d outside 0..n_q=%d", n_sel, n_q);
  SA_REQUIRE(n_sel == 0 || (batch->sel_seq && batch->sel_pos && batch->sel_of), SA_ERR_INVALID_ARG,
             "layer_stack: shared selection without sel_seq/sel_pos/sel_of");
  const bool shared_sel = n_sel > 0;
  const int32_t n_rows = shared_sel ? n_sel : n_q;            // rows of scores and top-k
  const int32_t* r_seq = shared_sel ? batch->sel_seq : batch->q_seq;
  const int32_t* r_pos = shared_sel ? batch->sel_pos : batch->q_pos;
  const size_t need = sa_layer_stack_workspace_size(n_q, ld, k);
  SA_REQUIRE(ws && ws_bytes >= need, SA_ERR_WORKSPACE, "layer_stack: workspace of %zu bytes, %zu needed", ws_bytes,
             need);
  SA_REQUIRE(((uintptr_t)ws & 255u) == 0, SA_ERR_INVALID_ARG, "layer_stack: workspace not 256-byte aligned");
  // Check every layer before enqueuing anything.
  for (int l = 0; l < n_layers; ++l) {
    const sa_layer_desc& L = layers[l];
    int32_t rc;
    if (L.is_full) {
      rc = check_indexer_args(L.q_idx, L.w, L.k_idx, batch->seq_start, batch->seq_len, r_seq, r_pos, n_rows,
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
  p += align256(mla_workspace_size(n_q, k));
  int32_t* sel_idx = (int32_t*)p;

  hipStream_t st = (hipStream_t)stream;
  const int32_t* cur_idx = nullptr;
  bool rec_idx = false, rec_topk = false, rec_attn = false;
  int32_t rc;
  // Decode batches score one query per workgroup column; batches with at
  // least 16 queries per sequence (chunked prefill) use the query-blocked
  // indexer.  The top-k then runs its own first-digit histogram pass over the
  // scores.  The decode indexer also clears the top-k's histograms and
  // counters on the side, which saves the top-k a launch of its own for that.
  const int ialgo = indexer_algo(n_rows, batch->n_seq, 0);
  // Queries that share their sequences' rows (chunked prefill, the same test
  // as the indexer's choice): the attention's gathers keep the rows cached.
  const bool shared_rows = indexer_algo(n_q, batch->n_seq, 0) == 2;
  uint32_t* clear = nullptr;
  int64_t n_clear = 0;
  if (ialgo == 1) topk_clear_range(topk_ws, n_rows, ld, &clear, &n_clear);
  if ((rc = debug_batch(batch->seq_start, batch->seq_len, batch->q_seq, batch->q_pos, n_q, batch->n_seq, ld, st)))
    return rc;
  if (shared_sel) {
    if ((rc = debug_batch(batch->seq_start, batch->seq_len, r_seq, r_pos, n_rows, batch->n_seq, ld, st))) return rc;
    if ((rc = debug_share(batch->sel_of, n_sel, batch->q_seq, batch->sel_seq, n_q, st))) return rc;
  }
  for (int l = 0; l < n_layers; ++l) {
    const sa_layer_desc& L = layers[l];
    if (L.is_full) {
      const bool ev = events && !rec_idx && events->indexer_begin && events->indexer_end;
      if (ev && (rc = record(events->indexer_begin, st))) return rc;
      rc = launch_indexer(L.q_idx, L.w, L.k_idx, L.k_scale, batch->seq_start, batch->seq_len, r_seq, r_pos, n_rows,
                          batch->n_seq, scores, ld, ialgo, st, clear, n_clear);
      if (rc) return rc;
      if (ev && (rc = record(events->indexer_end, st))) return rc;
      rec_idx |= ev;
      const bool evt = events && !rec_topk && events->topk_begin && events->topk_end;
      if (evt && (rc = record(events->topk_begin, st))) return rc;
      rc = launch_topk(scores, ld, r_pos, n_rows, k, shared_sel ? sel_idx : L.idx, topk_ws, 0, st, ialgo == 1);
      if (rc) return rc;
      // each query's rows: the selecting query's, cut at the query's position
      if (shared_sel && (rc = launch_share(sel_idx, n_sel, k, batch->sel_of, batch->q_pos, n_q, L.idx, st))) return rc;
      if ((rc = debug_idx(L.idx, n_q, k, batch->q_pos, nullptr, st))) return rc;
      if (evt && (rc = record(events->topk_end, st))) return rc;
      rec_topk |= evt;
      cur_idx = L.idx;
    }
    const bool eva = events && !rec_attn && events->attn_begin && events->attn_end;
    if (eva && (rc = record(events->attn_begin, st))) return rc;
    // consecutive layers put their bf16 partial states in alternate halves of
    // the region, so a layer's streaming stores do not land on lines the
    // previous layer's merge has just read into the L2
    rc = launch_mla(L.q_abs, L.kv, L.kv_scale, batch->seq_start, batch->q_seq, cur_idx, n_q, k, L.w_uv, scale, L.out,
                    nullptr, mla_ws, st, shared_rows, l & 1);
    if (rc) return rc;
    if (eva && (rc = record(events->attn_end, st))) return rc;
    rec_attn |= eva;
  }
  return SA_OK;
}

int32_t sa_share_selection(const int32_t* sel_idx, int32_t n_sel, int32_t k, const int32_t* sel_of,
                           const int32_t* q_pos, int32_t n_q, int32_t* idx, sa_stream_t stream) {
  SA_REQUIRE(n_q >= 0 && n_sel >= 0, SA_ERR_INVALID_ARG, "share_selection: negative count");
  SA_REQUIRE(k >= 1 && k <= SA_MAX_TOPK, SA_ERR_INVALID_ARG, "share_selection: k=%d outside 1..%d", k, SA_MAX_TOPK);
  if (n_q == 0) return SA_OK;
  SA_REQUIRE(n_sel >= 1, SA_ERR_INVALID_ARG, "share_selection: queries without selecting rows");
  SA_REQUIRE(sel_idx && sel_of && q_pos && idx, SA_ERR_INVALID_ARG, "share_selection: null pointer argument");
  SA_REQUIRE(n_q <= 0x7fffffff, SA_ERR_UNSUPPORTED, "share_selection: grid too large");
  hipStream_t st = (hipStream_t)stream;
  int32_t rc = debug_share(sel_of, n_sel, nullptr, nullptr, n_q, st);
  if (rc) return rc;
  return launch_share(sel_idx, n_sel, k, sel_of, q_pos, n_q, idx, st);
}

int32_t sa_q_project(const void* c_q, const void* w_qb, const void* w_iq, const void* w_iw, const int32_t* pos,
                     int32_t n, void* q, void* q_idx, float* w, sa_stream_t stream) {
  SA_REQUIRE(n >= 0, SA_ERR_INVALID_ARG, "q_project: negative n");
  if (n == 0) return SA_OK;
  SA_REQUIRE(c_q && w_qb && pos && q, SA_ERR_INVALID_ARG, "q_project: null pointer argument");
  const bool idx_part = w_iq || w_iw || q_idx || w;
  SA_REQUIRE(!idx_part || (w_iq && w_iw && q_idx && w), SA_ERR_INVALID_ARG,
             "q_project: the indexer part needs all of w_iq, w_iw, q_idx and w (or none)");
  SA_REQUIRE(aligned16(c_q) && aligned16(w_qb) && aligned16(q) &&
                 (!idx_part || (aligned16(w_iq) && aligned16(w_iw) && aligned16(q_idx) && aligned16(w))),
             SA_ERR_INVALID_ARG, "q_project: tensors not 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  int32_t rc = debug_cache(pos, nullptr, n, st);
  if (rc) return rc;
  return launch_q_project(c_q, w_qb, w_iq, w_iw, pos, n, q, q_idx, w, st);
}

int32_t sa_q_absorb(const void* q, const void* w_uk_t, int32_t n, void* q_abs, sa_stream_t stream) {
  SA_REQUIRE(n >= 0, SA_ERR_INVALID_ARG, "q_absorb: negative n");
  if (n == 0) return SA_OK;
  SA_REQUIRE(q && w_uk_t && q_abs, SA_ERR_INVALID_ARG, "q_absorb: null pointer argument");
  SA_REQUIRE(aligned16(q) && aligned16(w_uk_t) && aligned16(q_abs), SA_ERR_INVALID_ARG,
             "q_absorb: tensors not 16-byte aligned");
  return launch_q_absorb(q, w_uk_t, n, q_abs, (hipStream_t)stream);
}

// Per-device address of `scratch`, looked up once per device with that
// device current (the first sa_layer_stack_noalloc call on it).
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

static int32_t scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    set_error("layer_stack_noalloc: no usable current device");
    return SA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      set_error("layer_stack_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                hipGetErrorString(e));
      return SA_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}

size_t sa_layer_stack_noalloc_max_bytes(void) { return SA_NOALLOC_SCRATCH_BYTES; }

int32_t sa_layer_stack_noalloc(const sa_layer_desc* layers, int32_t n_layers, const sa_batch_desc* batch, int32_t k,
                               float scale, const sa_stage_events* events, sa_stream_t stream) {
  SA_REQUIRE(layers && batch, SA_ERR_INVALID_ARG, "layer_stack_noalloc: null descriptor");
  SA_REQUIRE(k >= 1 && k <= SA_MAX_TOPK, SA_ERR_INVALID_ARG, "layer_stack_noalloc: k=%d outside 1..%d", k,
             SA_MAX_TOPK);
  if (n_layers <= 0 || batch->n_q <= 0) return sa_layer_stack(layers, n_layers, batch, k, scale, nullptr, 0, events,
                                                              stream);
  const size_t need = sa_layer_stack_workspace_size(batch->n_q, batch->ld, k);
  SA_REQUIRE(need <= (size_t)SA_NOALLOC_SCRATCH_BYTES, SA_ERR_WORKSPACE,
             "layer_stack_noalloc: %d queries with score rows of %lld need %zu bytes of workspace, more than the "
             "%zu-byte static scratch (use sa_layer_stack with a workspace)",
             batch->n_q, (long long)batch->ld, need, (size_t)SA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  int32_t rc = scratch_for_current_device(&ws);
  if (rc) return rc;
  return sa_layer_stack(layers, n_layers, batch, k, scale, ws, SA_NOALLOC_SCRATCH_BYTES, events, stream);
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
  int32_t rc = debug_cache(pos, dst, n, (hipStream_t)stream);
  if (rc) return rc;
  return launch_cache_write(kv_a, gamma, k_raw, ln_w, ln_b, pos, dst, n, kv_cache, k_cache, (hipStream_t)stream);
}

}  // extern "C"
