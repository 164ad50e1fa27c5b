/*
 * sparse_mla.h -- C ABI of the MI355X (gfx950) indexer-selected sparse MLA
 * library (libsparse_mla.so).
 *
 * The hot path of one attention layer, as described for GLM-5.2 on the pages
 * this library was built from:
 *   models.inteligile.com "GLM-5.2 / Model techniques map", section "Checked
 *     in its code", rows "Indexer-selected sparse attention (DeepSeek Sparse
 *     Attention)" and "Multi-head latent attention";
 *   hermosaai "GLM 5.2", sections "78 layers, IndexShare pattern" and
 *     "MLA + DSA with IndexShare";
 *   llm-architectures-explained "GLM-5.2", section "Every architecture field";
 *   llm-atlas "GLM-5.2", section "Champs bruts du config.json".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Shapes are fixed to the model's configuration: 32 indexer heads of 128,
 * 64 attention heads, cache rows of 576 = 512 latent + 64 rope, 256 value
 * dims, selections of at most 2048 positions.
 *
 * Sequences are packed: a cache (indexer keys or latent rows) is one array of
 * rows, and row seq_start[b] + s holds position s of sequence b (seq_start is
 * int64, so caches may exceed 2^31 rows).  Query t belongs to sequence
 * q_seq[t] and sits at position q_pos[t]; its causal set is positions
 * 0 .. q_pos[t] (diagonal included).
 *
 * Memory: every pointer is caller-owned DEVICE memory, contiguous, row-major,
 * with a 16-byte-aligned base.  bf16 tensors are passed as void*.  The
 * library never allocates or frees device memory, never synchronises the
 * host, and keeps no pointer after a call returns.  Scratch memory comes from
 * a caller-provided workspace whose size the matching *_workspace_size()
 * function returns.
 *
 * Streams: every call enqueues its kernels on `stream` (a hipStream_t; NULL
 * is the default stream) and returns immediately.  Calls are therefore safe
 * to capture in a HIP graph.  Two calls that share a workspace must be
 * ordered on one stream.
 *
 * Errors: every call returns SA_OK (0) or a negative sa_status.  Argument
 * checks happen on the host before anything is enqueued; a rejected call
 * enqueues nothing.  sa_last_error_message() gives a thread-local description
 * of the last failure.  Preconditions that depend on device data (q_pos below
 * the sequence length, q_pos < ld, finite inputs, idx entries in the causal
 * set) are documented per call and are not checked.
 */
#ifndef SPARSE_MLA_H
#define SPARSE_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque HIP handles (layout-compatible with hipStream_t / hipEvent_t). */
typedef struct ihipStream_t* sa_stream_t;
typedef struct ihipEvent_t* sa_event_t;

enum sa_status {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = -1,   /* null pointer, negative size, k out of range, ... */
  SA_ERR_UNSUPPORTED = -2,   /* a request outside the fixed configuration */
  SA_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
  SA_ERR_HIP = -4            /* a HIP launch or runtime call failed */
};

enum {
  SA_INDEX_HEADS = 32,       /* index_n_heads */
  SA_INDEX_DIM = 128,        /* index_head_dim */
  SA_MAX_TOPK = 2048,        /* index_topk */
  SA_HEADS = 64,             /* num_attention_heads */
  SA_LATENT = 512,           /* kv_lora_rank */
  SA_ROPE = 64,              /* qk_rope_head_dim */
  SA_ROW = 576,              /* SA_LATENT + SA_ROPE: one cache row */
  SA_VDIM = 256              /* v_head_dim */
};

/* Library version, (major << 16) | (minor << 8) | patch. */
int32_t sa_version(void);

/* Static text for a status code. */
const char* sa_status_string(int32_t status);

/* Thread-local text describing the last failed call on this thread ("" if none). */
const char* sa_last_error_message(void);

/*
 * sa_indexer_score -- indexer scores of each query against its causal keys.
 *
 * Defines (the pages give the indexer's shapes -- index_n_heads heads of
 * index_head_dim and one key per token shared by all heads, "Indexer-selected
 * sparse attention" row -- and the score is taken as):
 *     scores[t, s] = sum_h w[t, h] * max(0, q_idx[t, h, :] . k_idx[seq_start[q_seq[t]] + s, :])
 * for 0 <= s <= q_pos[t], and scores[t, s] = -inf for q_pos[t] < s < ld.
 * Products of bf16 values are exact in fp32; sums are fp32.
 *
 *   q_idx     bf16  [n_q, 32, 128]   indexer queries
 *   w         fp32  [n_q, 32]        per-query head weights
 *   k_idx     bf16  [total_rows, 128] packed indexer keys
 *   seq_start int64 [n_seq]          first row of each sequence
 *   q_seq     int32 [n_q]            sequence of each query (0 <= q_seq < n_seq)
 *   q_pos     int32 [n_q]            position of each query (0 <= q_pos < ld,
 *                                    and below its sequence's length)
 *   scores    fp32  [n_q, ld]        output; every entry is written
 *   ld        row length of scores (>= 1, < 2^31)
 * n_q = 0 is a no-op.
 */
int32_t sa_indexer_score(const void* q_idx, const float* w, const void* k_idx,
                         const int64_t* seq_start, const int32_t* q_seq, const int32_t* q_pos,
                         int32_t n_q, int32_t n_seq, float* scores, int64_t ld,
                         sa_stream_t stream);

/*
 * sa_topk_select -- exact top-k positions of each score row.
 *
 * Defines ("Indexer-selected sparse attention" row: the kept count is
 * min(index_topk, number of scores), returned as int32 positions): row t keeps
 * the k_eff = min(k, q_pos[t] + 1) largest scores[t, 0 .. q_pos[t]].  Equal
 * scores go to the lower position (the pages state no tie order; this is the
 * reading taken); -0.0 and +0.0 are equal.  The kept positions are written to
 * idx[t, 0 .. k_eff) in ascending order and idx[t, k_eff .. k) = -1.
 * The result is deterministic.  NaN scores are not allowed.
 *
 *   scores  fp32  [n_q, ld]   (entries beyond q_pos[t] are not read)
 *   q_pos   int32 [n_q]       0 <= q_pos[t] < ld
 *   k       1 .. 2048
 *   idx     int32 [n_q, k]    output
 *   ws      workspace of at least sa_topk_workspace_size(n_q, ld, k) bytes
 */
size_t sa_topk_workspace_size(int32_t n_q, int64_t ld, int32_t k);
int32_t sa_topk_select(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q, int32_t k,
                       int32_t* idx, void* ws, size_t ws_bytes, sa_stream_t stream);

/*
 * sa_mla_sparse_attn -- absorbed multi-head latent attention over selected
 * rows, then the per-head value up-projection.
 *
 * Defines ("Multi-head latent attention" row: a 512-wide latent after
 * kv_a_layernorm plus a 64-wide decoupled rope key per token, kv_b_proj
 * splitting per head into 192 key rows and 256 value rows; the key half is
 * folded into the query, so q_abs is 576 wide, and the value half W_UV is
 * applied after attention; plain softmax with no sink and no output gate):
 * for query t, head h, over the rows R_j = kv[seq_start[q_seq[t]] + idx[t, j]]
 * with idx[t, j] >= 0 (entries of -1 are skipped):
 *     z_j  = scale * (q_abs[t, h, :] . R_j)                (576 dims)
 *     obar = sum_j softmax(z)_j * R_j[0 .. 512)
 *     out[t, h, :] = bf16_rne(W_UV[h] @ obar)              ([256, 512] @ [512])
 * Softmax is computed in fp32 with a running maximum; the softmax weights
 * may enter the value product as bf16.  A row with no selected entry gives 0.
 *
 *   q_abs   bf16  [n_q, 64, 576]
 *   kv      bf16  [total_rows, 576] packed cache rows of this layer
 *   idx     int32 [n_q, k]    positions in 0 .. q_pos[t], or -1
 *   k       1 .. 2048
 *   w_uv    bf16  [64, 256, 512]
 *   scale   softmax scale (1/sqrt(256) = 1/16 for this model)
 *   out     bf16  [n_q, 64, 256]  output
 *   lse     fp32  [n_q, 64] or NULL: natural-log log-sum-exp of z (-inf if empty)
 *   ws      workspace of at least sa_mla_workspace_size(n_q, k) bytes
 */
size_t sa_mla_workspace_size(int32_t n_q, int32_t k);
int32_t sa_mla_sparse_attn(const void* q_abs, const void* kv, const int64_t* seq_start,
                           const int32_t* q_seq, const int32_t* idx, int32_t n_q, int32_t k,
                           const void* w_uv, float scale, void* out, float* lse,
                           void* ws, size_t ws_bytes, sa_stream_t stream);

/*
 * sa_layer_stack -- the hot path over a stack of layers with IndexShare.
 *
 * Defines (hermosaai "GLM 5.2", "MLA + DSA with IndexShare": a full layer runs
 * the indexer and picks the top 2048 positions per query; the following shared
 * layers reuse that selection instead of scoring again): layers run in order;
 * a full layer (is_full != 0) runs sa_indexer_score and sa_topk_select into its
 * own idx, a shared layer uses the idx of the latest full layer before it; every
 * layer then runs sa_mla_sparse_attn with its own q_abs, kv and w_uv.  layers[0]
 * must be full.  sa_layer_is_full() gives the model's own pattern.
 *
 * Fields of sa_layer_desc (device pointers):
 *   full layers only: q_idx bf16 [n_q,32,128], w fp32 [n_q,32], k_idx bf16 [rows,128],
 *                     idx int32 [n_q, k] (output: this layer's selection)
 *   every layer:      q_abs bf16 [n_q,64,576], kv bf16 [rows,576], w_uv bf16 [64,256,512],
 *                     out bf16 [n_q,64,256] (output)
 * sa_batch_desc: seq_start int64 [n_seq], q_seq int32 [n_q], q_pos int32 [n_q], the
 * counts, and ld (score row length, > max q_pos).
 * events: optional (NULL or any NULL member = not recorded); hipEvents recorded on
 * `stream` just before and after the named stage of the FIRST layer where it runs.
 *   ws  workspace of at least sa_layer_stack_workspace_size(n_q, ld, k) bytes
 */
typedef struct sa_layer_desc {
  int32_t is_full;
  const void* q_idx;
  const float* w;
  const void* k_idx;
  int32_t* idx;
  const void* q_abs;
  const void* kv;
  const void* w_uv;
  void* out;
} sa_layer_desc;

typedef struct sa_batch_desc {
  const int64_t* seq_start;
  const int32_t* q_seq;
  const int32_t* q_pos;
  int32_t n_q;
  int32_t n_seq;
  int64_t ld;
} sa_batch_desc;

typedef struct sa_stage_events {
  sa_event_t indexer_begin, indexer_end;
  sa_event_t topk_begin, topk_end;
  sa_event_t attn_begin, attn_end;
} sa_stage_events;

size_t sa_layer_stack_workspace_size(int32_t n_q, int64_t ld, int32_t k);
int32_t sa_layer_stack(const sa_layer_desc* layers, int32_t n_layers, const sa_batch_desc* batch,
                       int32_t k, float scale, void* ws, size_t ws_bytes,
                       const sa_stage_events* events, sa_stream_t stream);

/* IndexShare pattern of the 78-layer model: 1 if layer runs its own indexer
 * (layers 0-2, then every layer l with l mod 4 == 2), else 0; -1 if layer < 0. */
int32_t sa_layer_is_full(int32_t layer);

/*
 * sa_cache_write -- the step before the path: turn n new tokens' projections
 * into their cache rows (and, optionally, their indexer keys).
 *
 * Defines ("Multi-head latent attention" row: kv_a_layernorm, an RMSNorm over
 * the 512-wide latent, and a decoupled 64-wide rope key; "QK normalization"
 * row: k_norm, a LayerNorm of the indexer key projection; "Partial RoPE" and
 * "YaRN RoPE scaling" rows: 64 rotated dims, default rope type, theta 8e6;
 * llm-atlas config: rms_norm_eps 1e-5, rope_interleave, indexer_rope_interleave):
 *     kv_cache[dst[i], 0:512]   = latent / sqrt(mean(latent^2) + 1e-5) * gamma
 *     kv_cache[dst[i], 512:576] = rope(kv_a[i, 512:576], pos[i])
 *     k_cache[dst[i], :]        = LN(k_raw[i]) * ln_w + ln_b, then
 *                                 dims 64..127 <- rope(dims 64..127, pos[i])
 * where rope turns each adjacent pair (2j, 2j + 1) by pos * 8e6^(-2j / 64)
 * and LN uses the population variance and eps 1e-5.  The pages give no eps
 * for k_norm and do not say which half of the indexer key turns: this takes
 * rms_norm_eps and the last 64 dims (the main attention's nope/rope order).
 * Computed in fp64; each stored value is rounded once to bf16 (through fp32,
 * both steps to nearest even).
 *
 *   kv_a      bf16  [n, 576]  kv_a_proj output (512 latent, then 64 rope key), 16-byte aligned
 *   gamma     bf16  [512]     kv_a_layernorm weight, 16-byte aligned
 *   k_raw     bf16  [n, 128]  indexer key projection, or NULL to skip the indexer key
 *   ln_w      bf16  [128]     k_norm weight (ignored when k_raw is NULL)
 *   ln_b      bf16  [128]     k_norm bias   (ignored when k_raw is NULL)
 *   pos       int32 [n]       position of each token within its sequence (>= 0)
 *   dst       int64 [n]       row of each token in kv_cache / k_cache (distinct rows)
 *   kv_cache  bf16  [*, 576]  written at rows dst[i] only, 16-byte aligned
 *   k_cache   bf16  [*, 128]  written at rows dst[i] only (ignored when k_raw is NULL)
 * Everything is device memory owned by the caller; nothing is kept after the
 * call.  n = 0 launches nothing.  Rows in range and distinct are preconditions
 * the call does not check (checking would need the data on the host).
 */
int32_t sa_cache_write(const void* kv_a, const void* gamma, const void* k_raw, const void* ln_w,
                       const void* ln_b, const int32_t* pos, const int64_t* dst, int32_t n,
                       void* kv_cache, void* k_cache, sa_stream_t stream);

/*
 * Variants that pin an internal algorithm, for tests and measurements.
 * algo 0 = automatic (what the entry points above use).
 *   indexer: 1 = one query per workgroup (streams keys once per query),
 *            2 = query blocks sharing key tiles (MFMA over queries x heads);
 *            automatic picks 2 when n_q >= 64 and n_q >= 16 * n_seq (at least
 *            16 queries per sequence on average), else 1.
 *   topk:    1 = rows split over many workgroups with candidate compaction,
 *            2 = one workgroup per row, full radix passes (the exact fallback).
 * Returns SA_ERR_INVALID_ARG for an unknown algo.
 */
int32_t sa_indexer_score_algo(const void* q_idx, const float* w, const void* k_idx,
                              const int64_t* seq_start, const int32_t* q_seq, const int32_t* q_pos,
                              int32_t n_q, int32_t n_seq, float* scores, int64_t ld,
                              int32_t algo, sa_stream_t stream);
int32_t sa_topk_select_algo(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q,
                            int32_t k, int32_t* idx, void* ws, size_t ws_bytes, int32_t algo,
                            sa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MLA_H */
