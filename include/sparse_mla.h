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
 * of the last failure.  The shapes themselves are compile-time constants (the
 * enum below), so the host checks cover counts, pointers, alignment, k, ld,
 * the workspace size and grid limits.  Preconditions that depend on device
 * data (q_seq < n_seq, q_pos below its sequence's length and below ld, idx
 * entries in the causal set, sequences shorter than SA_MAX_SEQ_LEN, no NaN
 * scores) are documented per call.  Release builds do not check them (that
 * would need the data on the host, i.e. a synchronisation); the SA_DEBUG
 * build (libsparse_mla_debug.so) checks them on the device inside every call
 * and reports the first violation through sa_debug_check().  The indexer
 * never reads past its sequence's keys even when q_pos violates them: it
 * clamps the causal set at seq_len - 1.
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
  SA_ERR_HIP = -4,           /* a HIP launch or runtime call failed */
  SA_ERR_DEBUG = -5          /* SA_DEBUG build: a device-side precondition check failed */
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

/* Longest sequence (rows of one layer's cache) the attention gather
 * addresses: row offsets within a sequence are 32-bit byte offsets of
 * 1152-byte rows, so position * 1152 + 1151 < 2^32.  The model's 1,048,576
 * tokens are well inside. */
#define SA_MAX_SEQ_LEN 3728270

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
 *   seq_len   int32 [n_seq]          cached keys of each sequence (0 .. SA_MAX_SEQ_LEN)
 *   q_seq     int32 [n_q]            sequence of each query (0 <= q_seq < n_seq)
 *   q_pos     int32 [n_q]            position of each query (0 <= q_pos < ld,
 *                                    and q_pos < seq_len[q_seq])
 *   scores    fp32  [n_q, ld]        output; every entry is written
 *   ld        row length of scores (>= 1, < 2^31)
 * n_q = 0 is a no-op.  Keys are read only at positions below seq_len: a query
 * whose q_pos breaks q_pos < seq_len gets -inf from seq_len on (and the
 * SA_DEBUG build reports it).
 */
int32_t sa_indexer_score(const void* q_idx, const float* w, const void* k_idx,
                         const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq,
                         const int32_t* q_pos, int32_t n_q, int32_t n_seq, float* scores, int64_t ld,
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
 *   scores  fp32  [n_q, ld]   (entries beyond q_pos[t] may hold anything: they
 *                             may be read but never affect the result)
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
 *   idx     int32 [n_q, k]    positions in 0 .. q_pos[t], or -1 (positions
 *                             below SA_MAX_SEQ_LEN: the gather's row offsets
 *                             within a sequence are 32-bit)
 *   k       1 .. 2048
 *   w_uv    bf16  [64, 256, 512]
 *   scale   softmax scale (1/sqrt(256) = 1/16 for this model)
 *   out     bf16  [n_q, 64, 256]  output
 *   lse     fp32  [n_q, 64] or NULL: natural-log log-sum-exp of z (-inf if empty)
 *   ws      workspace of at least sa_mla_workspace_size(n_q, k) bytes
 */
size_t sa_mla_workspace_size(int32_t n_q, int32_t k);
/* How sa_mla_sparse_attn (and its FP8 variant) slices each query's selection
 * for n_q queries of k entries: *n_sp slices of *kps entries (the last may be
 * shorter, none is empty), slice s taking entries s * kps .. of each idx row;
 * with *n_sp > 1 the slices' partial softmax states are combined by a
 * log-sum-exp merge.  For workspace planning and error analysis. */
int32_t sa_mla_split_info(int32_t n_q, int32_t k, int32_t* n_sp, int32_t* kps);
/* The precision of those partial states: 0 (one slice, none), 32 (fp32), or
 * 16 (each slice's unnormalised weighted row sum rounded to bf16, round to
 * nearest even, before the merge; used for one 32-head block per workgroup and
 * 2..8 slices, i.e. decode batches of 16..63 queries at k = 2048).  A negative
 * status for arguments outside the ranges above.  For error analysis. */
int32_t sa_mla_partial_bits(int32_t n_q, int32_t k);
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
 *   FP8 caches:       k_scale / kv_scale non-NULL: k_idx / kv hold E4M3 codes (see the
 *                     FP8 calls below) and these are their per-row scales; NULL: bf16.
 * sa_batch_desc: seq_start int64 [n_seq], seq_len int32 [n_seq], q_seq int32 [n_q],
 * q_pos int32 [n_q], the counts, and ld (score row length, > max q_pos; at most
 * SA_MAX_SEQ_LEN, so every selected position is one the gather can address).
 *
 * Shared selection for speculative / multi-token-prediction decode (llm-atlas
 * "GLM-5.2", config field index_share_for_mtp_iteration; hermosaai "GLM 5.2",
 * "78 layers, IndexShare pattern": the Multi-Token Prediction layer serves
 * speculative decoding).  With n_sel = 0 every query selects for itself.  With
 * 1 <= n_sel <= n_q, full layers run the indexer and top-k only for n_sel
 * selecting queries (sequence sel_seq[s], position sel_pos[s]; the full
 * layers' q_idx and w then hold n_sel rows), and query t uses the selection of
 * selecting query sel_of[t] cut at its own position (sa_share_selection): the
 * draft tokens of a sequence verified in one step share one indexer pass,
 * normally the one of their last token, whose causal set holds the others'.
 * Preconditions: 0 <= sel_of[t] < n_sel, sel_seq[sel_of[t]] == q_seq[t], the
 * selecting queries obey the batch rules; the idx outputs of full layers hold
 * the per-query rows.
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
  const float* k_scale;     /* non-NULL: k_idx holds FP8 codes [rows, 128] with these scales [rows] */
  const float* kv_scale;    /* non-NULL: kv holds FP8 codes [rows, 576] with these scales [rows] */
} sa_layer_desc;

typedef struct sa_batch_desc {
  const int64_t* seq_start;
  const int32_t* seq_len;
  const int32_t* q_seq;
  const int32_t* q_pos;
  int32_t n_q;
  int32_t n_seq;
  int64_t ld;
  int32_t n_sel;            /* 0: no shared selection */
  const int32_t* sel_seq;   /* [n_sel] */
  const int32_t* sel_pos;   /* [n_sel] */
  const int32_t* sel_of;    /* [n_q] */
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

/*
 * sa_layer_stack_noalloc -- sa_layer_stack for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same call without a workspace argument.  Its
 * workspace is a static device array of SA_NOALLOC_SCRATCH_BYTES (64 MiB) per
 * GPU, part of the library's code object, held until the process ends; the
 * call allocates and frees nothing.  A batch whose
 * sa_layer_stack_workspace_size(n_q, ld, k) exceeds that size is rejected with
 * SA_ERR_WORKSPACE before anything is enqueued (64 MiB holds, e.g., 16
 * queries over 131,072-position rows, or 64 over 32,768).  Every call on one
 * GPU shares that GPU's array and leaves its contents behind (the call clears
 * what it needs at zero itself): two calls that overlap on one GPU (on
 * different streams, or from different threads) race and must not be issued.
 * The first call on a device looks up the array's address on that device.
 * Results equal sa_layer_stack's bit for bit.
 */
#define SA_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t sa_layer_stack_noalloc_max_bytes(void);
int32_t sa_layer_stack_noalloc(const sa_layer_desc* layers, int32_t n_layers, const sa_batch_desc* batch,
                               int32_t k, float scale, const sa_stage_events* events, sa_stream_t stream);

/*
 * sa_share_selection -- per-token selection rows from shared ones (the step
 * sa_layer_stack takes for a shared selection, see sa_batch_desc).
 *
 * Defines (the reading of index_share_for_mtp_iteration above): token t takes
 * row sel_of[t] of sel_idx and keeps its entries p with 0 <= p <= q_pos[t],
 * in the row's order, then -1 padding:
 *   idx[t, :] = [p in sel_idx[sel_of[t], :] if 0 <= p <= q_pos[t]] + [-1, ...]
 *
 *   sel_idx int32 [n_sel, k]   shared rows (positions, -1 padding; any order)
 *   sel_of  int32 [n_q]        0 <= sel_of[t] < n_sel
 *   q_pos   int32 [n_q]
 *   k       1 .. 2048
 *   idx     int32 [n_q, k]     output (must not overlap sel_idx)
 * Exact integer work; deterministic.
 */
int32_t sa_share_selection(const int32_t* sel_idx, int32_t n_sel, int32_t k, const int32_t* sel_of,
                           const int32_t* q_pos, int32_t n_q, int32_t* idx, sa_stream_t stream);

/*
 * sa_q_project -- the query projections of n new tokens from their q_lora
 * activation (the step before sa_indexer_score and sa_mla_sparse_attn on the
 * query side).
 *
 * Defines ("Multi-head latent attention" row: a q_lora_rank = 2048
 * bottleneck; "Partial RoPE" row: each head's query is [192 nope ; 64 rope]
 * and only the rope part turns; "Indexer-selected sparse attention" row: 32
 * indexer heads of 128; llm-atlas config: qk_head_dim 256, rope_interleave,
 * indexer_rope_interleave, rope_theta 8e6):
 *     q[t]     = bf16(W_QB c_q[t]) as [64][256]; dims 192..255 of each head
 *                turned in pairs (2j, 2j+1) by pos[t] * 8e6^(-2j/64)
 *     q_idx[t] = bf16(W_IQ c_q[t]) as [32][128]; dims 64..127 turned the same way
 *     w[t]     = W_IW c_q[t] (fp32)
 * The pages print neither the indexer query's nor the head weights' source;
 * both are taken from q_lora, and the indexer query turns its last 64 dims like
 * the indexer key (sa_cache_write).  Sums in fp32; each stored bf16 value is
 * rounded to nearest even; the pairs turn in fp64 from the rounded values and
 * are rounded again.
 *
 *   c_q    bf16 [n, 2048]          q_lora activation
 *   w_qb   bf16 [64 * 256, 2048]   q_b_proj weight (rows: head-major, [192 nope ; 64 rope])
 *   w_iq   bf16 [32 * 128, 2048]   indexer query weight, or NULL
 *   w_iw   bf16 [32, 2048]         head-weight projection, or NULL
 *   pos    int32 [n]               token positions (>= 0)
 *   q      bf16 [n, 64, 256]       output
 *   q_idx  bf16 [n, 32, 128]       output, or NULL
 *   w      fp32 [n, 32]            output, or NULL
 * w_iq, w_iw, q_idx and w are all given or all NULL (NULL: only q, e.g. for a
 * layer that reuses another layer's selection).  Every pointer 16-byte aligned.
 */
int32_t sa_q_project(const void* c_q, const void* w_qb, const void* w_iq, const void* w_iw,
                     const int32_t* pos, int32_t n, void* q, void* q_idx, float* w,
                     sa_stream_t stream);

/*
 * sa_q_absorb -- fold the key half of kv_b_proj into the query.
 *
 * Defines ("Multi-head latent attention" row: kv_b_proj maps the 512-wide
 * latent to, per head, 192 key rows W_UK[h] and 256 value rows): with
 * q_nope = q[t, h, 0:192] and q_rope = q[t, h, 192:256],
 *     q_abs[t, h, 0:512]   = bf16(W_UK[h]^T q_nope)      (fp32 sums)
 *     q_abs[t, h, 512:576] = q_rope
 * so that q_abs[t, h] . [latent ; k_rope] = q_nope . (W_UK[h] latent) +
 * q_rope . k_rope: the explicit logit over the cache row.
 *
 *   q       bf16 [n, 64, 256]   (sa_q_project's output)
 *   w_uk_t  bf16 [64, 512, 192] W_UK[h]^T per head: element [h][c][d] =
 *                               kv_b_proj.weight[h * 448 + d][c] (the transpose
 *                               of each head's 192 key rows, arranged once when
 *                               the weights are loaded)
 *   q_abs   bf16 [n, 64, 576]   output (sa_mla_sparse_attn's q_abs)
 */
int32_t sa_q_absorb(const void* q, const void* w_uk_t, int32_t n, void* q_abs, sa_stream_t stream);

/*
 * FP8 caches (models.inteligile.com techniques map, "inference quantization":
 * FP8 inference; llm-atlas "GLM-5.2", "Faits clés": precision fp8).  The pages
 * give no format or scaling; the reading taken: OCP E4M3 codes (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits, subnormals m * 2^-9, largest
 * finite magnitude 448 = code 0x7E) with one fp32 scale per cache row (per
 * 576-wide latent row, per 128-wide indexer key).  A stored row means
 * scale * value(code); it halves the bytes the decode path streams.
 *
 * sa_quantize_rows_fp8 -- rows of bf16 values to codes and scales:
 *     scale = max_i |x_i| / 448 (fp32, correctly rounded; 1 for an all-zero row)
 *     code_i = E4M3 nearest to x_i / scale (fp32 quotient, ties to the even
 *              code, magnitudes above 448 saturating to 448; zero is 0x00)
 *   src       bf16 [n_rows, d], d = 576 (cache rows) or 128 (indexer keys)
 *   dst_rows  int64 [n_rows] or NULL: row i goes to row dst_rows[i] of codes/scales
 *   codes     uint8 [*, d], scales fp32 [*]
 * Bit-exact integer decisions (the same fp32 quotient on any conforming
 * implementation).
 *
 * sa_fp8_decode -- n codes (n a multiple of 16) to their bf16 values (exact,
 * unscaled): the decoder the FP8 kernels use.
 *
 * sa_indexer_score_fp8 / sa_indexer_score_fp8_algo -- sa_indexer_score (and its
 * algo variant) over keys stored as codes k_codes uint8 [rows, 128] with
 * k_scale fp32 [rows]: the key of row r is k_scale[r] * value(k_codes[r]).
 * Computed as k_scale[r] times the score of the decoded codes (ReLU commutes
 * with a positive scale), the codes exact in bf16.
 *
 * sa_mla_sparse_attn_fp8 -- sa_mla_sparse_attn over cache rows stored as codes
 * kv_codes uint8 [rows, 576] with kv_scale fp32 [rows]: row r is
 * kv_scale[r] * value(kv_codes[r]).  Each logit is the decoded row's logit
 * times the row's scale, and the softmax weight enters the value product
 * multiplied by the scale (bf16), the normaliser summing the weights alone.
 * Same workspace as sa_mla_sparse_attn.
 */
int32_t sa_quantize_rows_fp8(const void* src, int64_t n_rows, int32_t d, const int64_t* dst_rows,
                             void* codes, float* scales, sa_stream_t stream);
int32_t sa_fp8_decode(const void* codes, int64_t n, void* out, sa_stream_t stream);
int32_t sa_indexer_score_fp8(const void* q_idx, const float* w, const void* k_codes, const float* k_scale,
                             const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq,
                             const int32_t* q_pos, int32_t n_q, int32_t n_seq, float* scores, int64_t ld,
                             sa_stream_t stream);
int32_t sa_indexer_score_fp8_algo(const void* q_idx, const float* w, const void* k_codes, const float* k_scale,
                                  const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq,
                                  const int32_t* q_pos, int32_t n_q, int32_t n_seq, float* scores, int64_t ld,
                                  int32_t algo, sa_stream_t stream);
int32_t sa_mla_sparse_attn_fp8(const void* q_abs, const void* kv_codes, const float* kv_scale,
                               const int64_t* seq_start, const int32_t* q_seq, const int32_t* idx, int32_t n_q,
                               int32_t k, const void* w_uv, float scale, void* out, float* lse, void* ws,
                               size_t ws_bytes, sa_stream_t stream);

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
 *            2 = one workgroup per row, full radix passes (the exact fallback);
 *            automatic picks 2 for rows of at most 12,288 scores (ld), else 1.
 * Returns SA_ERR_INVALID_ARG for an unknown algo.
 */
int32_t sa_indexer_score_algo(const void* q_idx, const float* w, const void* k_idx,
                              const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq,
                              const int32_t* q_pos, int32_t n_q, int32_t n_seq, float* scores,
                              int64_t ld, int32_t algo, sa_stream_t stream);

/*
 * Device-side precondition checks (the SA_DEBUG build).
 *
 * In libsparse_mla_debug.so (built with -DSA_DEBUG) every entry point above
 * also enqueues, on its stream and before its own kernels, a check of the
 * preconditions that depend on device data:
 *   batch:   0 <= q_seq[t] < n_seq; 0 <= q_pos[t] < seq_len[q_seq[t]];
 *            q_pos[t] < ld; 0 <= seq_len[b] <= SA_MAX_SEQ_LEN; seq_start[b] >= 0
 *   top-k:   0 <= q_pos[t] < ld; no NaN in scores[t, 0 .. q_pos[t]]
 *   attention: -1 <= idx[t, j] < SA_MAX_SEQ_LEN (and, inside sa_layer_stack,
 *            idx[t, j] <= q_pos[t]); q_seq[t] >= 0
 *   shared selection: 0 <= sel_of[t] < n_sel; sel_seq[sel_of[t]] == q_seq[t]
 *            (and the selecting queries obey the batch rules)
 *   cache write: pos[i] >= 0, dst[i] >= 0;  query projection: pos[t] >= 0
 * The first violation (and a count of all of them) is kept in a device-side
 * record.  The check kernels only read; the call's own kernels still run.
 *
 * sa_debug_check(stream) waits for `stream`, reads the record and clears it.
 * It returns SA_OK when nothing was violated since the last check, and
 * SA_ERR_DEBUG otherwise, with sa_last_error_message() naming the check, the
 * query or sequence, and the offending value.  In the release library it does
 * nothing and returns SA_ERR_UNSUPPORTED.  sa_debug_enabled() is 1 in the
 * SA_DEBUG build, 0 otherwise.
 *
 * sa_debug_check_host runs the batch and attention-index checks above on
 * HOST arrays (same rules, same messages), in both builds: for callers that
 * keep the batch description on the host, and to exercise the checks without
 * a GPU.  idx may be NULL (k is then ignored).  Returns SA_OK or SA_ERR_DEBUG;
 * SA_ERR_INVALID_ARG for null arrays with a non-zero count.
 */
int32_t sa_debug_enabled(void);
int32_t sa_debug_check(sa_stream_t stream);
int32_t sa_debug_check_host(const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq,
                            const int32_t* q_pos, int32_t n_q, int32_t n_seq, int64_t ld,
                            const int32_t* idx, int32_t k);
int32_t sa_topk_select_algo(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q,
                            int32_t k, int32_t* idx, void* ws, size_t ws_bytes, int32_t algo,
                            sa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MLA_H */
