// Device-side precondition checks of the SA_DEBUG build, sa_debug_check, and
// the host-array variant of the same checks.
//
// The checks cover what the release library documents but cannot check
// without the data on the host: queries inside their sequence and inside the
// score rows, sequences short enough for the attention gather's 32-bit row
// offsets, selection entries inside the causal set, scores without NaN
// (models.inteligile.com "GLM-5.2 / Model techniques map", "Checked in its
// code", row "Indexer-selected sparse attention": each query keeps at most
// index_topk of its causal positions, as int32 positions).  The check kernels
// only read the caller's data and record the first violation in a per-device
// word array; they never stop the call's own kernels.
#include <stdio.h>

#include "debug_checks.h"
#include "sa_common.h"

namespace sa_dbg {

// The record: [0] first code, [1] item, [2] slot, [3] value, [4] count.
__device__ uint32_t g_rec[kRecWords];

__device__ __forceinline__ void report(uint32_t code, uint32_t item, uint32_t slot, int64_t val) {
  atomicAdd(&g_rec[4], 1u);
  if (atomicCAS(&g_rec[0], 0u, code) == 0u) {
    g_rec[1] = item;
    g_rec[2] = slot;
    g_rec[3] = (uint32_t)val;
  }
}

__global__ void batch_kernel(const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq,
                             const int32_t* q_pos, int32_t n_q, int32_t n_seq, int64_t ld) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n = n_q > n_seq ? n_q : n_seq;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    int64_t val = 0;
    if (i < n_seq) {
      const uint32_t c = check_sequence(seq_start[i], seq_len[i], &val);
      if (c) report(c, (uint32_t)i, 0, val);
    }
    if (i < n_q) {
      const uint32_t c = check_query(q_seq[i], q_pos[i], seq_len, n_seq, ld, &val);
      if (c) report(c, (uint32_t)i, 0, val);
    }
  }
}

// Selection entries; q_pos may be null (causal bound unknown), q_seq may be
// null (not checked).
__global__ void idx_kernel(const int32_t* idx, int32_t n_q, int32_t k, const int32_t* q_pos, const int32_t* q_seq) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n = (int64_t)n_q * k;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int32_t t = (int32_t)(i / k), j = (int32_t)(i - (int64_t)t * k);
    int64_t val = 0;
    if (j == 0 && q_seq && q_seq[t] < 0) report(Q_SEQ_RANGE, (uint32_t)t, 0, q_seq[t]);
    const uint32_t c = check_idx(idx[i], q_pos ? q_pos[t] : -1, &val);
    if (c) report(c, (uint32_t)t, (uint32_t)j, val);
  }
}

// The part of each score row the top-k reads: q_pos first, then NaN.
__global__ void scores_kernel(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q) {
  for (int32_t t = blockIdx.x; t < n_q; t += gridDim.x) {
    const int32_t p = q_pos[t];
    if (p < 0 || (int64_t)p >= ld) {
      if (threadIdx.x == 0) report(p < 0 ? Q_POS_NEG : Q_POS_BEYOND_LD, (uint32_t)t, 0, p);
      continue;
    }
    const float* row = scores + (int64_t)t * ld;
    for (int64_t s = threadIdx.x; s <= p; s += blockDim.x)
      if (row[s] != row[s]) report(SCORE_NAN, (uint32_t)t, (uint32_t)s, s);
  }
}

__global__ void share_kernel(const int32_t* sel_of, int32_t n_sel, const int32_t* q_seq, const int32_t* sel_seq,
                             int32_t n_q) {
  for (int32_t t = blockIdx.x * blockDim.x + threadIdx.x; t < n_q; t += gridDim.x * blockDim.x) {
    int64_t val = 0;
    const uint32_t c = check_share(sel_of[t], n_sel, q_seq ? q_seq[t] : 0, q_seq ? sel_seq : nullptr, &val);
    if (c) report(c, (uint32_t)t, 0, val);
  }
}

__global__ void cache_kernel(const int32_t* pos, const int64_t* dst, int32_t n) {
  for (int32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    if (pos[i] < 0) report(CACHE_POS_NEG, (uint32_t)i, 0, pos[i]);
    if (dst && dst[i] < 0) report(CACHE_DST_NEG, (uint32_t)i, 0, dst[i]);
  }
}

}  // namespace sa_dbg

namespace sa_host {

static int dbg_grid(int64_t n, int threads) {
  const int64_t g = (n + threads - 1) / threads;
  return (int)(g < 1 ? 1 : (g > 1024 ? 1024 : g));
}

// Hooks called by the entry points before their own kernels.  They enqueue
// the checks in the SA_DEBUG build and do nothing otherwise.
int32_t debug_batch(const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq, const int32_t* q_pos,
                    int32_t n_q, int32_t n_seq, int64_t ld, hipStream_t stream) {
#ifdef SA_DEBUG
  const int64_t n = n_q > n_seq ? n_q : n_seq;
  if (n <= 0) return SA_OK;
  hipLaunchKernelGGL(sa_dbg::batch_kernel, dim3(dbg_grid(n, 256)), dim3(256), 0, stream, seq_start, seq_len, q_seq,
                     q_pos, n_q, n_seq, ld);
  return check_launch("debug batch check");
#else
  (void)seq_start, (void)seq_len, (void)q_seq, (void)q_pos, (void)n_q, (void)n_seq, (void)ld, (void)stream;
  return SA_OK;
#endif
}

int32_t debug_idx(const int32_t* idx, int32_t n_q, int32_t k, const int32_t* q_pos, const int32_t* q_seq,
                  hipStream_t stream) {
#ifdef SA_DEBUG
  if (n_q <= 0 || k <= 0) return SA_OK;
  hipLaunchKernelGGL(sa_dbg::idx_kernel, dim3(dbg_grid((int64_t)n_q * k, 256)), dim3(256), 0, stream, idx, n_q, k,
                     q_pos, q_seq);
  return check_launch("debug index check");
#else
  (void)idx, (void)n_q, (void)k, (void)q_pos, (void)q_seq, (void)stream;
  return SA_OK;
#endif
}

int32_t debug_scores(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q, hipStream_t stream) {
#ifdef SA_DEBUG
  if (n_q <= 0) return SA_OK;
  hipLaunchKernelGGL(sa_dbg::scores_kernel, dim3(n_q < 1024 ? n_q : 1024), dim3(256), 0, stream, scores, ld, q_pos,
                     n_q);
  return check_launch("debug score check");
#else
  (void)scores, (void)ld, (void)q_pos, (void)n_q, (void)stream;
  return SA_OK;
#endif
}

// q_seq / sel_seq may be null (the standalone sharing call has no
// sequences): then only the range of sel_of is checked.
int32_t debug_share(const int32_t* sel_of, int32_t n_sel, const int32_t* q_seq, const int32_t* sel_seq, int32_t n_q,
                    hipStream_t stream) {
#ifdef SA_DEBUG
  if (n_q <= 0) return SA_OK;
  hipLaunchKernelGGL(sa_dbg::share_kernel, dim3(dbg_grid(n_q, 256)), dim3(256), 0, stream, sel_of, n_sel, q_seq,
                     sel_seq, n_q);
  return check_launch("debug shared-selection check");
#else
  (void)sel_of, (void)n_sel, (void)q_seq, (void)sel_seq, (void)n_q, (void)stream;
  return SA_OK;
#endif
}

int32_t debug_cache(const int32_t* pos, const int64_t* dst, int32_t n, hipStream_t stream) {
#ifdef SA_DEBUG
  if (n <= 0) return SA_OK;
  hipLaunchKernelGGL(sa_dbg::cache_kernel, dim3(dbg_grid(n, 256)), dim3(256), 0, stream, pos, dst, n);
  return check_launch("debug cache-write check");
#else
  (void)pos, (void)dst, (void)n, (void)stream;
  return SA_OK;
#endif
}

static int32_t fail_record(const uint32_t* rec) {
  set_error("debug check failed: %s (item %u, slot %u, value %d); %u violation(s) since the last check",
            sa_dbg::code_name(rec[0]), rec[1], rec[2], (int32_t)rec[3], rec[4]);
  return SA_ERR_DEBUG;
}

}  // namespace sa_host

using namespace sa_host;

extern "C" {

int32_t sa_debug_enabled(void) {
#ifdef SA_DEBUG
  return 1;
#else
  return 0;
#endif
}

int32_t sa_debug_check(sa_stream_t stream) {
#ifdef SA_DEBUG
  hipStream_t st = (hipStream_t)stream;
  uint32_t rec[sa_dbg::kRecWords] = {};
  const uint32_t zero[sa_dbg::kRecWords] = {};
  if (hipMemcpyFromSymbolAsync(rec, HIP_SYMBOL(sa_dbg::g_rec), sizeof rec, 0, hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipMemcpyToSymbolAsync(HIP_SYMBOL(sa_dbg::g_rec), zero, sizeof zero, 0, hipMemcpyHostToDevice, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    set_error("sa_debug_check: cannot read the check record: %s", hipGetErrorString(hipGetLastError()));
    return SA_ERR_HIP;
  }
  return rec[0] ? fail_record(rec) : SA_OK;
#else
  (void)stream;
  set_error("sa_debug_check: this library was built without SA_DEBUG (load libsparse_mla_debug.so)");
  return SA_ERR_UNSUPPORTED;
#endif
}

int32_t sa_debug_check_host(const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq,
                            const int32_t* q_pos, int32_t n_q, int32_t n_seq, int64_t ld, const int32_t* idx,
                            int32_t k) {
  if (n_q < 0 || n_seq < 0 || (idx && k < 0)) {
    set_error("sa_debug_check_host: negative count");
    return SA_ERR_INVALID_ARG;
  }
  if ((n_seq > 0 && (!seq_start || !seq_len)) || (n_q > 0 && (!q_seq || !q_pos))) {
    set_error("sa_debug_check_host: null array with a non-zero count");
    return SA_ERR_INVALID_ARG;
  }
  uint32_t rec[sa_dbg::kRecWords] = {};
  auto note = [&](uint32_t code, uint32_t item, uint32_t slot, int64_t val) {
    ++rec[4];
    if (!rec[0]) {
      rec[0] = code;
      rec[1] = item;
      rec[2] = slot;
      rec[3] = (uint32_t)val;
    }
  };
  int64_t val = 0;
  for (int32_t b = 0; b < n_seq; ++b) {
    const uint32_t c = sa_dbg::check_sequence(seq_start[b], seq_len[b], &val);
    if (c) note(c, (uint32_t)b, 0, val);
  }
  for (int32_t t = 0; t < n_q; ++t) {
    const uint32_t c = sa_dbg::check_query(q_seq[t], q_pos[t], seq_len, n_seq, ld, &val);
    if (c) note(c, (uint32_t)t, 0, val);
  }
  if (idx) {
    for (int32_t t = 0; t < n_q; ++t)
      for (int32_t j = 0; j < k; ++j) {
        const uint32_t c = sa_dbg::check_idx(idx[(int64_t)t * k + j], q_pos[t], &val);
        if (c) note(c, (uint32_t)t, (uint32_t)j, val);
      }
  }
  return rec[0] ? fail_record(rec) : SA_OK;
}

}  // extern "C"
