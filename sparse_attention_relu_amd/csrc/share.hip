// Selection shared by a group of query tokens (MTP / speculative decode).
//
// llm-atlas "GLM-5.2", "Champs bruts du config.json": index_share_for_mtp_iteration
// is true; hermosaai "GLM 5.2", "78 layers, IndexShare pattern": one
// Multi-Token Prediction layer serves speculative decoding.  A group of draft
// tokens of one sequence takes one selection (made for a selecting query of
// the group); each token keeps the selected positions at or before its own
// position, in the row's order, followed by -1 padding.
//
// share_kernel: one workgroup of 256 threads per token row.  Thread i reads
// slots 8i .. 8i+7 of the source row (k <= 2048), flags the kept entries, and
// a workgroup prefix sum of the flag counts gives each kept entry its output
// slot; the rest of the row is -1.
#include "sa_common.h"

namespace sa {

constexpr int kShareThreads = 256;
constexpr int kSharePer = kMaxTopk / kShareThreads;     // 8 slots per thread

__global__ __launch_bounds__(kShareThreads) void share_kernel(const int32_t* __restrict__ sel_idx, int32_t n_sel,
                                                              int32_t k, const int32_t* __restrict__ sel_of,
                                                              const int32_t* __restrict__ q_pos,
                                                              int32_t* __restrict__ idx) {
  const int t = blockIdx.x;
  __shared__ int sh_wave[kShareThreads / 64];
  // sel_of[t] outside [0, n_sel) breaks a precondition (the SA_DEBUG build
  // reports it); clamped, the row read stays inside sel_idx.
  const int src = min(max(sel_of[t], 0), n_sel - 1);
  const int p = q_pos[t];
  const int32_t* row = sel_idx + (int64_t)src * k;
  int32_t* out = idx + (int64_t)t * k;
  const int j0 = (int)threadIdx.x * kSharePer;
  int v[kSharePer];
  int n_keep = 0;
#pragma unroll
  for (int u = 0; u < kSharePer; ++u) {
    const int j = j0 + u;
    v[u] = j < k ? row[j] : -1;
    if (v[u] < 0 || v[u] > p) v[u] = -1;
    n_keep += v[u] >= 0;
  }
  // workgroup exclusive prefix sum of n_keep: a scan within each of the 4
  // waves with shuffles, then the waves' totals through LDS
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = n_keep;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) sh_wave[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += sh_wave[w];
  const int total = sh_wave[0] + sh_wave[1] + sh_wave[2] + sh_wave[3];
  int slot = base + incl - n_keep;
#pragma unroll
  for (int u = 0; u < kSharePer; ++u)
    if (v[u] >= 0) out[slot++] = v[u];
  for (int j = total + (int)threadIdx.x; j < k; j += kShareThreads) out[j] = -1;
}

}  // namespace sa

namespace sa_host {

int32_t launch_share(const int32_t* sel_idx, int32_t n_sel, int32_t k, const int32_t* sel_of, const int32_t* q_pos,
                     int32_t n_q, int32_t* idx, hipStream_t stream) {
  if (n_q <= 0) return SA_OK;
  hipLaunchKernelGGL(sa::share_kernel, dim3(n_q), dim3(sa::kShareThreads), 0, stream, sel_idx, n_sel, k, sel_of, q_pos,
                     idx);
  return check_launch("share_kernel");
}

}  // namespace sa_host
