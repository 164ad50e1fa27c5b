// Exact top-k selection of indexer score rows for gfx950.
//
// Row t keeps the k_eff = min(k, q_pos[t] + 1) largest scores[t, 0..q_pos[t]],
// equal scores going to the lower position, written in ascending position
// order and padded with -1 (models.inteligile.com "GLM-5.2 / Model techniques
// map", "Checked in its code", row "Indexer-selected sparse attention": the kept
// count is min(index_topk, number of scores), as int32 positions; the tie order
// is the reading taken where the pages are silent).
//
// Scores become order-preserving uint32 keys (-0.0 folded onto +0.0).  A
// position s is kept iff its composite key (key(s) << 32) | ~s ranks among the
// k_eff largest composites: composites are unique, so the tie rule is built
// in and every step below is an exact integer radix select.
//
// Path 1 (many workgroups per row, used by default):
//   hist     rows x chunks: 4096-bin histogram of the top 12 key bits (LDS,
//            then global atomics); the last chunk of a row to finish finds the
//            bin b1 holding the k_eff-th largest key.
//   compact  rows x chunks: positions in bins above b1 are kept outright;
//            those in b1 become candidates (composite keys), up to a capacity.
//   finish   one workgroup per row: radix select over the candidates for the
//            remaining count, then a bitonic sort of the kept positions.
// Path 2 (one workgroup per row; also the exact fallback of path 1 when the
//   candidates overflow): three radix passes over the row give the exact
//   k_eff-th largest key K*, then one ordered pass keeps every key > K* and the
//   lowest-positioned keys == K*, writing them in position order.
#include "sa_common.h"

namespace sa {

constexpr int kBins1 = 4096;           // top 12 bits of the key
constexpr int kChunk = 4096;           // elements per workgroup in path 1
constexpr int kHistThreads = 256;
constexpr int kFinThreads = 1024;

// Per-row state words in the workspace.
enum { ST_B1 = 0, ST_ABOVE, ST_NCAND, ST_SELCNT, ST_CANDCNT, ST_DONE, ST_WORDS = 8 };

struct TopkWs {
  uint32_t* hist;    // [n_q][kBins1]
  int32_t* state;    // [n_q][ST_WORDS]
  int32_t* sel;      // [n_q][kMaxTopk]
  uint64_t* cand;    // [n_q][cap]
  int64_t cap;
};

// Inclusive scan over a workgroup of NT threads (NT a multiple of 64).
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* sh_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) sh_wave[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int x = lane < NT / 64 ? sh_wave[lane] : 0;
#pragma unroll
    for (int o = 1; o < NT / 64; o <<= 1) {
      const int u = __shfl_up(x, o, 64);
      if (lane >= o) x += u;
    }
    if (lane < NT / 64) sh_wave[lane] = x;
  }
  __syncthreads();
  if (wave > 0) v += sh_wave[wave - 1];
  __syncthreads();
  return v;
}

// Given a histogram (bins ordered by increasing key), find the bin d holding
// the need-th largest element: count(bins > d) < need <= count(bins >= d).
// Returns d and writes count(bins > d) to *above.  All NT threads call it.
template <int NT, int NB>
__device__ int find_bin(const uint32_t* hist, int need, int* above_out, int* sh_wave, int* sh_res) {
  constexpr int PER = NB / NT;      // bins per thread, scanned from the top
  const int tid = threadIdx.x;
  int local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) local += (int)hist[NB - 1 - (tid * PER + i)];
  const int incl = block_inclusive_scan<NT>(local, sh_wave);
  const int excl = incl - local;
  if (excl < need && need <= incl) {
    int run = excl;
    for (int i = 0; i < PER; ++i) {
      const int b = NB - 1 - (tid * PER + i);
      const int c = (int)hist[b];
      if (run + c >= need) {
        sh_res[0] = b;
        sh_res[1] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  const int d = sh_res[0];
  *above_out = sh_res[1];
  __syncthreads();
  return d;
}

// ----------------------------------------------------------------- path 1
__global__ void topk_zero_kernel(uint32_t* __restrict__ hist, int32_t* __restrict__ state, int64_t n_hist,
                                 int64_t n_state) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_hist; i += stride) hist[i] = 0u;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_state; i += stride) state[i] = 0;
}

__global__ __launch_bounds__(kHistThreads) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                                   const int32_t* __restrict__ q_pos, int k,
                                                                   int n_chunks, TopkWs ws) {
  const int t = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x - t * n_chunks;
  const int64_t n_t = (int64_t)q_pos[t] + 1;
  if (n_t <= k) return;      // every position is kept: nothing to select
  __shared__ uint32_t h[kBins1];
  __shared__ int sh_wave[kHistThreads / 64];
  __shared__ int sh_res[2];
  __shared__ int sh_last;
  for (int i = threadIdx.x; i < kBins1; i += kHistThreads) h[i] = 0u;
  __syncthreads();
  const float* row = scores + (int64_t)t * ld;
  const int64_t b0 = (int64_t)chunk * kChunk;
  const int64_t b1 = min(b0 + (int64_t)kChunk, n_t);
  for (int64_t s = b0 + threadIdx.x; s < b1; s += kHistThreads) atomicAdd(&h[score_key(row[s]) >> 20], 1u);
  __syncthreads();
  uint32_t* gh = ws.hist + (int64_t)t * kBins1;
  for (int i = threadIdx.x; i < kBins1; i += kHistThreads)
    if (h[i]) atomicAdd(&gh[i], h[i]);
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) sh_last = atomicAdd(&ws.state[(int64_t)t * ST_WORDS + ST_DONE], 1) == n_chunks - 1;
  __syncthreads();
  if (!sh_last) return;
  __threadfence();
  // Last chunk of this row: locate the bin of the k-th largest key.
  for (int i = threadIdx.x; i < kBins1; i += kHistThreads)
    h[i] = __hip_atomic_load(&gh[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int above;
  const int d = find_bin<kHistThreads, kBins1>(h, k, &above, sh_wave, sh_res);
  if (threadIdx.x == 0) {
    int32_t* st = ws.state + (int64_t)t * ST_WORDS;
    st[ST_B1] = d;
    st[ST_ABOVE] = above;
    st[ST_NCAND] = (int)h[d];
  }
}

__global__ __launch_bounds__(kHistThreads) void topk_compact_kernel(const float* __restrict__ scores, int64_t ld,
                                                                      const int32_t* __restrict__ q_pos, int k,
                                                                      int n_chunks, TopkWs ws) {
  const int t = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x - t * n_chunks;
  const int64_t n_t = (int64_t)q_pos[t] + 1;
  if (n_t <= k) return;
  int32_t* st = ws.state + (int64_t)t * ST_WORDS;
  const uint32_t bin = (uint32_t)st[ST_B1];
  const bool take_cand = st[ST_NCAND] <= ws.cap;
  const float* row = scores + (int64_t)t * ld;
  const int64_t b0 = (int64_t)chunk * kChunk;
  const int64_t b1 = min(b0 + (int64_t)kChunk, n_t);
  int32_t* sel = ws.sel + (int64_t)t * kMaxTopk;
  uint64_t* cand = ws.cand + (int64_t)t * ws.cap;
  const int lane = threadIdx.x & 63;
  const uint64_t lanemask_lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // Uniform trip count per wave so the ballots see every lane.
  for (int64_t base = b0; base < b1; base += kHistThreads) {
    const int64_t s = base + threadIdx.x;
    uint32_t key = 0;
    bool valid = s < b1;
    if (valid) key = score_key(row[s]);
    const uint32_t d = key >> 20;
    const bool is_above = valid && d > bin;
    const bool is_cand = valid && take_cand && d == bin;
    const uint64_t ma = __ballot(is_above);
    const uint64_t mc = __ballot(is_cand);
    int base_a = 0, base_c = 0;
    if (lane == 0) {
      if (ma) base_a = atomicAdd(&st[ST_SELCNT], __popcll(ma));
      if (mc) base_c = atomicAdd(&st[ST_CANDCNT], __popcll(mc));
    }
    base_a = __shfl(base_a, 0, 64);
    base_c = __shfl(base_c, 0, 64);
    if (is_above) sel[base_a + __popcll(ma & lanemask_lt)] = (int32_t)s;
    if (is_cand) cand[base_c + __popcll(mc & lanemask_lt)] = ((uint64_t)key << 32) | (uint32_t)~(uint32_t)s;
  }
}

// ------------------------------------------------------- finishing (1 WG/row)
// Bitonic sort of n (<= 2048) ints in LDS, ascending; entries n.. are padded.
__device__ void bitonic_sort_2048(int* v, int n) {
  for (int i = n + threadIdx.x; i < 2 * kFinThreads; i += kFinThreads) v[i] = 0x7fffffff;
  __syncthreads();
  for (int size = 2; size <= 2 * kFinThreads; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int i = threadIdx.x;
      const int lo = 2 * i - (i & (stride - 1));
      const int hi = lo + stride;
      const bool up = ((lo & size) == 0);
      const int a = v[lo], b = v[hi];
      if ((a > b) == up) {
        v[lo] = b;
        v[hi] = a;
      }
      __syncthreads();
    }
  }
}

// Exact selection over a whole row by one workgroup (path 2 / fallback):
// writes idx[0..k_eff) in ascending position order.
__device__ void select_row_exact(const float* __restrict__ row, int64_t n_t, int k_eff, int32_t* __restrict__ idx,
                                 uint32_t* h, int* sh_wave, int* sh_res) {
  uint32_t prefix = 0, mask = 0;
  int need = k_eff;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  for (int p = 0; p < 3; ++p) {
    const int sh = shifts[p];
    const uint32_t dmask = (1u << widths[p]) - 1u;
    for (int i = threadIdx.x; i < kBins1; i += kFinThreads) h[i] = 0u;
    __syncthreads();
    for (int64_t s = threadIdx.x; s < n_t; s += kFinThreads) {
      const uint32_t key = score_key(row[s]);
      if ((key & mask) == prefix) atomicAdd(&h[(key >> sh) & dmask], 1u);
    }
    __syncthreads();
    int above;
    const int d = find_bin<kFinThreads, kBins1>(h, need, &above, sh_wave, sh_res);
    need -= above;
    prefix |= (uint32_t)d << sh;
    mask |= dmask << sh;
  }
  // prefix is now the exact k_eff-th largest key K*; `need` keys equal to K*
  // are kept (the lowest positions), every key above K* is kept.
  const uint32_t kstar = prefix;
  const int need_eq = need;
  constexpr int E = 4;
  int out_base = 0, eq_base = 0;
  for (int64_t blk = 0; blk < n_t; blk += (int64_t)E * kFinThreads) {
    const int64_t s0 = blk + (int64_t)threadIdx.x * E;
    uint32_t keys[E];
    int c_gt = 0, c_eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      keys[e] = (s0 + e < n_t) ? score_key(row[s0 + e]) : 0u;
      const bool ok = s0 + e < n_t;
      c_gt += ok && keys[e] > kstar;
      c_eq += ok && keys[e] == kstar;
    }
    const int eq_incl = block_inclusive_scan<kFinThreads>(c_eq, sh_wave);
    int eq_rank = eq_base + eq_incl - c_eq;     // rank among equal keys before this thread's first
    int c_out = 0;
    bool take[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ok = s0 + e < n_t;
      take[e] = false;
      if (ok && keys[e] > kstar) take[e] = true;
      else if (ok && keys[e] == kstar) {
        take[e] = eq_rank < need_eq;
        ++eq_rank;
      }
      c_out += take[e];
    }
    const int out_incl = block_inclusive_scan<kFinThreads>(c_out, sh_wave);
    int slot = out_base + out_incl - c_out;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (take[e] && slot < k_eff) idx[slot++] = (int32_t)(s0 + e);
    // totals for the next block (last thread's inclusive values)
    if (threadIdx.x == kFinThreads - 1) {
      sh_res[0] = eq_incl;
      sh_res[1] = out_incl;
    }
    __syncthreads();
    eq_base += sh_res[0];
    out_base += sh_res[1];
    __syncthreads();
    (void)c_gt;
  }
}

__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(const float* __restrict__ scores, int64_t ld,
                                                                    const int32_t* __restrict__ q_pos, int k,
                                                                    int32_t* __restrict__ idx, TopkWs ws,
                                                                    int force_exact) {
  const int t = blockIdx.x;
  const int64_t n_t = (int64_t)q_pos[t] + 1;
  int32_t* out = idx + (int64_t)t * k;
  __shared__ uint32_t h[kBins1];
  __shared__ int v[2 * kFinThreads];
  __shared__ int sh_wave[kFinThreads / 64];
  __shared__ int sh_res[2];
  __shared__ int sh_cnt;
  if (n_t <= k) {
    for (int i = threadIdx.x; i < k; i += kFinThreads) out[i] = i < n_t ? i : -1;
    return;
  }
  const int k_eff = k;
  const float* row = scores + (int64_t)t * ld;
  const int32_t* st = ws.state + (int64_t)t * ST_WORDS;
  if (force_exact || st[ST_NCAND] > ws.cap) {
    select_row_exact(row, n_t, k_eff, out, h, sh_wave, sh_res);
    return;
  }
  const int n_above = st[ST_ABOVE];
  const int n_cand = st[ST_NCAND];
  int remaining = k_eff - n_above;
  const int32_t* sel = ws.sel + (int64_t)t * kMaxTopk;
  for (int i = threadIdx.x; i < n_above; i += kFinThreads) v[i] = sel[i];
  // Radix select among candidates on the 52 bits below the shared 12-bit bin.
  const uint64_t* cand = ws.cand + (int64_t)t * ws.cap;
  uint64_t prefix = (uint64_t)st[ST_B1] << 52;
  uint64_t mask = 0xfffull << 52;
  const int shifts[7] = {44, 36, 28, 20, 12, 4, 0};
  for (int p = 0; p < 7; ++p) {
    const int sh = shifts[p];
    const uint64_t dmask = p < 6 ? 0xffull : 0xfull;
    for (int i = threadIdx.x; i < 1024; i += kFinThreads) h[i] = 0u;   // digit bins live in h[0..256)
    __syncthreads();
    for (int i = threadIdx.x; i < n_cand; i += kFinThreads) {
      const uint64_t c = cand[i];
      if ((c & mask) == prefix) atomicAdd(&h[(c >> sh) & dmask], 1u);
    }
    __syncthreads();
    int above;
    const int d = find_bin<kFinThreads, 1024>(h, remaining, &above, sh_wave, sh_res);
    const int in_bin = (int)h[d];
    remaining -= above;
    prefix |= (uint64_t)d << sh;
    mask |= dmask << sh;
    __syncthreads();
    if (in_bin == remaining) break;
  }
  if (threadIdx.x == 0) sh_cnt = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n_cand; i += kFinThreads) {
    const uint64_t c = cand[i];
    if ((c & mask) >= prefix) {
      const int slot = atomicAdd(&sh_cnt, 1);
      if (n_above + slot < k_eff) v[n_above + slot] = (int)(~(uint32_t)c);
    }
  }
  __syncthreads();
  bitonic_sort_2048(v, k_eff);
  for (int i = threadIdx.x; i < k; i += kFinThreads) out[i] = i < k_eff ? v[i] : -1;
}

}  // namespace sa

namespace sa_host {

static int64_t topk_cap(int64_t ld) {
  int64_t cap = ld / 16;
  if (cap < 4096) cap = 4096;
  if (cap > 65536) cap = 65536;
  return cap;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t topk_workspace_size(int32_t n_q, int64_t ld, int32_t k) {
  (void)k;
  const int64_t cap = topk_cap(ld);
  return align256((size_t)n_q * sa::kBins1 * 4) + align256((size_t)n_q * sa::ST_WORDS * 4) +
         align256((size_t)n_q * sa::kMaxTopk * 4) + align256((size_t)n_q * cap * 8);
}

int32_t launch_topk(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q, int32_t k, int32_t* idx,
                    void* ws, int algo, hipStream_t stream) {
  if (algo == 0) algo = 1;
  sa::TopkWs w;
  uint8_t* p = (uint8_t*)ws;
  w.cap = topk_cap(ld);
  w.hist = (uint32_t*)p;
  p += align256((size_t)n_q * sa::kBins1 * 4);
  w.state = (int32_t*)p;
  p += align256((size_t)n_q * sa::ST_WORDS * 4);
  w.sel = (int32_t*)p;
  p += align256((size_t)n_q * sa::kMaxTopk * 4);
  w.cand = (uint64_t*)p;
  const int n_chunks = (int)((ld + sa::kChunk - 1) / sa::kChunk);
  if ((int64_t)n_chunks * n_q > 0x7fffffff) {
    set_error("topk: too many chunks");
    return SA_ERR_UNSUPPORTED;
  }
  if (algo == 1) {
    const int64_t n_hist = (int64_t)n_q * sa::kBins1, n_state = (int64_t)n_q * sa::ST_WORDS;
    const int64_t zb64 = (n_hist + 255) / 256;
    const int zb = (int)(zb64 < 4096 ? zb64 : 4096);
    hipLaunchKernelGGL(sa::topk_zero_kernel, dim3(zb), dim3(256), 0, stream, w.hist, w.state, n_hist, n_state);
    int32_t rc = check_launch("topk_zero_kernel");
    if (rc) return rc;
    hipLaunchKernelGGL(sa::topk_hist_kernel, dim3(n_chunks * n_q), dim3(sa::kHistThreads), 0, stream, scores, ld,
                       q_pos, k, n_chunks, w);
    if ((rc = check_launch("topk_hist_kernel"))) return rc;
    hipLaunchKernelGGL(sa::topk_compact_kernel, dim3(n_chunks * n_q), dim3(sa::kHistThreads), 0, stream, scores,
                       ld, q_pos, k, n_chunks, w);
    if ((rc = check_launch("topk_compact_kernel"))) return rc;
    hipLaunchKernelGGL(sa::topk_finish_kernel, dim3(n_q), dim3(sa::kFinThreads), 0, stream, scores, ld, q_pos, k,
                       idx, w, 0);
    return check_launch("topk_finish_kernel");
  }
  hipLaunchKernelGGL(sa::topk_finish_kernel, dim3(n_q), dim3(sa::kFinThreads), 0, stream, scores, ld, q_pos, k, idx,
                     w, 1);
  return check_launch("topk_finish_kernel");
}

}  // namespace sa_host
