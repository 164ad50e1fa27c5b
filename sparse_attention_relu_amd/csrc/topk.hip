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
// Path 1 (many workgroups per row, the automatic choice for rows longer than
// kPath2MaxLd):
//   hist     rows x chunks: 4096-bin histogram of the top 12 key bits (LDS,
//            then global atomics).  Inside sa_layer_stack the decode
//            indexer zeroes the histograms and counters on the side.
//   compact  rows x chunks, one pass with the chunk in registers: every
//            workgroup reads the finished histogram and finds the bin b1 that
//            holds the k_eff-th largest key (no hand-off between workgroups;
//            with large chunks a one-workgroup-per-row bin kernel finds it
//            once and the compaction reads it from the row's state words);
//            positions in bins above b1 are kept outright, those in b1 become
//            candidates (composite keys); one atomic per workgroup and counter
//            reserves the output slots.
//   finish   one workgroup per row: the candidates go to LDS, a radix select
//            finds the remaining count among them, and the kept positions are
//            put in ascending order by an LDS bitmap (rows up to 2^18
//            positions), a two-level bitmap (one 128-bit map per occupied
//            bucket of 128 positions, rows up to 2^20) or a bitonic sort
//            (longer rows).
// Path 2 (one workgroup per row; the automatic choice for short rows, and the
//   exact fallback of path 1 when the candidates overflow their capacity):
//   three radix passes over the row give
//   the exact k_eff-th largest key K*, then one ordered pass keeps every
//   key > K* and the lowest-positioned keys == K*, writing them in order.
#include "topk_common.h"

namespace sa {

constexpr int kHistThreads = 1024;
// Path 1 reads PER scores per thread, a chunk of PER x 1024 per workgroup:
// 8 (8192-score chunks) for decode batches; when the rows would give more
// than kManyChunks such workgroups (chunked prefill: 4096 rows of 131,072),
// where each workgroup's fixed chain (its row's histogram, the bin search,
// the slot reservation) would otherwise outweigh its share of the scores,
// 32 in the histogram and 16 in the compaction (whose registers at 32 would
// leave room for one workgroup per CU instead of two).
constexpr int kPerSmall = 8, kPerLargeHist = 32, kPerLargeCompact = 16;
constexpr int64_t kManyChunks = 4096;
constexpr int kFinThreads = 1024;
constexpr int kLdsCand = 8192;         // candidates staged in LDS by the finish kernel
constexpr int kPreCand = 1024;         // candidate slots the finish kernel requests with the counts
constexpr int kFinBins = 2048;         // 11-bit digits in the finish kernel
constexpr int kBitmapBits = 1 << 18;   // rows up to this length are emitted in order from an LDS bitmap
constexpr int kSparseSpan = 128;       // longer rows, up to kSparseBits: buckets of 128 positions,
constexpr int kSparseWords = kSparseSpan / 32;
constexpr int kSparseBits = 1 << 20;   // one 4-word bitmap per occupied bucket
constexpr int kSparseBuckets = kSparseBits / kSparseSpan;
constexpr int64_t kPath2MaxLd = 12288; // the automatic choice takes path 2 for rows up to this length
static_assert(kMaxTopk % kFinThreads == 0, "the finish kernel loads the kept positions in whole rounds");
static_assert(kSparseBuckets <= kBitmapBits / 32 && kSparseWords * kMaxTopk <= 2 * kLdsCand && kMaxTopk <= kBins1,
              "the two-level bitmap reuses the bitmap, candidate and histogram arrays");

// ----------------------------------------------------------------- path 1
__global__ void topk_zero_kernel(uint32_t* __restrict__ a, int64_t n_a, int32_t* __restrict__ b, int64_t n_b) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_a; i += stride) a[i] = 0u;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_b; i += stride) b[i] = 0;
}

// Path 1's chunk loads: v[j] = row[b0 + threadIdx.x + kHistThreads j];
// returns the row's length q_pos[t] + 1.  Small chunks (decode batches, one or
// two workgroups per CU, each a chain of round trips) are requested beside the
// length, one round trip instead of two: entries past the row's end are read
// within the row stride and ignored.  Large chunks (many workgroups per CU
// hide the chain) load after the length, as registers for 32 early loads
// would halve the workgroups a CU holds.
template <int kPer>
__device__ __forceinline__ int64_t load_chunk(const float* row, int64_t b0, int64_t ld, const int32_t* qp_ptr,
                                              float (&v)[kPer]) {
  if constexpr (kPer == kPerSmall) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) v[j] = row[min(b0 + threadIdx.x + kHistThreads * j, ld - 1)];
    const int qp = *qp_ptr;
    // (the empty statements keep the compiler from sinking the loads behind
    // the caller's branch on the length)
#pragma unroll
    for (int j = 0; j < kPer; ++j) asm volatile("" ::"v"(v[j]));
    asm volatile("" ::"s"(qp));
    return (int64_t)qp + 1;
  } else {
    const int64_t n_t = (int64_t)*qp_ptr + 1;
    if (b0 < n_t) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int64_t s = b0 + threadIdx.x + kHistThreads * j;
        v[j] = s < n_t ? row[s] : 0.f;
      }
    }
    return n_t;
  }
}

template <int kPer>
__global__ __launch_bounds__(kHistThreads) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                                   const int32_t* __restrict__ q_pos, int k,
                                                                   int n_chunks, TopkWs ws) {
  const int t = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x - t * n_chunks;
  const int64_t b0 = (int64_t)chunk * (kPer * kHistThreads);
  const float* row = scores + (int64_t)t * ld;
  float v[kPer];
  const int64_t n_t = load_chunk<kPer>(row, b0, ld, q_pos + t, v);
  if (n_t <= k || b0 >= n_t) return;      // take-all rows need no histogram
  __shared__ uint32_t h[kBins1];
  for (int i = threadIdx.x; i < kBins1; i += kHistThreads) h[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (b0 + threadIdx.x + kHistThreads * j < n_t) atomicAdd(&h[score_key(v[j]) >> 20], 1u);
  __syncthreads();
  uint32_t* gh = ws.hist + (int64_t)t * kBins1;
  for (int i = threadIdx.x; i < kBins1; i += kHistThreads)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Large chunks: the bin of the k-th largest key is found once per row, by one
// workgroup, and recorded in the row's state words (bin, keys above it, keys
// in it) for the compaction and the finish.
__global__ __launch_bounds__(kHistThreads) void topk_bin_kernel(const int32_t* __restrict__ q_pos, int k, TopkWs ws) {
  const int t = blockIdx.x;
  const FirstHist<kHistThreads> fh = load_first_hist<kHistThreads>(ws, t);   // beside the length
  const int64_t n_t = (int64_t)q_pos[t] + 1;
  if (n_t <= k) return;                   // take-all rows have no histogram
  __shared__ __align__(16) uint32_t h[kBins1];
  __shared__ int sh_wave[kHistThreads / 64];
  __shared__ int sh_res[2];
  int above, n_cand;
  const int bin = first_digit_bin<kHistThreads>(fh, k, h, sh_wave, sh_res, &above, &n_cand);
  if (threadIdx.x == 0) {
    int32_t* st = ws.state + (int64_t)t * ST_WORDS;
    st[ST_B1] = bin;
    st[ST_ABOVE] = above;
    st[ST_NCAND] = n_cand;
  }
}

// kBinDone: topk_bin_kernel has recorded the row's bin (large chunks: 8 or
// more workgroups per row would each repeat the 16 KB histogram read and the
// workgroup-wide bin search); otherwise every workgroup of the row finds the
// bin from the row's histogram (cheaper than a cross-workgroup hand-off) and
// chunk 0 records it.
template <int kPer, bool kBinDone>
__global__ __launch_bounds__(kHistThreads) void topk_compact_kernel(const float* __restrict__ scores, int64_t ld,
                                                                      const int32_t* __restrict__ q_pos, int k,
                                                                      int n_chunks, TopkWs ws) {
  const int t = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x - t * n_chunks;
  const int64_t b0 = (int64_t)chunk * (kPer * kHistThreads);
  const float* row = scores + (int64_t)t * ld;
  int32_t* st = ws.state + (int64_t)t * ST_WORDS;
  float v[kPer];
  FirstHist<kHistThreads> fh;
  int rec_bin = 0, rec_cand = 0;
  if constexpr (kBinDone) {
    rec_bin = st[ST_B1];
    rec_cand = st[ST_NCAND];
  } else if constexpr (kPer == kPerSmall) {
    fh = load_first_hist<kHistThreads>(ws, t);   // beside the chunk
  }
  const int64_t n_t = load_chunk<kPer>(row, b0, ld, q_pos + t, v);
  if (n_t <= k || b0 >= n_t) return;
  if constexpr (!kBinDone && kPer != kPerSmall) fh = load_first_hist<kHistThreads>(ws, t);
  __shared__ __align__(16) uint32_t h[kBins1];
  __shared__ int sh_wave[kHistThreads / 64];
  __shared__ int sh_res[2];
  __shared__ int sh_base[2];
  uint32_t bin;
  int n_cand;
  if constexpr (kBinDone) {
    bin = (uint32_t)rec_bin;
    n_cand = rec_cand;
  } else {
    int above;
    bin = (uint32_t)first_digit_bin<kHistThreads>(fh, k, h, sh_wave, sh_res, &above, &n_cand);
    if (chunk == 0 && threadIdx.x == 0) {
      st[ST_B1] = (int)bin;
      st[ST_ABOVE] = above;
      st[ST_NCAND] = n_cand;
    }
  }
  const bool take_cand = n_cand <= ws.cap;
  uint32_t above_mask = 0, cand_mask = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const bool ok = b0 + threadIdx.x + kHistThreads * j < n_t;
    const uint32_t d = score_key(v[j]) >> 20;
    above_mask |= (uint32_t)(ok && d > bin) << j;
    cand_mask |= (uint32_t)(ok && take_cand && d == bin) << j;
  }
  const int packed = (__popc(above_mask) << 16) | __popc(cand_mask);
  int total;
  const int incl = block_inclusive_scan<kHistThreads>(packed, sh_wave, &total);
  const int excl = incl - packed;
  if (threadIdx.x == 0) {
    const int ta = total >> 16, tc = total & 0xffff;
    sh_base[0] = ta ? atomicAdd(&st[ST_SELCNT], ta) : 0;
    sh_base[1] = tc ? atomicAdd(&st[ST_CANDCNT], tc) : 0;
  }
  __syncthreads();
  int slot_a = sh_base[0] + (excl >> 16);
  int slot_c = sh_base[1] + (excl & 0xffff);
  int32_t* sel = ws.sel + (int64_t)t * kMaxTopk;
  uint64_t* cand = ws.cand + (int64_t)t * ws.cap;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t s = (uint32_t)(b0 + threadIdx.x + kHistThreads * j);
    // (slots stay below kMaxTopk and cap whenever the histogram is complete;
    // the checks keep inconsistent workspace contents from writing out of range)
    if ((above_mask >> j) & 1u) {
      if (slot_a < kMaxTopk) sel[slot_a] = (int32_t)s;
      ++slot_a;
    }
    if ((cand_mask >> j) & 1u) {
      if (slot_c < ws.cap) cand[slot_c] = ((uint64_t)score_key(v[j]) << 32) | (uint32_t)~s;
      ++slot_c;
    }
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
    int c_eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ok = s0 + e < n_t;
      keys[e] = ok ? score_key(row[s0 + e]) : 0u;
      c_eq += ok && keys[e] == kstar;
    }
    int eq_tot, out_tot;
    const int eq_incl = block_inclusive_scan<kFinThreads>(c_eq, sh_wave, &eq_tot);
    int eq_rank = eq_base + eq_incl - c_eq;     // rank among equal keys of this thread's first
    int c_out = 0;
    bool take[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ok = s0 + e < n_t;
      take[e] = false;
      if (ok && keys[e] > kstar) {
        take[e] = true;
      } else if (ok && keys[e] == kstar) {
        take[e] = eq_rank < need_eq;
        ++eq_rank;
      }
      c_out += take[e];
    }
    const int out_incl = block_inclusive_scan<kFinThreads>(c_out, sh_wave, &out_tot);
    int slot = out_base + out_incl - c_out;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (take[e] && slot < k_eff) idx[slot++] = (int32_t)(s0 + e);
    eq_base += eq_tot;
    out_base += out_tot;
  }
}

// Radix select among n_cand candidate composites (all in first-digit bin b1):
// the `remaining` largest are kept.  Works on the 52 composite bits below the
// shared 12-bit bin, 11 bits at a time (20 key bits, then position bits only
// while keys tie across the boundary).  Returns (prefix, mask): a candidate c
// is kept iff (c & mask) >= prefix (composites are unique, so exactly
// `remaining` of them).  h needs kFinBins entries.
struct Kept {
  uint64_t prefix, mask;
};
__device__ Kept select_candidates(const uint64_t* cand, int n_cand, uint32_t b1, int remaining, uint32_t* h,
                                  int* sh_wave, int* sh_res) {
  uint64_t prefix = (uint64_t)b1 << 52;
  uint64_t mask = 0xfffull << 52;
  const int shifts[5] = {41, 30, 19, 8, 0};
  for (int p = 0; p < 5; ++p) {
    const int sh = shifts[p];
    const uint64_t dmask = p < 4 ? 0x7ffull : 0xffull;
    for (int i = threadIdx.x; i < kFinBins; i += kFinThreads) h[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n_cand; i += kFinThreads) {
      const uint64_t c = cand[i];
      if ((c & mask) == prefix) atomicAdd(&h[(c >> sh) & dmask], 1u);
    }
    __syncthreads();
    int above;
    const int d = find_bin<kFinThreads, kFinBins>(h, remaining, &above, sh_wave, sh_res);
    const int in_bin = (int)h[d];
    remaining -= above;
    prefix |= (uint64_t)d << sh;
    mask |= dmask << sh;
    __syncthreads();
    if (in_bin == remaining) break;     // the whole boundary bin is kept
  }
  return Kept{prefix, mask};
}

// Ascending emission of the positions set in words[0 .. n_words), bit j of
// word i standing for position base(i) + j (base increasing with i): thread i
// owns a run of words; a prefix sum of their popcounts gives its first output
// slot.  Slots past the set bits (up to k) get -1.
template <class Base>
__device__ void emit_words(const uint32_t* words, int n_words, Base base, int32_t* __restrict__ out, int k,
                           int* sh_wave) {
  const int per = (n_words + kFinThreads - 1) / kFinThreads;
  const int w0 = min((int)threadIdx.x * per, n_words), w1 = min(w0 + per, n_words);
  int cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __popc(words[i]);
  int total;
  int slot = block_inclusive_scan<kFinThreads>(cnt, sh_wave, &total) - cnt;
  for (int i = w0; i < w1; ++i) {
    uint32_t bits = words[i];
    const int b0 = base(i);
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (slot >= 0 && slot < k) out[slot] = b0 + b;
      ++slot;
    }
  }
  for (int i = total + threadIdx.x; i < k; i += kFinThreads) out[i] = -1;
}

// Ascending emission of the distinct positions v[0 .. n_v) (n_v <= kMaxTopk)
// of a row of n_t <= kSparseBits positions, through a two-level bitmap: the
// 128-position buckets that hold a position are flagged (flag: kSparseBuckets
// words), numbered in order by a prefix sum (bucket_of: the bucket of each
// number, at most n_v of them), and each position sets its bit in the 4-word
// bitmap of its bucket's number (words: 4 kMaxTopk words); the words are then
// emitted in order.  Entries outside [0, n_t) are dropped.
__device__ void emit_sparse(const int* v, int n_v, int64_t n_t, uint32_t* flag, uint32_t* words, int* bucket_of,
                            int32_t* __restrict__ out, int k, int* sh_wave) {
  const int n_b = (int)((n_t + kSparseSpan - 1) / kSparseSpan);
  for (int i = threadIdx.x; i < n_b; i += kFinThreads) flag[i] = 0u;
  for (int i = threadIdx.x; i < kSparseWords * kMaxTopk; i += kFinThreads) words[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < n_v; i += kFinThreads) {
    const int p = v[i];
    if (p >= 0 && p < n_t) flag[p / kSparseSpan] = 1u;
  }
  __syncthreads();
  // thread i numbers a run of buckets; a flag becomes its bucket's number
  const int per = (n_b + kFinThreads - 1) / kFinThreads;
  const int b0 = min((int)threadIdx.x * per, n_b), b1 = min(b0 + per, n_b);
  int cnt = 0;
  for (int b = b0; b < b1; ++b) cnt += (int)flag[b];
  int n_used;
  int num = block_inclusive_scan<kFinThreads>(cnt, sh_wave, &n_used) - cnt;
  for (int b = b0; b < b1; ++b)
    if (flag[b]) {
      flag[b] = (uint32_t)num;
      bucket_of[num] = b;
      ++num;
    }
  __syncthreads();
  for (int i = threadIdx.x; i < n_v; i += kFinThreads) {
    const int p = v[i];
    if (p >= 0 && p < n_t)
      atomicOr(&words[kSparseWords * flag[p / kSparseSpan] + (p % kSparseSpan) / 32], 1u << (p & 31));
  }
  __syncthreads();
  emit_words(words, kSparseWords * n_used,
             [&](int i) { return bucket_of[i / kSparseWords] * kSparseSpan + (i % kSparseWords) * 32; }, out, k,
             sh_wave);
}

__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(const float* __restrict__ scores, int64_t ld,
                                                                    const int32_t* __restrict__ q_pos, int k,
                                                                    int32_t* __restrict__ idx, TopkWs ws,
                                                                    int force_exact) {
  const int t = blockIdx.x;
  // After path 1, everything the row may need is requested in one round
  // trip, beside its length and counts: all kMaxTopk kept-position slots and
  // the first kPreCand candidate slots (cap >= kPreCand); what lies past the
  // counts is ignored.
  const int32_t* sel = ws.sel + (int64_t)t * kMaxTopk;
  const uint64_t* gcand = ws.cand + (int64_t)t * ws.cap;
  int sv[kMaxTopk / kFinThreads] = {};
  uint64_t cv[kPreCand / kFinThreads] = {};
  if (!force_exact) {
#pragma unroll
    for (int u = 0; u < kMaxTopk / kFinThreads; ++u) sv[u] = sel[threadIdx.x + kFinThreads * u];
#pragma unroll
    for (int u = 0; u < kPreCand / kFinThreads; ++u) cv[u] = gcand[threadIdx.x + kFinThreads * u];
  }
  const int32_t* st = ws.state + (int64_t)t * ST_WORDS;
  const int st_ncand = st[ST_NCAND], st_above = st[ST_ABOVE], st_b1 = st[ST_B1];
  const int qp = q_pos[t];
  // (the empty statement keeps the compiler from sinking the count loads
  // behind the branch on the row's length: all four arrive together)
  asm volatile("" ::"s"(st_ncand), "s"(st_above), "s"(st_b1), "s"(qp));
  const int64_t n_t = (int64_t)qp + 1;
  int32_t* out = idx + (int64_t)t * k;
  __shared__ __align__(16) uint32_t h[kBins1];
  __shared__ int v[2 * kFinThreads];
  __shared__ uint64_t lc[kLdsCand];
  __shared__ uint32_t bm[kBitmapBits / 32];
  __shared__ int sh_wave[kFinThreads / 64];
  __shared__ int sh_res[2];
  __shared__ int sh_cnt;
  if (n_t <= k) {
    for (int i = threadIdx.x; i < k; i += kFinThreads) out[i] = i < n_t ? i : -1;
    return;
  }
  const int k_eff = k;
  const float* row = scores + (int64_t)t * ld;
  if (force_exact || st_ncand > ws.cap) {
    select_row_exact(row, n_t, k_eff, out, h, sh_wave, sh_res);
    return;
  }
  // Counts come from the compaction; clamped so that inconsistent workspace
  // contents cannot index out of range.
  const int n_above = min(max(st_above, 0), k_eff - 1);
  const int n_cand = (int)min((int64_t)max(st_ncand, 0), ws.cap);
  const bool in_lds = n_cand <= kLdsCand;
  const bool ordered_by_bitmap = n_t <= kBitmapBits;
  const int n_words = (int)((n_t + 31) >> 5);
  // kept positions: n_above < kMaxTopk = 2 x kFinThreads
#pragma unroll
  for (int u = 0; u < kMaxTopk / kFinThreads; ++u)
    if ((int)threadIdx.x + kFinThreads * u >= n_above) sv[u] = -1;
  if (ordered_by_bitmap) {
    for (int i = threadIdx.x; i < n_words; i += kFinThreads) bm[i] = 0u;
  } else {
#pragma unroll
    for (int u = 0; u < kMaxTopk / kFinThreads; ++u) {
      const int i = (int)threadIdx.x + kFinThreads * u;
      if (i < n_above) v[i] = sv[u];
    }
  }
  if (in_lds) {
#pragma unroll
    for (int u = 0; u < kPreCand / kFinThreads; ++u) {
      const int i = (int)threadIdx.x + kFinThreads * u;
      if (i < n_cand) lc[i] = cv[u];
    }
    for (int i = kPreCand + threadIdx.x; i < n_cand; i += kFinThreads) lc[i] = gcand[i];
  }
  __syncthreads();
  if (ordered_by_bitmap)
#pragma unroll
    for (int u = 0; u < kMaxTopk / kFinThreads; ++u) {
      const int s = sv[u];
      if (s >= 0 && s < n_t) atomicOr(&bm[s >> 5], 1u << (s & 31));
    }
  const uint64_t* cand = in_lds ? lc : gcand;
  const Kept kept = select_candidates(cand, n_cand, (uint32_t)st_b1, k_eff - n_above, h, sh_wave, sh_res);
  if (threadIdx.x == 0) sh_cnt = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n_cand; i += kFinThreads) {
    const uint64_t c = cand[i];
    if ((c & kept.mask) >= kept.prefix) {
      const int s = (int)(~(uint32_t)c);
      if (ordered_by_bitmap) {
        if (s >= 0 && s < n_t) atomicOr(&bm[s >> 5], 1u << (s & 31));
      } else {
        const int slot = atomicAdd(&sh_cnt, 1);
        if (n_above + slot < k_eff) v[n_above + slot] = s;
      }
    }
  }
  __syncthreads();
  if (!ordered_by_bitmap && n_t <= kSparseBits) {
    const int n_v = min(n_above + sh_cnt, k_eff);
    emit_sparse(v, n_v, n_t, bm, reinterpret_cast<uint32_t*>(lc), reinterpret_cast<int*>(h), out, k, sh_wave);
    return;
  }
  if (!ordered_by_bitmap) {
    bitonic_sort_2048(v, k_eff);
    for (int i = threadIdx.x; i < k; i += kFinThreads) out[i] = i < k_eff ? v[i] : -1;
    return;
  }
  emit_words(bm, n_words, [](int i) { return i << 5; }, out, k, sh_wave);
}

}  // namespace sa

namespace sa_host {

static int64_t topk_cap(int64_t ld) {
  static_assert(sa::kPreCand <= 4096 && sa::kPreCand % sa::kFinThreads == 0,
                "the finish kernel reads kPreCand candidate slots unconditionally");
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

sa::TopkWs topk_carve(void* ws, int32_t n_q, int64_t ld) {
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
  return w;
}

// Zero the histogram and state words (adjacent in the carve), plus n_extra
// int32 words at `extra` (counters of other kernels sharing the launch).
int32_t topk_zero(const sa::TopkWs& w, int32_t* extra, int64_t n_extra, hipStream_t stream) {
  const int64_t n_a = (int64_t)((uint8_t*)w.sel - (uint8_t*)w.hist) / 4;
  const int64_t zb64 = (n_a + 255) / 256;
  const int zb = (int)(zb64 < 2048 ? zb64 : 2048);
  hipLaunchKernelGGL(sa::topk_zero_kernel, dim3(zb), dim3(256), 0, stream, w.hist, n_a, extra, n_extra);
  return check_launch("topk_zero_kernel");
}

int32_t topk_zero_words(int32_t* p, int64_t n, hipStream_t stream) {
  const int64_t zb64 = (n + 255) / 256;
  const int zb = (int)(zb64 < 2048 ? (zb64 > 0 ? zb64 : 1) : 2048);
  hipLaunchKernelGGL(sa::topk_zero_kernel, dim3(zb), dim3(256), 0, stream, (uint32_t*)nullptr, (int64_t)0, p, n);
  return check_launch("topk_zero_kernel");
}

// Whether a batch of n_q rows of ld takes path 1's large chunks.
static bool topk_large_chunks(int32_t n_q, int64_t ld) {
  const int64_t small = (ld + sa::kPerSmall * sa::kHistThreads - 1) / (sa::kPerSmall * sa::kHistThreads);
  return small * n_q > sa::kManyChunks;
}

static int64_t topk_chunks(int64_t ld, int per) { return (ld + per * sa::kHistThreads - 1) / (per * sa::kHistThreads); }

// Everything after the first-digit histogram: compaction and finish.
static int32_t topk_after_hist(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q, int32_t k,
                               int32_t* idx, const sa::TopkWs& w, bool large, hipStream_t stream) {
  if (large) {
    hipLaunchKernelGGL(sa::topk_bin_kernel, dim3(n_q), dim3(sa::kHistThreads), 0, stream, q_pos, k, w);
    int32_t rc = check_launch("topk_bin_kernel");
    if (rc) return rc;
    const int n_chunks = (int)topk_chunks(ld, sa::kPerLargeCompact);
    hipLaunchKernelGGL((sa::topk_compact_kernel<sa::kPerLargeCompact, true>), dim3(n_chunks * n_q),
                       dim3(sa::kHistThreads), 0, stream, scores, ld, q_pos, k, n_chunks, w);
  } else {
    const int n_chunks = (int)topk_chunks(ld, sa::kPerSmall);
    hipLaunchKernelGGL((sa::topk_compact_kernel<sa::kPerSmall, false>), dim3(n_chunks * n_q), dim3(sa::kHistThreads), 0,
                       stream, scores, ld, q_pos, k, n_chunks, w);
  }
  int32_t rc = check_launch("topk_compact_kernel");
  if (rc) return rc;
  hipLaunchKernelGGL(sa::topk_finish_kernel, dim3(n_q), dim3(sa::kFinThreads), 0, stream, scores, ld, q_pos, k, idx, w,
                     0);
  return check_launch("topk_finish_kernel");
}

// Words that path 1 needs at zero before it starts (histograms and state
// words, adjacent in the carve).
void topk_clear_range(void* ws, int32_t n_q, int64_t ld, uint32_t** p, int64_t* n) {
  const sa::TopkWs w = topk_carve(ws, n_q, ld);
  *p = w.hist;
  *n = (int64_t)((uint8_t*)w.sel - (uint8_t*)w.hist) / 4;
}

// cleared: path 1's words (topk_clear_range) are already zero in stream order.
int32_t launch_topk(const float* scores, int64_t ld, const int32_t* q_pos, int32_t n_q, int32_t k, int32_t* idx,
                    void* ws, int algo, hipStream_t stream, bool cleared) {
  // Automatic choice: one kernel and one workgroup per row (path 2) for short
  // rows, whose three radix passes over at most 12,288 scores cost less than
  // path 1's three launches (4 rows of 4096: 10.8 against 20.7 us; 16 of 8192:
  // 15.4 against 22.6 us; even at 16,384); path 1 from there on.
  if (algo == 0) algo = ld <= sa::kPath2MaxLd ? 2 : 1;
  sa::TopkWs w = topk_carve(ws, n_q, ld);
  const bool large = topk_large_chunks(n_q, ld);
  // (the compaction's chunks are the smaller ones)
  if (topk_chunks(ld, large ? sa::kPerLargeCompact : sa::kPerSmall) * n_q > 0x7fffffff) {
    set_error("topk: too many chunks");
    return SA_ERR_UNSUPPORTED;
  }
  if (algo == 1) {
    int32_t rc = cleared ? SA_OK : topk_zero(w, nullptr, 0, stream);
    if (rc) return rc;
    if (large) {
      const int64_t n_chunks = topk_chunks(ld, sa::kPerLargeHist);
      hipLaunchKernelGGL(sa::topk_hist_kernel<sa::kPerLargeHist>, dim3((unsigned)(n_chunks * n_q)),
                         dim3(sa::kHistThreads), 0, stream, scores, ld, q_pos, k, (int)n_chunks, w);
    } else {
      const int64_t n_chunks = topk_chunks(ld, sa::kPerSmall);
      hipLaunchKernelGGL(sa::topk_hist_kernel<sa::kPerSmall>, dim3((unsigned)(n_chunks * n_q)), dim3(sa::kHistThreads),
                         0, stream, scores, ld, q_pos, k, (int)n_chunks, w);
    }
    if ((rc = check_launch("topk_hist_kernel"))) return rc;
    return topk_after_hist(scores, ld, q_pos, n_q, k, idx, w, large, stream);
  }
  hipLaunchKernelGGL(sa::topk_finish_kernel, dim3(n_q), dim3(sa::kFinThreads), 0, stream, scores, ld, q_pos, k, idx,
                     w, 1);
  return check_launch("topk_finish_kernel");
}

}  // namespace sa_host
