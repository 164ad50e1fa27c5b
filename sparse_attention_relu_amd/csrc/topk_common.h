// Pieces of the radix top-k: workspace layout, score keys, workgroup scans
// and the bin search.
#pragma once

#include "sa_common.h"

namespace sa {

constexpr int kBins1 = 4096;           // first digit: top 12 bits of the key

// Per-row state words in the top-k workspace.
enum { ST_B1 = 0, ST_ABOVE, ST_NCAND, ST_SELCNT, ST_CANDCNT, ST_DONE, ST_WORDS = 8 };

struct TopkWs {
  uint32_t* hist;    // [n_q][kBins1]   first-digit histogram (zeroed before use)
  int32_t* state;    // [n_q][ST_WORDS] (zeroed before use)
  int32_t* sel;      // [n_q][kMaxTopk] positions kept outright
  uint64_t* cand;    // [n_q][cap]      candidates (key << 32 | ~position)
  int64_t cap;
};

// Inclusive scan over the 64 lanes of a wave in registers (DPP, no LDS round
// trip): prefix sums within each row of 16 lanes (row_shr 1, 2, 4, 8; lanes
// without a source add 0), then lane 15 of rows 0 and 2 is added to rows 1 and
// 3 (row_bcast:15), then lane 31 to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

// Inclusive scan over a workgroup of NT threads (NT a multiple of 64).
// *total receives the workgroup sum.  sh_wave needs NT/64 ints.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* sh_wave, int* total = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_inclusive_scan(v);
  if (lane == 63) sh_wave[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int x = lane < NT / 64 ? sh_wave[lane] : 0;
    x = wave_inclusive_scan(x);
    if (lane < NT / 64) sh_wave[lane] = x;
  }
  __syncthreads();
  if (wave > 0) v += sh_wave[wave - 1];
  if (total) *total = sh_wave[NT / 64 - 1];
  __syncthreads();
  return v;
}

// Given a histogram (bins ordered by increasing key), find the bin d holding
// the need-th largest element: count(bins > d) < need <= count(bins >= d).
// Returns d and writes count(bins > d) to *above.  All NT threads call it.
// need is clamped into [1, total] (total >= 1), so a bin is always found and
// every later index stays in range even if the counts were inconsistent.
template <int NT, int NB>
__device__ int find_bin(const uint32_t* hist, int need, int* above_out, int* sh_wave, int* sh_res) {
  constexpr int PER = NB / NT;      // bins per thread, scanned from the top
  const int tid = threadIdx.x;
  int local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) local += (int)hist[NB - 1 - (tid * PER + i)];
  int total;
  const int incl = block_inclusive_scan<NT>(local, sh_wave, &total);
  if (total <= 0) {                 // empty histogram: lowest bin, nothing above
    *above_out = 0;
    return 0;
  }
  need = min(max(need, 1), total);
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

// Locate the bin of the k-th largest key from a row's complete first-digit
// histogram (built by an earlier kernel, so plain loads see it).  NT threads;
// each holds kBins1 / 4 / NT groups of four bins, requested by
// load_first_hist; first_digit_bin puts them in h (kBins1 entries of LDS),
// returns the bin and writes *above = keys in higher bins, *n_cand = keys in
// the bin.
template <int NT>
struct FirstHist {
  u32x4 q[kBins1 / 4 / NT];
};

template <int NT>
__device__ __forceinline__ FirstHist<NT> load_first_hist(const TopkWs& ws, int t) {
  const u32x4* gh = reinterpret_cast<const u32x4*>(ws.hist + (int64_t)t * kBins1);
  FirstHist<NT> r;
#pragma unroll
  for (int i = 0; i < kBins1 / 4 / NT; ++i) r.q[i] = gh[threadIdx.x + NT * i];
  return r;
}

template <int NT>
__device__ int first_digit_bin(const FirstHist<NT>& fh, int k, uint32_t* h, int* sh_wave, int* sh_res, int* above,
                               int* n_cand) {
  u32x4* hh = reinterpret_cast<u32x4*>(h);
#pragma unroll
  for (int i = 0; i < kBins1 / 4 / NT; ++i) hh[threadIdx.x + NT * i] = fh.q[i];
  __syncthreads();
  const int d = find_bin<NT, kBins1>(h, k, above, sh_wave, sh_res);
  *n_cand = (int)h[d];
  return d;
}

}  // namespace sa
