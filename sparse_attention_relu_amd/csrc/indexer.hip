// Indexer score kernels for gfx950.
//
// scores[t, s] = sum_h w[t, h] * max(0, q[t, h, :] . k[seq(t), s, :]) over the
// causal set s <= q_pos[t], -inf beyond it (models.inteligile.com "GLM-5.2 /
// Model techniques map", "Checked in its code", row "Indexer-selected sparse
// attention (DeepSeek Sparse Attention)": 32 heads of 128 against one key per
// token shared by every head).
//
// Both kernels put the 32 heads of one query on the M side of
// v_mfma_f32_32x32x16_bf16 and 32 keys on the N side, so one accumulator tile
// holds every head of one query for 32 keys: each lane owns one key column and
// 16 of the 32 head rows, and the ReLU + weighted head sum is 16 in-lane
// max/fma pairs plus one exchange with the lane 32 away.  The contraction
// dimension (128) is consumed in 8 steps of 16; the split of each 16-wide step
// between the two half-waves is the same for both operands, which is all the
// sum needs.
//
//   indexer_decode_kernel   one query per workgroup column: streams that
//                           query's keys once (decode: every query has its own
//                           sequence).  HBM-bound: 256 B of keys per 8 KFLOP.
//   indexer_prefill_kernel  16 queries of one sequence share each key tile staged
//                           in LDS: the dense contraction of chunked prefill.
#include "fp8.h"
#include "sa_common.h"

namespace sa {

// ---------------------------------------------------------------- helpers
// Rows of the 32x32 accumulator owned by a lane: element i of the 16-vector
// is row 8*(i/4) + 4*(lane/32) + (i%4), column lane%32.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// max(x, 0) of a finite float as one integer max of its bits: negative
// values (and -0.0) have the sign bit set, so they compare below 0 as int32.
// (A float max would also be preceded by a NaN-quieting max in IEEE mode.)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ float relu_weighted_sum(const f32x16& acc, const float (&wr)[16]) {
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) part = fmaf(wr[i], relu(acc[i]), part);
  return part + __shfl_xor(part, 32, 64);
}

// This lane's 16 heads of the sum (accumulator element i is head
// acc_row(i, lane)); the other 16 heads are in the lane 32 away.
__device__ __forceinline__ float relu_weighted_part(const f32x16& acc, const float (&wr)[16]) {
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) part = fmaf(wr[i], relu(acc[i]), part);
  return part;
}

// ------------------------------------------------------------ decode kernel
// A workgroup covers 128 consecutive keys of one query's sequence: at each of
// its 2 steps the 2 waves take the next 64 keys (32 each, 8 KB), staged
// through wave-private LDS into the MFMA, with the next step's loads in
// flight.
constexpr int kDecWaves = 2;
constexpr int kDecSteps = 2;
constexpr int kDecChunk = kDecWaves * 32 * kDecSteps;     // keys per workgroup
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kKeyPitch = 272;                            // LDS bytes per key row (256 + 16 pad)

struct DecArgs {
  const uint16_t* q_idx;
  const float* w;
  const uint16_t* k_idx;    // bf16 keys [rows][128], or E4M3 codes [rows][128] (FP8)
  const float* k_scale;     // FP8: one scale per key row
  const int64_t* seq_start;
  const int32_t* seq_len;
  const int32_t* q_seq;
  const int32_t* q_pos;
  float* scores;
  int64_t ld;
  int n_chunks;
  uint32_t* clear;     // optional: words set to zero on the side (the next kernel's counters)
  int64_t n_clear;
};

// FP8: the keys are E4M3 codes with one fp32 scale per key; they are decoded
// to bf16 (exact) on their way into the staging LDS, and each score is the
// codes' score times the key's scale (ReLU commutes with a positive scale).
template <bool FP8>
__global__ __launch_bounds__(kDecThreads) void indexer_decode_kernel(DecArgs A) {
  constexpr int kG = FP8 ? 4 : 8;          // 16-byte key pieces per lane per step
  // side job: clear the caller's words (a grid-stride loop over all workgroups)
  for (int64_t i = (int64_t)blockIdx.x * kDecThreads + threadIdx.x; i < A.n_clear; i += (int64_t)gridDim.x * kDecThreads)
    A.clear[i] = 0u;
  const int t = blockIdx.x / A.n_chunks;
  const int chunk = blockIdx.x - t * A.n_chunks;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int seq = A.q_seq[t];
  // the causal set, clamped to the sequence's keys (q_pos < seq_len is a
  // precondition; the clamp keeps a violation from reading other rows)
  const int64_t pos = min((int64_t)A.q_pos[t], (int64_t)A.seq_len[seq] - 1);
  const int64_t c0 = (int64_t)chunk * kDecChunk;
  float* srow = A.scores + (int64_t)t * A.ld;
  if (c0 > pos) {
    const int64_t end = min(c0 + (int64_t)kDecChunk, A.ld);
    for (int64_t s = c0 + threadIdx.x; s < end; s += kDecThreads) srow[s] = -INFINITY;
    return;
  }
  __shared__ __align__(16) uint8_t lds[kDecWaves][32 * kKeyPitch];
  __shared__ float sh_w[kIdxHeads];

  // step it of this wave covers keys c0 + (4 it + wave) * 32 .. +31; keys
  // and score columns are handled relative to c0 in 32 bits
  const int wlast = (int)min(pos - c0, (int64_t)kDecChunk - 1);       // last valid key
  const int wend = (int)min(A.ld - c0, (int64_t)kDecChunk);          // columns of this chunk in the row
  const int64_t row0 = A.seq_start[seq] + c0;
  const uint16_t* kb = A.k_idx + row0 * kIdxDim;
  const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(A.k_idx) + row0 * kIdxDim;
  float* sc0 = srow + c0;
  const int n_it = kDecSteps;
  uint8_t* my = lds[wave];
  auto key_of = [&](int it) { return (it * kDecWaves + wave) * 32; };

  // Loads past the causal bound re-read the last valid key (always in bounds);
  // their scores are replaced by -inf, so no load needs a branch.  Keys are
  // read once: streaming loads keep them from displacing cached data.
  auto load = [&](u32x4 (&g)[kG], float& ks, int it) {
    if (FP8) {
#pragma unroll
      for (int j = 0; j < kG; ++j) {       // 8 keys of 128 codes per piece index j
        const int key = min(key_of(it) + 8 * j + (lane >> 3), wlast);
        g[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb8 + key * kIdxDim + (lane & 7) * 16));
      }
      ks = A.k_scale[row0 + min(key_of(it) + (lane & 31), wlast)];
    } else {
#pragma unroll
      for (int j = 0; j < kG; ++j) {
        const int key = min(key_of(it) + 4 * j + (lane >> 4), wlast);
        g[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + key * kIdxDim + (lane & 15) * 8));
      }
    }
  };

  // The query (32 head rows, laid out like a block of 32 keys) is read from
  // global memory once per workgroup into wave 0's staging buffer, and the
  // head weights into sh_w; every wave takes its operands from there.  The
  // first two key blocks of each wave are requested before that (loads
  // complete in order, so staging the query waits only for the query).
  const uint16_t* qt = A.q_idx + (int64_t)t * kIdxHeads * kIdxDim;
  constexpr int kQPieces = kIdxHeads * kIdxDim * 2 / 16 / kDecThreads;    // 16-byte pieces per thread
  static_assert(kQPieces * kDecThreads * 16 == kIdxHeads * kIdxDim * 2, "query pieces");
  u32x4 qv[kQPieces];
#pragma unroll
  for (int u = 0; u < kQPieces; ++u) {
    const int f = (int)threadIdx.x + kDecThreads * u;   // 16-byte piece: head f / 16, chunk f % 16
    qv[u] = ld16(qt + (f >> 4) * kIdxDim + (f & 15) * 8);
  }
  const float wv = A.w[(int64_t)t * kIdxHeads + (threadIdx.x & (kIdxHeads - 1))];
  // Prefetches are unconditional (clamped to the last valid step) so the
  // loads stay in order and each step waits only for its own data.
  u32x4 g0[kG], g1[kG];
  float ks0 = 1.f, ks1 = 1.f;
  load(g0, ks0, 0);
  load(g1, ks1, 1);
#pragma unroll
  for (int u = 0; u < kQPieces; ++u) {
    const int f = (int)threadIdx.x + kDecThreads * u;
    *reinterpret_cast<u32x4*>(lds[0] + (f >> 4) * kKeyPitch + (f & 15) * 16) = qv[u];
  }
  sh_w[threadIdx.x & (kIdxHeads - 1)] = wv;     // every thread (equal values): no branch, no late load
  lds_barrier();
  // A operand: head lane % 32, dims 16 s + 8 (lane / 32) .. +8 (chunk 2 s + lane / 32)
  bf16x8 a[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    a[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(lds[0] + (lane & 31) * kKeyPitch + (2 * s + (lane >> 5)) * 16));
  float wr[16];         // weights of this lane's accumulator rows
#pragma unroll
  for (int i = 0; i < 16; ++i) wr[i] = sh_w[acc_row(i, lane)];
  // wave 0 stages keys in lds[0] from here on
  lds_barrier();

  auto step = [&](const u32x4 (&g)[kG], float ks, int it) {
    if (FP8) {
#pragma unroll
      for (int j = 0; j < kG; ++j) {       // codes 16c .. 16c + 15 -> bf16 chunks 2c, 2c + 1
        u32x4 lo, hi;
        e4m3x16_to_bf16x16(g[j], lo, hi);
        uint8_t* dst = my + (8 * j + (lane >> 3)) * kKeyPitch + (lane & 7) * 32;
        *reinterpret_cast<u32x4*>(dst) = lo;
        *reinterpret_cast<u32x4*>(dst + 16) = hi;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kG; ++j)
        *reinterpret_cast<u32x4*>(my + (4 * j + (lane >> 4)) * kKeyPitch + (lane & 15) * 16) = g[j];
    }
    wave_lds_fence();
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 b = *reinterpret_cast<const u32x4*>(my + (lane & 31) * kKeyPitch + (2 * s + (lane >> 5)) * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], as_bf16x8(b), acc, 0, 0, 0);
    }
    wave_lds_fence();
    const float sc = FP8 ? relu_weighted_sum(acc, wr) * ks : relu_weighted_sum(acc, wr);
    const int key = key_of(it) + (lane & 31);
    if (lane < 32 && key < wend) sc0[key] = key <= wlast ? sc : -INFINITY;
  };

  static_assert(kDecSteps % 2 == 0, "steps alternate between two register sets");
#pragma unroll
  for (int it = 0; it < n_it; it += 2) {
    step(g0, ks0, it);
    if (it + 2 < n_it) load(g0, ks0, it + 2);
    step(g1, ks1, it + 1);
    if (it + 3 < n_it) load(g1, ks1, it + 3);
  }
}

// ----------------------------------------------------------- prefill kernel
constexpr int kPfQ = 16;           // queries per workgroup (2 per wave)
constexpr int kPfThreads = kPfQ * 32;
constexpr int kPfKT = 128;         // keys per tile
constexpr int kKeyBytes = kIdxDim * 2;
constexpr int kPfSplit = 16384;    // keys per workgroup

// FP8: E4M3 key codes with one fp32 scale per key; a tile's codes are
// decoded to bf16 (exact) when stored to LDS, its scales staged beside it,
// and each score multiplied by its key's scale.
template <bool FP8>
__global__ __launch_bounds__(kPfThreads, 512 / kPfThreads) void indexer_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
    const float* __restrict__ k_scale, const int64_t* __restrict__ seq_start, const int32_t* __restrict__ seq_len, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int n_q, float* __restrict__ scores, int64_t ld, int n_splits) {
  // Workgroups are dealt to the 8 XCDs round-robin (bid % 8).  Give each XCD a
  // contiguous run of the split-major work list, so the workgroups resident on
  // one XCD share the same 4 MB key split in that XCD's L2.
  const int n_wg = (int)gridDim.x;
  const int item = (n_wg & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (n_wg >> 3) + (int)(blockIdx.x >> 3);
  const int n_qb = n_wg / n_splits;
  const int split = item / n_qb;
  const int qb = item - split * n_qb;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t s0 = (int64_t)split * kPfSplit;
  const int64_t s1 = min(s0 + (int64_t)kPfSplit, ld);
  const int t_base = qb * kPfQ;

  __shared__ __align__(16) uint8_t lds[2][kPfKT * kKeyPitch];
  __shared__ float sh_ks[FP8 ? 2 : 1][FP8 ? kPfKT : 1];   // FP8: the tiles' key scales
  __shared__ int sh_seq[kPfQ];
  __shared__ int sh_pos[kPfQ];
  __shared__ int sh_done[kPfQ];
  __shared__ __align__(16) float sh_w[kPfQ][kIdxHeads];   // head weights, staged for the register copies
  {
    const int t = min(t_base + (int)(threadIdx.x >> 5), n_q - 1);
    sh_w[threadIdx.x >> 5][threadIdx.x & 31] = w[(int64_t)t * kIdxHeads + (threadIdx.x & 31)];
  }
  if (threadIdx.x < kPfQ) {
    const int t = t_base + threadIdx.x;
    const int sq = t < n_q ? q_seq[t] : -1;
    sh_seq[threadIdx.x] = sq;
    // causal set clamped to the sequence's keys (-1: no key; the row is all -inf)
    sh_pos[threadIdx.x] = t < n_q ? min(q_pos[t], seq_len[sq] - 1) : -1;
    sh_done[threadIdx.x] = t < n_q ? 0 : 1;
  }
  __syncthreads();

  // This wave's two queries: A operands in registers.
  bf16x8 a[2][8];
  int64_t pos[2];
  int seq[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int lq = 2 * wave + qq;
    const int t = min(t_base + lq, n_q - 1);
    pos[qq] = sh_pos[lq];
    seq[qq] = sh_seq[lq];
    const uint16_t* qt = q_idx + (int64_t)t * kIdxHeads * kIdxDim;
#pragma unroll
    for (int s = 0; s < 8; ++s) a[qq][s] = as_bf16x8(ld16(qt + (lane & 31) * kIdxDim + 16 * s + 8 * (lane >> 5)));
  }
  // Head weights of this lane's accumulator rows, for both queries (32
  // registers; reading them from LDS at every column was 0.7-1.3% slower).
  float wr[2][16];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq)
#pragma unroll
    for (int i = 0; i < 16; ++i) wr[qq][i] = sh_w[2 * wave + qq][acc_row(i, lane)];
  // The query operands are in before the key loop starts.  Without this wait
  // the compiler, which tracks load counters per register, places waits for
  // them inside the loop, where (the counter being in order) they also wait
  // for the next tile's prefetch and the score stores in every tile: about
  // 40% of the MFMA time.
  SA_WAIT_VMCNT(0);

  // Queries of one block may belong to several sequences: handle one sequence
  // per pass, the others' rows stay untouched in that pass.
#pragma unroll 1
  for (int pass = 0; pass < kPfQ; ++pass) {
    int cur = -1;
    int64_t maxpos = -1;
    for (int i = 0; i < kPfQ; ++i)
      if (!sh_done[i] && cur < 0) cur = sh_seq[i];
    if (cur < 0) break;
    for (int i = 0; i < kPfQ; ++i)
      if (!sh_done[i] && sh_seq[i] == cur) maxpos = max(maxpos, (int64_t)sh_pos[i]);
    // (queries past n_q have seq -1; a query with no key has pos -1 and
    // gets -inf everywhere)
    const bool act0 = seq[0] == cur;
    const bool act1 = seq[1] == cur;
    const uint16_t* kbase = k_idx + seq_start[cur] * kIdxDim;
    const int64_t cend = min(s1, maxpos + 1);              // keys that need a product
    const int n_tiles = cend > s0 ? (int)((cend - s0 + kPfKT - 1) / kPfKT) : 0;
    // Score rows of this wave's queries from key s0 on; positions relative to
    // s0 (clamped into [-1, kPfSplit]), so the tile loop uses 32-bit offsets.
    const int span = (int)(s1 - s0);
    float* srow0 = scores + (int64_t)(t_base + 2 * wave) * ld + s0;
    float* srow1 = srow0 + ld;
    const int rpos0 = (int)max(min(pos[0] - s0, (int64_t)kPfSplit), (int64_t)-1);
    const int rpos1 = (int)max(min(pos[1] - s0, (int64_t)kPfSplit), (int64_t)-1);
    const int rmax = (int)max(min(maxpos - s0, (int64_t)kPfSplit), (int64_t)-1);
    const uint16_t* kseg = kbase + s0 * kIdxDim;
    const uint8_t* kseg8 = reinterpret_cast<const uint8_t*>(k_idx) + (seq_start[cur] + s0) * kIdxDim;
    const float* kssg = FP8 ? k_scale + seq_start[cur] + s0 : nullptr;

    // Key tiles go global -> registers -> LDS (double-buffered): the loads of
    // tile i + 1 are issued before the products of tile i and stored to LDS
    // after them.
    constexpr int kPieces = kPfKT * (FP8 ? kIdxDim : kKeyBytes) / 16 / kPfThreads;   // 16-byte pieces per thread
    u32x4 ga[kPieces];
    float gks = 1.f;                   // FP8: the scale of key threadIdx.x of the tile
    auto load_tile = [&](u32x4 (&g)[kPieces], int tile) {
#pragma unroll
      for (int j = 0; j < kPieces; ++j) {
        const int flat = j * kPfThreads + threadIdx.x;     // 16-byte piece within the tile
        // keys past the last needed one re-read that key (their scores are -inf)
        if (FP8) {
          const int rkey = min(tile * kPfKT + (flat >> 3), rmax);
          g[j] = ld16(kseg8 + rkey * kIdxDim + (flat & 7) * 16);
        } else {
          const int rkey = min(tile * kPfKT + (flat >> 4), rmax);
          g[j] = ld16(kseg + rkey * kIdxDim + (flat & 15) * 8);
        }
      }
      if (FP8 && threadIdx.x < kPfKT) gks = kssg[min(tile * kPfKT + (int)threadIdx.x, rmax)];
    };
    auto store_tile = [&](const u32x4 (&g)[kPieces], int buf) {
#pragma unroll
      for (int j = 0; j < kPieces; ++j) {
        const int flat = j * kPfThreads + threadIdx.x;
        if (FP8) {                     // codes 16c .. 16c + 15 -> bf16 chunks 2c, 2c + 1
          u32x4 lo, hi;
          e4m3x16_to_bf16x16(g[j], lo, hi);
          uint8_t* dst = lds[buf] + (flat >> 3) * kKeyPitch + (flat & 7) * 32;
          *reinterpret_cast<u32x4*>(dst) = lo;
          *reinterpret_cast<u32x4*>(dst + 16) = hi;
        } else {
          *reinterpret_cast<u32x4*>(lds[buf] + (flat >> 4) * kKeyPitch + (flat & 15) * 16) = g[j];
        }
      }
      if (FP8 && threadIdx.x < kPfKT) sh_ks[buf][threadIdx.x] = gks;
    };
    // Products of key column n (32 keys) of the tile in LDS buffer buf, for
    // both queries.
    auto column = [&](f32x16 (&acc)[2], int buf, int n) {
      u32x4 b[8];                       // the column's operands, read before its products
#pragma unroll
      for (int s = 0; s < 8; ++s)
        b[s] = *reinterpret_cast<const u32x4*>(lds[buf] + (n * 32 + (lane & 31)) * kKeyPitch +
                                               (2 * s + (lane >> 5)) * 16);
      acc[0] = f32x16{};
      acc[1] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][s], as_bf16x8(b[s]), acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][s], as_bf16x8(b[s]), acc[1], 0, 0, 0);
      }
    };
    // ReLU sums and stores of column n of a tile (skipped for tile < 0).
    // Lanes 0..31 finish the first query's scores of the column's 32 keys,
    // lanes 32..63 the second query's: one exchange, one store.
    const bool hi = lane >= 32;
    const bool act_l = hi ? act1 : act0;
    const int rpos_l = hi ? rpos1 : rpos0;
    float* srow_l = hi ? srow1 : srow0;
    auto finish = [&](const f32x16 (&acc)[2], int tile, int n) {
      float sc = sum_halves(relu_weighted_part(acc[0], wr[0]), relu_weighted_part(acc[1], wr[1]));
      if (FP8) sc *= sh_ks[tile & 1][n * 32 + (lane & 31)];
      const int rkey = tile * kPfKT + n * 32 + (lane & 31);
      // streaming store: the score rows are read back only by the next kernel
      if (act_l && tile >= 0 && rkey < span) __builtin_nontemporal_store(rkey <= rpos_l ? sc : -INFINITY, &srow_l[rkey]);
    };
    // Software pipeline over the key columns of a tile: each column is
    // finished during the products of the next one (the last column of a tile
    // during the next tile's first), so the MFMA pipe has work while the ReLU
    // sums run.  Columns alternate between the two accumulator sets.
    constexpr int kCols = kPfKT / 32;
    static_assert(kCols % 2 == 0, "an even number of key columns per tile");
    f32x16 acc0[2], acc1[2] = {f32x16{}, f32x16{}};
    auto products = [&](int tile) {
      const int buf = tile & 1;
#pragma unroll
      for (int c = 0; c < kCols; c += 2) {
        column(acc0, buf, c);
        finish(acc1, c == 0 ? tile - 1 : tile, c == 0 ? kCols - 1 : c - 1);
        column(acc1, buf, c + 1);
        finish(acc0, tile, c);
      }
    };
    if (n_tiles > 0) {
      load_tile(ga, 0);
      store_tile(ga, 0);
    }
    __syncthreads();
    // The next tile's loads and stores are unconditional (the last tile
    // re-reads itself into the idle buffer): with a branch around them the
    // compiler cannot tell that the loads it waits for at the store were
    // issued on the same path, and waits for every outstanding memory
    // operation, score stores included, at the top of each tile.
#pragma unroll 1
    for (int tile = 0; tile < n_tiles; ++tile) {
      load_tile(ga, min(tile + 1, n_tiles - 1));
      products(tile);
      store_tile(ga, (tile + 1) & 1);
      __syncthreads();
    }
    if (n_tiles > 0) finish(acc1, n_tiles - 1, kCols - 1);
    // keys of this split past the last needed tile: -inf for the active queries
    for (int r = n_tiles * kPfKT + lane; r < span; r += 64) {
      if (act0) srow0[r] = -INFINITY;
      if (act1) srow1[r] = -INFINITY;
    }
    __syncthreads();
    if (threadIdx.x < kPfQ && sh_seq[threadIdx.x] == cur) sh_done[threadIdx.x] = 1;
    __syncthreads();
  }
}

}  // namespace sa

// ------------------------------------------------------------------ launchers
namespace sa_host {

// Automatic choice: the query-blocked kernel pays off only when its 16-query
// blocks share a sequence, i.e. when the batch holds at least 16 queries per
// sequence on average (chunked prefill); batches of decode queries, one or a
// few per sequence, stream each query's keys (64 queries of 64 sequences run
// 80x faster that way than as 16-sequence blocks).
int indexer_algo(int32_t n_q, int32_t n_seq, int algo) {
  if (algo != 0) return algo;
  return (n_q >= 64 && (int64_t)n_q >= 16 * (int64_t)(n_seq > 0 ? n_seq : 1)) ? 2 : 1;
}

// clear / n_clear: words the decode kernel (algo 1) sets to zero on the side;
// the caller passes none with algo 2.
// k_scale != NULL: k_idx holds E4M3 codes with one scale per key.
int32_t launch_indexer(const void* q_idx, const float* w, const void* k_idx, const float* k_scale,
                       const int64_t* seq_start, const int32_t* seq_len, const int32_t* q_seq, const int32_t* q_pos,
                       int32_t n_q, int32_t n_seq, float* scores, int64_t ld, int algo, hipStream_t stream,
                       uint32_t* clear, int64_t n_clear) {
  algo = indexer_algo(n_q, n_seq, algo);
  if (algo != 1 && n_clear > 0) {
    set_error("indexer: only the decode kernel clears words on the side");
    return SA_ERR_INVALID_ARG;
  }
  if (algo == 1) {
    const int n_chunks = (int)((ld + sa::kDecChunk - 1) / sa::kDecChunk);
    const int64_t grid = (int64_t)n_chunks * n_q;
    if (grid > 0x7fffffff) {
      set_error("indexer: grid of %lld workgroups is too large", (long long)grid);
      return SA_ERR_UNSUPPORTED;
    }
    sa::DecArgs A{(const uint16_t*)q_idx, w, (const uint16_t*)k_idx, k_scale, seq_start, seq_len, q_seq, q_pos,
                  scores, ld, n_chunks, clear, n_clear > 0 ? n_clear : 0};
    if (k_scale)
      hipLaunchKernelGGL(sa::indexer_decode_kernel<true>, dim3((unsigned)grid), dim3(sa::kDecThreads), 0, stream, A);
    else
      hipLaunchKernelGGL(sa::indexer_decode_kernel<false>, dim3((unsigned)grid), dim3(sa::kDecThreads), 0, stream, A);
    return check_launch("indexer_decode_kernel");
  }
  const int n_splits = (int)((ld + sa::kPfSplit - 1) / sa::kPfSplit);
  const int n_qb = (n_q + sa::kPfQ - 1) / sa::kPfQ;
  const int64_t grid = (int64_t)n_splits * n_qb;
  if (grid > 0x7fffffff) {
    set_error("indexer: grid of %lld workgroups is too large", (long long)grid);
    return SA_ERR_UNSUPPORTED;
  }
  if (k_scale)
    hipLaunchKernelGGL(sa::indexer_prefill_kernel<true>, dim3((unsigned)grid), dim3(sa::kPfThreads), 0, stream,
                       (const uint16_t*)q_idx, w, (const uint16_t*)k_idx, k_scale, seq_start, seq_len, q_seq, q_pos,
                       n_q, scores, ld, n_splits);
  else
    hipLaunchKernelGGL(sa::indexer_prefill_kernel<false>, dim3((unsigned)grid), dim3(sa::kPfThreads), 0, stream,
                       (const uint16_t*)q_idx, w, (const uint16_t*)k_idx, k_scale, seq_start, seq_len, q_seq, q_pos,
                       n_q, scores, ld, n_splits);
  return check_launch("indexer_prefill_kernel");
}

}  // namespace sa_host
