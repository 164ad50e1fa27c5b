// Absorbed sparse MLA attention and the W_UV up-projection for gfx950.
//
// For query t, head h, over the selected cache rows R_j (576 = 512 latent +
// 64 rope; models.inteligile.com "GLM-5.2 / Model techniques map", "Checked
// in its code", rows "Multi-head latent attention" and "Indexer-selected
// sparse attention"; softmax in fp32 with no sink and no output gate, rows
// "Learnable attention sink" and "Gated attention output"):
//     z_j = scale * q_abs[t, h] . R_j,  obar = softmax(z) @ R[:, :512],
//     out[t, h] = bf16(W_UV[h] @ obar).
//
// mla_attn_kernel: for decode batches below 64 queries one workgroup per
// (query, slice of the selection, group of 32 heads), the two head groups of a
// slice gathering the same rows at the same time through one XCD's L2; from
// 64 queries on one workgroup per (query, slice) for both groups, which share
// every gathered tile (the same code with two head blocks).  The slice is
// consumed in 32-row tiles by 4 score waves and 4 output waves working one tile
// apart:
//   - the output waves gather each tile (36 KB) with 16-byte direct-to-LDS
//     loads into a 3-buffer ring, so two tiles are in flight without registers.
//     A tile buffer is latent-quarter-major, [4 quarters][32 rows][256 B] and
//     then [32 rows][128 B] of rope, so output wave w refills exactly the
//     quarter it reads and can issue the next gather as soon as its own reads
//     of the old tile are done, while the score waves are still in QK^T;
//   - score wave w computes the partial S^T[32 rows x 32 heads] = R . Q^T over
//     dims 144w..144w+143 with v_mfma_f32_32x32x16_bf16 (R from LDS, Q^T in
//     registers); after an exchange through LDS it runs the online softmax of
//     heads 8w..8w+7 of the group in base 2 (the running max is only moved
//     when a tile exceeds it by more than 2^8, so rescaling is rare) and puts
//     its bf16 weights and any rescale factors in LDS;
//   - output wave w accumulates O^T[latent dims 128w..128w+127 x 32 heads] +=
//     V^T . P^T of the previous tile with v_mfma_f32_32x32x16_bf16: the 32 rows
//     are the contraction, the V^T operand is assembled from 8-byte row pieces
//     with byte permutes (rows and dims are permuted consistently in both
//     operands, no transpose through LDS), P^T comes from the score waves.
// Within a quarter row (16 chunks of 16 bytes) chunk c of row r sits at slot
// c ^ (r & 15), within a rope row (8 chunks) at slot c ^ ((r >> 1) & 7): the
// 16 lanes of one operand read hit 16 different bank groups.
// With one slice per query the workgroup normalises and writes the latent
// average obar (bf16); with several, each writes its partial state.  With
// one 32-head block per workgroup and 2..8 slices (16..63 decode queries)
// the partial states are bf16 and head-major, and mla_merge_wuv_kernel
// merges them inside the W_UV launch; otherwise they are fp32 in register
// tile order and mla_merge_kernel (up to 8 slices), mla_merge_wide_kernel
// (more slices, i.e. few queries) or mla_merge_split_kernel (more slices and
// at most two queries) combines them into obar.
// mla_wuv_kernel: one workgroup per (head, 64 value rows) stages that 64 x 512
// slice of W_UV in LDS and multiplies it with obar^T, 16 queries per
// v_mfma_f32_16x16x32_bf16 column block, rounding the output to bf16.
#include <atomic>

#include "fp8.h"
#include "sa_common.h"

namespace sa {

constexpr int kAttnWaves = 4;
constexpr int kTile = 32;                  // rows per tile
constexpr int kRowBytes = kRow * 2;        // 1152
constexpr int kTileBytes = kTile * kRowBytes;                     // 36,864
constexpr int kQuarterBytes = kTile * 256;                        // one latent quarter (128 dims) of a tile
constexpr int kRopeOff = 4 * kQuarterBytes;                       // the tile's rope block
constexpr int kRing = 3;                   // LDS tile buffers (two tiles in flight)
constexpr int kLoadsPerWave = kTileBytes / 1024 / kAttnWaves;    // 9 direct-to-LDS loads of 1 KB
constexpr float kRescaleSlack = 8.0f;      // log2 units
constexpr int kMaxSp = 32;
constexpr int kCpolNt = 2;                 // cache-policy operand of global_load_lds: non-temporal

__device__ __forceinline__ uint32_t perm_lo(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
__device__ __forceinline__ uint32_t perm_hi(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }

// Byte offset in a tile buffer of 16-byte chunk c (0..71) of row r.
__device__ __forceinline__ int tile_chunk_offset(int r, int c) {
  return c < 64 ? (c >> 4) * kQuarterBytes + r * 256 + 16 * ((c & 15) ^ (r & 15))
                : kRopeOff + r * 128 + 16 * ((c - 64) ^ ((r >> 1) & 7));
}

struct AttnArgs {
  const uint16_t* q_abs;
  const uint16_t* kv;
  const int64_t* seq_start;
  const int32_t* q_seq;
  const int32_t* idx;
  int k;
  int n_q;
  int n_sp;
  int kps;               // selection entries per slice (multiple of kTile)
  float scale_log2;      // scale * log2(e)
  float* part_o;         // n_sp > 1: [n_q][n_sp] blocks of 64 x 512 fp32 in register-tile order, or with
                         // part_bf16 [n_q][n_sp][64][512] bf16 (unnormalised, head-major)
  float* part_ml;        // [n_q][n_sp][64][2]     (max in log2 units, sum)
  uint16_t* obar;        // [n_q][64][512] bf16 latent average
  float* lse;            // [n_q][64] or null
  const float* kv_scale; // FP8 rows: kv holds E4M3 codes [rows][576] and this one scale per row
  int part_bf16;         // partial states in bf16, head-major (merged by mla_merge_wuv_kernel)
};

constexpr int kMaxSlice = 2048;
constexpr int kHeadGroup = 32;             // heads per block (two blocks per query)
constexpr size_t kRingBytes = (size_t)kRing * kTileBytes;                  // 110,592
// per block of 32 heads:
constexpr size_t kSBytes = 4 * 4 * 64 * 16;                               // partial S^T of each score wave
constexpr size_t kPBytes = 2 * kHeadGroup * 80;                           // bf16 weights, double-buffered, 80 B per head
constexpr size_t kAlphaBytes = 2 * kHeadGroup * 4;                        // rescale factors
constexpr size_t kMlBytes = kHeadGroup * 2 * 4;                           // (m, l) per head at the end
constexpr size_t kFlagBytes = 2 * 4 * 4;
// LDS of a workgroup with NB blocks of 32 heads (NB = 2: 162,848 bytes)
constexpr size_t kScBytes = (size_t)kRing * kTile * 4;                      // FP8 rows: each staged row's scale
template <int NB, bool FP8 = false>
constexpr size_t attn_smem() {
  return kRingBytes + NB * (kSBytes + kPBytes + kAlphaBytes + kMlBytes) + kFlagBytes + kMaxSlice * 4 +
         (FP8 ? kScBytes : 0);
}
static_assert(attn_smem<2, true>() <= 160 * 1024, "two head blocks fit the LDS of a CU");
constexpr int kAttnThreads = 512;          // 4 score waves + 4 output waves

// Slot of the 4-row group p (rows 4p..4p+3) in a head's weight entry: the
// output waves read groups (4ks + hl, 4ks + 2 + hl) as one 16-byte operand.
__device__ __forceinline__ int p_slot(int p) { return (p & 4) | ((p & 1) << 1) | ((p >> 1) & 1); }

// x combined over the 8 lanes of an aligned group, every lane gets the result
// (DPP: mirror within the 8, then swap neighbours, then swap pairs).
template <typename Op>
__device__ __forceinline__ float reduce8(float x, Op op) {
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false)));   // row_half_mirror
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xb1, 0xf, 0xf, false)));    // quad_perm 1,0,3,2
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4e, 0xf, 0xf, false)));    // quad_perm 2,3,0,1
  return x;
}

// NB = 1: one workgroup per (query, slice, group of 32 heads); NB = 2: one per
// (query, slice) for all 64 heads, the two blocks of 32 heads sharing every
// gathered tile (half the gathers and steps per head, twice the products per
// step).  Head block blk of a workgroup is head group hg + blk.
//
// FP8 (kv holds E4M3 codes, one fp32 scale per row): the output waves gather
// 576-byte code rows and their scales into registers one step ahead and land
// them in the same tile buffers decoded to bf16 (exact), with the scales in
// sclds; the score waves scale each logit by its row's scale and feed
// p_j * scale_j to the value product, while the softmax sum keeps p_j: the
// attention of the rows scale_j * value(codes_j).
//
// CACHED: the row gathers use the default cache policy instead of streaming
// loads, for batches whose queries share their sequences' rows (chunked
// prefill: 4096 queries of one sequence gather each of its rows about 64
// times per layer, and these repeats then hit in the caches).
template <int NB, bool FP8, bool CACHED>
__global__ __launch_bounds__(kAttnThreads, 1) void mla_attn_kernel(AttnArgs A) {
  // Workgroups are dealt to the 8 XCDs round-robin (bid % 8): give each XCD a
  // contiguous run of (query, slice, head group) items, so the two head
  // groups of a slice gather the same rows through one L2 at the same time.
  const int n_wg = (int)gridDim.x;
  const int item = (n_wg & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (n_wg >> 3) + (int)(blockIdx.x >> 3);
  const int hg = NB == 1 ? (item & 1) : 0;
  const int ts = NB == 1 ? (item >> 1) : item;
  const int t = ts / A.n_sp;
  const int sp = ts - t * A.n_sp;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int w = wave & 3;                       // dim quarter of QK (score waves) / latent quarter (output waves)
  const int l32 = lane & 31, hl = lane >> 5;    // MFMA column / row within the 32x32 tile, and lane half

  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* ring = smem;
  // [NB][4 waves][4 row groups][64 lanes, lane l at slot l ^ 2 (2 group + l / 32)]
  f32x4* slds = reinterpret_cast<f32x4*>(smem + kRingBytes);
  uint8_t* sm2 = smem + kRingBytes + NB * kSBytes;
  u32x2* plds = reinterpret_cast<u32x2*>(sm2);                             // [2][NB * 32 heads][10 slots, 8 used]
  float* alds = reinterpret_cast<float*>(sm2 + NB * kPBytes);              // [2][NB * 32 heads]
  int* flds = reinterpret_cast<int*>(sm2 + NB * (kPBytes + kAlphaBytes));  // [2][4 score waves]
  float* mlds = reinterpret_cast<float*>(sm2 + NB * (kPBytes + kAlphaBytes) + kFlagBytes);   // [NB * 32][2]
  int32_t* spos = reinterpret_cast<int32_t*>(sm2 + NB * (kPBytes + kAlphaBytes + kMlBytes) + kFlagBytes);
  float* sclds = reinterpret_cast<float*>(spos + kMaxSlice);                 // FP8: [kRing][32] row scales

  const int j0 = sp * A.kps;
  const int j1 = min(A.k, j0 + A.kps);
  const int n_sel = max(j1 - j0, 0);
  // The slice's positions: loaded first, stored to LDS once the score waves
  // have also issued their query loads (so the two round trips overlap).
  int pv[kMaxSlice / kAttnThreads];
  if (n_sel > 0) {
    const int32_t* irow = A.idx + (int64_t)t * A.k + j0;
#pragma unroll
    for (int u = 0; u < kMaxSlice / kAttnThreads; ++u)
      pv[u] = irow[min((int)threadIdx.x + kAttnThreads * u, n_sel - 1)];
  }
  // Entries past the slice, up to the end of its last tile (at least one
  // tile), read as padding (-1): validity is then just position >= 0.
  const int n_tiles = (n_sel + kTile - 1) / kTile;
  const int n_stage = max(n_tiles, 1) * kTile;
  auto store_positions = [&]() {
#pragma unroll
    for (int u = 0; u < kMaxSlice / kAttnThreads; ++u) {
      const int j = (int)threadIdx.x + kAttnThreads * u;
      if (j < n_stage) spos[j] = j < n_sel ? pv[u] : -1;
    }
  };

  // Both roles pass the same sequence of workgroup barriers: B0 (positions
  // staged), B1 (tile 0 staged), then per step BAR_s and BAR_p, then BAR_end.
  //
  // Products use v_mfma_f32_32x32x16_bf16 (lane l: A row / B column l % 32,
  // contraction slots 8 (l / 32) .. +8; result element i of lane l is row
  // 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32).
  if (wave < 4) {
    // =========================== score waves: QK^T and the online softmax of tile `step`
    // S^T[32 rows x 32 heads] is split over the 576 dims: wave w takes dims
    // 144w .. 144w + 143 (9 steps of 16).  Q operand: head 32hg + l32, dims
    // 144w + 16s + 8hl .. +8.
    bf16x8 qb[NB][9];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const uint16_t* qp = A.q_abs + ((int64_t)t * kHeads + kHeadGroup * (hg + blk) + l32) * kRow + 144 * w + 8 * hl;
#pragma unroll
      for (int s = 0; s < 9; ++s) qb[blk][s] = as_bf16x8(ld16(qp + 16 * s));
    }
    store_positions();
    // The staged positions must be visible; the query loads stay in flight.
    lds_barrier();                                                     // B0
    // R operand: row l32, 16-byte chunk 18w + 2s + hl.
    int roff[9];
#pragma unroll
    for (int s = 0; s < 9; ++s) roff[s] = tile_chunk_offset(l32, 18 * w + 2 * s + hl);
    // Softmax ownership: this wave finishes heads 8w .. 8w + 7 of the group;
    // lane (hd, p) = (lane / 8, lane % 8) takes head 8w + hd and rows
    // 4p .. 4p + 3, i.e. elements 4 (p / 2) .. +3 of result column
    // 8w + hd + 32 (p % 2).
    const int hd = lane >> 3, pq = lane & 7;
    const int hloc = 8 * w + hd;
    const int src_lane = hloc + 32 * (pq & 1);
    const int ig = pq >> 1;
    float m_run[NB], l_run[NB];               // softmax state of head hloc of each block (lane-partial sum)
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      m_run[blk] = -INFINITY;
      l_run[blk] = 0.f;
    }
    lds_barrier();                                                     // B1: tile 0 staged
#pragma unroll 1
    for (int tile = 0; tile <= n_tiles; ++tile) {
      const bool active = tile < n_tiles;
      const uint8_t* cur = ring + (tile % kRing) * kTileBytes;
      const int pb_i = tile & 1;
      const int jt = tile * kTile;
      if (active) {
        // ---- partial S^T = R . Q^T over this wave's dims, 32 heads, 32 rows.
        u32x4 ra[9];            // all of this wave's row chunks of the tile, read up front
#pragma unroll
        for (int s = 0; s < 9; ++s)
          ra[s] = *reinterpret_cast<const u32x4*>(cur + roff[s]);
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          f32x16 acc = {};
#pragma unroll
          for (int s = 0; s < 9; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ra[s]), qb[blk][s], acc, 0, 0, 0);
#pragma unroll
          for (int g = 0; g < 4; ++g)
            slds[((blk * 4 + w) * 4 + g) * 64 + (lane ^ (2 * (2 * g + hl)))] =
                f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
        }
        // Issue order: the 9 operand reads, then the products, then the
        // partial stores.  Left alone, the scheduler interleaves the reads
        // with the products and keeps only one or two of them in flight.
        __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);        // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 9 * NB, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x200, 4 * NB, 0);   // LDS writes
      }
      lds_barrier();                                                   // BAR_s
      if (active) {
        // full scores of this lane's 4 rows: sum of the 4 waves' partials
        // (the swizzle puts the 16 lanes of a read on 16 bank groups)
        const int src_sw = src_lane ^ (2 * pq);
        const u32x4 pos4 = *reinterpret_cast<const u32x4*>(spos + jt + 4 * pq);
        f32x4 rs4 = {1.f, 1.f, 1.f, 1.f};        // FP8: the scales of this lane's 4 rows
        if constexpr (FP8) rs4 = *reinterpret_cast<const f32x4*>(sclds + (tile % kRing) * kTile + 4 * pq);
        f32x4 sp4[NB][4];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) sp4[blk][w2] = slds[((blk * 4 + w2) * 4 + ig) * 64 + src_sw];
        // every read above goes out before the first sum: one LDS round trip
        __builtin_amdgcn_sched_barrier(0);
        float x[NB][4];
        float tmax[NB];
        bool bump[NB];
        bool bump_any = false;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          const f32x4 s4 = ((sp4[blk][0] + sp4[blk][1]) + sp4[blk][2]) + sp4[blk][3];
          // ---- online softmax of head hloc of the block over rows jt + 4pq .. +3
          tmax[blk] = -INFINITY;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[blk][j] = (int)pos4[j] >= 0 ? (FP8 ? s4[j] * (rs4[j] * A.scale_log2) : s4[j] * A.scale_log2) : -INFINITY;
            tmax[blk] = fmaxf(tmax[blk], x[blk][j]);
          }
          tmax[blk] = reduce8(tmax[blk], [](float a, float b) { return fmaxf(a, b); });
          bump[blk] = tmax[blk] > m_run[blk] + kRescaleSlack;
          bump_any |= bump[blk];
        }
        // One flag per wave and step covers its heads in every block, so when
        // it is set every block's factor is written (1 where nothing moved).
        const bool any_bump = __any(bump_any);
        if (any_bump) {
#pragma unroll
          for (int blk = 0; blk < NB; ++blk) {
            const float alpha = bump[blk] ? (m_run[blk] == -INFINITY ? 0.f : fast_exp2(m_run[blk] - tmax[blk])) : 1.f;
            if (bump[blk]) m_run[blk] = tmax[blk];
            l_run[blk] *= alpha;
            alds[pb_i * NB * kHeadGroup + blk * kHeadGroup + hloc] = alpha;   // the 8 lanes of a head store the same value
          }
        }
        flds[pb_i * 4 + w] = any_bump ? 1 : 0;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          // masked rows have x = -inf and weight exp2(-inf) = 0; m_run is -inf
          // only while every row so far was masked
          const float m_use = m_run[blk] == -INFINITY ? 0.f : m_run[blk];
          float p[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            p[j] = fast_exp2(x[blk][j] - m_use);
            l_run[blk] += p[j];
          }
          if constexpr (FP8)
            plds[((pb_i * NB + blk) * kHeadGroup + hloc) * 10 + p_slot(pq)] =
                u32x2{pack_bf16x2(p[0] * rs4[0], p[1] * rs4[1]), pack_bf16x2(p[2] * rs4[2], p[3] * rs4[3])};
          else
            plds[((pb_i * NB + blk) * kHeadGroup + hloc) * 10 + p_slot(pq)] =
                u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
        }
      }
      lds_barrier();                                                   // BAR_p
    }
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      // Head hloc of the block: sum over the 8 lanes that share it.
      const float lsum = reduce8(l_run[blk], [](float a, float b) { return a + b; });
      if (pq == 0) {
        const int head = kHeadGroup * (hg + blk) + hloc;
        mlds[(blk * kHeadGroup + hloc) * 2 + 0] = m_run[blk];
        mlds[(blk * kHeadGroup + hloc) * 2 + 1] = lsum;
        if (A.n_sp == 1) {
          if (A.lse)
            A.lse[(int64_t)t * kHeads + head] = lsum > 0.f ? (m_run[blk] + __log2f(lsum)) * 0.69314718055994531f : -INFINITY;
        } else {
          const int64_t pbase = ((int64_t)t * A.n_sp + sp) * kHeads;
          A.part_ml[(pbase + head) * 2 + 0] = m_run[blk];
          A.part_ml[(pbase + head) * 2 + 1] = lsum;
        }
      }
    }
    lds_barrier();                                                     // BAR_end
    return;
  }
  // =========================== output waves: O^T += V^T . P^T of tile `step - 1`
  // Wave w owns latent dims 128w .. 128w+127 for the 32 heads: result tile mt
  // holds dims 128w + 4m + mt (m = result row) of heads 32hg + n.  The 32
  // rows of a tile are two contraction steps ks of 16; slot 8hl + e of step
  // ks is row 16ks + 8 (e >> 2) + 4hl + (e & 3) in both operands (the score
  // waves' weight slots 4ks + 2hl and +1 hold exactly these rows).  The V^T
  // operand of lane (m = l32, hl) takes 8 bytes (dims 4m .. 4m+3) of each of
  // its 8 rows and byte permutes form the four dim tiles mt.
  // Direct-to-LDS gather of the tiles, issued by these waves, 16 bytes per
  // lane: loads u < 8 of wave w fill quarter w of rows 4u .. 4u + 3 (1 KB),
  // load 8 the rope of rows 8w .. 8w + 7; each lane fetches the row chunk
  // whose swizzled slot it fills.
  const uint8_t* rows_b = reinterpret_cast<const uint8_t*>(A.kv + A.seq_start[A.q_seq[t]] * kRow);
  int lrow[kLoadsPerWave], lcol[kLoadsPerWave];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = 4 * u + (lane >> 4);
    lrow[u] = r;
    lcol[u] = 16 * (16 * w + ((lane & 15) ^ (r & 15)));
  }
  {
    const int r = 8 * w + (lane >> 3);
    lrow[8] = r;
    lcol[8] = 16 * (64 + ((lane & 7) ^ ((r >> 1) & 7)));
  }
  auto read_pos = [&](int tile, int (&pos)[kLoadsPerWave]) {
    const int jt = min(tile, max(n_tiles - 1, 0)) * kTile;
#pragma unroll
    for (int u = 0; u < kLoadsPerWave; ++u) pos[u] = spos[jt + lrow[u]];
  };
  auto issue_at = [&](int tile, const int (&pos)[kLoadsPerWave]) {
    uint8_t* b = ring + (tile % kRing) * kTileBytes;
#pragma unroll
    for (int u = 0; u < kLoadsPerWave; ++u) {
      // padding entries read row 0; byte offsets within the sequence stay
      // below 2^32 for sequences below 3.7M rows.  Cache policy: streaming
      // (non-temporal) unless CACHED, as in decode batches the rows are dead
      // after this step's two head groups (-1.5 us per launch against the
      // default policy).
      const int p = pos[u] >= 0 ? pos[u] : 0;
      const uint32_t off = (uint32_t)p * (uint32_t)kRowBytes + (uint32_t)lcol[u];
      uint8_t* dst = b + (u < 8 ? w * kQuarterBytes + 1024 * u : kRopeOff + 1024 * w);
      __builtin_amdgcn_global_load_lds((const void*)(rows_b + off), (__attribute__((address_space(3))) void*)dst, 16,
                                       0, CACHED ? 0 : kCpolNt);
    }
  };
  auto issue = [&](int tile) {
    // every position first (one LDS round trip), then the loads
    int pos[kLoadsPerWave];
    read_pos(tile, pos);
    issue_at(tile, pos);
  };
  // Streaming gathers take the positions of the tile they issue from
  // registers, read one step earlier while the products ran, so the loads go
  // out as soon as the operand reads are back (about -0.5 us per launch on
  // 16-query decode steps).  With cached gathers (chunked prefill) that
  // measured slower, and the positions are read just before the loads.
  constexpr bool kPosAhead = !FP8 && !CACHED;
  // V^T operand: 8-byte read of row rho = 16ks + 8(e >> 2) + 4hl + (e & 3),
  // dims 128w + 4 l32 .. +3 (chunk 16w + l32 / 2, half l32 & 1); rho & 15 is
  // 8(e >> 2) + 4hl + (e & 3) for every ks.
  int voff[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) voff[e] = tile_chunk_offset(8 * (e >> 2) + 4 * hl + (e & 3), 16 * w + (l32 >> 1)) + 8 * (l32 & 1);
  f32x16 o[NB][4];               // O^T tiles of each head block: dim tiles mt
#pragma unroll
  for (int blk = 0; blk < NB; ++blk)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) o[blk][mt] = f32x16{};
  // FP8 gather: per tile this wave loads quarter w of every row's latent
  // codes (rows 8u + lane / 8, 16 codes at 16 (lane % 8), u = 0..3), the rope
  // codes of rows 8w .. 8w + 7 (row 8w + (lane % 32) / 4, 16 codes at
  // 16 (lane % 4); the upper half-wave repeats the lower) and the scales of
  // rows 8w .. 8w + 7 (every lane loads row 8w + lane % 8), one step ahead,
  // into registers; land8 decodes them into the tile buffer.
  const uint8_t* rows8 = reinterpret_cast<const uint8_t*>(A.kv) + A.seq_start[A.q_seq[t]] * kRow;
  const float* scl = FP8 ? A.kv_scale + A.seq_start[A.q_seq[t]] : nullptr;
  u32x4 g8l[4], g8r;
  float g8s = 1.f;
  auto issue8 = [&](int tile) {
    const int jt = tile * kTile;
    int pl[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pl[u] = spos[jt + 8 * u + (lane >> 3)];
    const int pr = spos[jt + 8 * w + ((lane & 31) >> 2)];
    const int ps = spos[jt + 8 * w + (lane & 7)];
    // (streaming loads unless CACHED, as for the bf16 rows)
    auto ld_row = [](const uint8_t* p) {
      if constexpr (CACHED) return *reinterpret_cast<const u32x4*>(p);
      else return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    };
#pragma unroll
    for (int u = 0; u < 4; ++u)
      g8l[u] = ld_row(rows8 + (uint32_t)max(pl[u], 0) * (uint32_t)kRow + (uint32_t)(128 * w + 16 * (lane & 7)));
    g8r = ld_row(rows8 + (uint32_t)max(pr, 0) * (uint32_t)kRow + (uint32_t)(kLatent + 16 * (lane & 3)));
    g8s = scl[max(ps, 0)];
  };
  auto land8 = [&](int tile) {
    uint8_t* b = ring + (tile % kRing) * kTileBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) {           // codes 16c .. 16c + 15 -> bf16 chunks 2c, 2c + 1 of quarter w
      const int r = 8 * u + (lane >> 3);
      const int c = 16 * w + 2 * (lane & 7);
      u32x4 lo, hi;
      e4m3x16_to_bf16x16(g8l[u], lo, hi);
      *reinterpret_cast<u32x4*>(b + tile_chunk_offset(r, c)) = lo;
      *reinterpret_cast<u32x4*>(b + tile_chunk_offset(r, c + 1)) = hi;
    }
    if (lane < 32) {
      const int r = 8 * w + (lane >> 2);
      const int c = 64 + 2 * (lane & 3);
      u32x4 lo, hi;
      e4m3x16_to_bf16x16(g8r, lo, hi);
      *reinterpret_cast<u32x4*>(b + tile_chunk_offset(r, c)) = lo;
      *reinterpret_cast<u32x4*>(b + tile_chunk_offset(r, c + 1)) = hi;
    }
    if (lane < 8) sclds[(tile % kRing) * kTile + 8 * w + lane] = g8s;
  };
  store_positions();
  lds_barrier();                                                       // B0
  if constexpr (FP8) {
    if (n_tiles > 0) {
      issue8(0);
      __builtin_amdgcn_s_waitcnt(0);      // (vmcnt(0): tile 0's codes are in)
      land8(0);
      if (n_tiles > 1) issue8(1);
    }
  } else {
    // Only tiles of the slice are gathered (no clamped re-reads past its
    // end), so each wait below names exactly the loads still allowed out.
    if (n_tiles > 0) issue(0);
    if (n_tiles > 1) {
      issue(1);
      SA_WAIT_VMCNT(kLoadsPerWave);      // tile 0 is in (tile 1 may still be in flight)
    } else {
      SA_WAIT_VMCNT(0);
    }
  }
  lds_barrier();                                                       // B1
  // weights / rescale of head l32 come from score wave l32 / 8
  const int pw = l32 >> 3;
  int npos[kLoadsPerWave];        // kPosAhead: positions of the next tile to gather
  if constexpr (kPosAhead) read_pos(2, npos);
#pragma unroll 1
  for (int step = 0; step <= n_tiles; ++step) {
    // Operands of tile step - 1 are read before BAR_s; its products run after
    // BAR_s, beside the score waves' softmax.  Once this wave's reads have
    // returned, its quarter (and its rope rows) of that buffer are dead: the
    // score waves finished tile step - 1 before the previous BAR_s and no other
    // output wave reads this quarter.  So the gather of tile step + 2 into it
    // is issued here, while the score waves are still in QK^T of tile step.
    const bool pv_step = step > 0;
    const int tile = step - 1;
    const int pb_i = tile & 1;
    u32x2 v[2][8];
    u32x4 pt[NB][2];
    int fl = 0;
    float al[NB];
    if (pv_step) {
      const uint8_t* cur = ring + (tile % kRing) * kTileBytes;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[ks][e] = *reinterpret_cast<const u32x2*>(cur + 16 * ks * 256 + voff[e]);
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          pt[blk][ks] = *reinterpret_cast<const u32x4*>(plds + ((pb_i * NB + blk) * kHeadGroup + l32) * 10 + 4 * ks + 2 * hl);
        al[blk] = alds[pb_i * NB * kHeadGroup + blk * kHeadGroup + l32];   // meaningful only where the flag is set
      }
      fl = flds[pb_i * 4 + pw];
    }
    if (!FP8 && step + 2 < n_tiles) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if constexpr (kPosAhead) issue_at(step + 2, npos);
      else issue(step + 2);
    }
    lds_barrier();                                                     // BAR_s
    if (pv_step) {
      if (__any(fl)) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          const float sc = fl ? al[blk] : 1.f;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) o[blk][mt] *= sc;
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int d = mt >> 1;
          u32x4 av;
          if (mt & 1) {
            av[0] = perm_hi(v[ks][0][d], v[ks][1][d]);
            av[1] = perm_hi(v[ks][2][d], v[ks][3][d]);
            av[2] = perm_hi(v[ks][4][d], v[ks][5][d]);
            av[3] = perm_hi(v[ks][6][d], v[ks][7][d]);
          } else {
            av[0] = perm_lo(v[ks][0][d], v[ks][1][d]);
            av[1] = perm_lo(v[ks][2][d], v[ks][3][d]);
            av[2] = perm_lo(v[ks][4][d], v[ks][5][d]);
            av[3] = perm_lo(v[ks][6][d], v[ks][7][d]);
          }
#pragma unroll
          for (int blk = 0; blk < NB; ++blk)
            o[blk][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(pt[blk][ks]), o[blk][mt], 0, 0, 0);
        }
      }
    }
    // tile step + 1 must be in before the next step's QK (step + 2 stays in flight)
    if constexpr (FP8) {
      // its buffer held tile step - 2, whose last reads (this wave's V operands)
      // were at step - 1; then tile step + 2's loads go out behind it
      if (step + 1 < n_tiles) {
        __builtin_amdgcn_s_waitcnt(0);    // (vmcnt(0): tile step + 1's codes are in)
        land8(step + 1);
        if (step + 2 < n_tiles) issue8(step + 2);
      }
    } else {
      if constexpr (kPosAhead)
        if (step + 1 < n_tiles) read_pos(step + 3, npos);   // issued next step
      // tile step + 1 must be in; tile step + 2, if any, stays in flight
      if (step + 2 < n_tiles)
        SA_WAIT_VMCNT(kLoadsPerWave);
      else if (step + 1 < n_tiles)
        SA_WAIT_VMCNT(0);
    }
    lds_barrier();                                                     // BAR_p
  }
  // Partial accumulators in register-tile order: [t][sp][hg][w][mt][a][lane]
  // x 4 values (b = 0..3), so every store instruction writes 1 KB contiguously.
  // Streaming stores: the partials go out as they are written instead of
  // being written back from L2 when the kernel ends (-1 us per launch).  They
  // need no (m, l), so they are issued before BAR_end, beside the score waves'
  // last softmax.
  if (A.n_sp > 1 && A.part_bf16) {
    // Head-major bf16 partials, so the fused merge reads one head's 512
    // dims as 1 KB: this wave's 32 heads x 128 dims go through its own
    // quarter of ring buffer blk (no load targets the ring after the last
    // step, and no other wave touches that quarter) as [32 heads][256 B],
    // 16-byte chunk q of head r at slot q ^ (r & 15), and leave as 256-byte
    // runs per head (four heads per store instruction), before the closing
    // barrier like the fp32 partials.  (Assembling whole 1 KB head rows from
    // the four waves and storing them after the barrier measured 0.7 us per
    // 4-layer step slower.)
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      uint8_t* tb = ring + blk * kTileBytes + w * kQuarterBytes;
      const f32x16* ot = o[blk];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int bh = 0; bh < 2; ++bh) {            // dims 32a + 16hl + 8bh .. +7 of the quarter: chunk 4a + 2hl + bh
          const int i0 = 4 * a + 2 * bh;
          const u32x4 pk = {pack_bf16x2(ot[0][i0], ot[1][i0]), pack_bf16x2(ot[2][i0], ot[3][i0]),
                            pack_bf16x2(ot[0][i0 + 1], ot[1][i0 + 1]), pack_bf16x2(ot[2][i0 + 1], ot[3][i0 + 1])};
          *reinterpret_cast<u32x4*>(tb + l32 * 256 + 16 * ((4 * a + 2 * hl + bh) ^ (l32 & 15))) = pk;
        }
      }
    }
    wave_lds_fence();
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const uint8_t* tb = ring + blk * kTileBytes + w * kQuarterBytes;
      uint16_t* pb = reinterpret_cast<uint16_t*>(A.part_o) +
                     (((int64_t)t * A.n_sp + sp) * kHeads + kHeadGroup * (hg + blk)) * kLatent + 128 * w;
      u32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4), q = lane & 15;
        v[i] = *reinterpret_cast<const u32x4*>(tb + r * 256 + 16 * (q ^ (r & 15)));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_nontemporal_store(v[i], reinterpret_cast<u32x4*>(pb + (4 * i + (lane >> 4)) * kLatent + 8 * (lane & 15)));
    }
  } else if (A.n_sp > 1) {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x4* po = reinterpret_cast<f32x4*>(A.part_o) + ((((int64_t)t * A.n_sp + sp) * 2 + hg + blk) * 4 + w) * 16 * 64;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          __builtin_nontemporal_store(
              f32x4{o[blk][mt][4 * a], o[blk][mt][4 * a + 1], o[blk][mt][4 * a + 2], o[blk][mt][4 * a + 3]},
              &po[(mt * 4 + a) * 64 + lane]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);         // the partial stores are out before the workgroup ends
  lds_barrier();                                                       // BAR_end: (m, l) of every head
  // Result element 4a + b of tile mt is dim 128w + 32a + 16hl + 4b + mt of
  // head 32hg + l32: for each a a lane holds 16 consecutive dims.
  if (A.n_sp == 1) {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const float L = mlds[(blk * kHeadGroup + l32) * 2 + 1];
      const float inv = L > 0.f ? 1.f / L : 0.f;
      uint16_t* ob = A.obar + ((int64_t)t * kHeads + kHeadGroup * (hg + blk) + l32) * kLatent + 128 * w + 16 * hl;
      const f32x16* ot = o[blk];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int bh = 0; bh < 2; ++bh) {            // dims 8bh .. 8bh + 7 of the 16: b = 2bh, 2bh + 1
          const int i0 = 4 * a + 2 * bh;
          const u32x4 pk = {pack_bf16x2(ot[0][i0] * inv, ot[1][i0] * inv), pack_bf16x2(ot[2][i0] * inv, ot[3][i0] * inv),
                            pack_bf16x2(ot[0][i0 + 1] * inv, ot[1][i0 + 1] * inv),
                            pack_bf16x2(ot[2][i0 + 1] * inv, ot[3][i0 + 1] * inv)};
          *reinterpret_cast<u32x4*>(ob + 32 * a + 8 * bh) = pk;
        }
      }
    }
  }
}

// Merge of the slices' partial softmax states: obar = sum_s a_s O_s / sum_s a_s l_s
// with a_s = 2^(m_s - max m).  Partials are in the attention kernel's register
// tile order.  One workgroup per (query, latent quarter w, head group hg, dim
// tile pair mp), dealt to the XCDs like the attention kernel's items; thread
// (a, lane) owns dim tiles mt = 2mp, 2mp + 1 of head 32hg + (lane & 31), i.e.
// dims 128w + 32a + 16 (lane >> 5) + 4b + mt, and reads them for 8 slices at
// a time (one rescale per batch).
constexpr int kMergeBatch = 8;         // slices read per round trip

__global__ __launch_bounds__(256) void mla_merge_kernel(AttnArgs A) {
  const int n_wg = (int)gridDim.x;
  const int item = (n_wg & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (n_wg >> 3) + (int)(blockIdx.x >> 3);
  const int t = item >> 4;
  const int w = (item >> 2) & 3;
  const int hg = (item >> 1) & 1;
  const int mp = item & 1;
  const int a = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l32 = lane & 31, hl = lane >> 5;
  const int head = kHeadGroup * hg + l32;
  const int n_sp = A.n_sp;
  // slice s adds s * 2 * 4 * 1024; tile mt + 1 adds 4 * 64
  const f32x4* src = reinterpret_cast<const f32x4*>(A.part_o) + (((int64_t)t * n_sp * 2 + hg) * 4 + w) * 1024 +
                     (2 * mp * 4 + a) * 64 + lane;
  const float2* mlp = reinterpret_cast<const float2*>(A.part_ml) + (int64_t)t * n_sp * kHeads + head;
  float M = -INFINITY, L = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_sp; s0 += kMergeBatch) {
    f32x4 v0[kMergeBatch], v1[kMergeBatch];
    float2 ml[kMergeBatch];
    // slices past n_sp are not loaded (a uniform branch): clamped re-reads
    // would pass 4x the bytes through the load path at 2 slices
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      ml[u] = float2{-INFINITY, 0.f};
      v0[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      v1[u] = v0[u];
      if (s0 + u < n_sp) {
        const int s = s0 + u;
        ml[u] = mlp[(int64_t)s * kHeads];
        v0[u] = src[(int64_t)s * 8192];
        v1[u] = src[(int64_t)s * 8192 + 256];
      }
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (s0 + u < n_sp) mb = fmaxf(mb, ml[u].x);
    if (mb > M) {                       // new running maximum (never taken while every slice is empty)
      const float c = M == -INFINITY ? 0.f : fast_exp2(M - mb);
      acc0 *= c;
      acc1 *= c;
      L *= c;
      M = mb;
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float wt = (s0 + u < n_sp && ml[u].x != -INFINITY) ? fast_exp2(ml[u].x - M) : 0.f;
      L = fmaf(wt, ml[u].y, L);
      acc0 += wt * v0[u];
      acc1 += wt * v1[u];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  // acc0[b] is dim 128w + 32a + 16hl + 4b + 2mp, acc1[b] the next dim
  uint16_t* ob = A.obar + ((int64_t)t * kHeads + head) * kLatent + 128 * w + 32 * a + 16 * hl + 2 * mp;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    *reinterpret_cast<uint32_t*>(ob + 4 * b) = pack_bf16x2(acc0[b] * inv, acc1[b] * inv);
  if (A.lse && w == 0 && mp == 0 && a == 0 && hl == 0)
    A.lse[(int64_t)t * kHeads + head] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// The same merge for more than 8 slices (few queries): work item
// qb = ((hg * 4 + w) * 2 + mp) * 4 + a of a query, the same dims per lane as
// above; G = 2 or 4 waves split an item's slices, at most 8 each (one round
// trip), and their partial merges are combined through LDS, so one query's 32
// slices take one round trip over 64 workgroups instead of four over 16.
constexpr int kMergeWaves = 4;
static_assert(kMergeBatch * kMergeWaves >= kMaxSp, "a workgroup's waves cover every slice");

__host__ __device__ inline int merge_groups(int n_sp) { return n_sp <= 2 * kMergeBatch ? 2 : 4; }

__global__ __launch_bounds__(kMergeWaves * 64) void mla_merge_wide_kernel(AttnArgs A) {
  const int n_sp = A.n_sp;
  const int G = merge_groups(n_sp);
  const int n_wg = (int)gridDim.x;
  const int item = (n_wg & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (n_wg >> 3) + (int)(blockIdx.x >> 3);
  const int t = item / (16 * G);
  const int j = item - t * 16 * G;
  const int g = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int qb = j * (kMergeWaves / G) + g / G;   // this wave's item
  const int sg = g % G;                           // and its share of the slices
  const int hg = qb >> 5, w = (qb >> 3) & 3, mp = (qb >> 2) & 1, a = qb & 3;
  const int l32 = lane & 31, hl = lane >> 5;
  const int head = kHeadGroup * hg + l32;
  const int per = (n_sp + G - 1) / G;
  const int s_lo = sg * per, s_hi = min(n_sp, s_lo + per);
  // slice s adds s * 2 * 4 * 1024; tile mt + 1 adds 4 * 64
  const f32x4* src = reinterpret_cast<const f32x4*>(A.part_o) + (((int64_t)t * n_sp * 2 + hg) * 4 + w) * 1024 +
                     (2 * mp * 4 + a) * 64 + lane;
  const float2* mlp = reinterpret_cast<const float2*>(A.part_ml) + (int64_t)t * n_sp * kHeads + head;
  f32x4 v0[kMergeBatch], v1[kMergeBatch];
  float2 ml[kMergeBatch];
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) {
    const int s = min(s_lo + u, n_sp - 1);
    ml[u] = mlp[(int64_t)s * kHeads];
    v0[u] = src[(int64_t)s * 8192];
    v1[u] = src[(int64_t)s * 8192 + 256];
  }
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u)
    if (s_lo + u < s_hi) M = fmaxf(M, ml[u].x);
  float L = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) {
    const float wt = (s_lo + u < s_hi && ml[u].x != -INFINITY) ? fast_exp2(ml[u].x - M) : 0.f;
    L = fmaf(wt, ml[u].y, L);
    acc0 += wt * v0[u];
    acc1 += wt * v1[u];
  }
  {
    // combine the G waves of an item: [wave][field][lane]
    __shared__ float part[kMergeWaves][10][64];
    part[g][0][lane] = M;
    part[g][1][lane] = L;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      part[g][2 + b][lane] = acc0[b];
      part[g][6 + b][lane] = acc1[b];
    }
    __syncthreads();
    if (sg != 0) return;
    float Mt = -INFINITY;
    for (int q = g; q < g + G; ++q) Mt = fmaxf(Mt, part[q][0][lane]);
    float Lt = 0.f;
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
    for (int q = g; q < g + G; ++q) {
      const float mq = part[q][0][lane];
      const float c = mq != -INFINITY ? fast_exp2(mq - Mt) : 0.f;   // waves without slices have M = -inf
      Lt = fmaf(c, part[q][1][lane], Lt);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        o0[b] = fmaf(c, part[q][2 + b][lane], o0[b]);
        o1[b] = fmaf(c, part[q][6 + b][lane], o1[b]);
      }
    }
    M = Mt;
    L = Lt;
    acc0 = o0;
    acc1 = o1;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  // acc0[b] is dim 128w + 32a + 16hl + 4b + 2mp, acc1[b] the next dim
  uint16_t* ob = A.obar + ((int64_t)t * kHeads + head) * kLatent + 128 * w + 32 * a + 16 * hl + 2 * mp;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    *reinterpret_cast<uint32_t*>(ob + 4 * b) = pack_bf16x2(acc0[b] * inv, acc1[b] * inv);
  if (A.lse && w == 0 && mp == 0 && a == 0 && hl == 0)
    A.lse[(int64_t)t * kHeads + head] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// The merge for one or two queries with many slices (the decode of one long
// sequence): 64 items per query are too few workgroups to stream the partial
// states at the chip's rate, so each item is split 4 ways by lane.  Workgroup
// (item, quarter q) takes lanes 16q .. 16q + 15 of the item; thread (g, i)
// (i = lane within the quarter, g = 0..15) merges slices g, g + 16, and the 16
// groups of a lane are combined through LDS.  Same dims per lane and the same
// arithmetic as the merges above.
constexpr int kSplitMaxQ = 2;          // queries up to which this merge is used
static_assert(kMaxSp <= 32, "two slices per thread cover every slice");

__global__ __launch_bounds__(256) void mla_merge_split_kernel(AttnArgs A) {
  const int n_wg = (int)gridDim.x;
  const int wg = (n_wg & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (n_wg >> 3) + (int)(blockIdx.x >> 3);
  const int t = wg >> 8;                          // 64 items x 4 quarters per query
  const int qb = (wg >> 2) & 63, qq = wg & 3;
  const int hg = qb >> 5, w = (qb >> 3) & 3, mp = (qb >> 2) & 1, a = qb & 3;
  const int i = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int lane = 16 * qq + i;                   // lane of the item (the attention's register lane)
  const int l32 = lane & 31, hl = lane >> 5;
  const int head = kHeadGroup * hg + l32;
  const int n_sp = A.n_sp;
  const f32x4* src = reinterpret_cast<const f32x4*>(A.part_o) + (((int64_t)t * n_sp * 2 + hg) * 4 + w) * 1024 +
                     (2 * mp * 4 + a) * 64 + lane;
  const float2* mlp = reinterpret_cast<const float2*>(A.part_ml) + (int64_t)t * n_sp * kHeads + head;
  f32x4 v0[2], v1[2];
  float2 ml[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int s = g + 16 * u;
    ml[u] = float2{-INFINITY, 0.f};
    v0[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    v1[u] = v0[u];
    if (s < n_sp) {
      ml[u] = mlp[(int64_t)s * kHeads];
      v0[u] = src[(int64_t)s * 8192];
      v1[u] = src[(int64_t)s * 8192 + 256];
    }
  }
  float M = fmaxf(ml[0].x, ml[1].x), L = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float wt = ml[u].x != -INFINITY ? fast_exp2(ml[u].x - M) : 0.f;
    L = fmaf(wt, ml[u].y, L);
    acc0 += wt * v0[u];
    acc1 += wt * v1[u];
  }
  __shared__ float part[10][16][16];              // [field][group][lane in quarter]
  part[0][g][i] = M;
  part[1][g][i] = L;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    part[2 + b][g][i] = acc0[b];
    part[6 + b][g][i] = acc1[b];
  }
  __syncthreads();
  if (g != 0) return;
  float Mt = -INFINITY;
  for (int q = 0; q < 16; ++q) Mt = fmaxf(Mt, part[0][q][i]);
  float Lt = 0.f;
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < 16; ++q) {
    const float mq = part[0][q][i];
    const float c = mq != -INFINITY ? fast_exp2(mq - Mt) : 0.f;   // groups without slices have M = -inf
    Lt = fmaf(c, part[1][q][i], Lt);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      o0[b] = fmaf(c, part[2 + b][q][i], o0[b]);
      o1[b] = fmaf(c, part[6 + b][q][i], o1[b]);
    }
  }
  const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
  // o0[b] is dim 128w + 32a + 16hl + 4b + 2mp, o1[b] the next dim
  uint16_t* ob = A.obar + ((int64_t)t * kHeads + head) * kLatent + 128 * w + 32 * a + 16 * hl + 2 * mp;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    *reinterpret_cast<uint32_t*>(ob + 4 * b) = pack_bf16x2(o0[b] * inv, o1[b] * inv);
  if (A.lse && w == 0 && mp == 0 && a == 0 && hl == 0)
    A.lse[(int64_t)t * kHeads + head] = Lt > 0.f ? (Mt + __log2f(Lt)) * 0.69314718055994531f : -INFINITY;
}

// ------------------------------------------------------------------ W_UV
struct WuvArgs {
  const uint16_t* obar;     // [n_q][64][512] bf16
  const uint16_t* w_uv;     // [64][256][512] bf16
  uint16_t* out;            // [n_q][64][256] bf16
  int n_q;
};

constexpr int kWuvQ = 16;                       // queries per block (MFMA N)
// ROWS value rows per workgroup (ROWS / 16 waves), the query blocks split
// QSPLIT ways: 64 x 1 for decode batches (the W_UV slice dominates a
// workgroup's bytes); 128 x 2 from kWuvWideQ queries on, where each
// workgroup streams every obar row of its head and the per-CU rate bounds
// the kernel, so twice the value rows per obar byte halve those bytes.
template <int ROWS>
constexpr size_t wuv_smem() { return (size_t)(ROWS + 2 * kWuvQ) * kLatent * 2; }   // 96 or 160 KB
constexpr int kWuvWideQ = 512;

// One workgroup per (head, ROWS value rows, 1 / QSPLIT of the query blocks).
// Its W_UV rows and, block by block, the obar rows of 16 queries are staged in
// LDS with 1 KB direct-to-LDS loads (one 512-wide row each, chunks swizzled by
// row so the MFMA operand reads are conflict-free).  Wave w multiplies value
// rows 16w..16w+15 with each block.
template <int ROWS, int QSPLIT>
__global__ __launch_bounds__(ROWS * 4) void mla_wuv_kernel(WuvArgs W) {
  constexpr int kWaves = ROWS / 16;
  constexpr int kRowBlocks = kVdim / ROWS;
  constexpr int kBlkLoads = kWuvQ / kWaves;            // obar rows each wave stages per block
  static_assert(kVdim % ROWS == 0 && kWuvQ % kWaves == 0, "value-row blocks and staging shares");
  extern __shared__ __align__(16) uint8_t smem[];
  const int bx = (int)blockIdx.x;
  const int h = bx / (kRowBlocks * QSPLIT);
  const int rest = bx - h * (kRowBlocks * QSPLIT);
  const int vb = (rest / QSPLIT) * ROWS;
  const int qs = rest % QSPLIT;
  const int n_blk_all = (W.n_q + kWuvQ - 1) / kWuvQ;
  const int per = (n_blk_all + QSPLIT - 1) / QSPLIT;
  const int b0 = qs * per, b1 = min(b0 + per, n_blk_all);
  if (b0 >= b1) return;                                 // (before any load)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  uint8_t* wl = smem;                                   // [ROWS rows][1 KB]
  uint8_t* ol = smem + ROWS * 1024;                     // [2 buffers][16 rows][1 KB]
  // Row r of a staged block: lane p fills slot p with chunk p ^ (r & 15).
  auto stage_row = [&](uint8_t* dst_row, const uint16_t* src_row, int r) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(src_row) + 16 * (lane ^ (r & 15));
    __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst_row, 16, 0, 0);
  };
  const uint16_t* wsrc = W.w_uv + ((int64_t)h * kVdim + vb) * kLatent;
#pragma unroll
  for (int u = 0; u < 16; ++u) stage_row(wl + (16 * w + u) * 1024, wsrc + (int64_t)(16 * w + u) * kLatent, u);
  auto stage_block = [&](int b) {
#pragma unroll
    for (int u = 0; u < kBlkLoads; ++u) {
      const int r = kBlkLoads * w + u;
      const int tq = min(b * kWuvQ + r, W.n_q - 1);
      stage_row(ol + (((b - b0) & 1) * kWuvQ + r) * 1024, W.obar + ((int64_t)tq * kHeads + h) * kLatent, r);
    }
  };
  stage_block(b0);
  // Operand reads: row l16 (value row 16w + l16, or query l16), chunk 4s + g.
  // Byte offset of chunk 4s + g of row l16: 16 ((4s + g) ^ l16) = 64 s ^ rd.
  const int rd = 16 * (g ^ l16);
  bf16x8 wa[16];
  for (int b = b0; b < b1; ++b) {
    if (b + 1 < b1) {
      stage_block(b + 1);
      SA_WAIT_VMCNT(kBlkLoads);
    } else {
      SA_WAIT_VMCNT(0);
    }
    lds_barrier();
    if (b == b0) {
#pragma unroll
      for (int s = 0; s < 16; ++s)
        wa[s] = *reinterpret_cast<const bf16x8*>(wl + (16 * w + l16) * 1024 + ((16 * (4 * s)) ^ rd));
    }
    const uint8_t* orow = ol + (((b - b0) & 1) * kWuvQ + l16) * 1024;
    bf16x8 ob[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) ob[s] = *reinterpret_cast<const bf16x8*>(orow + ((16 * (4 * s)) ^ rd));
    // every operand read above goes out before the first product: one LDS
    // round trip per block instead of several
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[s], ob[s], acc, 0, 0, 0);
    // acc[j] = out[t = 16b + l16][h][vb + 16w + 4g + j]
    const int tq = b * kWuvQ + l16;
    if (tq < W.n_q) {
      const u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *reinterpret_cast<u32x2*>(W.out + ((int64_t)tq * kHeads + h) * kVdim + vb + 16 * w + 4 * g) = pk;
    }
    lds_barrier();                      // buffer (b - b0) & 1 is refilled by the next iteration's staging
  }
}

// ------------------------------------------------------- merge + W_UV in one
// For decode batches whose selections are split into 2..8 slices: the merge
// of the slices' bf16 head-major partial states is done by the workgroups of
// the W_UV product itself, one launch per layer instead of two.  One
// workgroup of 512 threads per (head, 64 value rows): all eight waves stage
// its 64 KB of W_UV in LDS (8 rows each; with 16 rows on each of the first
// four the step took 0.8 us longer) and the first four run the products;
// for each block of 16 queries thread (query rq, 16-dim chunk c)
// reads that chunk of the head's partial states for every slice (32 B each,
// one round trip per 8 slices), combines them with the log-sum-exp weights
// 2^(m_s - max m) and writes the bf16 latent average into the LDS row the
// products read.  Each partial state is read by the four workgroups of its
// head (against 128 value rows per workgroup, the 256 workgroups share the
// loads over every CU: -0.9 us per 4-layer step).
struct MergeWuvArgs {
  const uint16_t* part_o;   // [n_q][n_sp][64][512] bf16, unnormalised
  const float* part_ml;     // [n_q][n_sp][64][2]: max (log2 units), sum
  const uint16_t* w_uv;     // [64][256][512]
  uint16_t* out;            // [n_q][64][256]
  float* lse;               // [n_q][64] or null
  int n_q, n_sp;
};
constexpr int kMwRows = 64;
constexpr int kMwThreads = 512;
static_assert(kMwThreads == kWuvQ * (kLatent / 16), "one thread per (query of the block, 16-dim chunk)");
constexpr int kMwMaxSp = kMergeBatch;     // slices merged per round trip (and at most)
constexpr size_t kMwSmem = (size_t)(kMwRows + kWuvQ) * kLatent * 2;   // 80 KB

__global__ __launch_bounds__(kMwThreads) void mla_merge_wuv_kernel(MergeWuvArgs W) {
  extern __shared__ __align__(16) uint8_t smem[];
  // the four workgroups of a head (value rows 64j .. 64j + 63) are 64 apart,
  // so the round-robin dealing puts them on one XCD, where the repeated
  // reads of the head's partial states can hit that XCD's L2
  const int h = (int)blockIdx.x & (kHeads - 1);
  const int vb = ((int)blockIdx.x >> 6) * kMwRows;
  constexpr int kWaves = kMwRows / 16;      // waves that run the products
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  uint8_t* wl = smem;                                   // [64 rows][1 KB]
  uint8_t* ol = smem + kMwRows * 1024;                  // [16 rows][1 KB]: the block's latent averages
  // W_UV rows as in mla_wuv_kernel, kMwRows / 8 per wave: lane p of row r
  // fills slot p with chunk p ^ (r & 15)
  const uint16_t* wsrc = W.w_uv + ((int64_t)h * kVdim + vb) * kLatent;
#pragma unroll
  for (int u = 0; u < kMwRows / 8; ++u) {
    const int r = (kMwRows / 8) * w + u;
    const uint8_t* src = reinterpret_cast<const uint8_t*>(wsrc + (int64_t)r * kLatent) + 16 * (lane ^ (r & 15));
    __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(wl + r * 1024),
                                     16, 0, 0);
  }
  const int rq = threadIdx.x >> 5, c = threadIdx.x & 31;
  const int rd = 16 * (g ^ l16);
  const int64_t slice_stride = (int64_t)kHeads * kLatent / 8;      // in 16-byte units
  bf16x8 wa[16];
  const int n_blk = (W.n_q + kWuvQ - 1) / kWuvQ;
  for (int b = 0; b < n_blk; ++b) {
    const int tq = min(b * kWuvQ + rq, W.n_q - 1);
    const u32x4* src =
        reinterpret_cast<const u32x4*>(W.part_o + ((int64_t)tq * W.n_sp * kHeads + h) * kLatent + 16 * c);
    const float2* mlp = reinterpret_cast<const float2*>(W.part_ml) + (int64_t)tq * W.n_sp * kHeads + h;
    float M = -INFINITY, L = 0.f;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    for (int s0 = 0; s0 < W.n_sp; s0 += kMwMaxSp) {
      u32x4 v[kMwMaxSp][2];
      float2 ml[kMwMaxSp];
#pragma unroll
      for (int u = 0; u < kMwMaxSp; ++u) {
        ml[u] = float2{-INFINITY, 0.f};
        v[u][0] = u32x4{0u, 0u, 0u, 0u};
        v[u][1] = v[u][0];
        if (s0 + u < W.n_sp) {
          ml[u] = mlp[(int64_t)(s0 + u) * kHeads];
          v[u][0] = src[(s0 + u) * slice_stride];
          v[u][1] = src[(s0 + u) * slice_stride + 1];
        }
      }
      float mb = M;
#pragma unroll
      for (int u = 0; u < kMwMaxSp; ++u) mb = fmaxf(mb, ml[u].x);
      if (mb > M) {                       // new running maximum (never taken while every slice is empty)
        const float cf = M == -INFINITY ? 0.f : fast_exp2(M - mb);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] *= cf;
        L *= cf;
        M = mb;
      }
#pragma unroll
      for (int u = 0; u < kMwMaxSp; ++u) {
        const float wt = ml[u].x != -INFINITY ? fast_exp2(ml[u].x - M) : 0.f;
        L = fmaf(wt, ml[u].y, L);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int e = 0; e < 4; ++e) {         // dims 16c + 8k2 + 2e, +1
            const uint32_t x = v[u][k2][e];
            acc[8 * k2 + 2 * e] = fmaf(wt, __uint_as_float(x << 16), acc[8 * k2 + 2 * e]);
            acc[8 * k2 + 2 * e + 1] = fmaf(wt, __uint_as_float(x & 0xffff0000u), acc[8 * k2 + 2 * e + 1]);
          }
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint8_t* orow = ol + rq * 1024;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {      // chunk 2c + k2 of row rq at slot (2c + k2) ^ rq
      const float* x = acc + 8 * k2;
      const u32x4 pk = {pack_bf16x2(x[0] * inv, x[1] * inv), pack_bf16x2(x[2] * inv, x[3] * inv),
                        pack_bf16x2(x[4] * inv, x[5] * inv), pack_bf16x2(x[6] * inv, x[7] * inv)};
      *reinterpret_cast<u32x4*>(orow + 16 * ((2 * c + k2) ^ rq)) = pk;
    }
    if (W.lse && vb == 0 && c == 0 && b * kWuvQ + rq < W.n_q)
      W.lse[(int64_t)(b * kWuvQ + rq) * kHeads + h] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
    SA_WAIT_VMCNT(0);                     // (the W_UV rows, on the first block)
    lds_barrier();
    if (w < kWaves) {
      if (b == 0) {
#pragma unroll
        for (int s = 0; s < 16; ++s)
          wa[s] = *reinterpret_cast<const bf16x8*>(wl + (16 * w + l16) * 1024 + ((16 * (4 * s)) ^ rd));
      }
      const uint8_t* qrow = ol + l16 * 1024;
      bf16x8 ob[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) ob[s] = *reinterpret_cast<const bf16x8*>(qrow + ((16 * (4 * s)) ^ rd));
      __builtin_amdgcn_sched_barrier(0);
      f32x4 o4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 16; ++s) o4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[s], ob[s], o4, 0, 0, 0);
      // o4[j] = out[16b + l16][h][vb + 16w + 4g + j]
      const int to = b * kWuvQ + l16;
      if (to < W.n_q) {
        const u32x2 pk = {pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3])};
        *reinterpret_cast<u32x2*>(W.out + ((int64_t)to * kHeads + h) * kVdim + vb + 16 * w + 4 * g) = pk;
      }
    }
    lds_barrier();                        // the block's rows are rewritten by the next block's merge
  }
}

}  // namespace sa

namespace sa_host {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Head blocks per attention workgroup: 2 (all 64 heads share every gathered
// tile, half the tile steps per head) from 64 queries on; 1 (a workgroup per
// 32 heads, so twice the workgroups per slice) for smaller decode batches,
// where two head blocks would need twice the slices, and so twice the partial
// states, for the same parallelism (16 queries: 0.209 against 0.189 ms per
// 4-layer step; 64 queries: 0.320 against 0.338 ms).
constexpr int kTwoBlockMinQ = 64;
int mla_head_blocks(int32_t n_q) { return n_q >= kTwoBlockMinQ ? 2 : 1; }

// The slicing of each query's selection: n_sp slices of kps entries (a
// multiple of the 32-row tile; the last slice may be shorter).  About one
// workgroup per CU; a slice keeps at least two tiles; the slice count is
// recomputed from the rounded slice length so no slice is empty.
void mla_split(int32_t n_q, int32_t k, int* n_sp_out, int* kps_out) {
  const int target = mla_head_blocks(n_q) == 2 ? 256 : 128;
  int n_sp = (target + n_q - 1) / n_q;
  const int max_sp = (k + 63) / 64;
  if (n_sp > max_sp) n_sp = max_sp;
  if (n_sp > sa::kMaxSp) n_sp = sa::kMaxSp;
  if (n_sp < 1) n_sp = 1;
  int kps = (k + n_sp - 1) / n_sp;
  kps = (kps + sa::kTile - 1) / sa::kTile * sa::kTile;
  *n_sp_out = (k + kps - 1) / kps;
  *kps_out = kps;
}

// Partial states: none with one slice; bf16 head-major, merged inside the
// W_UV launch, for one head block and 2..8 slices (decode batches of 16..63
// queries); fp32 register-tile order with a merge launch otherwise.
int mla_partial_bits(int32_t n_q, int32_t k) {
  int n_sp, kps;
  mla_split(n_q, k, &n_sp, &kps);
  if (n_sp == 1) return 0;
  return (mla_head_blocks(n_q) == 1 && n_sp <= sa::kMwMaxSp) ? 16 : 32;
}

int mla_n_splits(int32_t n_q, int32_t k) {
  int n_sp, kps;
  mla_split(n_q, k, &n_sp, &kps);
  return n_sp;
}

struct MlaWs {
  float* part_o;
  float* part_ml;
  uint16_t* obar;
};

static MlaWs mla_carve(void* ws, int32_t n_q, int n_sp) {
  MlaWs m;
  uint8_t* p = (uint8_t*)ws;
  m.obar = (uint16_t*)p;
  p += align256((size_t)n_q * sa::kHeads * sa::kLatent * 2);
  m.part_ml = (float*)p;
  p += n_sp > 1 ? align256((size_t)n_q * n_sp * sa::kHeads * 2 * 4) : 0;
  m.part_o = (float*)p;
  return m;
}

size_t mla_workspace_size(int32_t n_q, int32_t k) {
  const int n_sp = mla_n_splits(n_q, k);
  size_t s = align256((size_t)n_q * sa::kHeads * sa::kLatent * 2);
  if (n_sp > 1) s += align256((size_t)n_q * n_sp * sa::kHeads * 2 * 4) + align256((size_t)n_q * n_sp * sa::kHeads * sa::kLatent * 4);
  return s;
}

// hipFuncSetAttribute is per device; remember which devices have been set up.
static std::atomic<uint64_t> g_attr_set{0};

// kv_scale != NULL: kv holds E4M3 codes [rows][576] with one scale per row.
// shared_rows: the batch's queries share their sequences' rows (the caller
// knows the sequence count), so the gathers keep them in the caches.
template <int NB, bool FP8>
static void launch_attn(bool cached, int64_t grid, size_t smem, hipStream_t stream, const sa::AttnArgs& A) {
  if (cached)
    hipLaunchKernelGGL((sa::mla_attn_kernel<NB, FP8, true>), dim3((unsigned)grid), dim3(sa::kAttnThreads), smem,
                       stream, A);
  else
    hipLaunchKernelGGL((sa::mla_attn_kernel<NB, FP8, false>), dim3((unsigned)grid), dim3(sa::kAttnThreads), smem,
                       stream, A);
}

template <int NB, bool FP8>
static hipError_t reserve_attn_lds() {
  const int smem = (int)sa::attn_smem<NB, FP8>();
  hipError_t e = hipFuncSetAttribute((const void*)sa::mla_attn_kernel<NB, FP8, false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)sa::mla_attn_kernel<NB, FP8, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            smem);
  return e;
}

int32_t launch_mla(const void* q_abs, const void* kv, const float* kv_scale, const int64_t* seq_start,
                   const int32_t* q_seq, const int32_t* idx, int32_t n_q, int32_t k, const void* w_uv, float scale,
                   void* out, float* lse, void* ws, hipStream_t stream, bool shared_rows, int part_half) {
  int n_sp, kps;
  mla_split(n_q, k, &n_sp, &kps);
  MlaWs m = mla_carve(ws, n_q, n_sp);
  const bool part_bf16 = mla_partial_bits(n_q, k) == 16;
  // bf16 partial states take half of the fp32 region; part_half picks which
  if (part_bf16 && part_half)
    m.part_o = reinterpret_cast<float*>(reinterpret_cast<uint16_t*>(m.part_o) + (size_t)n_q * n_sp * sa::kHeads * sa::kLatent);
  sa::AttnArgs A;
  A.q_abs = (const uint16_t*)q_abs;
  A.kv = (const uint16_t*)kv;
  A.seq_start = seq_start;
  A.q_seq = q_seq;
  A.idx = idx;
  A.k = k;
  A.n_q = n_q;
  A.n_sp = n_sp;
  A.kps = kps;
  A.scale_log2 = scale * sa::kLog2e;
  A.part_o = m.part_o;
  A.part_ml = m.part_ml;
  A.obar = m.obar;
  A.lse = lse;
  A.kv_scale = kv_scale;
  A.part_bf16 = part_bf16 ? 1 : 0;
  const int nb = mla_head_blocks(n_q);
  const bool fp8 = kv_scale != nullptr;
  const size_t smem = nb == 2 ? (fp8 ? sa::attn_smem<2, true>() : sa::attn_smem<2>())
                              : (fp8 ? sa::attn_smem<1, true>() : sa::attn_smem<1>());
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    set_error("mla: hipGetDevice failed");
    return SA_ERR_HIP;
  }
  const uint64_t bit = 1ull << (dev & 63);
  if (!(g_attr_set.load() & bit)) {
    if (reserve_attn_lds<1, false>() != hipSuccess || reserve_attn_lds<2, false>() != hipSuccess ||
        reserve_attn_lds<1, true>() != hipSuccess || reserve_attn_lds<2, true>() != hipSuccess ||
        hipFuncSetAttribute((const void*)sa::mla_wuv_kernel<64, 1>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sa::wuv_smem<64>()) != hipSuccess ||
        hipFuncSetAttribute((const void*)sa::mla_wuv_kernel<128, 2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sa::wuv_smem<128>()) != hipSuccess ||
        hipFuncSetAttribute((const void*)sa::mla_merge_wuv_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sa::kMwSmem) != hipSuccess) {
      set_error("mla: cannot reserve %zu bytes of LDS", smem);
      return SA_ERR_HIP;
    }
    g_attr_set.fetch_or(bit);
  }
  const int64_t grid = (int64_t)n_q * n_sp * (nb == 2 ? 1 : 2);
  const bool wide = n_sp > sa::kMergeBatch;
  const int64_t merge_grid = (int64_t)n_q * 16 * (wide ? sa::merge_groups(n_sp) : 1);
  if (grid > 0x7fffffff || merge_grid > 0x7fffffff) {
    set_error("mla: grid too large");
    return SA_ERR_UNSUPPORTED;
  }
  if (nb == 2 && fp8)
    launch_attn<2, true>(shared_rows, grid, smem, stream, A);
  else if (nb == 2)
    launch_attn<2, false>(shared_rows, grid, smem, stream, A);
  else if (fp8)
    launch_attn<1, true>(shared_rows, grid, smem, stream, A);
  else
    launch_attn<1, false>(shared_rows, grid, smem, stream, A);
  int32_t rc = check_launch("mla_attn_kernel");
  if (rc) return rc;
  if (A.part_bf16) {
    sa::MergeWuvArgs M{(const uint16_t*)m.part_o, m.part_ml, (const uint16_t*)w_uv, (uint16_t*)out, lse, n_q, n_sp};
    hipLaunchKernelGGL(sa::mla_merge_wuv_kernel, dim3(sa::kHeads * (sa::kVdim / sa::kMwRows)), dim3(sa::kMwThreads),
                       sa::kMwSmem, stream, M);
    return check_launch("mla_merge_wuv_kernel");
  }
  if (n_sp > 1) {
    if (wide && n_q <= sa::kSplitMaxQ) {
      hipLaunchKernelGGL(sa::mla_merge_split_kernel, dim3((unsigned)(n_q * 256)), dim3(256), 0, stream, A);
      if ((rc = check_launch("mla_merge_split_kernel"))) return rc;
    } else {
      if (wide)
        hipLaunchKernelGGL(sa::mla_merge_wide_kernel, dim3((unsigned)merge_grid), dim3(sa::kMergeWaves * 64), 0, stream,
                           A);
      else
        hipLaunchKernelGGL(sa::mla_merge_kernel, dim3((unsigned)merge_grid), dim3(256), 0, stream, A);
      if ((rc = check_launch(wide ? "mla_merge_wide_kernel" : "mla_merge_kernel"))) return rc;
    }
  }
  sa::WuvArgs W{m.obar, (const uint16_t*)w_uv, (uint16_t*)out, n_q};
  if (n_q >= sa::kWuvWideQ)
    hipLaunchKernelGGL((sa::mla_wuv_kernel<128, 2>), dim3(sa::kHeads * 2 * 2), dim3(512), sa::wuv_smem<128>(), stream,
                       W);
  else
    hipLaunchKernelGGL((sa::mla_wuv_kernel<64, 1>), dim3(sa::kHeads * 4), dim3(256), sa::wuv_smem<64>(), stream, W);
  return check_launch("mla_wuv_kernel");
}

}  // namespace sa_host
