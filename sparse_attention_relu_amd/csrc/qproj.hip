// Query side for gfx950: the projections that produce the hot path's query
// inputs from the q_lora activation.
//
//   q      = bf16(W_QB c_q)             per head [192 nope ; 64 rope], the rope
//                                       part turned at the token's position
//   q_idx  = bf16(W_IQ c_q)             32 heads x 128, dims 64..127 turned
//   w      = W_IW c_q                   32 head weights, fp32
//   q_abs  = [bf16(W_UK[h]^T q_nope[h]) ; q_rope[h]]   per head (absorption)
//
// models.inteligile.com "GLM-5.2 / Model techniques map", "Checked in its
// code", rows "Multi-head latent attention" (q_lora_rank bottleneck; kv_b_proj
// holds, per head, qk_nope_head_dim key rows and v_head_dim value rows),
// "Partial RoPE" (the per-head split [192 nope ; 64 rope]) and
// "Indexer-selected sparse attention" (32 indexer heads of 128);
// llm-architectures-explained "GLM-5.2", "Every architecture field"
// (q_lora_rank 2,048); llm-atlas "GLM-5.2", config fields qk_head_dim,
// rope_interleave, indexer_rope_interleave.  The pages print neither the
// indexer query's nor the head weights' source; both are taken from the same
// q_lora activation, and the indexer query turns its last 64 dims like the
// indexer key.  Each projection's output is rounded to bf16 once (the head
// weights stay fp32); the rope pairs turn from those bf16 values in fp64 and
// are rounded again.
//
// Every product is a "weights x tokens" contraction with both operands K-
// contiguous (nn.Linear weights [rows][K]; W_UK is taken pre-arranged as
// W_UK^T [64][512][192], its transpose per head, so the absorption is the same
// kind of product).  Weights sit on the M side of v_mfma_f32_16x16x32_bf16
// and tokens on the N side, so each lane of the 16x16 result holds 4
// consecutive weight rows of one token: a rope pair (2j, 2j + 1) is in one
// lane.
//
//   qgemm_skinny_kernel  decode batches (16 or 32 tokens per token block):
//                        each wave streams its share of K (64-wide blocks w,
//                        w + 4, ...) for 96 (projection) or 64 (absorption)
//                        weight rows straight into MFMA operand registers,
//                        3 blocks in flight, no LDS and no barrier in the
//                        loop; the 4 waves' partial tiles are summed through
//                        LDS at the end.  HBM-bound on the weights.
//   qgemm_tiled_kernel   prefill batches: 128 or 256 weight rows x 128 tokens
//                        per workgroup, K chunks staged in LDS by direct
//                        global -> LDS loads (a ring of stages), waves of
//                        64 x 64: 128 x 128 tiles and 64-wide chunks in two
//                        stages for the projection, 256 x 128 tiles and
//                        32-wide chunks in three stages for the absorption.
#include <atomic>
#include <cmath>

#include "rope.h"
#include "sa_common.h"

namespace sa {

constexpr int kQThreads = 256;
constexpr int kQModeBf16 = 0;        // bf16 (RNE)
constexpr int kQModeRope = 1;        // bf16, rows r % period >= rope_start turned in pairs
constexpr int kQModeF32 = 2;         // fp32

struct QSeg {
  const uint16_t* w;   // [rows][lda] weights of this segment (+ batch * w_batch)
  void* out;           // token t: out + t * ldo (+ batch * o_batch), element = segment row
  int64_t ldo;
  int rows;            // a multiple of 4
  int mblocks;         // workgroups along this segment's rows
  int mode;
  int period, rope_start;
};

struct QArgs {
  const uint16_t* x;   // tokens [n][ldx] (+ batch * x_batch), K contiguous
  int64_t ldx, x_batch, w_batch, o_batch;
  int lda, K, n;
  int n_seg;
  QSeg seg[3];
  const int32_t* pos;  // [n] token positions (rope)
  // absorption: the rope part rides along, copied by the first m-block of
  // each (head, token block): dst + t * dst_ld + b * dst_batch <- src (64 values)
  const uint16_t* copy_src;
  uint16_t* copy_dst;
  int64_t copy_src_ld, copy_dst_ld, copy_src_batch, copy_dst_batch;
  double inv_freq[32];   // theta^(-2j / 64)
};

__device__ __forceinline__ double bf16_bits_to_f64(uint32_t h) { return (double)__uint_as_float(h << 16); }

// The segment of workgroup row-block mb (uniform), and mb within it.
__device__ __forceinline__ int q_segment(const QArgs& A, int& mb) {
  int s = 0;
  if (A.n_seg > 1 && mb >= A.seg[0].mblocks) {
    mb -= A.seg[0].mblocks;
    s = 1;
    if (A.n_seg > 2 && mb >= A.seg[1].mblocks) {
      mb -= A.seg[1].mblocks;
      s = 2;
    }
  }
  return s;
}

// Store rows r .. r + 3 (segment rows, r a multiple of 4) of token t.
__device__ __forceinline__ void q_store4(const QArgs& A, const QSeg& S, int b, int r, int t, f32x4 v) {
#pragma clang fp contract(off)
  if (r >= S.rows || t >= A.n) return;
  if (S.mode == kQModeF32) {
    float* o = reinterpret_cast<float*>(S.out) + (int64_t)b * A.o_batch + (int64_t)t * S.ldo + r;
    *reinterpret_cast<f32x4*>(o) = v;
    return;
  }
  uint16_t* o = reinterpret_cast<uint16_t*>(S.out) + (int64_t)b * A.o_batch + (int64_t)t * S.ldo + r;
  const int hr = S.mode == kQModeRope ? r % S.period : 0;
  if (S.mode == kQModeRope && hr >= S.rope_start) {
    const int p = A.pos[t];
    const int j = (hr - S.rope_start) >> 1;
    uint32_t pk[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      double x0 = bf16_bits_to_f64(f32_to_bf16_rne(v[2 * q]));
      double x1 = bf16_bits_to_f64(f32_to_bf16_rne(v[2 * q + 1]));
      double sn, cs;
      turn_sincos(p, A.inv_freq[j + q], sn, cs);
      rope_pair(x0, x1, sn, cs);
      pk[q] = pack_bf16x2((float)x0, (float)x1);
    }
    *reinterpret_cast<u32x2*>(o) = u32x2{pk[0], pk[1]};
  } else {
    *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

// The 64-value rope part of each token of the block (absorption only).
__device__ __forceinline__ void q_copy_rope(const QArgs& A, int b, int n0, int n_tok) {
  for (int i = threadIdx.x; i < n_tok * 8; i += blockDim.x) {
    const int t = n0 + (i >> 3);
    if (t >= A.n) continue;
    const u32x4 v = ld16(A.copy_src + (int64_t)b * A.copy_src_batch + (int64_t)t * A.copy_src_ld + (i & 7) * 8);
    *reinterpret_cast<u32x4*>(A.copy_dst + (int64_t)b * A.copy_dst_batch + (int64_t)t * A.copy_dst_ld + (i & 7) * 8) = v;
  }
}

// ------------------------------------------------------------ decode batches
// K is consumed in 64-wide blocks dealt to the 4 waves in turn (blocks w,
// w + 4, ...).  Within a block the two 32-wide MFMA steps take their
// contraction slots from k = 64 blk + 16 kg + 8 j (j = step, kg = lane / 16),
// the same order for both operands, so each lane reads 32 contiguous bytes
// of a row and the 4 lanes of a row read its whole 128-byte line.
// 16-row weight tiles per workgroup: the projection takes 6 (96 rows: its
// 20,512 rows make 215 workgroups, one per CU), the absorption 4 (64 rows
// per head block, 512 workgroups: 7.36 against 7.66 us for 2 and 7.68 for 8
// at 16 tokens).
constexpr int kSkTMProject = 6, kSkTMAbsorb = 4;
constexpr int kSkDepth = 3;          // 64-wide blocks in flight per wave

// KPW > 0: K is exactly 4 KPW blocks (every wave has KPW of them) and the
// block loop is unrolled at compile time, so every load is unconditional and
// the compiler waits for each block's loads alone.  With a runtime count
// (KPW = 0) the loads sit behind branches, and the compiler, unable to count
// what is outstanding, waits for everything before each block: one block in
// flight instead of kSkDepth.
template <int TN, int KPW, int TM>   // 16 TN tokens and 16 TM weight rows per workgroup
__global__ __launch_bounds__(kQThreads) void qgemm_skinny_kernel(QArgs A) {
  int mb = blockIdx.x;
  const int si = q_segment(A, mb);
  const QSeg& S = si == 0 ? A.seg[0] : (si == 1 ? A.seg[1] : A.seg[2]);
  const int b = blockIdx.z;
  const int m0 = mb * 16 * TM, n0 = blockIdx.y * 16 * TN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, kg = lane >> 4;
  if (A.copy_dst && mb == 0) q_copy_rope(A, b, n0, 16 * TN);
  // operand row pointers: weight row m0 + 16 tm + l16, token n0 + 16 tn + l16
  // (clamped into range; their results are not stored), lane offset 16 kg
  const uint16_t* wp[TM];
  const uint16_t* xp[TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
    wp[tm] = S.w + (int64_t)b * A.w_batch + (int64_t)min(m0 + 16 * tm + l16, S.rows - 1) * A.lda + 16 * kg;
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
    xp[tn] = A.x + (int64_t)b * A.x_batch + (int64_t)min(n0 + 16 * tn + l16, A.n - 1) * A.ldx + 16 * kg;
  const int n_blk = A.K / 64;
  const int n_my = (n_blk - wave + 3) / 4;      // this wave's blocks: wave, wave + 4, ...
  f32x4 acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 ra[kSkDepth][TM][2], rb[kSkDepth][TN][2];
  auto load = [&](int slot, int i) {
    const int k = 64 * (wave + 4 * i);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        ra[slot][tm][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp[tm] + k + 8 * j));
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int j = 0; j < 2; ++j) rb[slot][tn][j] = ld16(xp[tn] + k + 8 * j);
  };
  auto products = [&](int u) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ra[u][tm][j]), as_bf16x8(rb[u][tn][j]),
                                                                acc[tm][tn], 0, 0, 0);
  };
  if constexpr (KPW > 0) {
    static_assert(KPW >= kSkDepth, "the unrolled loop starts with kSkDepth blocks in flight");
    // (the scheduling barriers keep each block's loads where they are
    // written; left free, the scheduler sinks them next to their use)
#pragma unroll
    for (int u = 0; u < kSkDepth; ++u) load(u, u);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      products(i % kSkDepth);
      if (i + kSkDepth < KPW) load(i % kSkDepth, i + kSkDepth);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int u = 0; u < kSkDepth; ++u)
      if (u < n_my) load(u, u);
    for (int i = 0; i < n_my; i += kSkDepth) {
#pragma unroll
      for (int u = 0; u < kSkDepth; ++u) {
        if (i + u < n_my) {
          products(u);
          if (i + u + kSkDepth < n_my) load(u, i + u + kSkDepth);
        }
      }
    }
  }
  // sum the 4 waves' partial tiles: wave w finishes tiles tm = w, w + 4, ...
  __shared__ f32x4 part[4][TM][TN][64];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) part[wave][tm][tn][lane] = acc[tm][tn];
  __syncthreads();
  for (int tm = wave; tm < TM; tm += 4) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      f32x4 v = part[0][tm][tn][lane];
#pragma unroll
      for (int w2 = 1; w2 < 4; ++w2) v += part[w2][tm][tn][lane];
      q_store4(A, S, b, m0 + 16 * tm + 4 * kg, n0 + 16 * tn + l16, v);
    }
  }
}

// ----------------------------------------------------------- prefill batches
// BM weight rows x 128 tokens per workgroup (BM / 64 x 2 waves of 64 x 64), K
// in BK-wide chunks through a ring of STAGES LDS stages filled by direct
// global -> LDS loads, STAGES - 1 chunks ahead of the products.  A stage
// holds each row's BK values as 16-byte chunks, chunk c of row r at slot
// ti_slot(r, c): the lanes of each 128-byte phase of an operand read hit 32
// different banks.
// (launch bounds: WPC workgroups of (BM / 64) x 2 waves per CU)
template <int BM>
constexpr int ti_threads() { return 64 * (BM / 64) * 2; }
template <int BM, int WPC>
constexpr int ti_waves_per_simd() { return (BM / 64) * 2 * WPC / 4; }

template <int BM, int BK, int STAGES>
struct TiCfg {
  static constexpr int kBN = 128;
  static constexpr int kWM = BM / 64;                  // wave rows
  static constexpr int kWaves = kWM * (kBN / 64);
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRowB = BK * 2;                 // bytes per staged row
  static constexpr int kChunks = kRowB / 16;           // 16-byte chunks per staged row
  static constexpr int kStageB = (BM + kBN) * kRowB;
  static constexpr int kLoads = kStageB / 16 / kThreads;   // 16-byte direct loads per thread per stage
  static constexpr size_t kSmem = (size_t)STAGES * kStageB;
  static_assert(kChunks == 4 || kChunks == 8, "64- or 128-byte rows");
  static_assert(kStageB % (1024 * kWaves) == 0, "whole 1 KB loads per wave");
  static_assert(STAGES >= 2, "at least one chunk ahead");
  static_assert(kThreads == ti_threads<BM>(), "launch bounds");
};
constexpr int kTiTM = 4, kTiTN = 4;                     // 16x16 tiles per wave (64 x 64)

// Configurations (interleaved A/B at 4096 tokens, identical outputs):
// the projection (K = 2048) takes 128 x 128 tiles, 64-wide chunks in two
// stages, two workgroups per CU: 473 us, against 520-723 us for 32-wide chunks
// (2-4 stages, 2-4 workgroups per CU) or 256-row tiles.  The absorption
// (K = 192 per head, three chunks: the tile's fixed costs dominate) takes
// 256 x 128 tiles, 32-wide chunks in three stages, two workgroups per CU:
// 222 against 253 us.
struct TiProject {
  static constexpr int kSkTM = kSkTMProject;
  static constexpr int kBM = 128, kBK = 64, kStages = 2, kWpc = 2;
};
struct TiAbsorb {
  static constexpr int kSkTM = kSkTMAbsorb;
  static constexpr int kBM = 256, kBK = 32, kStages = 3, kWpc = 2;
};

template <int BM, int BK, int STAGES, int WPC>
__global__ __attribute__((amdgpu_flat_work_group_size(1, ti_threads<BM>()),
                          amdgpu_waves_per_eu(ti_waves_per_simd<BM, WPC>()))) void qgemm_tiled_kernel(QArgs A) {
  using C = TiCfg<BM, BK, STAGES>;
  constexpr int kCh = C::kChunks;
  auto ti_slot = [](int r, int c) { return kCh == 8 ? c ^ (r & 7) : c ^ ((r >> 1) & 3); };
  extern __shared__ __align__(16) uint8_t qsm[];
  int mb = blockIdx.x;
  const int si = q_segment(A, mb);
  const QSeg& S = si == 0 ? A.seg[0] : (si == 1 ? A.seg[1] : A.seg[2]);
  const int b = blockIdx.z;
  const int m0 = mb * BM, n0 = blockIdx.y * C::kBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % C::kWM, wn = wave / C::kWM;
  const int l16 = lane & 15, kg = lane >> 4;
  if (A.copy_dst && mb == 0) q_copy_rope(A, b, n0, C::kBN);
  const uint16_t* W = S.w + (int64_t)b * A.w_batch;
  const uint16_t* X = A.x + (int64_t)b * A.x_batch;
  // Load u of this wave fills the 1 KB of staged rows from row
  // (1024 / kRowB) (kWaves u + wave) on (rows 0..BM-1 weights, then tokens):
  // lane p -> row + p / kChunks, slot p % kChunks, which holds the chunk that
  // ti_slot maps there.
  const uint16_t* src[C::kLoads];
  int dst[C::kLoads];
#pragma unroll
  for (int u = 0; u < C::kLoads; ++u) {
    const int row = (1024 / C::kRowB) * (C::kWaves * u + wave) + lane / kCh;
    const int chunk = ti_slot(row, lane % kCh);          // (the mapping is its own inverse)
    src[u] = row < BM ? W + (int64_t)min(m0 + row, S.rows - 1) * A.lda + 8 * chunk
                      : X + (int64_t)min(n0 + row - BM, A.n - 1) * A.ldx + 8 * chunk;
    dst[u] = 1024 * (C::kWaves * u + wave);              // the instruction's 1 KB, lane p at + 16 p
  }
  const int nk = A.K / BK;
  auto issue = [&](int kc) {                             // chunk kc (clamped) into its stage
    const int kk = min(kc, nk - 1);
    uint8_t* st = qsm + (size_t)(kc % STAGES) * C::kStageB;
#pragma unroll
    for (int u = 0; u < C::kLoads; ++u)
      __builtin_amdgcn_global_load_lds((const void*)(src[u] + kk * BK),
                                       (__attribute__((address_space(3))) void*)(st + dst[u]), 16, 0, 0);
  };
  f32x4 acc[kTiTM][kTiTN];
#pragma unroll
  for (int tm = 0; tm < kTiTM; ++tm)
#pragma unroll
    for (int tn = 0; tn < kTiTN; ++tn) acc[tm][tn] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < STAGES - 1; ++c) issue(c);
  SA_WAIT_VMCNT(C::kLoads * (STAGES - 2));               // chunk 0 is in
  __syncthreads();
  // operand rows of this lane: weight row 64 wm + 16 tm + l16, token row
  // BM + 64 wn + 16 tn + l16; chunk 4 s + kg
  const int rA = 64 * wm + l16, rB = BM + 64 * wn + l16;
#pragma unroll 1
  for (int kc = 0; kc < nk; ++kc) {
    issue(kc + STAGES - 1);                              // into the stage read at kc - 1
    const uint8_t* st = qsm + (size_t)(kc % STAGES) * C::kStageB;
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      const int c = 4 * s + kg;
      bf16x8 a[kTiTM], bb[kTiTN];
#pragma unroll
      for (int tm = 0; tm < kTiTM; ++tm) {
        const int r = rA + 16 * tm;
        a[tm] = *reinterpret_cast<const bf16x8*>(st + r * C::kRowB + 16 * ti_slot(r, c));
      }
#pragma unroll
      for (int tn = 0; tn < kTiTN; ++tn) {
        const int r = rB + 16 * tn;
        bb[tn] = *reinterpret_cast<const bf16x8*>(st + r * C::kRowB + 16 * ti_slot(r, c));
      }
#pragma unroll
      for (int tm = 0; tm < kTiTM; ++tm)
#pragma unroll
        for (int tn = 0; tn < kTiTN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tm], bb[tn], acc[tm][tn], 0, 0, 0);
    }
    SA_WAIT_VMCNT(C::kLoads * (STAGES - 2));             // chunk kc + 1 is in
    __syncthreads();                                     // and every wave is done with chunk kc's stage
  }
  SA_WAIT_VMCNT(0);                                      // (the clamped trailing loads land before the end)
#pragma unroll
  for (int tm = 0; tm < kTiTM; ++tm)
#pragma unroll
    for (int tn = 0; tn < kTiTN; ++tn)
      q_store4(A, S, b, m0 + 64 * wm + tm * 16 + 4 * kg, n0 + 64 * wn + tn * 16 + l16, acc[tm][tn]);
}

}  // namespace sa

namespace sa_host {

static bool q_skinny(int32_t n) { return n <= 64; }

static void fill_inv_freq(double* f) {
  for (int j = 0; j < 32; ++j) f[j] = std::pow(8.0e6, -(double)(2 * j) / 64.0);
}

template <class T>
using TiOf = sa::TiCfg<T::kBM, T::kBK, T::kStages>;

template <class T>
static const void* ti_kernel() {
  return (const void*)sa::qgemm_tiled_kernel<T::kBM, T::kBK, T::kStages, T::kWpc>;
}

// hipFuncSetAttribute is per device; remember which devices have been set up.
static std::atomic<uint64_t> g_q_attr_set{0};

static int32_t q_reserve_lds() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    set_error("query side: hipGetDevice failed");
    return SA_ERR_HIP;
  }
  const uint64_t bit = 1ull << (dev & 63);
  if (g_q_attr_set.load() & bit) return SA_OK;
  if (hipFuncSetAttribute(ti_kernel<sa::TiProject>(), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)TiOf<sa::TiProject>::kSmem) != hipSuccess ||
      hipFuncSetAttribute(ti_kernel<sa::TiAbsorb>(), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)TiOf<sa::TiAbsorb>::kSmem) != hipSuccess) {
    set_error("query side: cannot reserve the tiled product's LDS");
    return SA_ERR_HIP;
  }
  g_q_attr_set.fetch_or(bit);
  return SA_OK;
}

// T: the tiled product's configuration for batches above the skinny limit.
template <class T>
static int32_t q_launch(sa::QArgs& A, int n_batch, hipStream_t stream) {
  const bool sk = q_skinny(A.n);
  const int sk_tn = A.n <= 16 ? 1 : 2;        // 16 or 32 tokens per skinny workgroup
  const int bm = sk ? 16 * T::kSkTM : T::kBM, bn = sk ? 16 * sk_tn : TiOf<T>::kBN;
  int64_t mblocks = 0;
  for (int s = 0; s < A.n_seg; ++s) {
    A.seg[s].mblocks = (A.seg[s].rows + bm - 1) / bm;
    mblocks += A.seg[s].mblocks;
  }
  const int64_t nblocks = (A.n + bn - 1) / bn;
  if (mblocks > 0x7fffffff || nblocks > 65535 || n_batch > 65535) {
    set_error("query side: grid too large (%lld x %lld x %d)", (long long)mblocks, (long long)nblocks, n_batch);
    return SA_ERR_UNSUPPORTED;
  }
  fill_inv_freq(A.inv_freq);
  const dim3 grid((unsigned)mblocks, (unsigned)nblocks, (unsigned)n_batch);
  if (sk) {
    const bool k2048 = A.K == 2048;      // q_lora_rank: 8 blocks per wave, unrolled
    constexpr int TM = T::kSkTM;
    if (sk_tn == 1 && k2048)
      hipLaunchKernelGGL((sa::qgemm_skinny_kernel<1, 8, TM>), grid, dim3(sa::kQThreads), 0, stream, A);
    else if (k2048)
      hipLaunchKernelGGL((sa::qgemm_skinny_kernel<2, 8, TM>), grid, dim3(sa::kQThreads), 0, stream, A);
    else if (sk_tn == 1)
      hipLaunchKernelGGL((sa::qgemm_skinny_kernel<1, 0, TM>), grid, dim3(sa::kQThreads), 0, stream, A);
    else
      hipLaunchKernelGGL((sa::qgemm_skinny_kernel<2, 0, TM>), grid, dim3(sa::kQThreads), 0, stream, A);
    return check_launch("qgemm_skinny_kernel");
  }
  const int32_t rc = q_reserve_lds();
  if (rc) return rc;
  hipLaunchKernelGGL((sa::qgemm_tiled_kernel<T::kBM, T::kBK, T::kStages, T::kWpc>), grid, dim3(TiOf<T>::kThreads),
                     TiOf<T>::kSmem, stream, A);
  return check_launch("qgemm_tiled_kernel");
}

int32_t launch_q_project(const void* c_q, const void* w_qb, const void* w_iq, const void* w_iw, const int32_t* pos,
                         int32_t n, void* q, void* q_idx, float* w, hipStream_t stream) {
  sa::QArgs A{};
  A.x = (const uint16_t*)c_q;
  A.ldx = 2048;
  A.lda = 2048;
  A.K = 2048;
  A.n = n;
  A.pos = pos;
  A.seg[0] = sa::QSeg{(const uint16_t*)w_qb, q, sa::kHeads * 256, sa::kHeads * 256, 0, sa::kQModeRope, 256, 192};
  A.n_seg = 1;
  if (w_iq) {
    A.seg[1] = sa::QSeg{(const uint16_t*)w_iq, q_idx, sa::kIdxHeads * sa::kIdxDim, sa::kIdxHeads * sa::kIdxDim, 0,
                        sa::kQModeRope, sa::kIdxDim, sa::kIdxDim - 64};
    A.seg[2] = sa::QSeg{(const uint16_t*)w_iw, w, sa::kIdxHeads, sa::kIdxHeads, 0, sa::kQModeF32, 0, 0};
    A.n_seg = 3;
  }
  return q_launch<sa::TiProject>(A, 1, stream);
}

int32_t launch_q_absorb(const void* q, const void* w_uk_t, int32_t n, void* q_abs, hipStream_t stream) {
  sa::QArgs A{};
  A.x = (const uint16_t*)q;
  A.ldx = sa::kHeads * 256;
  A.x_batch = 256;
  A.w_batch = (int64_t)sa::kLatent * 192;
  A.o_batch = sa::kRow;
  A.lda = 192;
  A.K = 192;
  A.n = n;
  A.seg[0] = sa::QSeg{(const uint16_t*)w_uk_t, q_abs, (int64_t)sa::kHeads * sa::kRow, sa::kLatent, 0, sa::kQModeBf16, 0, 0};
  A.n_seg = 1;
  A.copy_src = (const uint16_t*)q + 192;
  A.copy_dst = (uint16_t*)q_abs + sa::kLatent;
  A.copy_src_ld = sa::kHeads * 256;
  A.copy_dst_ld = (int64_t)sa::kHeads * sa::kRow;
  A.copy_src_batch = 256;
  A.copy_dst_batch = sa::kRow;
  return q_launch<sa::TiAbsorb>(A, sa::kHeads, stream);
}

}  // namespace sa_host
