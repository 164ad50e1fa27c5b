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
// mla_attn_kernel: one workgroup per (query, group of 16 heads, slice of the
// selection); its 4 waves take 16-row tiles of the slice in turn and merge
// their running (max, sum, accumulator) in LDS at the end.  Per tile a wave
//   - gathers 16 rows (18 KB) with 16-byte loads into wave-private LDS, the
//     next tile's loads in flight while the current one is computed (the
//     slice's positions are staged in LDS first, so no load waits on another);
//   - S^T[16 rows x 16 heads] = R . Q^T with v_mfma_f32_16x16x32_bf16 over the
//     576 dims (R from LDS, Q^T held in registers for the whole slice);
//   - runs the online softmax in base 2; the running maximum is only moved
//     when a tile exceeds it by more than 2^8, so the accumulator is rarely
//     rescaled;
//   - O^T[512 dims x 16 heads] += V^T . P^T with v_mfma_f32_16x16x16_bf16:
//     the 16 keys of the tile are the contraction, P^T comes straight out of
//     the S^T accumulator layout (each lane holds 4 keys of one head), and the
//     V^T operand is assembled from the lane's own row chunks with byte
//     permutes (dims are permuted consistently, no LDS transpose).
// With one slice per query the workgroup normalises and writes the latent
// average obar (bf16) itself; with several, each writes a partial state and
// mla_merge_kernel combines them.
// mla_wuv_kernel: one workgroup per (head, 64 value rows) holds that 64 x 512
// slice of W_UV in registers and multiplies it with obar^T, 16 queries per
// v_mfma_f32_16x16x32_bf16 column block, rounding the output to bf16.
#include <atomic>

#include "sa_common.h"

namespace sa {

constexpr int kAttnWaves = 4;
constexpr int kTile = 16;                 // rows per wave tile
constexpr int kRowPitch = 1168;           // LDS bytes per gathered row (1152 + 16)
constexpr int kHg = 4;                    // head groups of 16
constexpr float kRescaleSlack = 8.0f;     // log2 units

// Orders a wave's LDS writes before its reads of other lanes' data (LDS-only:
// in-flight global loads are not waited for).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t perm_lo(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
__device__ __forceinline__ uint32_t perm_hi(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }

struct AttnArgs {
  const uint16_t* q_abs;
  const uint16_t* kv;
  const int64_t* seq_start;
  const int32_t* q_seq;
  const int32_t* idx;
  int k;
  int n_q;
  int n_sp;
  int kps;               // selection entries per slice (multiple of 64)
  float scale_log2;      // scale * log2(e)
  float* part_o;         // [n_q][4][n_sp][16][512]   (n_sp > 1)
  float* part_ml;        // [n_q][4][n_sp][16][2]     (max in log2 units, sum)
  uint16_t* obar;        // [n_q][64][512] bf16 latent average
  float* lse;            // [n_q][64] or null
};

constexpr int kMaxSlice = 2048;
constexpr size_t kAttnTileBytes = (size_t)kAttnWaves * 2 * kTile * kRowPitch;     // 149,504
constexpr size_t kAttnSmem = kAttnTileBytes + kMaxSlice * 4;                      // + staged positions

__global__ __launch_bounds__(256, 1) void mla_attn_kernel(AttnArgs A) {
  // Workgroup -> (query t, slice sp, head group hg).  The 4 head groups of a
  // (t, sp) pair gather the same rows; their ids differ by multiples of 8 so
  // they land on the same XCD (round-robin dispatch) and share its L2.
  const int bid = blockIdx.x;
  const int pair = (bid >> 5) * 8 + (bid & 7);
  const int hg = (bid >> 3) & 3;
  if (pair >= A.n_q * A.n_sp) return;
  const int t = pair / A.n_sp;
  const int sp = pair - t * A.n_sp;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;

  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* buf0 = smem + wave * (2 * kTile * kRowPitch);
  uint8_t* buf1 = buf0 + kTile * kRowPitch;
  int32_t* spos = reinterpret_cast<int32_t*>(smem + kAttnTileBytes);

  const int j0 = sp * A.kps;
  const int j1 = min(A.k, j0 + A.kps);
  const int n_sel = max(j1 - j0, 0);
  if (n_sel > 0) {
    // Stage the slice's positions (all loads issued before any is used).
    const int32_t* irow = A.idx + (int64_t)t * A.k + j0;
    int pv[kMaxSlice / 256];
#pragma unroll
    for (int u = 0; u < kMaxSlice / 256; ++u) pv[u] = irow[min((int)threadIdx.x + 256 * u, n_sel - 1)];
#pragma unroll
    for (int u = 0; u < kMaxSlice / 256; ++u)
      if ((int)threadIdx.x + 256 * u < n_sel) spos[threadIdx.x + 256 * u] = pv[u];
  }

  // Q^T operand for this wave's 16 heads: head hg*16 + l16, dims 32s + 8g .. +8.
  bf16x8 qb[18];
  {
    const uint16_t* qp = A.q_abs + ((int64_t)t * kHeads + hg * 16 + l16) * kRow + 8 * g;
#pragma unroll
    for (int s = 0; s < 18; ++s) qb[s] = as_bf16x8(ld16(qp + 32 * s));
  }
  const uint16_t* rows = A.kv + A.seq_start[A.q_seq[t]] * kRow;
  const int n_tiles = (n_sel + kTile - 1) / kTile;
  __syncthreads();

  // Gather of one tile into registers: 16 chunks of the latent (keys 4g+i,
  // dims 8m..8m+7 with m = l16 + 16b) and 2 chunks of the rope part (key l16,
  // dims 512 + 32u + 8g).  Padding entries (-1) and slots past the slice read
  // row 0 and are masked out of the softmax.
  u32x4 gv[16], gr[2];
  const int last_sel = max(n_sel - 1, 0);
  auto row_of = [&](int j) {      // branch-free: out-of-slice or padding entries read row 0
    const int p = spos[min(j, last_sel)];
    return (j < n_sel && p >= 0) ? p : 0;
  };
  auto gather = [&](int tile) {
    const int jt = tile * kTile;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t* r = rows + (int64_t)row_of(jt + 4 * g + i) * kRow;
#pragma unroll
      for (int b = 0; b < 4; ++b) gv[4 * i + b] = ld16(r + 8 * (l16 + 16 * b));
    }
    const uint16_t* rr = rows + (int64_t)row_of(jt + l16) * kRow + kLatent;
#pragma unroll
    for (int u = 0; u < 2; ++u) gr[u] = ld16(rr + 32 * u + 8 * g);
  };
  auto stash = [&](uint8_t* buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        *reinterpret_cast<u32x4*>(buf + (4 * g + i) * kRowPitch + 16 * (l16 + 16 * b)) = gv[4 * i + b];
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *reinterpret_cast<u32x4*>(buf + l16 * kRowPitch + 2 * kLatent + 64 * u + 16 * g) = gr[u];
  };

  f32x4 o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Wave w takes tiles w, w+4, ...  (the first gather is unconditional so that
  // every path into the loop has drained the same loads)
  int tile = wave;
  gather(min(tile, max(n_tiles - 1, 0)));
  stash(buf0);
  wave_lds_sync();
  uint8_t* cur = buf0;
  uint8_t* nxt = buf1;
#pragma unroll 1
  for (; tile < n_tiles; tile += kAttnWaves) {
    // Next tile's gather, unconditional (clamped) so the loads stay in order.
    gather(min(tile + kAttnWaves, n_tiles - 1));
    bool valid[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = tile * kTile + 4 * g + i;
      valid[i] = j < n_sel && spos[min(j, last_sel)] >= 0;
    }
    // S^T = R . Q^T over 576 dims.
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 18; ++st) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(cur + l16 * kRowPitch + 64 * st + 16 * g);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), qb[st], s, 0, 0, 0);
    }
    // Online softmax (base 2), head = l16, keys 4g + i.
    float x[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = valid[i] ? s[i] * A.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const bool bump = tmax > m_run + kRescaleSlack;
    if (__any(bump)) {
      const float new_m = bump ? tmax : m_run;
      const float alpha = (bump && m_run != -INFINITY) ? fast_exp2(m_run - new_m) : (bump ? 0.f : 1.f);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] *= alpha;
      m_run = new_m;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = x[i] == -INFINITY ? 0.f : fast_exp2(x[i] - m_run);
      l_run += p[i];
    }
    const u32x2 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    const s16x4 pt = as_s16x4(pb);
    // O^T += V^T . P^T: tile (b, e) covers dims 8(r + 16b) + e for rows r = 0..15.
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      u32x4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = *reinterpret_cast<const u32x4*>(cur + (4 * g + i) * kRowPitch + 16 * (l16 + 16 * b));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = e >> 1;
        u32x2 av;
        if (e & 1) {
          av[0] = perm_hi(v[0][d], v[1][d]);
          av[1] = perm_hi(v[2][d], v[3][d]);
        } else {
          av[0] = perm_lo(v[0][d], v[1][d]);
          av[1] = perm_lo(v[2][d], v[3][d]);
        }
        o[8 * b + e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_s16x4(av), pt, o[8 * b + e], 0, 0, 0);
      }
    }
    stash(nxt);
    wave_lds_sync();
    uint8_t* tmp = cur;
    cur = nxt;
    nxt = tmp;
  }
  // Reduce the sum over the 4 lanes that share a head.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  // Merge the 4 waves in LDS (reusing the tile buffers).
  __syncthreads();
  float* lo = reinterpret_cast<float*>(smem);                  // [4][16][512]
  float* lml = lo + kAttnWaves * 16 * kLatent;                 // [4][16][2]
  float* lw = lml + kAttnWaves * 16 * 2;                       // [4][16] merge weights
  float* lhs = lw + kAttnWaves * 16;                           // [16][2]  merged (max, sum)
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dim = 32 * g + 8 * jj + 128 * b + e;
        lo[(wave * 16 + l16) * kLatent + dim] = o[8 * b + e][jj];
      }
  if (g == 0) {
    lml[(wave * 16 + l16) * 2 + 0] = m_run;
    lml[(wave * 16 + l16) * 2 + 1] = l_run;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const int hh = threadIdx.x;
    float M = -INFINITY;
    for (int w2 = 0; w2 < kAttnWaves; ++w2) M = fmaxf(M, lml[(w2 * 16 + hh) * 2]);
    float L = 0.f;
    for (int w2 = 0; w2 < kAttnWaves; ++w2) {
      const float m = lml[(w2 * 16 + hh) * 2];
      const float a = m == -INFINITY ? 0.f : fast_exp2(m - M);
      lw[w2 * 16 + hh] = a;
      L = fmaf(a, lml[(w2 * 16 + hh) * 2 + 1], L);
    }
    lhs[hh * 2] = M;
    lhs[hh * 2 + 1] = L;
    if (A.n_sp == 1) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      for (int w2 = 0; w2 < kAttnWaves; ++w2) lw[w2 * 16 + hh] *= inv;
      if (A.lse) A.lse[(int64_t)t * kHeads + hg * 16 + hh] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f
                                                                      : -INFINITY;
    }
  }
  __syncthreads();
  if (A.n_sp == 1) {
    // One slice: normalise and write obar (bf16) directly.
    uint16_t* ob = A.obar + ((int64_t)t * kHeads + hg * 16) * kLatent;
    for (int i = threadIdx.x; i < 16 * kLatent / 2; i += 256) {
      const int hh = (2 * i) / kLatent, dim = 2 * i - hh * kLatent;
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kAttnWaves; ++w2) {
        const float a = lw[w2 * 16 + hh];
        v0 = fmaf(a, lo[(w2 * 16 + hh) * kLatent + dim], v0);
        v1 = fmaf(a, lo[(w2 * 16 + hh) * kLatent + dim + 1], v1);
      }
      *reinterpret_cast<uint32_t*>(ob + hh * kLatent + dim) = pack_bf16x2(v0, v1);
    }
    return;
  }
  // Several slices: write this slice's partial state ...
  const int64_t gbase = ((int64_t)t * kHg + hg) * A.n_sp;
  const int64_t pbase = (gbase + sp) * 16;
  for (int i = threadIdx.x; i < 16 * kLatent / 4; i += 256) {
    const int hh = (4 * i) / kLatent, dim = 4 * i - hh * kLatent;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w2 = 0; w2 < kAttnWaves; ++w2) {
      const float a = lw[w2 * 16 + hh];
      const f32x4 x = *reinterpret_cast<const f32x4*>(lo + (w2 * 16 + hh) * kLatent + dim);
      acc += a * x;
    }
    *reinterpret_cast<f32x4*>(A.part_o + (pbase + hh) * kLatent + dim) = acc;
  }
  if (threadIdx.x < 16) {
    A.part_ml[(pbase + threadIdx.x) * 2 + 0] = lhs[threadIdx.x * 2];
    A.part_ml[(pbase + threadIdx.x) * 2 + 1] = lhs[threadIdx.x * 2 + 1];
  }
}

// Merge of the slices' partial softmax states: obar = sum_s a_s O_s / sum_s a_s l_s
// with a_s = 2^(m_s - max m).  One workgroup per (query, head group, 64 dims);
// each thread owns one head and 4 dims and issues all its loads at once.
constexpr int kMaxSp = 8;

__global__ __launch_bounds__(256) void mla_merge_kernel(AttnArgs A) {
  const int blk = blockIdx.x;
  const int dblk = blk & 7;
  const int hg = (blk >> 3) & 3;
  const int t = blk >> 5;
  const int hh = threadIdx.x >> 4;
  const int dim = dblk * 64 + (threadIdx.x & 15) * 4;
  const int64_t gbase = ((int64_t)t * kHg + hg) * A.n_sp;
  float m[kMaxSp], l[kMaxSp];
  f32x4 o[kMaxSp];
#pragma unroll
  for (int s2 = 0; s2 < kMaxSp; ++s2) {
    const int sc = min(s2, A.n_sp - 1);
    m[s2] = A.part_ml[((gbase + sc) * 16 + hh) * 2];
    l[s2] = A.part_ml[((gbase + sc) * 16 + hh) * 2 + 1];
    o[s2] = *reinterpret_cast<const f32x4*>(A.part_o + ((gbase + sc) * 16 + hh) * kLatent + dim);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s2 = 0; s2 < kMaxSp; ++s2) M = fmaxf(M, m[s2]);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < kMaxSp; ++s2) {
    const float a = (s2 < A.n_sp && m[s2] != -INFINITY) ? fast_exp2(m[s2] - M) : 0.f;
    L = fmaf(a, l[s2], L);
    acc += a * o[s2];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  acc *= inv;
  const u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  *reinterpret_cast<u32x2*>(A.obar + ((int64_t)t * kHeads + hg * 16 + hh) * kLatent + dim) = pk;
  if (A.lse && dblk == 0 && (threadIdx.x & 15) == 0)
    A.lse[(int64_t)t * kHeads + hg * 16 + hh] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// ------------------------------------------------------------------ W_UV
struct WuvArgs {
  const uint16_t* obar;     // [n_q][64][512] bf16
  const uint16_t* w_uv;     // [64][256][512] bf16
  uint16_t* out;            // [n_q][64][256] bf16
  int n_q;
};

__global__ __launch_bounds__(256) void mla_wuv_kernel(WuvArgs W) {
  const int h = blockIdx.x >> 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int v0 = (blockIdx.x & 3) * 64 + wave * 16;          // this wave's 16 value rows
  // A operand: W_UV[h][v0 + l16][32s + 8g .. +8], held for every query block.
  bf16x8 wa[16];
  const uint16_t* wp = W.w_uv + ((int64_t)h * kVdim + v0 + l16) * kLatent + 8 * g;
#pragma unroll
  for (int s = 0; s < 16; ++s) wa[s] = as_bf16x8(ld16(wp + 32 * s));
  for (int tb = 0; tb < W.n_q; tb += 16) {
    const int t = min(tb + l16, W.n_q - 1);
    const uint16_t* op = W.obar + ((int64_t)t * kHeads + h) * kLatent + 8 * g;
    bf16x8 ob[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) ob[s] = as_bf16x8(ld16(op + 32 * s));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[s], ob[s], acc, 0, 0, 0);
    // acc[j] = out[t = tb + l16][h][v0 + 4g + j]
    if (tb + l16 < W.n_q) {
      const u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *reinterpret_cast<u32x2*>(W.out + ((int64_t)(tb + l16) * kHeads + h) * kVdim + v0 + 4 * g) = pk;
    }
  }
}

}  // namespace sa

namespace sa_host {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int mla_n_splits(int32_t n_q, int32_t k) {
  const int target = 256;                      // one workgroup per CU
  int n_sp = (target + 4 * n_q - 1) / (4 * n_q);
  const int max_sp = (k + 63) / 64;
  if (n_sp > max_sp) n_sp = max_sp;
  if (n_sp > sa::kMaxSp) n_sp = sa::kMaxSp;
  if (n_sp < 1) n_sp = 1;
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
  p += n_sp > 1 ? align256((size_t)n_q * 4 * n_sp * 16 * 2 * 4) : 0;
  m.part_o = (float*)p;
  return m;
}

size_t mla_workspace_size(int32_t n_q, int32_t k) {
  const int n_sp = mla_n_splits(n_q, k);
  size_t s = align256((size_t)n_q * sa::kHeads * sa::kLatent * 2);
  if (n_sp > 1) s += align256((size_t)n_q * 4 * n_sp * 16 * 2 * 4) + align256((size_t)n_q * 4 * n_sp * 16 * sa::kLatent * 4);
  return s;
}

// hipFuncSetAttribute is per device; remember which devices have been set up.
static std::atomic<uint64_t> g_attr_set{0};

int32_t launch_mla(const void* q_abs, const void* kv, const int64_t* seq_start, const int32_t* q_seq,
                   const int32_t* idx, int32_t n_q, int32_t k, const void* w_uv, float scale, void* out, float* lse,
                   void* ws, hipStream_t stream) {
  const int n_sp = mla_n_splits(n_q, k);
  int kps = (k + n_sp - 1) / n_sp;
  kps = (kps + 63) / 64 * 64;
  MlaWs m = mla_carve(ws, n_q, n_sp);
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
  const size_t smem = sa::kAttnSmem;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    set_error("mla: hipGetDevice failed");
    return SA_ERR_HIP;
  }
  const uint64_t bit = 1ull << (dev & 63);
  if (!(g_attr_set.load() & bit)) {
    if (hipFuncSetAttribute((const void*)sa::mla_attn_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem) != hipSuccess) {
      set_error("mla: cannot reserve %zu bytes of LDS", smem);
      return SA_ERR_HIP;
    }
    g_attr_set.fetch_or(bit);
  }
  const int64_t pairs = (int64_t)n_q * n_sp;
  const int64_t grid = (pairs + 7) / 8 * 32;
  if (grid > 0x7fffffff) {
    set_error("mla: grid too large");
    return SA_ERR_UNSUPPORTED;
  }
  hipLaunchKernelGGL(sa::mla_attn_kernel, dim3((unsigned)grid), dim3(256), smem, stream, A);
  int32_t rc = check_launch("mla_attn_kernel");
  if (rc) return rc;
  if (n_sp > 1) {
    hipLaunchKernelGGL(sa::mla_merge_kernel, dim3((unsigned)(n_q * 32)), dim3(256), 0, stream, A);
    if ((rc = check_launch("mla_merge_kernel"))) return rc;
  }
  sa::WuvArgs W{m.obar, (const uint16_t*)w_uv, (uint16_t*)out, n_q};
  hipLaunchKernelGGL(sa::mla_wuv_kernel, dim3(sa::kHeads * 4), dim3(256), 0, stream, W);
  return check_launch("mla_wuv_kernel");
}

}  // namespace sa_host
