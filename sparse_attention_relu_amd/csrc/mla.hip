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
//     next tile's loads in flight while the current one is computed;
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
// mla_combine_wuv_kernel: one workgroup per (head, 64 value rows) keeps its
// 64 x 512 slice of W_UV in registers, merges the slices' partial softmax
// states of each query and applies the up-projection, rounding to bf16.
#include <atomic>

#include "sa_common.h"

namespace sa {

constexpr int kAttnWaves = 4;
constexpr int kTile = 16;                 // rows per wave tile
constexpr int kRowPitch = 1168;           // LDS bytes per gathered row (1152 + 16)
constexpr int kHg = 4;                    // head groups of 16
constexpr float kRescaleSlack = 8.0f;     // log2 units

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
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
  float* part_o;         // [n_q][4][n_sp][16][512]
  float* part_ml;        // [n_q][4][n_sp][16][2]  (max in log2 units, sum)
};

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

  // Q^T operand for this wave's 16 heads: head hg*16 + l16, dims 32s + 8g .. +8.
  bf16x8 qb[18];
  {
    const uint16_t* qp = A.q_abs + ((int64_t)t * kHeads + hg * 16 + l16) * kRow + 8 * g;
#pragma unroll
    for (int s = 0; s < 18; ++s) qb[s] = as_bf16x8(ld16(qp + 32 * s));
  }
  const uint16_t* rows = A.kv + A.seq_start[A.q_seq[t]] * kRow;
  const int32_t* irow = A.idx + (int64_t)t * A.k;
  const int j0 = sp * A.kps;
  const int j1 = min(A.k, j0 + A.kps);
  const int n_tiles = j1 > j0 ? (j1 - j0 + kTile - 1) / kTile : 0;

  // Gather of one tile into registers: 16 chunks of the latent (keys 4g+i,
  // dims 8m..8m+7 with m = l16 + 16b) and 2 chunks of the rope part (key l16,
  // dims 512 + 32u + 8g).
  u32x4 gv[16], gr[2];
  int my_pos[4];          // selection entries of keys 4g + i of the current tile (for masking)
  auto gather = [&](int tile) {
    const int jt = j0 + tile * kTile;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = jt + 4 * g + i;
      const int p = j < j1 ? irow[j] : -1;
      const uint16_t* r = rows + (int64_t)max(p, 0) * kRow;
#pragma unroll
      for (int b = 0; b < 4; ++b) gv[4 * i + b] = ld16(r + 8 * (l16 + 16 * b));
    }
    const int jr = jt + l16;
    const int pr = jr < j1 ? irow[jr] : -1;
    const uint16_t* rr = rows + (int64_t)max(pr, 0) * kRow + kLatent;
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

  // Wave w takes tiles w, w+4, ...
  int tile = wave;
  if (tile < n_tiles) {
    gather(tile);
    stash(buf0);
  }
  wave_lds_sync();
  uint8_t* cur = buf0;
  uint8_t* nxt = buf1;
#pragma unroll 1
  for (; tile < n_tiles; tile += kAttnWaves) {
    const bool more = tile + kAttnWaves < n_tiles;
    if (more) gather(tile + kAttnWaves);
    // Valid keys of this tile for this lane: keys 4g + i.
    const int jt = j0 + tile * kTile;
    bool valid[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = jt + 4 * g + i;
      valid[i] = j < j1 && irow[j] >= 0;
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
    if (more) stash(nxt);
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
  const int64_t pbase = (((int64_t)t * kHg + hg) * A.n_sp + sp) * 16;
  for (int i = threadIdx.x; i < 16 * kLatent; i += 256) {
    const int hh = i / kLatent, dim = i - hh * kLatent;
    float mw[kAttnWaves], M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < kAttnWaves; ++w2) {
      mw[w2] = lml[(w2 * 16 + hh) * 2];
      M = fmaxf(M, mw[w2]);
    }
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kAttnWaves; ++w2) {
      const float a = mw[w2] == -INFINITY ? 0.f : fast_exp2(mw[w2] - M);
      acc = fmaf(a, lo[(w2 * 16 + hh) * kLatent + dim], acc);
      lsum = fmaf(a, lml[(w2 * 16 + hh) * 2 + 1], lsum);
    }
    A.part_o[(pbase + hh) * kLatent + dim] = acc;
    if (dim == 0) {
      A.part_ml[(pbase + hh) * 2 + 0] = M;
      A.part_ml[(pbase + hh) * 2 + 1] = lsum;
    }
  }
}

// ------------------------------------------------------------ combine + W_UV
constexpr int kQB = 16;                     // queries per batch
constexpr int kObarPitch = 132;             // floats per 128-wide quarter (+4 pad)

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  const uint16_t* w_uv;
  int n_q;
  int n_sp;
  uint16_t* out;        // [n_q][64][256]
  float* lse;           // [n_q][64] or null
};

__global__ __launch_bounds__(256) void mla_combine_wuv_kernel(CombineArgs C) {
  const int h = blockIdx.x >> 2;
  const int vblk = blockIdx.x & 3;
  const int tid = threadIdx.x;
  const int v = vblk * 64 + (tid >> 2);
  const int cq = tid & 3;
  const int hg = h >> 4, hh = h & 15;

  // W_UV[h][v][128 cq .. +128) as 64 packed bf16 pairs.
  u32x4 wreg[16];
  {
    const uint16_t* wp = C.w_uv + ((int64_t)h * kVdim + v) * kLatent + 128 * cq;
#pragma unroll
    for (int i = 0; i < 16; ++i) wreg[i] = ld16(wp + 8 * i);
  }
  __shared__ float obar[kQB * 4 * kObarPitch];
  __shared__ float wgt[kQB * 32];
  __shared__ float lse_sh[kQB];

  for (int q0 = 0; q0 < C.n_q; q0 += kQB) {
    const int nqb = min(kQB, C.n_q - q0);
    // Softmax-state merge weights per (query, slice).
    if (tid < nqb) {
      const int t = q0 + tid;
      const float* ml = C.part_ml + (((int64_t)t * kHg + hg) * C.n_sp) * 16 * 2;
      float M = -INFINITY;
      for (int sp = 0; sp < C.n_sp; ++sp) M = fmaxf(M, ml[(sp * 16 + hh) * 2]);
      float L = 0.f;
      for (int sp = 0; sp < C.n_sp; ++sp) {
        const float m = ml[(sp * 16 + hh) * 2];
        const float a = m == -INFINITY ? 0.f : fast_exp2(m - M);
        wgt[tid * 32 + sp] = a;
        L = fmaf(a, ml[(sp * 16 + hh) * 2 + 1], L);
      }
      const float inv = L > 0.f ? 1.f / L : 0.f;
      for (int sp = 0; sp < C.n_sp; ++sp) wgt[tid * 32 + sp] *= inv;
      lse_sh[tid] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
    }
    __syncthreads();
    for (int i = tid; i < nqb * kLatent; i += 256) {
      const int tq = i / kLatent, c = i - tq * kLatent;
      const int t = q0 + tq;
      const float* po = C.part_o + ((((int64_t)t * kHg + hg) * C.n_sp) * 16 + hh) * kLatent + c;
      float acc = 0.f;
      for (int sp = 0; sp < C.n_sp; ++sp) acc = fmaf(wgt[tq * 32 + sp], po[(int64_t)sp * 16 * kLatent], acc);
      obar[tq * 4 * kObarPitch + (c >> 7) * kObarPitch + (c & 127)] = acc;
    }
    __syncthreads();
    for (int tq = 0; tq < nqb; ++tq) {
      const float* ob = obar + tq * 4 * kObarPitch + cq * kObarPitch;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t wv = wreg[i][d];
          acc = fmaf(__uint_as_float(wv << 16), ob[8 * i + 2 * d], acc);
          acc = fmaf(__uint_as_float(wv & 0xffff0000u), ob[8 * i + 2 * d + 1], acc);
        }
      }
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      if (cq == 0) C.out[((int64_t)(q0 + tq) * kHeads + h) * kVdim + v] = (uint16_t)f32_to_bf16_rne(acc);
    }
    if (C.lse && vblk == 0 && tid < nqb) C.lse[(int64_t)(q0 + tid) * kHeads + h] = lse_sh[tid];
    __syncthreads();
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
  if (n_sp > 32) n_sp = 32;
  if (n_sp < 1) n_sp = 1;
  return n_sp;
}

size_t mla_workspace_size(int32_t n_q, int32_t k) {
  const int n_sp = mla_n_splits(n_q, k);
  return align256((size_t)n_q * 4 * n_sp * 16 * sa::kLatent * 4) + align256((size_t)n_q * 4 * n_sp * 16 * 2 * 4);
}

// hipFuncSetAttribute is per device; remember which devices have been set up.
static std::atomic<uint64_t> g_attr_set{0};

int32_t launch_mla(const void* q_abs, const void* kv, const int64_t* seq_start, const int32_t* q_seq,
                   const int32_t* idx, int32_t n_q, int32_t k, const void* w_uv, float scale, void* out, float* lse,
                   void* ws, hipStream_t stream) {
  const int n_sp = mla_n_splits(n_q, k);
  int kps = (k + n_sp - 1) / n_sp;
  kps = (kps + 63) / 64 * 64;
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
  A.part_o = (float*)ws;
  A.part_ml = (float*)((uint8_t*)ws + align256((size_t)n_q * 4 * n_sp * 16 * sa::kLatent * 4));
  const size_t smem = (size_t)sa::kAttnWaves * 2 * sa::kTile * sa::kRowPitch;   // 149,504 B
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
  sa::CombineArgs C;
  C.part_o = A.part_o;
  C.part_ml = A.part_ml;
  C.w_uv = (const uint16_t*)w_uv;
  C.n_q = n_q;
  C.n_sp = n_sp;
  C.out = (uint16_t*)out;
  C.lse = lse;
  hipLaunchKernelGGL(sa::mla_combine_wuv_kernel, dim3(sa::kHeads * 4), dim3(256), 0, stream, C);
  return check_launch("mla_combine_wuv_kernel");
}

}  // namespace sa_host
