// Cache write for gfx950: the step before the path.  Each new token's
// kv_a_proj output (512 latent + 64 rope-key values) becomes its 576-wide
// cache row, and its indexer-key projection (128 values) its indexer key.
//
//   row[0:512]   = RMSNorm(latent) * gamma, eps = rms_norm_eps = 1e-5
//   row[512:576] = the 64-dim key with interleaved RoPE: pair (2i, 2i + 1)
//                  turned by p * theta^(-2i / 64), theta = 8e6
//   key[0:128]   = LayerNorm(k) * weight + bias (population variance, same eps),
//                  then dims 64..127 turned like the rope key
//
// models.inteligile.com "GLM-5.2 / Model techniques map", "Checked in its
// code", rows "Multi-head latent attention" (kv_a_layernorm over the 512-dim
// latent, decoupled rope key), "QK normalization" (k_norm, a LayerNorm of the
// indexer key), "Partial RoPE" and "YaRN RoPE scaling" (64 rotated dims,
// default rope type, rope_theta 8e6); llm-atlas "GLM-5.2", config fields
// rms_norm_eps, rope_interleave, indexer_rope_interleave.  The pages give no
// eps for k_norm and do not say which half of the indexer key turns; this
// takes rms_norm_eps and the last 64 dims (the order of the main attention's
// nope/rope split).
//
// The arithmetic is done in fp64 (the kernel moves 2.8 KB per token and
// spends a few hundred flops on it): the RoPE angles reach 10^6 rad at
// million-token positions, where fp32 would keep no correct digit of the
// angle.  The angle is reduced to [-pi, pi] first (Cody-Waite, 2 pi in three
// parts, the first two short enough that their products with the turn count
// are exact), so sin and cos take their short path.  The 32 frequencies are
// computed once on the host in fp64.  Each stored value is rounded once,
// fp64 -> fp32 -> bf16, both steps to nearest even.  Expressions are not
// contracted into fused multiply-adds; the norms multiply by one reciprocal
// square root (within an fp64 ulp of dividing by the root).
#include <math.h>

#include <cmath>

#include "rope.h"
#include "sa_common.h"

namespace sa {

constexpr int kCwWaves = 4;                 // tokens per workgroup: one wave each
constexpr double kNormEps = 1e-5;
constexpr double kRopeTheta = 8.0e6;

struct CacheWriteArgs {
  const uint16_t* kv_a;    // [n][576] bf16: kv_a_proj output of the new tokens
  const uint16_t* gamma;   // [512] bf16: kv_a_layernorm weight
  const uint16_t* k_raw;   // [n][128] bf16: indexer key projection, or null
  const uint16_t* ln_w;    // [128] bf16: k_norm weight
  const uint16_t* ln_b;    // [128] bf16: k_norm bias
  const int32_t* pos;      // [n]: position of each token in its sequence
  const int64_t* dst;      // [n]: row of each token in the caches
  uint16_t* kv_cache;      // [*][576] bf16
  uint16_t* k_cache;       // [*][128] bf16
  int n;
  double inv_freq[kRope / 2];   // theta^(-2i / 64)
};

__device__ __forceinline__ double bf16_to_f64(uint32_t h) { return (double)__uint_as_float(h << 16); }

// One DPP move of a double (its two halves).
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, kCtrl, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), kCtrl, 0xf, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, l);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Sum over the 64 lanes, the same value on every lane: within each row of 16
// by DPP exchanges (lane ^ 1, lane ^ 2, then the mirror images within 8 and
// within 16 lanes; both partners add the same two operands), then the four
// row sums in one fixed order.
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<0xB1>(v);      // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(v);      // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(v);     // row_half_mirror
  v += dpp_f64<0x140>(v);     // row_mirror
  return ((readlane_f64(v, 0) + readlane_f64(v, 16)) + readlane_f64(v, 32)) + readlane_f64(v, 48);
}

__device__ __forceinline__ uint32_t pack2(double a, double b) { return pack_bf16x2((float)a, (float)b); }

__global__ __launch_bounds__(kCwWaves * 64) void cache_write_kernel(CacheWriteArgs A) {
#pragma clang fp contract(off)
  const int t = blockIdx.x * kCwWaves + (threadIdx.x >> 6);
  if (t >= A.n) return;                    // whole waves leave together
  const int lane = threadIdx.x & 63;
  const uint16_t* src = A.kv_a + (int64_t)t * kRow;
  // Every load is issued first, so the token costs one round trip (the
  // stores below could alias the inputs as far as the compiler knows, so it
  // would not move later loads above them).
  const int p = A.pos[t];
  const int64_t row = A.dst[t];
  const u32x4 xv = ld16(src + 8 * lane);                                      // latent 8l .. 8l + 7
  const u32x4 gv = ld16(A.gamma + 8 * lane);
  const uint32_t kv = *reinterpret_cast<const uint32_t*>(src + kLatent + 2 * (lane & 31));   // rope pair l % 32
  uint32_t kr = 0, wv = 0, bv = 0;                                            // indexer dims 2l, 2l + 1
  if (A.k_raw) {
    kr = *reinterpret_cast<const uint32_t*>(A.k_raw + (int64_t)t * kIdxDim + 2 * lane);
    wv = *reinterpret_cast<const uint32_t*>(A.ln_w + 2 * lane);
    bv = *reinterpret_cast<const uint32_t*>(A.ln_b + 2 * lane);
  }
  uint16_t* out = A.kv_cache + row * kRow;
  // Lane l turns pair l % 32: lanes 0..31 for the rope key, 32..63 for the
  // indexer key's last 64 dims; one sine and cosine per lane.
  double sn, cs;
  turn_sincos(p, A.inv_freq[lane & 31], sn, cs);

  // Latent: lane l holds values 8l .. 8l + 7.
  double x[8], g[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16_to_f64(xv[j] & 0xffffu);
    x[2 * j + 1] = bf16_to_f64(xv[j] >> 16);
    g[2 * j] = bf16_to_f64(gv[j] & 0xffffu);
    g[2 * j + 1] = bf16_to_f64(gv[j] >> 16);
  }
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
  const double inv_rms = 1.0 / sqrt(wave_sum(ss) / (double)kLatent + kNormEps);
  u32x4 yv;
#pragma unroll
  for (int j = 0; j < 4; ++j) yv[j] = pack2(x[2 * j] * inv_rms * g[2 * j], x[2 * j + 1] * inv_rms * g[2 * j + 1]);
  *reinterpret_cast<u32x4*>(out + 8 * lane) = yv;

  // Rope key: lane i < 32 turns pair i.
  if (lane < kRope / 2) {
    double k0 = bf16_to_f64(kv & 0xffffu), k1 = bf16_to_f64(kv >> 16);
    rope_pair(k0, k1, sn, cs);
    *reinterpret_cast<uint32_t*>(out + kLatent + 2 * lane) = pack2(k0, k1);
  }

  // Indexer key: LayerNorm over the 128 dims, then lanes 32..63 (dims
  // 64..127) turn pair l - 32.
  if (A.k_raw) {
    const double a0 = bf16_to_f64(kr & 0xffffu), a1 = bf16_to_f64(kr >> 16);
    const double mean = wave_sum(a0 + a1) / (double)kIdxDim;
    const double d0 = a0 - mean, d1 = a1 - mean;
    const double inv_sd = 1.0 / sqrt(wave_sum(d0 * d0 + d1 * d1) / (double)kIdxDim + kNormEps);
    double y0 = d0 * inv_sd * bf16_to_f64(wv & 0xffffu) + bf16_to_f64(bv & 0xffffu);
    double y1 = d1 * inv_sd * bf16_to_f64(wv >> 16) + bf16_to_f64(bv >> 16);
    if (lane >= kIdxDim / 4) rope_pair(y0, y1, sn, cs);
    *reinterpret_cast<uint32_t*>(A.k_cache + row * kIdxDim + 2 * lane) = pack2(y0, y1);
  }
}

}  // namespace sa

namespace sa_host {

int32_t launch_cache_write(const void* kv_a, const void* gamma, const void* k_raw, const void* ln_w, const void* ln_b,
                           const int32_t* pos, const int64_t* dst, int32_t n, void* kv_cache, void* k_cache,
                           hipStream_t stream) {
  sa::CacheWriteArgs A{(const uint16_t*)kv_a, (const uint16_t*)gamma, (const uint16_t*)k_raw,
                       (const uint16_t*)ln_w, (const uint16_t*)ln_b, pos, dst,
                       (uint16_t*)kv_cache, (uint16_t*)k_cache, n, {}};
  for (int i = 0; i < sa::kRope / 2; ++i) A.inv_freq[i] = std::pow(sa::kRopeTheta, -(double)(2 * i) / (double)sa::kRope);
  const int grid = (n + sa::kCwWaves - 1) / sa::kCwWaves;
  hipLaunchKernelGGL(sa::cache_write_kernel, dim3(grid), dim3(sa::kCwWaves * 64), 0, stream, A);
  return check_launch("cache_write_kernel");
}

}  // namespace sa_host
