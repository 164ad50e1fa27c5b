// FP8 row quantizer and code decoder for gfx950.
//
// A cache row (576-wide latent + rope, or a 128-wide indexer key) becomes
// E4M3 codes and one fp32 scale (models.inteligile.com "GLM-5.2 / Model
// techniques map", "inference quantization": FP8 inference; llm-atlas
// "GLM-5.2", "Faits clés": precision fp8; the pages give no format or scaling,
// the reading taken is below):
//   scale  = amax_i |x_i| / 448          (fp32, correctly rounded; 1 if amax = 0)
//   code_i = E4M3 nearest to x_i / scale (fp32 quotient, ties to even code,
//                                         saturating at +-448)
// The row means scale * value(code).
//
// quantize_kernel: one wave per row; lane l holds 16-byte chunks l and l + 64
// (8 bf16 values each), the row maximum is a wave reduction, each chunk's 8
// codes leave as one 8-byte store.
#include "fp8.h"

namespace sa {

constexpr int kQzWaves = 4;

__global__ __launch_bounds__(kQzWaves * 64) void quantize_kernel(const uint16_t* __restrict__ src, int64_t n_rows,
                                                                  int d, const int64_t* __restrict__ dst_rows,
                                                                  uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int64_t r = (int64_t)blockIdx.x * kQzWaves + (threadIdx.x >> 6);
  if (r >= n_rows) return;                      // whole waves leave together
  const int lane = threadIdx.x & 63;
  const int n_chunk = d / 8;
  const uint16_t* row = src + r * d;
  u32x4 v[2];
  float amax = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = lane + 64 * h;
    v[h] = c < n_chunk ? ld16(row + 8 * c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax = fmaxf(amax, fabsf(__uint_as_float(v[h][i] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(v[h][i] & 0xffff0000u)));
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
  const int64_t out = dst_rows ? dst_rows[r] : r;
  if (lane == 0) scales[out] = scale;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = lane + 64 * h;
    if (c >= n_chunk) continue;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = f32_to_e4m3(__uint_as_float(v[h][i] << 16) / scale);
      const uint32_t hi = f32_to_e4m3(__uint_as_float(v[h][i] & 0xffff0000u) / scale);
      w[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
    }
    *reinterpret_cast<u32x2*>(codes + out * d + 8 * c) = u32x2{w[0], w[1]};
  }
}

// codes [n] -> bf16 values [n] (unscaled), 16 codes per thread.
__global__ void fp8_decode_kernel(const uint8_t* __restrict__ codes, int64_t n16, uint16_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x) {
    u32x4 lo, hi;
    e4m3x16_to_bf16x16(ld16(codes + 16 * i), lo, hi);
    *reinterpret_cast<u32x4*>(out + 16 * i) = lo;
    *reinterpret_cast<u32x4*>(out + 16 * i + 8) = hi;
  }
}

}  // namespace sa

namespace sa_host {

int32_t launch_quantize(const void* src, int64_t n_rows, int32_t d, const int64_t* dst_rows, void* codes, float* scales,
                        hipStream_t stream) {
  const int64_t grid = (n_rows + sa::kQzWaves - 1) / sa::kQzWaves;
  if (grid > 0x7fffffff) {
    set_error("quantize: grid too large");
    return SA_ERR_UNSUPPORTED;
  }
  hipLaunchKernelGGL(sa::quantize_kernel, dim3((unsigned)grid), dim3(sa::kQzWaves * 64), 0, stream,
                     (const uint16_t*)src, n_rows, d, dst_rows, (uint8_t*)codes, scales);
  return check_launch("quantize_kernel");
}

int32_t launch_fp8_decode(const void* codes, int64_t n, void* out, hipStream_t stream) {
  const int64_t n16 = n / 16;
  const int64_t g = (n16 + 255) / 256;
  hipLaunchKernelGGL(sa::fp8_decode_kernel, dim3((unsigned)(g < 1 ? 1 : (g > 4096 ? 4096 : g))), dim3(256), 0, stream,
                     (const uint8_t*)codes, n16, (uint16_t*)out);
  return check_launch("fp8_decode_kernel");
}

}  // namespace sa_host
