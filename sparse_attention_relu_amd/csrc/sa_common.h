// Shared device helpers for the gfx950 kernels of libsparse_mla.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sparse_mla.h"

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kIdxHeads = SA_INDEX_HEADS;
constexpr int kIdxDim = SA_INDEX_DIM;
constexpr int kMaxTopk = SA_MAX_TOPK;
constexpr int kHeads = SA_HEADS;
constexpr int kLatent = SA_LATENT;
constexpr int kRope = SA_ROPE;
constexpr int kRow = SA_ROW;
constexpr int kVdim = SA_VDIM;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ s16x4 as_s16x4(u32x2 v) { return __builtin_bit_cast(s16x4, v); }

// 16-byte global load (plain vector load; the compiler emits global_load_dwordx4).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// fp32 -> bf16 with round-to-nearest-even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats to packed bf16 (lo in bits 0..15) with gfx950's
// v_cvt_pk_bf16_f32: round to nearest even under the default rounding mode,
// the same result as f32_to_bf16_rne for every non-NaN input.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Order-preserving map of an fp32 score to uint32: a > b (as floats) iff
// key(a) > key(b); -0.0 is folded onto +0.0 so equal values tie.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that completes this wave's LDS instructions first but
// leaves the direct-to-LDS tile loads in flight (__syncthreads, and even an
// LDS-scoped fence, would wait for them: they are tracked as memory writes).
// Tile loads are waited for explicitly with SA_WAIT_VMCNT.  The "memory"
// clobber keeps the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Orders a wave's LDS writes before its reads of other lanes' data (and the
// reads before the next writes).  LDS-only: in-flight global loads are not
// waited for.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(n) leaving the other counters unconstrained (gfx9 encoding).
#define SA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8))

// Half-wave sums with v_permlane32_swap (a VALU exchange of the wave's two
// 32-lane halves; no LDS round trip): returns p[l] + p[l + 32] in lanes
// l < 32 and q[l - 32] + q[l] in lanes l >= 32.  With q = p every lane gets
// the sum of its lane pair.
__device__ __forceinline__ float sum_halves(float p, float q) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(q), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace sa

// Host-side error plumbing shared by the launchers.
namespace sa_host {
void set_error(const char* fmt, ...);
int32_t check_launch(const char* what);
}  // namespace sa_host
