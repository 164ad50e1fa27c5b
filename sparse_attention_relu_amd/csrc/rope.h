// fp64 rotary-embedding helpers shared by the kernels that turn rope pairs
// (the cache write and the query projection): interleaved pairs (2i, 2i + 1)
// turned by p * theta^(-2i / 64), theta = 8e6 (models.inteligile.com
// "GLM-5.2 / Model techniques map", rows "Partial RoPE" and "YaRN RoPE
// scaling"; llm-atlas "GLM-5.2", rope_interleave).  The angles reach 10^6 rad
// at million-token positions, where fp32 keeps no correct digit of the angle,
// so the turn is computed in fp64 after an exact reduction to [-pi, pi].
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace sa {

// sin and cos of p * f: the angle (|p f| < 2^31) less k whole turns,
// k = rint(angle / 2 pi) < 2^29, with 2 pi = C1 + C2 + C3 where C1 and C2
// have 24 significant bits, so k C1 and k C2 are exact.
__device__ __forceinline__ void turn_sincos(int p, double f, double& s, double& c) {
#pragma clang fp contract(off)
  constexpr double kC1 = 6.2831854820251465;        // float(2 pi)
  constexpr double kC2 = -1.7484555314695172e-07;   // float(2 pi - C1)
  constexpr double kC3 = -6.8604979977715316e-15;   // 2 pi - C1 - C2
  constexpr double kInv2Pi = 0.15915494309189535;
  const double a = (double)p * f;
  const double k = rint(a * kInv2Pi);
  const double r = ((a - k * kC1) - k * kC2) - k * kC3;
  sincos(r, &s, &c);
}

// Pair (x0, x1) turned by the angle with sine s and cosine c.
__device__ __forceinline__ void rope_pair(double& x0, double& x1, double s, double c) {
#pragma clang fp contract(off)
  const double y0 = x0 * c - x1 * s;
  const double y1 = x0 * s + x1 * c;
  x0 = y0;
  x1 = y1;
}

}  // namespace sa
