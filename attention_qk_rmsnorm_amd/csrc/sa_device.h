// sa_device.h -- small device helpers shared by the kernels of libsinkattn.
#pragma once

#include "sa_internal.h"

namespace sa {

// Document holding token t: the largest n < D with cu[n] <= t, for 0 <= t < T.
// Empty documents (cu[n] == cu[n+1]) are skipped because the search keeps the
// last index whose start is <= t.
__device__ inline int doc_of_token(const int32_t* __restrict__ cu, int D, int t) {
  int lo = 0, hi = D - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// sin and cos of the NeoX RoPE angle p * inv_freq (flint.layers,
// FlintAttention._apply_rope).  The product is formed and reduced modulo 2*pi
// in fp64 so positions up to 2^31 keep a fp32-accurate angle; the reduced
// angle then goes through the accurate fp32 sincos.
__device__ inline void rope_sincos(int p, double inv_freq, float* s, float* c) {
  const double two_pi = 6.283185307179586476925286766559;
  const double inv_two_pi = 0.15915494309189533576888376337251;
  double ang = (double)p * inv_freq;
  ang -= two_pi * rint(ang * inv_two_pi);
  sincosf((float)ang, s, c);
}

// sin and cos of the RoPE angle for the bf16 paths: the angle is carried in
// revolutions (p * inv_freq / 2pi), reduced to [-1/2, 1/2] in fp64, and fed
// to v_sin_f32 / v_cos_f32, which take revolutions.  Their error (~1e-6) is far
// below the bf16 rounding the rotated vector gets next.
__device__ inline void rope_sincos_rev(int p, double inv_freq_rev, float* s, float* c) {
  double r = (double)p * inv_freq_rev;
  r -= rint(r);
  const float rf = (float)r;
  *s = __builtin_amdgcn_sinf(rf);
  *c = __builtin_amdgcn_cosf(rf);
}

}  // namespace sa
