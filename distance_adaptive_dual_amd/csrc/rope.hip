// RoPE angle tables.
//
// Eq. (3) of "Dual Dimensionality for Local and Global Attention" rotates
// every key (and, read with Eq. (4), every query) at its own position.  The
// page fixes neither the pairing nor the base; the library uses rotate-half
// pairs (t, t + d_k/2) with theta_t = base^(-2t/d_k).
//
// At position 32k an fp32 product p * theta_t already carries ~4e-3 rad of
// error, so angles are formed in fp64 and split in two: cos/sin of
// (64*a) * theta_t and of b * theta_t (b < 64).  Kernels combine one entry of
// each with a complex multiply (error ~2 ulp of fp32).
#include <cmath>

#include "dar_common.hpp"

namespace dar {

// theta_t = 2^(-(2t/d_k) log2(base)) with log2(base) from the host; the angle
// is reduced by 2 pi (Cody-Waite: 2 pi as the double nearest to it plus the
// double nearest to the remainder, each subtracted by one fma) before sincos,
// which then takes its short-argument path.
__global__ void rope_tables_kernel(float2* __restrict__ lo, float2* __restrict__ hi, int half,
                                   int n_hi, double log2_base) {
  constexpr double kTwoPiHi = 6.283185307179586232, kTwoPiLo = 2.4492935982947064e-16;
  constexpr double kInvTwoPi = 0.15915494309189535;
  const int total = (64 + n_hi) * half;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += gridDim.x * blockDim.x) {
    const int row = idx / half, t = idx - row * half;
    const double theta = exp2(-(double)t / (double)half * log2_base);
    double ang;
    float2* dst;
    if (row < 64) {
      ang = (double)row * theta;
      dst = lo + idx;
    } else {
      ang = (double)(64L * (row - 64)) * theta;
      dst = hi + (idx - 64 * half);
    }
    const double k = rint(ang * kInvTwoPi);
    const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));
    double s, c;
    sincos(r, &s, &c);
    *dst = make_float2((float)c, (float)s);
  }
}

size_t rope_table_bytes(int d_k, long max_pos) {
  const long n_hi = (max_pos >> 6) + 1;
  const size_t b = sizeof(float2) * (size_t)(d_k / 2) * (size_t)(64 + n_hi);
  return (b + 255) & ~(size_t)255;
}

hipError_t launch_rope_tables(float2* lo, float2* hi, int d_k, long max_pos, float base,
                              hipStream_t s) {
  const int half = d_k / 2;
  const int n_hi = (int)((max_pos >> 6) + 1);
  const int total = (64 + n_hi) * half;
  const int threads = 256;
  int blocks = (total + threads - 1) / threads;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(rope_tables_kernel, dim3(blocks), dim3(threads), 0, s, lo, hi, half, n_hi,
                     std::log2((double)base));
  return hipGetLastError();
}

}  // namespace dar
