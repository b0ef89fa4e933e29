// RoPE on one interleaved pair, fp64 angle and rotation, one rounding to bf16.
//
// Pair i of a 64-wide rope vector, (x[2i], x[2i+1]), at absolute position p is
// rotated by theta_i = p * base^(-2i/64): y[2i] = x[2i] cos - x[2i+1] sin,
// y[2i+1] = x[2i+1] cos + x[2i] sin ([MLA80] = CSDN page "80 行 PyTorch 从零写
// DeepSeek 的 MLA", appendix A: build_rope / rotate_half / apply_rope pair the
// even and odd elements and share one frequency per pair).
//
// The angle reaches 65,543 rad at the longest contexts; an fp32 angle would
// carry an error of ~4e-3 rad there, so the angle, its reduction and the
// rotation run in fp64 and only the result is rounded.
#pragma once

#include <cmath>

#include "common.h"

namespace mla {

// Rotation frequencies base^(-2i/64) of the 32 pairs, computed on the host in
// fp64 and passed to the kernels by value.
struct RopeFreqs {
  double f[D_ROPE / 2];
};

inline RopeFreqs rope_freqs(double base) {
  RopeFreqs r;
  for (int i = 0; i < D_ROPE / 2; ++i) r.f[i] = std::pow(base, -(2.0 * i) / (double)D_ROPE);
  return r;
}

// sin and cos of x in fp64, |x| < 2^21 (the angles here stay below 2^17).
//  * Reduction after Cody and Waite: k = x 2/pi rounded to an integer,
//    r = x - k pi/2 with pi/2 = P1 + P2 + P3, where P1 and P2 carry at most
//    32 significant bits, so k P1 and k P2 are exact and the two leading
//    subtractions lose nothing; |r| <= pi/4 (plus rounding).
//  * sin r and cos r from their Taylor series about 0 through r^21 and r^22
//    (the first omitted terms are below 2^-80 on |r| <= pi/4), evaluated by
//    Horner's rule in r^2; coefficients are (-1)^n / (2n+1)! and
//    (-1)^n / (2n)! rounded to double.
//  * The quadrant k mod 4 swaps and negates: x = k pi/2 + r.
__device__ __forceinline__ void sincos_f64(double x, double& s, double& c) {
  constexpr double TWO_OVER_PI = 0x1.45f306dc9c883p-1;
  constexpr double P1 = 0x1.921fb544p+0;
  constexpr double P2 = 0x1.0b4611a6p-34;
  constexpr double P3 = 0x1.3198a2e037073p-69;
  const double kd = __builtin_rint(x * TWO_OVER_PI);
  double r = __builtin_fma(-kd, P1, x);
  r = __builtin_fma(-kd, P2, r);
  r = __builtin_fma(-kd, P3, r);
  const double r2 = r * r;
  // sin r = r + r r2 (S1 + r2 (S2 + ... + r2 S10)),  S_n = (-1)^n / (2n+1)!
  double ps = 1.9572941063391263e-20;
  ps = __builtin_fma(ps, r2, -8.22063524662433e-18);
  ps = __builtin_fma(ps, r2, 2.8114572543455206e-15);
  ps = __builtin_fma(ps, r2, -7.647163731819816e-13);
  ps = __builtin_fma(ps, r2, 1.6059043836821613e-10);
  ps = __builtin_fma(ps, r2, -2.505210838544172e-08);
  ps = __builtin_fma(ps, r2, 2.7557319223985893e-06);
  ps = __builtin_fma(ps, r2, -0.0001984126984126984);
  ps = __builtin_fma(ps, r2, 0.008333333333333333);
  ps = __builtin_fma(ps, r2, -0.16666666666666666);
  const double sr = __builtin_fma(r * r2, ps, r);
  // cos r = 1 + r2 (C1 + r2 (C2 + ... + r2 C11)),  C_n = (-1)^n / (2n)!
  double pc = -8.896791392450574e-22;
  pc = __builtin_fma(pc, r2, 4.110317623312165e-19);
  pc = __builtin_fma(pc, r2, -1.5619206968586225e-16);
  pc = __builtin_fma(pc, r2, 4.779477332387385e-14);
  pc = __builtin_fma(pc, r2, -1.1470745597729725e-11);
  pc = __builtin_fma(pc, r2, 2.08767569878681e-09);
  pc = __builtin_fma(pc, r2, -2.755731922398589e-07);
  pc = __builtin_fma(pc, r2, 2.48015873015873e-05);
  pc = __builtin_fma(pc, r2, -0.001388888888888889);
  pc = __builtin_fma(pc, r2, 0.041666666666666664);
  pc = __builtin_fma(pc, r2, -0.5);
  const double cr = __builtin_fma(r2, pc, 1.0);
  const int q = (int)(long long)kd & 3;   // x = k pi/2 + r, quadrant k mod 4
  const double sa = (q & 1) ? cr : sr, ca = (q & 1) ? sr : cr;
  s = (q & 2) ? -sa : sa;
  c = ((q + 1) & 2) ? -ca : ca;
}

// (cos, sin) of theta_i = pos * base^(-2i/64), fp64; inv_freq = base^(-2i/64).
__device__ __forceinline__ void rope_cos_sin(int pos, double inv_freq, double& c, double& s) {
  sincos_f64((double)pos * inv_freq, s, c);
}

// Rotate the bf16 pair packed in x_pair by (c, s); one rounding to bf16 each.
__device__ __forceinline__ uint32_t rope_rotate_bf16(uint32_t x_pair, double c, double s) {
  const double x0 = (double)bf16_to_f32((uint16_t)(x_pair & 0xffffu));
  const double x1 = (double)bf16_to_f32((uint16_t)(x_pair >> 16));
  const double y0 = x0 * c - x1 * s;
  const double y1 = x1 * c + x0 * s;
  return (uint32_t)f64_to_bf16(y0) | ((uint32_t)f64_to_bf16(y1) << 16);
}

// Rotate the bf16 pair packed in x_pair by (c, s); one rounding to fp32 each
// (the precision the FP8 quantizer starts from).
__device__ __forceinline__ void rope_rotate_f32(uint32_t x_pair, double c, double s, float& y0, float& y1) {
  const double x0 = (double)bf16_to_f32((uint16_t)(x_pair & 0xffffu));
  const double x1 = (double)bf16_to_f32((uint16_t)(x_pair >> 16));
  y0 = (float)(x0 * c - x1 * s);
  y1 = (float)(x1 * c + x0 * s);
}

__device__ __forceinline__ uint32_t rope_pair_bf16(uint32_t x_pair, int pos, double inv_freq) {
  double c, s;
  rope_cos_sin(pos, inv_freq, c, s);
  return rope_rotate_bf16(x_pair, c, s);
}

}  // namespace mla
