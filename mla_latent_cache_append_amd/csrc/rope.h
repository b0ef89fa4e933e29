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

#include "common.h"

namespace mla {

// (cos, sin) of theta_i = pos * base^(-2i/64), fp64.
__device__ __forceinline__ void rope_cos_sin(int pos, int i, double base, double& c, double& s) {
  const double theta = (double)pos * pow(base, -2.0 * (double)i / (double)D_ROPE);
  sincos(theta, &s, &c);
}

// Rotate the bf16 pair packed in x_pair by (c, s); one rounding to bf16 each.
__device__ __forceinline__ uint32_t rope_rotate_bf16(uint32_t x_pair, double c, double s) {
  const double x0 = (double)bf16_to_f32((uint16_t)(x_pair & 0xffffu));
  const double x1 = (double)bf16_to_f32((uint16_t)(x_pair >> 16));
  const double y0 = x0 * c - x1 * s;
  const double y1 = x1 * c + x0 * s;
  return (uint32_t)f64_to_bf16(y0) | ((uint32_t)f64_to_bf16(y1) << 16);
}

__device__ __forceinline__ uint32_t rope_pair_bf16(uint32_t x_pair, int pos, int i, double base) {
  double c, s;
  rope_cos_sin(pos, i, base, c, s);
  return rope_rotate_bf16(x_pair, c, s);
}

}  // namespace mla
