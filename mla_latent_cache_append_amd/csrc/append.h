// Append of one new token per wave into the paged latent cache, bf16 or
// FP8 rows: the bodies of the append kernels, also run by the fused
// append + absorb kernel. Token j is handled by one whole wavefront.
#pragma once

#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace mla {

// Row [c_kv | RoPE(k_pe)] of token j ([AUDIT] = llm-atlas page "DeepSeek MLA
// 吸收式缓存：真实权重执行与 FlashMLA 架构边界", §2.4: 512 latent + 64 decoupled
// rope key): lanes copy the 1,024-byte latent with one 16-byte load and store
// each; lanes 0..31 rotate the 32 rope pairs.
__device__ __forceinline__ void append_token(int j,
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const int32_t* __restrict__ pos, const int64_t* __restrict__ slot_mapping,
    uint16_t* __restrict__ pool, int64_t num_slots, int T, RopeFreqs fr) {
  const int lane = threadIdx.x & 63;
  if (j >= T) return;
  // every load is issued before the slot is known; the rotation overlaps
  // the slot's arrival
  const int64_t slot = slot_mapping[j];
  const u32x4 lat = *(const u32x4*)(c_kv + (int64_t)j * D_C + lane * 8);
  const int rl = lane & (D_ROPE / 2 - 1);
  const uint32_t x = *(const uint32_t*)(k_pe + (int64_t)j * D_ROPE + 2 * rl);
  const uint32_t y = rope_pair_bf16(x, pos[j], fr.f[rl]);
  if (slot < 0 || slot >= num_slots) return;  // outside the pool: no write
  uint16_t* row = pool + slot * D_K;
  *(u32x4*)(row + lane * 8) = lat;
  if (lane < D_ROPE / 2) *(uint32_t*)(row + D_C + 2 * lane) = y;
}

// Two-buffer layout ([AUDIT] §0 and §4.2: V3's absorbed decode writes the
// latent into kv_cache [B][max_seq][512] and the rotated rope key into
// pe_cache [B][max_seq][64] at [sequence][position]): the same row split in
// two, token j to [seq_idx[j]][pos[j]]. A sequence index outside [0, B) or a
// position outside [0, max_seq) skips the token.
__device__ __forceinline__ void append_token_kvpe(int j,
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ seq_idx,
    uint16_t* __restrict__ kv_cache, uint16_t* __restrict__ pe_cache, int B, int max_seq, int T, RopeFreqs fr) {
  const int lane = threadIdx.x & 63;
  if (j >= T) return;
  const int b = seq_idx[j], p = pos[j];
  const u32x4 lat = *(const u32x4*)(c_kv + (int64_t)j * D_C + lane * 8);
  const int rl = lane & (D_ROPE / 2 - 1);
  const uint32_t x = *(const uint32_t*)(k_pe + (int64_t)j * D_ROPE + 2 * rl);
  const uint32_t y = rope_pair_bf16(x, p, fr.f[rl]);
  if (b < 0 || b >= B || p < 0 || p >= max_seq) return;   // outside the caches: no write
  const int64_t row = (int64_t)b * max_seq + p;
  *(u32x4*)(kv_cache + row * D_C + lane * 8) = lat;
  if (lane < D_ROPE / 2) *(uint32_t*)(pe_cache + row * D_ROPE + 2 * lane) = y;
}

// fp32 -> E4M3 ("e4m3fn": exponent bias 7, 3 mantissa bits, largest finite
// 448, 0x7f NaN), nearest value with ties to the even mantissa, magnitudes
// above 448 saturated. Normal range (|u| >= 2^-6): round the fp32 mantissa
// to 3 bits in place (add 2^19 - 1 plus the kept lsb, clear 20 bits) and
// re-bias the exponent; a carry into the next binade is handled by the add.
// Below 2^-6 the grid step is 2^-9: u * 2^9 (exact) rounded to an integer
// (0..8; 8 is the code of 2^-6).
__device__ __forceinline__ uint32_t f32_to_e4m3(float u) {
  const uint32_t sign = (__float_as_uint(u) >> 24) & 0x80u;
  if (u != u) return 0x7Fu;
  const float a = fminf(fabsf(u), 448.f);
  uint32_t code;
  if (a >= 0x1p-6f) {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    code = ((((b >> 23) & 0xFFu) - 127u + 7u) << 3) | ((b >> 20) & 7u);
  } else {
    code = (uint32_t)__builtin_rintf(a * 512.f);
  }
  return sign | code;
}

// Token scale of the FP8 cache: the smallest power of two 2^k with
// amax / 2^k <= 448, k >= -124, 1 for amax = 0. With amax = 1.m 2^(eb-127):
// amax / 2^(eb-135) = 1.m * 256 is at most 448 while 1.m <= 1.75 (mantissa
// bits <= 0x600000), else one more power of two (one fewer always gives
// 1.m * 512 > 448). A subnormal amax gets the floor 2^-124. Every code
// times such a scale is a bf16 value, exactly.
__device__ __forceinline__ float fp8_token_scale(float amax) {
  if (!(amax > 0.f)) return 1.f;
  const uint32_t b = __float_as_uint(amax);
  const int eb = (int)((b >> 23) & 0xFFu);
  const int k = max(-124, eb - 135 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0));
  return __uint_as_float((uint32_t)(k + 127) << 23);
}

// One wave per token, as cache_append_kernel: lane l holds latent elements
// 8l..8l+7, lanes 0..31 also rope pair l; the row's absmax is a wave max.
__device__ __forceinline__ void append_token_fp8(int j,
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const int32_t* __restrict__ pos, const int64_t* __restrict__ slot_mapping,
    uint8_t* __restrict__ pool8, float* __restrict__ pool_scale, int64_t num_slots, int T, RopeFreqs fr) {
  const int lane = threadIdx.x & 63;
  if (j >= T) return;
  const int64_t slot = slot_mapping[j];
  const u32x4 lat = *(const u32x4*)(c_kv + (int64_t)j * D_C + lane * 8);
  const int rl = lane & (D_ROPE / 2 - 1);
  const uint32_t x = *(const uint32_t*)(k_pe + (int64_t)j * D_ROPE + 2 * rl);
  double c, s;
  rope_cos_sin(pos[j], fr.f[rl], c, s);
  float r0, r1;
  rope_rotate_f32(x, c, s, r0, r1);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32((uint16_t)(lat[i] & 0xffffu));
    v[2 * i + 1] = bf16_to_f32((uint16_t)(lat[i] >> 16));
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  if (lane < D_ROPE / 2) amax = fmaxf(amax, fmaxf(fabsf(r0), fabsf(r1)));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = fp8_token_scale(amax);
  if (slot < 0 || slot >= num_slots) return;  // outside the pool: no write
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= f32_to_e4m3(__fdiv_rn(v[i], scale)) << (8 * i);
    hi |= f32_to_e4m3(__fdiv_rn(v[4 + i], scale)) << (8 * i);
  }
  uint8_t* row = pool8 + slot * D_K;
  *(u32x2*)(row + lane * 8) = u32x2{lo, hi};
  if (lane < D_ROPE / 2) {
    const uint32_t pr = f32_to_e4m3(__fdiv_rn(r0, scale)) | (f32_to_e4m3(__fdiv_rn(r1, scale)) << 8);
    *(uint16_t*)(row + D_C + 2 * lane) = (uint16_t)pr;
  }
  if (lane == 0) pool_scale[slot] = scale;
}

}  // namespace mla
