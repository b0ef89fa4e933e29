// Device-side helpers shared by the libmla_absorb kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned int))));
typedef unsigned int u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned int))));

typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950 converts in
// hardware (v_cvt_pk_bf16_f32), two values per instruction, without branches.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// fp64 -> bf16 with a single rounding (nearest even) for normal-range values:
// round the 52-bit mantissa to 7 bits in the double itself, after which the
// value is exact in fp32 and its top 16 bits are the bf16 pattern.
__device__ __forceinline__ uint16_t f64_to_bf16(double d) {
  uint64_t u = (uint64_t)__double_as_longlong(d);
  if ((u & 0x7fffffffffffffffull) > 0x7ff0000000000000ull) return 0x7fc0u;
  const uint64_t lsb = (u >> 45) & 1ull;
  u += 0x00000fffffffffffull + lsb;
  u &= ~((1ull << 45) - 1ull);
  const float f = (float)__longlong_as_double((long long)u);
  return (uint16_t)(__float_as_uint(f) >> 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- MFMA
//
// v_mfma_f32_16x16x32_bf16, lane l, g = l / 16, c = l % 16:
//   A (16x32, MxK): a[j] = A[c][8g + j]      j = 0..7
//   B (32x16, KxN): b[j] = B[8g + j][c]
//   D (16x16):      d[i] = D[4g + i][c]      i = 0..3
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- LDS

// 16 bytes from LDS at a byte offset of an LDS base pointer.
__device__ __forceinline__ u32x4 lds_read_b128(const __attribute__((address_space(3))) char* base,
                                               uint32_t off) {
  return *(const __attribute__((address_space(3))) u32x4*)(base + off);
}

// Transposing 64-bit LDS read (ds_read_b64_tr_b16). Within each group of 16
// lanes, lane i supplies the address of 4 consecutive 16-bit elements; lane n
// of the group receives element n % 4 of the loads of lanes n / 4, 4 + n / 4,
// 8 + n / 4 and 12 + n / 4. With lane i loading row i / 4, columns 4 (i % 4)
// .. +3 of a row-major [row][16 col] block, lane n receives column n of rows
// 0..3: the transpose an MFMA operand needs when its K dimension is the
// row-major one.
__device__ __forceinline__ i16x4 lds_read_tr16_b64(const __attribute__((address_space(3))) char* base,
                                                   uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + off));
}

// Two transposing reads (4 rows each) joined into one 8-element MFMA operand.
__device__ __forceinline__ bf16x8 join_tr(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Buffer resource (V#) for raw 16-byte loads of `bytes` bytes at `base`:
// lanes whose offset + 16 exceeds `bytes` read zeros.
typedef unsigned int sgpr_x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ sgpr_x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return sgpr_x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, bytes, 0x00020000u};
}

// Buffer -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane
// l reads rsrc + voff + soff and its 16 bytes land at LDS byte address
// lds_wave_base + 16 l (lds_wave_base is wave-uniform, taken from M0).
//
// The copies are marked non-temporal (nt): every cache tile is read once per
// call, so they should not displace what the caches hold for later reads.
// Issued as inline asm on purpose: the compiler's wait-count pass cannot tell
// these LDS writes apart from the transposing LDS reads (ds_read_b64_tr_b16)
// and would drain every load in flight before each such read. The kernels
// order these copies themselves: s_waitcnt vmcnt(N) for the stage about to
// be read, then a barrier. M0 is set right before each copy; no compiled code
// in these kernels reads M0.
__device__ __forceinline__ void buffer_load_lds_16(sgpr_x4 rsrc, uint32_t voff, uint32_t soff,
                                                   uint32_t lds_wave_base) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen nt lds"
      :
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_wave_base)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const __attribute__((address_space(3))) void* p) {
  return (uint32_t)(uintptr_t)p;
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier for LDS traffic only: this wave's LDS writes complete,
// then s_barrier. Unlike __syncthreads() it does not wait for outstanding
// global / buffer loads, so tile loads stay in flight across it. (Data that
// buffer-to-LDS loads deliver is waited for separately with vmcnt.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace mla
