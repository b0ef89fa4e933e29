// Measurement probes for bench.py: what this GPU reaches on a plain stream
// read and on a back-to-back bf16 MFMA loop, reported next to the datasheet
// peaks. Not part of the decode path; built into its own library
// (libmla_probe.so) so that the decode library holds only the hot path.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Grid-stride read of n 16-byte words, eight loads in flight per thread; the
// XOR of everything read is stored only if it equals `magic` (never, for the
// buffers bench.py passes), so the loads cannot be dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n, u32x4* out,
                                                          uint32_t magic) {
  constexpr int U = 8;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * 256 * U;
  for (size_t base = (size_t)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
    u32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const size_t i = base + (size_t)k * 256;
      v[k] = i < n ? p[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= v[k];
  }
  if (acc.x == magic) out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Four independent chains of v_mfma_f32_32x32x16_bf16 per wave, `iters`
// rounds; one float per thread is stored only if it equals `magic`.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* out, float magic) {
  const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{threadIdx.x, 1u, 2u, 3u});
  const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{4u, 5u, threadIdx.x, 7u});
  f32x16 d0 = {}, d1 = {}, d2 = {}, d3 = {};
  for (int it = 0; it < iters; ++it) {
    d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d1, 0, 0, 0);
    d2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d2, 0, 0, 0);
    d3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d3, 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += d0[i] + d1[i] + d2[i] + d3[i];
  if (r == magic) out[(size_t)blockIdx.x * 256 + threadIdx.x] = r;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from device buffer `p`; `out` is a device
// buffer of at least 2048 * 256 * 16 bytes. Returns a hipError_t code.
int mla_probe_stream_read(const void* p, size_t bytes, void* out, void* stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(2048), dim3(256), 0, (hipStream_t)stream, (const u32x4*)p,
                     bytes / 16, (u32x4*)out, 0x9e3779b9u);
  return (int)hipGetLastError();
}

// `waves4` workgroups of 4 waves, each wave 4 * iters MFMAs of 32x32x16
// (32,768 flops each); `out` holds waves4 * 256 floats. Returns a hipError_t code.
int mla_probe_mfma(int waves4, int iters, void* out, void* stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(waves4), dim3(256), 0, (hipStream_t)stream, iters, (float*)out,
                     12345.678f);
  return (int)hipGetLastError();
}

}  // extern "C"
