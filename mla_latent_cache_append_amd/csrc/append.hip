// mla_cache_append: pack [c_kv | RoPE(k_pe)] rows into the paged latent cache.
//
// One wavefront per token: 64 lanes copy the 1,024-byte latent with one
// 16-byte load and store each; lanes 0..31 rotate the 32 rope pairs. The
// write is the 576-element row the pages cache per token per layer ([AUDIT] =
// llm-atlas page "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界",
// §2.4: 512 latent + 64 decoupled rope key).
#include "common.h"
#include "kernels.h"
#include "rope.h"
#include "append.h"

namespace mla {

__global__ __launch_bounds__(256) void cache_append_kernel(
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const int32_t* __restrict__ pos, const int64_t* __restrict__ slot_mapping,
    uint16_t* __restrict__ pool, int64_t num_slots, int T, RopeFreqs fr) {
  append_token(blockIdx.x * 4 + (threadIdx.x >> 6), c_kv, k_pe, pos, slot_mapping, pool, num_slots, T, fr);
}

// ------------------------------------------------------------- FP8 cache
//
// FP8 variant of the same row ([AUDIT] §6.1 lists an FP8 KV cache for the
// 576-wide MQA-mode kernels; the scale scheme is not given there). Each
// token's row v = [c_kv | RoPE(k_pe)] in fp32 (the latent exactly, the rope
// part rounded once from fp64) is stored as E4M3 codes of v / scale, the
// division IEEE fp32, with scale the smallest power of two that brings
// max|v| within 448 (see fp8_token_scale).

__global__ __launch_bounds__(256) void cache_append_fp8_kernel(
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const int32_t* __restrict__ pos, const int64_t* __restrict__ slot_mapping,
    uint8_t* __restrict__ pool8, float* __restrict__ pool_scale, int64_t num_slots, int T, RopeFreqs fr) {
  append_token_fp8(blockIdx.x * 4 + (threadIdx.x >> 6), c_kv, k_pe, pos, slot_mapping, pool8, pool_scale,
                   num_slots, T, fr);
}

hipError_t launch_cache_append_fp8(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* pos,
                                   const int64_t* slot_mapping, uint8_t* pool8, float* pool_scale,
                                   int64_t num_blocks, int32_t T, double rope_base, hipStream_t stream) {
  const int grid = (T + 3) / 4;
  hipLaunchKernelGGL(cache_append_fp8_kernel, dim3(grid), dim3(256), 0, stream, c_kv, k_pe, pos,
                     slot_mapping, pool8, pool_scale, num_blocks * BLOCK, T, rope_freqs(rope_base));
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void cache_append_kvpe_kernel(
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ seq_idx,
    uint16_t* __restrict__ kv_cache, uint16_t* __restrict__ pe_cache, int B, int max_seq, int T, RopeFreqs fr) {
  append_token_kvpe(blockIdx.x * 4 + (threadIdx.x >> 6), c_kv, k_pe, pos, seq_idx, kv_cache, pe_cache, B,
                    max_seq, T, fr);
}

hipError_t launch_cache_append_kvpe(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* pos,
                                    const int32_t* seq_idx, uint16_t* kv_cache, uint16_t* pe_cache, int32_t B,
                                    int32_t max_seq, int32_t T, double rope_base, hipStream_t stream) {
  const int grid = (T + 3) / 4;
  hipLaunchKernelGGL(cache_append_kvpe_kernel, dim3(grid), dim3(256), 0, stream, c_kv, k_pe, pos, seq_idx,
                     kv_cache, pe_cache, B, max_seq, T, rope_freqs(rope_base));
  return hipGetLastError();
}

hipError_t launch_cache_append(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* pos,
                               const int64_t* slot_mapping, uint16_t* pool, int64_t num_blocks,
                               int32_t T, double rope_base, hipStream_t stream) {
  const int grid = (T + 3) / 4;
  hipLaunchKernelGGL(cache_append_kernel, dim3(grid), dim3(256), 0, stream, c_kv, k_pe, pos,
                     slot_mapping, pool, num_blocks * BLOCK, T, rope_freqs(rope_base));
  return hipGetLastError();
}

}  // namespace mla
