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

namespace mla {

__global__ __launch_bounds__(256) void cache_append_kernel(
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const int32_t* __restrict__ pos, const int64_t* __restrict__ slot_mapping,
    uint16_t* __restrict__ pool, int64_t num_slots, int T, RopeFreqs fr) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
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

hipError_t launch_cache_append(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* pos,
                               const int64_t* slot_mapping, uint16_t* pool, int64_t num_blocks,
                               int32_t T, double rope_base, hipStream_t stream) {
  const int grid = (T + 3) / 4;
  hipLaunchKernelGGL(cache_append_kernel, dim3(grid), dim3(256), 0, stream, c_kv, k_pe, pos,
                     slot_mapping, pool, num_blocks * BLOCK, T, rope_freqs(rope_base));
  return hipGetLastError();
}

}  // namespace mla
