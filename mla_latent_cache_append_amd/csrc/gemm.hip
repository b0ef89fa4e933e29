// Per-head small GEMMs on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate):
//
//   mla_absorb_q : q_lat[n,h,:] = W_UK[h]^T q_nope[n,h,:]   (K = 128 -> 512 out)
//                  plus q_r = RoPE(q_pe[n,h,:], pos[n]) packed after it (576 wide)
//   mla_out_up   : o[n,h,:]     = W_UV[h]   o_lat[n,h,:]    (K = 512 -> 128 out)
//
// Sources: [AUDIT] = llm-atlas page "DeepSeek MLA 吸收式缓存：真实权重执行与
// FlashMLA 架构边界", §2.2 (W_K moved onto the query) and §2.3 (W_V applied
// after the weighted sum); [MLA80] = CSDN page "80 行 PyTorch 从零写 DeepSeek
// 的 MLA", §5 (absorbed decode: Q_abs by einsum with W_UK, ctx_latent then W_UV).
//
// Both are computed transposed (C^T = W^T-ish x activations^T) so that each
// lane's output is four consecutive features of one token: an 8-byte store.
#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace mla {

constexpr int AQ_COLS = 64;                  // latent columns per absorb workgroup
constexpr int AQ_CHUNKS = D_C / AQ_COLS;     // 8 workgroups per head
constexpr int AQ_LDS_STRIDE = D_NOPE + 8;    // padded row of the transposed W tile

// Blocks 0..N-1 rotate q_pe (one token each, dispatched first); the others
// each compute a [N x 64] column slice of q_lat for one head.
// W_UK[h] is stored [128 j][512 c] (rows of nn.Linear(d_c, H*d_nope).weight);
// the contraction runs over j, so each workgroup stages a [128 x 64] slice
// transposed into LDS as wt[c][j], making each MFMA A fragment (8 consecutive
// j of one c) a 16-byte LDS read.
__global__ __launch_bounds__(256) void absorb_q_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const int32_t* __restrict__ pos, const uint16_t* __restrict__ w_uk,
    uint16_t* __restrict__ q_out, int N, int H, double base) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[AQ_COLS * AQ_LDS_STRIDE];
  __shared__ double rot[D_ROPE / 2][2];
  if ((int)blockIdx.x < N) {
    // rope of one query token, all heads: q_out[n][h][512 + 2i .. +1]. The 32
    // (cos, sin) pairs depend only on the position: computed once, shared by
    // every head.
    const int n = blockIdx.x;
    if (threadIdx.x < D_ROPE / 2) rope_cos_sin(pos[n], threadIdx.x, base, rot[threadIdx.x][0], rot[threadIdx.x][1]);
    __syncthreads();
    for (int k = threadIdx.x; k < H * (D_ROPE / 2); k += blockDim.x) {
      const int h = k / (D_ROPE / 2), i = k % (D_ROPE / 2);
      const int64_t rowq = (int64_t)n * H + h;
      const uint32_t x = *(const uint32_t*)(q_pe + rowq * D_ROPE + 2 * i);
      *(uint32_t*)(q_out + rowq * D_K + D_C + 2 * i) = rope_rotate_bf16(x, rot[i][0], rot[i][1]);
    }
    return;
  }
  const int gb = blockIdx.x - N;
  const int h = gb / AQ_CHUNKS;
  const int c0 = (gb % AQ_CHUNKS) * AQ_COLS;
  const uint16_t* w = w_uk + (int64_t)h * D_NOPE * D_C;
  for (int k = threadIdx.x; k < D_NOPE * (AQ_COLS / 8); k += blockDim.x) {
    const int j = k / (AQ_COLS / 8);
    const int cc = (k % (AQ_COLS / 8)) * 8;
    const u32x4 v = *(const u32x4*)(w + (int64_t)j * D_C + c0 + cc);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      wt[(cc + e) * AQ_LDS_STRIDE + j] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  // A = W^T[M = column][K = j]: this wave's 16 columns, 4 k-steps of 32.
  bf16x8 af[D_NOPE / 32];
#pragma unroll
  for (int ks = 0; ks < D_NOPE / 32; ++ks)
    af[ks] = as_bf16x8(*(const u32x4*)&wt[(16 * wave + c) * AQ_LDS_STRIDE + 32 * ks + 8 * g]);
  for (int n0 = 0; n0 < N; n0 += 16) {
    const int n = n0 + c;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D_NOPE / 32; ++ks) {
      u32x4 bv = {0u, 0u, 0u, 0u};
      if (n < N) bv = *(const u32x4*)(q_nope + ((int64_t)n * H + h) * D_NOPE + 32 * ks + 8 * g);
      acc = mfma16x16x32(af[ks], as_bf16x8(bv), acc);
    }
    if (n < N) {
      // lane holds columns c0 + 16 wave + 4g + i (i = 0..3) of token n
      u32x2 out = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *(u32x2*)(q_out + ((int64_t)n * H + h) * D_K + c0 + 16 * wave + 4 * g) = out;
    }
  }
}

constexpr int OU_ROWS = 64;                 // W_UV rows (output features) per workgroup
constexpr int OU_CHUNKS = D_V / OU_ROWS;    // 2 workgroups per head

// W_UV[h] is stored [128 j][512 c] and the contraction runs over c, which is
// the contiguous axis of both W_UV and o_lat: every fragment is a 16-byte
// global load and no LDS is needed. Each wave keeps its 16 rows of W_UV (64
// VGPRs) and sweeps the tokens.
__global__ __launch_bounds__(256) void out_up_kernel(const uint16_t* __restrict__ o_lat,
                                                     const uint16_t* __restrict__ w_uv,
                                                     uint16_t* __restrict__ o, int N, int H) {
  const int h = blockIdx.x / OU_CHUNKS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int j0 = (blockIdx.x % OU_CHUNKS) * OU_ROWS + 16 * wave;
  const uint16_t* w = w_uv + ((int64_t)h * D_V + j0 + c) * D_C;
  bf16x8 af[D_C / 32];
#pragma unroll
  for (int ks = 0; ks < D_C / 32; ++ks) af[ks] = as_bf16x8(*(const u32x4*)(w + 32 * ks + 8 * g));
  for (int n0 = 0; n0 < N; n0 += 16) {
    const int n = n0 + c;
    const uint16_t* src = o_lat + ((int64_t)n * H + h) * D_C + 8 * g;
    // four independent accumulator chains keep the MFMA pipe busy
    f32x4 acc4[4] = {};
#pragma unroll
    for (int ks = 0; ks < D_C / 32; ++ks) {
      u32x4 bv = {0u, 0u, 0u, 0u};
      if (n < N) bv = *(const u32x4*)(src + 32 * ks);
      acc4[ks & 3] = mfma16x16x32(af[ks], as_bf16x8(bv), acc4[ks & 3]);
    }
    const f32x4 acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    if (n < N) {
      u32x2 out = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *(u32x2*)(o + ((int64_t)n * H + h) * D_V + j0 + 4 * g) = out;
    }
  }
}

hipError_t launch_absorb_q(const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                           const uint16_t* w_uk, uint16_t* q_out, int32_t N, int32_t H,
                           double rope_base, hipStream_t stream) {
  hipLaunchKernelGGL(absorb_q_kernel, dim3(H * AQ_CHUNKS + N), dim3(256), 0, stream, q_nope, q_pe,
                     pos, w_uk, q_out, N, H, rope_base);
  return hipGetLastError();
}

hipError_t launch_out_up(const uint16_t* o_lat, const uint16_t* w_uv, uint16_t* o, int32_t N,
                         int32_t H, hipStream_t stream) {
  hipLaunchKernelGGL(out_up_kernel, dim3(H * OU_CHUNKS), dim3(256), 0, stream, o_lat, w_uv, o, N,
                     H);
  return hipGetLastError();
}

}  // namespace mla
