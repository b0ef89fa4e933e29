// The projections around the attention, as plain bias-free linear maps
// y = x W^T (+ r) on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate).
//
// Source: [MLA80] = CSDN page "80 行 PyTorch 从零写 DeepSeek 的 MLA", §2: the
// layer's Wdq, Wuq, Wqr, Wdkv, Wkr and Wo are nn.Linear(bias=False) maps,
// weight stored [out][in]. The optional residual r serves a stack of layers
// (the stream a layer read plus what it returns).
//
// Decode multiplies a few tokens by a large weight, so the kernel is built
// to stream the weight once: a workgroup owns 16 output features x 32 tokens
// and its four waves split the contraction four ways (each wave a quarter of
// the input features), adding their partial sums through the LDS at the end.
// The output is computed transposed, y^T = W x^T, so that each lane's result
// is four consecutive features of one token: an 8-byte store.
#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int LIN_M = 16;   // output features per workgroup
constexpr int LIN_N = 32;   // tokens per workgroup (two 16-token MFMA tiles)

// x [N][K], w [M][K], r and y [N][M], all bf16. K is a multiple of 32 and M
// of 4. Rows past the last feature or token load a valid row (clamped); their
// results are not stored.
__global__ __launch_bounds__(256) void linear_kernel(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ w,
                                                     const uint16_t* r, uint16_t* y, int N, int K,
                                                     int M) {
  __shared__ float part[3][8][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int m0 = blockIdx.x * LIN_M, n0 = blockIdx.y * LIN_N;
  // A = W rows m0 + c, features 32 s + 8 g .. +7; B = x^T of tokens n0 + 16 t + c
  const uint16_t* wa = w + (int64_t)min(m0 + c, M - 1) * K + 8 * g;
  const uint16_t* xb0 = x + (int64_t)min(n0 + c, N - 1) * K + 8 * g;
  const uint16_t* xb1 = x + (int64_t)min(n0 + 16 + c, N - 1) * K + 8 * g;
  const int S = K / 32;
  const int s0 = (int)((int64_t)wave * S / 4), s1 = (int)((int64_t)(wave + 1) * S / 4);
  // two accumulators per token tile, alternating, so consecutive MFMAs do
  // not wait on each other's results
  f32x4 acc[2][2] = {};
  int s = s0;
  for (; s + 4 <= s1; s += 4) {
    u32x4 a[4], b0[4], b1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = *(const u32x4*)(wa + 32 * (s + u));
      b0[u] = *(const u32x4*)(xb0 + 32 * (s + u));
      b1[u] = *(const u32x4*)(xb1 + 32 * (s + u));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[0][u & 1] = mfma16x16x32(as_bf16x8(a[u]), as_bf16x8(b0[u]), acc[0][u & 1]);
      acc[1][u & 1] = mfma16x16x32(as_bf16x8(a[u]), as_bf16x8(b1[u]), acc[1][u & 1]);
    }
  }
  for (; s < s1; ++s) {
    const u32x4 a = *(const u32x4*)(wa + 32 * s);
    acc[0][0] = mfma16x16x32(as_bf16x8(a), as_bf16x8(*(const u32x4*)(xb0 + 32 * s)), acc[0][0]);
    acc[1][0] = mfma16x16x32(as_bf16x8(a), as_bf16x8(*(const u32x4*)(xb1 + 32 * s)), acc[1][0]);
  }
  f32x4 v[2] = {acc[0][0] + acc[0][1], acc[1][0] + acc[1][1]};
  // waves 1..3 hand their partial sums to wave 0 (slot [wave-1][t*4+i][lane])
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wave - 1][4 * t + i][lane] = v[t][i];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[t][i] += part[0][4 * t + i][lane] + part[1][4 * t + i][lane] + part[2][4 * t + i][lane];
    const int n = n0 + 16 * t + c, m = m0 + 4 * g;
    if (n >= N || m >= M) continue;
    const int64_t off = (int64_t)n * M + m;
    float o0 = v[t][0], o1 = v[t][1], o2 = v[t][2], o3 = v[t][3];
    if (r) {
      const u32x2 rv = *(const u32x2*)(r + off);
      o0 += bf16_to_f32((uint16_t)(rv[0] & 0xffffu));
      o1 += bf16_to_f32((uint16_t)(rv[0] >> 16));
      o2 += bf16_to_f32((uint16_t)(rv[1] & 0xffffu));
      o3 += bf16_to_f32((uint16_t)(rv[1] >> 16));
    }
    *(u32x2*)(y + off) = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
  }
}

hipError_t launch_linear(const uint16_t* x, const uint16_t* w, const uint16_t* r, uint16_t* y,
                         int32_t N, int32_t K, int32_t M, hipStream_t stream) {
  const dim3 grid((unsigned)((M + LIN_M - 1) / LIN_M), (unsigned)((N + LIN_N - 1) / LIN_N));
  hipLaunchKernelGGL(linear_kernel, grid, dim3(256), 0, stream, x, w, r, y, N, K, M);
  return hipGetLastError();
}

}  // namespace mla
