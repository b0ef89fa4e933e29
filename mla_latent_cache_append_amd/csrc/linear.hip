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
// and its sixteen waves take the 32-wide contraction steps in turn (wave w
// steps w, w + 16, ...; the loads of four steps in flight per wave), so that
// at any moment the workgroup reads one contiguous window of each weight
// row. The sixteen partial sums meet in the LDS and 256 threads add them up.
// The output is computed transposed, y^T = W x^T: lane results are
// consecutive features of one token.
#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int LIN_M = 16;      // output features per workgroup
constexpr int LIN_N = 32;      // tokens per workgroup (two 16-token MFMA tiles)
constexpr int LIN_WAVES = 16;  // waves per workgroup, each a slice of the contraction
constexpr int LIN_U = 4;       // steps per wave whose loads are in flight together

// x [N][K], w [M][K], r and y [N][M], all bf16. K is a multiple of 32 and M
// of 4. Rows past the last feature or token load a valid row (clamped); their
// results are not stored.
__global__ __launch_bounds__(64 * LIN_WAVES) void linear_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w,
                                                                const uint16_t* r, uint16_t* y, int N,
                                                                int K, int M) {
  __shared__ float part[LIN_WAVES][8][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int m0 = blockIdx.x * LIN_M, n0 = blockIdx.y * LIN_N;
  // A = W rows m0 + c, features 32 s + 8 g .. +7; B = x^T of tokens n0 + 16 t + c
  const uint16_t* wa = w + (int64_t)min(m0 + c, M - 1) * K + 8 * g;
  const uint16_t* xb0 = x + (int64_t)min(n0 + c, N - 1) * K + 8 * g;
  const uint16_t* xb1 = x + (int64_t)min(n0 + 16 + c, N - 1) * K + 8 * g;
  const int S = K / 32;
  // two accumulators per token tile, alternating, so consecutive MFMAs do
  // not wait on each other's results
  f32x4 acc[2][2] = {};
  for (int base = wave; base < S; base += LIN_WAVES * LIN_U) {
    u32x4 a[LIN_U], b0[LIN_U], b1[LIN_U];
#pragma unroll
    for (int u = 0; u < LIN_U; ++u) {
      const int ss = min(base + LIN_WAVES * u, S - 1);   // past the end: a valid step, not accumulated
      a[u] = *(const u32x4*)(wa + 32 * ss);
      b0[u] = *(const u32x4*)(xb0 + 32 * ss);
      b1[u] = *(const u32x4*)(xb1 + 32 * ss);
    }
#pragma unroll
    for (int u = 0; u < LIN_U; ++u) {
      if (base + LIN_WAVES * u < S) {
        acc[0][u & 1] = mfma16x16x32(as_bf16x8(a[u]), as_bf16x8(b0[u]), acc[0][u & 1]);
        acc[1][u & 1] = mfma16x16x32(as_bf16x8(a[u]), as_bf16x8(b1[u]), acc[1][u & 1]);
      }
    }
  }
  // partial sums: slot [wave][t*4+i][lane] holds feature m0 + 4 (lane/16) + i
  // of token n0 + 16 t + lane % 16
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][4 * t + i][lane] = acc[t][0][i] + acc[t][1][i];
  __syncthreads();
  if (threadIdx.x >= 256) return;
  // thread (p, t, l): features i = 2p, 2p+1 of slot lane l, token tile t
  const int l = threadIdx.x & 63, t = (threadIdx.x >> 6) & 1, p = threadIdx.x >> 7;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int q = 0; q < LIN_WAVES; ++q) {
    s0 += part[q][4 * t + 2 * p][l];
    s1 += part[q][4 * t + 2 * p + 1][l];
  }
  const int n = n0 + 16 * t + (l & 15), m = m0 + 4 * (l >> 4) + 2 * p;
  if (n >= N || m >= M) return;
  const int64_t off = (int64_t)n * M + m;
  if (r) {
    const uint32_t rv = *(const uint32_t*)(r + off);
    s0 += bf16_to_f32((uint16_t)(rv & 0xffffu));
    s1 += bf16_to_f32((uint16_t)(rv >> 16));
  }
  *(uint32_t*)(y + off) = pack_bf16x2(s0, s1);
}

hipError_t launch_linear(const uint16_t* x, const uint16_t* w, const uint16_t* r, uint16_t* y,
                         int32_t N, int32_t K, int32_t M, hipStream_t stream) {
  const dim3 grid((unsigned)((M + LIN_M - 1) / LIN_M), (unsigned)((N + LIN_N - 1) / LIN_N));
  hipLaunchKernelGGL(linear_kernel, grid, dim3(64 * LIN_WAVES), 0, stream, x, w, r, y, N, K, M);
  return hipGetLastError();
}

}  // namespace mla
