// The projections around the attention, as plain bias-free linear maps
// y = x W^T (+ r) on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate).
//
// Source: [MLA80] = CSDN page "80 行 PyTorch 从零写 DeepSeek 的 MLA", §2: the
// layer's Wdq, Wuq, Wqr, Wdkv, Wkr and Wo are nn.Linear(bias=False) maps,
// weight stored [out][in]. The optional residual r serves a stack of layers
// (the stream a layer read plus what it returns).
//
// Decode multiplies a few tokens by a large weight, so the kernel is built
// to stream the weight once: a workgroup owns 16 MT output features x 32
// tokens and its sixteen waves take the 32-wide contraction steps in turn (wave w
// steps w, w + 16, ...; the loads of four steps in flight per wave), so that
// at any moment the workgroup reads one contiguous window of each weight
// row. The sixteen partial sums meet in the LDS and 256 MT threads add them
// up. MT = 2 (two 16-feature tiles on each weight step, so each workgroup
// reads the activations once for twice the features) when that still gives
// at least 128 workgroups; MT = 1 otherwise, so that narrow maps keep more
// workgroups. Measured on Wo (7168 x 16384, 32 tokens): 62.7 us with MT = 2
// against 92.8 us with MT = 1; on 512 x 7168, MT = 1 is faster (25.8 us
// against 32.9 us).
// The output is computed transposed, y^T = W x^T: lane results are
// consecutive features of one token.
#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int LIN_N = 32;      // tokens per workgroup (two 16-token MFMA tiles)
constexpr int LIN_WAVES = 16;  // waves per workgroup, each a slice of the contraction
constexpr int LIN_U = 4;       // steps per wave whose loads are in flight together

// x [N][K], w [M][K], r and y [N][M], all bf16. K is a multiple of 32 and M
// of 4. Rows past the last feature or token load a valid row (clamped); their
// results are not stored.
template <int LIN_MT>
__global__ __launch_bounds__(64 * LIN_WAVES) void linear_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w,
                                                                const uint16_t* r, uint16_t* y, int N,
                                                                int K, int M) {
  constexpr int LIN_M = 16 * LIN_MT;   // output features per workgroup
  __shared__ float part[LIN_WAVES][8 * LIN_MT][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int m0 = blockIdx.x * LIN_M, n0 = blockIdx.y * LIN_N;
  // A = W rows m0 + 16 mt + c, features 32 s + 8 g .. +7; B = x^T of tokens n0 + 16 t + c
  const uint16_t* wa[LIN_MT];
#pragma unroll
  for (int mt = 0; mt < LIN_MT; ++mt) wa[mt] = w + (int64_t)min(m0 + 16 * mt + c, M - 1) * K + 8 * g;
  const uint16_t* xb0 = x + (int64_t)min(n0 + c, N - 1) * K + 8 * g;
  const uint16_t* xb1 = x + (int64_t)min(n0 + 16 + c, N - 1) * K + 8 * g;
  const int S = K / 32;
  // two accumulators per token tile, alternating, so consecutive MFMAs do
  // not wait on each other's results
  f32x4 acc[LIN_MT][2][2] = {};
  for (int base = wave; base < S; base += LIN_WAVES * LIN_U) {
    u32x4 a[LIN_U][LIN_MT], b0[LIN_U], b1[LIN_U];
#pragma unroll
    for (int u = 0; u < LIN_U; ++u) {
      const int ss = min(base + LIN_WAVES * u, S - 1);   // past the end: a valid step, not accumulated
#pragma unroll
      for (int mt = 0; mt < LIN_MT; ++mt) a[u][mt] = *(const u32x4*)(wa[mt] + 32 * ss);
      b0[u] = *(const u32x4*)(xb0 + 32 * ss);
      b1[u] = *(const u32x4*)(xb1 + 32 * ss);
    }
#pragma unroll
    for (int u = 0; u < LIN_U; ++u) {
      if (base + LIN_WAVES * u < S) {
#pragma unroll
        for (int mt = 0; mt < LIN_MT; ++mt) {
          acc[mt][0][u & 1] = mfma16x16x32(as_bf16x8(a[u][mt]), as_bf16x8(b0[u]), acc[mt][0][u & 1]);
          acc[mt][1][u & 1] = mfma16x16x32(as_bf16x8(a[u][mt]), as_bf16x8(b1[u]), acc[mt][1][u & 1]);
        }
      }
    }
  }
  // partial sums: slot [wave][8 mt + 4 t + i][lane] holds feature m0 + 16 mt + 4 (lane/16) + i
  // of token n0 + 16 t + lane % 16
#pragma unroll
  for (int mt = 0; mt < LIN_MT; ++mt)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wave][8 * mt + 4 * t + i][lane] = acc[mt][t][0][i] + acc[mt][t][1][i];
  __syncthreads();
  if (threadIdx.x >= 256 * LIN_MT) return;
  // thread (p, mt, t, l): features i = 2p, 2p+1 of slot lane l, feature tile mt, token tile t
  const int l = threadIdx.x & 63, t = (threadIdx.x >> 6) & 1, mt = (threadIdx.x >> 7) % LIN_MT,
            p = (threadIdx.x >> 7) / LIN_MT;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int q = 0; q < LIN_WAVES; ++q) {
    s0 += part[q][8 * mt + 4 * t + 2 * p][l];
    s1 += part[q][8 * mt + 4 * t + 2 * p + 1][l];
  }
  const int n = n0 + 16 * t + (l & 15), m = m0 + 16 * mt + 4 * (l >> 4) + 2 * p;
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
  const unsigned ny = (unsigned)((N + LIN_N - 1) / LIN_N);
  const unsigned nx2 = (unsigned)((M + 31) / 32);
  if ((int64_t)nx2 * ny >= 128) {
    hipLaunchKernelGGL(linear_kernel<2>, dim3(nx2, ny), dim3(64 * LIN_WAVES), 0, stream, x, w, r, y, N, K, M);
  } else {
    const dim3 grid((unsigned)((M + 15) / 16), ny);
    hipLaunchKernelGGL(linear_kernel<1>, grid, dim3(64 * LIN_WAVES), 0, stream, x, w, r, y, N, K, M);
  }
  return hipGetLastError();
}

}  // namespace mla
