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
// tokens and its sixteen waves take contraction steps in turn, so that at
// any moment the workgroup reads one contiguous window of each weight row.
// The sixteen partial sums meet in the LDS and 256 MT threads add them up.
// Two step shapes (the MFMA contracts over any 32 indices, as long as both
// operands use the same ones):
//   narrow steps: step s covers indices 32 s .. 32 s + 31, lane group g the 8
//     at 32 s + 8 g; four steps' loads in flight per wave;
//   wide steps (K a multiple of 128, up to 8192): step s covers 128 indices,
//     lane group g reads the 64 contiguous bytes at 128 s + 32 g and feeds
//     them to four MFMAs.
// Features per workgroup (16 MT): each workgroup streams its weight rows and
// the whole activation block, at a rate per workgroup that sets the time of
// these maps, so MT = 4 (64 features: half the activation bytes per weight
// byte of MT = 2) whenever that still leaves >= 224 workgroups; otherwise
// MT = 2 for wide outputs and MT = 1 for narrow ones.
// Maps with few workgroups also split the contraction over KS workgroups
// (grid z) when the caller gives a workspace: each writes its fp32 partial
// sums, and a second kernel adds the KS slices in a fixed order, adds the
// residual and rounds once. A long contraction on narrow steps (K >= 8192)
// takes MT = 4 with KS = 2 when that reaches 224 workgroups.
// Measured at 32 tokens (HIP-graph replays of 20 calls, us per call; the
// first figure is narrow steps, MT = 1 or 2, unsplit):
//   Wdkv 7168 -> 512: 23.3 -> 9.1 (wide steps, MT = 1, KS = 6)
//   Wkr 7168 -> 64: 23.2 -> ~9 (wide steps, MT = 1, KS = 18)
//   Wdq 7168 -> 1536: 23.6 -> 12.1 (wide steps, MT = 2, KS = 4)
//   Wuq 1536 -> 16384: 19.1 -> 11.8 (narrow steps, MT = 4, three in flight)
//   Wqr 1536 -> 8192: 10.0 -> 8.5 (wide steps, MT = 2; MT = 4 leaves 128
//     workgroups: 11.2)
//   Wo 16384 -> 7168: 59.3 -> 49.1 (narrow steps, MT = 4, KS = 2; unsplit
//     MT = 4 takes 88.6, so without a workspace it keeps MT = 2; wide
//     steps take 65-80, hence their bound on K)
// The output is computed transposed, y^T = W x^T: lane results are
// consecutive features of one token.
#include "common.h"
#include "kernels.h"

namespace mla {

// x [N][K], w [M][K], r and y [N][M], all bf16; ws [KS][N][M] fp32 when
// SPLIT. LIN_U narrow steps per wave have their loads in flight together.
// K is a multiple of the step width (32 or 128) and M of 4; split z
// takes steps [z S / KS, (z + 1) S / KS), never empty (KS <= S). Rows past
// the last feature or token load a valid row (clamped); their results are
// not stored.
template <int LIN_MT, bool WIDE, bool SPLIT, int LIN_U>
__global__ __launch_bounds__(64 * LIN_WAVES) __attribute__((amdgpu_waves_per_eu(4, 4))) void linear_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const uint16_t* r, uint16_t* y, float* ws,
    int N, int K, int M, int KS) {
  constexpr int LIN_M = 16 * LIN_MT;   // output features per workgroup
  constexpr int STEP = WIDE ? 128 : 32;
  __shared__ float part[LIN_WAVES][8 * LIN_MT][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int m0 = blockIdx.x * LIN_M, n0 = blockIdx.y * LIN_N, z = blockIdx.z;
  const int S = K / STEP;
  const int s_lo = (int)((int64_t)z * S / KS), s_hi = (int)((int64_t)(z + 1) * S / KS);
  // A = W rows m0 + 16 mt + c; B = x^T of tokens n0 + 16 t + c; lane group g's
  // first index within a step
  const int goff = WIDE ? 32 * g : 8 * g;
  const uint16_t* wa[LIN_MT];
#pragma unroll
  for (int mt = 0; mt < LIN_MT; ++mt) wa[mt] = w + (int64_t)min(m0 + 16 * mt + c, M - 1) * K + goff;
  const uint16_t* xb0 = x + (int64_t)min(n0 + c, N - 1) * K + goff;
  const uint16_t* xb1 = x + (int64_t)min(n0 + 16 + c, N - 1) * K + goff;
  // two accumulators per token tile, alternating, so consecutive MFMAs do
  // not wait on each other's results (with four feature tiles there are
  // eight independent chains already, and one each keeps the registers)
  constexpr int NA = LIN_MT >= 4 ? 1 : 2;
  f32x4 acc[LIN_MT][2][NA] = {};
  if constexpr (WIDE) {
    for (int ss = s_lo + wave; ss < s_hi; ss += LIN_WAVES) {
      u32x4 a[LIN_MT][4], b0[4], b1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int mt = 0; mt < LIN_MT; ++mt) a[mt][j] = *(const u32x4*)(wa[mt] + STEP * ss + 8 * j);
        b0[j] = *(const u32x4*)(xb0 + STEP * ss + 8 * j);
        b1[j] = *(const u32x4*)(xb1 + STEP * ss + 8 * j);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mt = 0; mt < LIN_MT; ++mt) {
          acc[mt][0][j % NA] = mfma16x16x32(as_bf16x8(a[mt][j]), as_bf16x8(b0[j]), acc[mt][0][j % NA]);
          acc[mt][1][j % NA] = mfma16x16x32(as_bf16x8(a[mt][j]), as_bf16x8(b1[j]), acc[mt][1][j % NA]);
        }
    }
  } else {
    for (int base = s_lo + wave; base < s_hi; base += LIN_WAVES * LIN_U) {
      u32x4 a[LIN_U][LIN_MT], b0[LIN_U], b1[LIN_U];
#pragma unroll
      for (int u = 0; u < LIN_U; ++u) {
        const int ss = min(base + LIN_WAVES * u, s_hi - 1);   // past the end: a valid step, not accumulated
#pragma unroll
        for (int mt = 0; mt < LIN_MT; ++mt) a[u][mt] = *(const u32x4*)(wa[mt] + STEP * ss);
        b0[u] = *(const u32x4*)(xb0 + STEP * ss);
        b1[u] = *(const u32x4*)(xb1 + STEP * ss);
      }
      // Every product is issued; a step past the end multiplies zeros (both
      // operands, so an inf in the clamped step's values adds nothing). A
      // branch here would let the compiler split the loads over the branches
      // and wait for each group in turn.
#pragma unroll
      for (int u = 0; u < LIN_U; ++u) {
        const bool live = base + LIN_WAVES * u < s_hi;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const u32x4 x0 = live ? b0[u] : zero, x1 = live ? b1[u] : zero;
#pragma unroll
        for (int mt = 0; mt < LIN_MT; ++mt) {
          const u32x4 wv = live ? a[u][mt] : zero;
          acc[mt][0][u % NA] = mfma16x16x32(as_bf16x8(wv), as_bf16x8(x0), acc[mt][0][u % NA]);
          acc[mt][1][u % NA] = mfma16x16x32(as_bf16x8(wv), as_bf16x8(x1), acc[mt][1][u % NA]);
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
      for (int i = 0; i < 4; ++i)
        part[wave][8 * mt + 4 * t + i][lane] = NA == 2 ? acc[mt][t][0][i] + acc[mt][t][NA - 1][i] : acc[mt][t][0][i];
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
  if constexpr (SPLIT) {
    *(float2*)(ws + (int64_t)z * N * M + off) = float2{s0, s1};
  } else {
    if (r) {
      const uint32_t rv = *(const uint32_t*)(r + off);
      s0 += bf16_to_f32((uint16_t)(rv & 0xffffu));
      s1 += bf16_to_f32((uint16_t)(rv >> 16));
    }
    *(uint32_t*)(y + off) = pack_bf16x2(s0, s1);
  }
}

// y = sum over z of ws[z] (z = 0, 1, ... in order) + r, one rounding; two
// features per thread. The slices are loaded eight at a time (indices past
// the last slice reload it and are not added), so a reduce of KS slices
// waits for ceil(KS / 8) memory round trips instead of KS. r may alias y
// (each element is read before it is written, by the same thread).
__global__ __launch_bounds__(256) void linear_reduce_kernel(const float* ws, const uint16_t* r, uint16_t* y,
                                                            int64_t NM, int KS) {
  constexpr int RB = 8;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 2;
  if (i >= NM) return;
  const uint32_t rv = r ? *(const uint32_t*)(r + i) : 0u;   // issued with the first slices
  float s0 = 0.f, s1 = 0.f;
  for (int z0 = 0; z0 < KS; z0 += RB) {
    float2 v[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) v[u] = *(const float2*)(ws + (int64_t)min(z0 + u, KS - 1) * NM + i);
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      if (z0 + u < KS) {
        s0 += v[u].x;
        s1 += v[u].y;
      }
    }
  }
  if (r) {
    s0 += bf16_to_f32((uint16_t)(rv & 0xffffu));
    s1 += bf16_to_f32((uint16_t)(rv >> 16));
  }
  *(uint32_t*)(y + i) = pack_bf16x2(s0, s1);
}

template <int MT, bool WIDE, int U>
static void launch_linear_t(const uint16_t* x, const uint16_t* w, const uint16_t* r, uint16_t* y, float* ws,
                            int32_t N, int32_t K, int32_t M, int ks, hipStream_t stream) {
  const dim3 grid((unsigned)((M + 16 * MT - 1) / (16 * MT)), (unsigned)((N + LIN_N - 1) / LIN_N), (unsigned)ks);
  if (ks == 1) {
    hipLaunchKernelGGL((linear_kernel<MT, WIDE, false, U>), grid, dim3(64 * LIN_WAVES), 0, stream, x, w, r, y,
                       nullptr, N, K, M, 1);
  } else {
    hipLaunchKernelGGL((linear_kernel<MT, WIDE, true, U>), grid, dim3(64 * LIN_WAVES), 0, stream, x, w, r, y, ws,
                       N, K, M, ks);
    const int64_t NM = (int64_t)N * M;
    hipLaunchKernelGGL(linear_reduce_kernel, dim3((unsigned)((NM / 2 + 255) / 256)), dim3(256), 0, stream, ws, r,
                       y, NM, ks);
  }
}

hipError_t launch_linear(const uint16_t* x, const uint16_t* w, const uint16_t* r, uint16_t* y, void* workspace,
                         size_t workspace_bytes, int32_t N, int32_t K, int32_t M, hipStream_t stream) {
  LinearPlan p = plan_linear(N, K, M, true);
  if (p.ks > 1 && (workspace == nullptr || workspace_bytes < p.ws_bytes)) p = plan_linear(N, K, M, false);
  float* ws = (float*)workspace;
  const int ks = p.ks;
  if (p.wide) {
    if (p.mt == 2) launch_linear_t<2, true, 1>(x, w, r, y, ws, N, K, M, ks, stream);
    else launch_linear_t<1, true, 1>(x, w, r, y, ws, N, K, M, ks, stream);
  } else if (p.mt == 4) {
    if (p.u == 3) launch_linear_t<4, false, 3>(x, w, r, y, ws, N, K, M, ks, stream);
    else launch_linear_t<4, false, 2>(x, w, r, y, ws, N, K, M, ks, stream);
  } else {
    if (p.mt == 2) launch_linear_t<2, false, 4>(x, w, r, y, ws, N, K, M, ks, stream);
    else launch_linear_t<1, false, 4>(x, w, r, y, ws, N, K, M, ks, stream);
  }
  return hipGetLastError();
}

}  // namespace mla
