// Attention over the latent cache in the expanded form, for long query
// chunks ([MLA80] §2: the model's forward expands per-head keys
// k_c = W_UK c_kv and values v = W_UV c_kv from the latent, concatenates the
// shared RoPE key and runs ordinary multi-head attention; [MLA80] §3 times
// prefill that way). The absorbed form does 2 H Lq L (576 + 512) flops per
// sequence; this one 2 L H 256 512 for the expansion plus 2 H Lq L (192 + 128)
// for the attention, so it wins once a chunk has a few hundred query tokens.
//
//   1. latent_gather_kernel: the sequence's cache rows out of the paged pool
//      into contiguous buffers, c [max_len][512] and k_r [max_len][64].
//   2. Two GEMMs per sequence (hipBLASLt: plain bf16 matrix products, fp32
//      accumulation, one rounding to bf16): K = c W_UK^T as [t][h 128 + j],
//      and V^T = W_UV c^T as [h 128 + j][t] (the layout the kernel's PV
//      product reads as its A operand).
//   3. mha_prefill_kernel: causal attention per (sequence, head, 256 query
//      rows, eight waves): 64-key tiles of K (with k_r) and V^T through the
//      LDS, scores in 32x32x16 bf16 MFMAs, online softmax in fp32,
//      O^T = V^T P^T.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <mutex>
#include <vector>

#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace mla {

namespace {

constexpr int XW = 8;                          // waves per workgroup
constexpr int XTHREADS = 64 * XW;              // 512
constexpr int XT = 64;                         // keys per tile (two 32-key blocks)
constexpr int XQ = 32 * XW;                    // query rows per workgroup, 32 per wave
constexpr int XQK = D_NOPE + D_ROPE;           // 192: key / query width
constexpr int K_STRIDE = 400;                  // LDS bytes per key row: 384, padded to 25 x 16
constexpr int VT_STRIDE = 136;                 // LDS bytes per value column: 128, padded to 17 x 8
constexpr int K_TILE = XT * K_STRIDE;          // 25,600
constexpr int VT_TILE = D_V * VT_STRIDE;       // 17,408
constexpr int X_STAGE = K_TILE + VT_TILE;      // 43,008
static_assert(2 * XTHREADS == XT * (D_NOPE / 8) && XTHREADS == XT * (D_ROPE / 8) &&
              2 * XTHREADS == D_V * (XT / 8), "tile loads: two content, one rope, two value chunks per thread");
constexpr float LN2F = 0.69314718055994530942f;

typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- gather
// One thread per 16-byte chunk of a 1,152-byte cache row: rows t < L of
// sequence b (blockIdx.y) into cg[b][t][0:512] and krg[b][t][0:64]; rows
// t >= L zero. A block id outside the pool gives NaN rows (the sequence's
// outputs come out NaN).
__global__ __launch_bounds__(256) void latent_gather_kernel(const uint16_t* pool, int64_t num_blocks,
                                                            const int32_t* block_table, int32_t max_blocks,
                                                            const int32_t* seq_lens, int32_t Lpad,
                                                            uint16_t* cg, uint16_t* krg) {
  const int b = blockIdx.y;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= (int64_t)Lpad * ROW_CHUNKS) return;
  const int t = (int)(c / ROW_CHUNKS), ch = (int)(c - (int64_t)t * ROW_CHUNKS);
  const int L = seq_lens[b];
  u32x4 v = {0u, 0u, 0u, 0u};
  if (t < L) {
    const int kb = t / BLOCK;
    const int blk = kb < max_blocks ? block_table[(int64_t)b * max_blocks + kb] : -1;
    if (blk >= 0 && (int64_t)blk < num_blocks)
      v = *(const u32x4*)(pool + ((int64_t)blk * BLOCK + t % BLOCK) * D_K + 8 * ch);
    else
      v = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
  }
  if (ch < D_C / 8)
    *(u32x4*)(cg + ((int64_t)b * Lpad + t) * D_C + 8 * ch) = v;
  else
    *(u32x4*)(krg + ((int64_t)b * Lpad + t) * D_ROPE + 8 * (ch - D_C / 8)) = v;
}

// ---------------------------------------------------------------- attention
struct MhaArgs {
  const uint16_t* q_nope;    // [B Lq][H][128]
  const uint16_t* q_pe;      // [B Lq][H][64], not rotated
  const int32_t* pos;        // [B Lq]: position of each query token (RoPE)
  const uint16_t* k;         // [B][Lpad][H 128]: expanded content keys
  const uint16_t* kr;        // [B][Lpad][64]: rotated rope keys
  const uint16_t* vt;        // [B][H 128][Lpad]: expanded values, transposed
  const int32_t* seq_lens;   // [B]
  uint16_t* o;               // [B Lq][H][128]
  float* lse;                // [B Lq][H] or null
  int32_t Lq, H, Lpad, max_len;
  float scale_log2;
  RopeFreqs fr;
};

// Workgroup (query block qb, head h; sequence b = blockIdx.y); wave w holds
// query rows 256 qb + 32 w + (l % 32); query row i sits at position
// L - Lq + i and sees keys t <= that position. Workgroup ids are dealt to the
// 8 XCDs round-robin; x is remapped so that the query blocks of one head,
// which read the same keys and values, run on one XCD and share its L2. MFMA layouts of
// v_mfma_f32_32x32x16_bf16 for lane l:
//   A (32x16): a[j] = A[l % 32][8 (l / 32) + j]
//   B (16x32): b[j] = B[8 (l / 32) + j][l % 32]
//   D (32x32): d[i] = D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32]
// Scores S^T = K Q^T per 32-key block kb: A = 32 keys x 16 features of K,
// B = Q^T, so score value v of block kb is key 32 kb + 8 (v / 4) + 4 (l / 32)
// + v % 4 of the tile for row l % 32; values 8 m .. 8 m + 7 of block kb are
// the B operand of O^T += V^T P^T for key slice kk = 2 kb + m with k-slot
// 8 (l / 32) + j <-> key 16 kk + 8 (j / 4) + 4 (l / 32) + j % 4, and V^T is
// read in that key order (two runs of four keys, 8 bytes each).
__global__ __launch_bounds__(XTHREADS, 1) void mha_prefill_kernel(MhaArgs a, int32_t nqb) {
  __shared__ __attribute__((aligned(16))) char smem[2 * X_STAGE];
  int unit = blockIdx.x;
  if ((gridDim.x & 7) == 0) unit = (unit & 7) * (int)(gridDim.x >> 3) + (unit >> 3);
  const int qb = unit % nqb, h = unit / nqb, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r32 = lane & 31, hf = lane >> 5;
  const int HD = a.H * D_NOPE;
  const int L = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
  const bool bad = L > a.max_len;
  const int Lc = max(0, min(L, a.max_len));    // keys present in the expanded buffers
  const int i = qb * XQ + 32 * wave + r32;      // this lane's query row
  const bool valid = i < a.Lq;
  const int prow = L - a.Lq + i;                // last key the row sees
  const int last = min(a.Lq, qb * XQ + XQ) - 1;
  const int kend = min(Lc, L - a.Lq + last + 1);
  const int ntiles = kend > 0 ? (kend + XT - 1) / XT : 0;

  // query fragments (B operand of S^T): row i, features 16 ks + 8 (l / 32) .. +7;
  // features 128.. are q_pe rotated to the row's position
  bf16x8 qf[XQK / 16];
  {
    const int64_t qrow = ((int64_t)b * a.Lq + (valid ? i : 0)) * a.H + h;
#pragma unroll
    for (int ks = 0; ks < D_NOPE / 16; ++ks) {
      u32x4 v = *(const u32x4*)(a.q_nope + qrow * D_NOPE + 16 * ks + 8 * hf);
      if (!valid) v = u32x4{0u, 0u, 0u, 0u};
      qf[ks] = as_bf16x8(v);
    }
    const int p = a.pos[(int64_t)b * a.Lq + (valid ? i : 0)];
#pragma unroll
    for (int ks = 0; ks < D_ROPE / 16; ++ks) {
      const int d = 16 * ks + 8 * hf;
      u32x4 v = *(const u32x4*)(a.q_pe + qrow * D_ROPE + d);
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = rope_pair_bf16(v[u], p, a.fr.f[d / 2 + u]);
      if (!valid) v = u32x4{0u, 0u, 0u, 0u};
      qf[D_NOPE / 16 + ks] = as_bf16x8(v);
    }
  }

  // tile j's keys 64 j .. +63 in registers, 16-byte chunks: two content
  // chunks (key c / 16, chunk c % 16 for c = tid, tid + 512), one rope chunk
  // (key tid / 8, chunk tid % 8) and two value chunks (column c / 8, keys
  // 8 (c % 8) .. +7); per-thread byte offsets are fixed, the tile moves a
  // wave-uniform base. Keys at or past Lc (tail tile only) read as zeros.
  struct Stage {
    u32x4 kc[2];
    u32x4 kr;
    u32x4 v[2];
  };
  const char* kbase = (const char*)(a.k + (int64_t)b * a.Lpad * HD + h * D_NOPE);
  const char* rbase = (const char*)(a.kr + (int64_t)b * a.Lpad * D_ROPE);
  const char* vbase = (const char*)(a.vt + ((int64_t)b * HD + h * D_NOPE) * a.Lpad);
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t c = tid + XTHREADS * u;
    koff[u] = (c / 16) * (uint32_t)HD * 2u + (c % 16) * 16u;
    voff[u] = (c / 8) * (uint32_t)a.Lpad * 2u + (c % 8) * 16u;
  }
  const uint32_t roff = (tid / 8) * (uint32_t)D_ROPE * 2u + (tid % 8) * 16u;
  auto load = [&](int j, Stage& st) {
    const int t0 = j * XT;
    const char* kb = kbase + (int64_t)t0 * HD * 2;
    const char* rb = rbase + (int64_t)t0 * D_ROPE * 2;
    const char* vb = vbase + (int64_t)t0 * 2;
    if (t0 + XT <= Lc) {
#pragma unroll
      for (int u = 0; u < 2; ++u) st.kc[u] = *(const u32x4*)(kb + koff[u]);
      st.kr = *(const u32x4*)(rb + roff);
#pragma unroll
      for (int u = 0; u < 2; ++u) st.v[u] = *(const u32x4*)(vb + voff[u]);
    } else {
      const int n = Lc - t0;   // keys of this tile present, 0 < n < 64
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < 2; ++u) st.kc[u] = (int)((tid + XTHREADS * u) / 16) < n ? *(const u32x4*)(kb + koff[u]) : z;
      st.kr = (int)(tid / 8) < n ? *(const u32x4*)(rb + roff) : z;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = 8 * (int)((tid + XTHREADS * u) % 8);
        u32x4 v = t < n ? *(const u32x4*)(vb + voff[u]) : z;
#pragma unroll
        for (int e = 0; e < 4; ++e) {   // keys t + 2e, t + 2e + 1
          if (t + 2 * e >= n) v[e] = 0u;
          else if (t + 2 * e + 1 >= n) v[e] &= 0xffffu;
        }
        st.v[u] = v;
      }
    }
  };
  auto store = [&](int s, const Stage& st) {
    lds_char* base = (lds_char*)smem + s * X_STAGE;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + XTHREADS * u;
      *(__attribute__((address_space(3))) u32x4*)(base + (c / 16) * K_STRIDE + 16 * (c % 16)) = st.kc[u];
    }
    *(__attribute__((address_space(3))) u32x4*)(base + (tid / 8) * K_STRIDE + 2 * D_NOPE + 16 * (tid % 8)) = st.kr;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + XTHREADS * u, col = c / 8, qq = c % 8;
      lds_char* p = base + K_TILE + col * VT_STRIDE + 16 * qq;
      *(__attribute__((address_space(3))) u32x2*)p = u32x2{st.v[u][0], st.v[u][1]};
      *(__attribute__((address_space(3))) u32x2*)(p + 8) = u32x2{st.v[u][2], st.v[u][3]};
    }
  };

  f32x16 O[D_V / 32];
#pragma unroll
  for (int cb = 0; cb < D_V / 32; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[cb][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  if (ntiles > 0) {
    Stage st;
    load(0, st);
    store(0, st);
  }
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    Stage nx;
    const bool more = j + 1 < ntiles;
    if (more) load(j + 1, nx);
    const lds_char* kst = (const lds_char*)smem + (j & 1) * X_STAGE;
    const lds_char* vst = kst + K_TILE;
    // the two key blocks' accumulator chains alternate, so no MFMA waits on
    // the one just before it
    f32x16 S[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) S[kb][v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < XQK / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 kf = *(const __attribute__((address_space(3))) u32x4*)(
            kst + (32 * kb + r32) * K_STRIDE + 2 * (16 * ks + 8 * hf));
        S[kb] = mfma32(as_bf16x8(kf), qf[ks], S[kb]);
      }
    // online softmax in log2 units: the max is taken over the raw scores
    // (the scale is positive), exponentials as exp2(s * scale - m); keys past
    // the row's position or past Lc masked
    const int t0 = j * XT;
    if (__any(t0 + XT - 1 > prow) || t0 + XT > Lc) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int tok = t0 + 32 * kb + 8 * (v >> 2) + 4 * hf + (v & 3);
          if (tok > prow || tok >= Lc) S[kb][v] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, S[kb][v]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt * a.scale_log2);
    const float mref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - mref);   // 0 while m_run = -inf
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        S[kb][v] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][v], a.scale_log2, -mref));
        ps += S[kb][v];
      }
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int cb = 0; cb < D_V / 32; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[cb][v] *= alpha;
    }
    bf16x8 P[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 w;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        w[jj] = pack_bf16x2(S[kk >> 1][8 * (kk & 1) + 2 * jj], S[kk >> 1][8 * (kk & 1) + 2 * jj + 1]);
      P[kk] = as_bf16x8(w);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int cb = 0; cb < D_V / 32; ++cb) {   // four accumulator chains in turn
        const lds_char* vp = vst + (32 * cb + r32) * VT_STRIDE + 2 * (16 * kk + 4 * hf);
        const u32x2 lo = *(const __attribute__((address_space(3))) u32x2*)vp;
        const u32x2 hi = *(const __attribute__((address_space(3))) u32x2*)(vp + 16);
        O[cb] = mfma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), P[kk], O[cb]);
      }
    if (more) store((j + 1) & 1, nx);
    __syncthreads();
  }

  // rows: o = O / l (bf16), lse = ln of the scaled scores' exponential sum
  const float l = l_run + __shfl_xor(l_run, 32);
  if (valid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* orow = a.o + (((int64_t)b * a.Lq + i) * a.H + h) * D_V;
#pragma unroll
    for (int cb = 0; cb < D_V / 32; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v0 = O[cb][4 * g] * inv, v1 = O[cb][4 * g + 1] * inv;
        float v2 = O[cb][4 * g + 2] * inv, v3 = O[cb][4 * g + 3] * inv;
        if (bad) v0 = v1 = v2 = v3 = NAN;
        *(u32x2*)(orow + 32 * cb + 8 * g + 4 * hf) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
      }
    if (a.lse && hf == 0) {
      float lv = l > 0.f ? (m_run + __log2f(l)) * LN2F : -INFINITY;
      if (bad) lv = NAN;
      a.lse[((int64_t)b * a.Lq + i) * a.H + h] = lv;
    }
  }
}

// ---------------------------------------------------------------- GEMMs
constexpr int MAX_DEVICES = 64;
std::mutex lt_mu;
hipblasLtHandle_t lt_handles[MAX_DEVICES];

// The algorithm hipBLASLt's heuristic picked for each GEMM shape on each
// device, so that repeated calls skip the query (about 15 us of host time per
// GEMM). A handful of shapes per run: searched linearly, the oldest dropped
// past LT_ALGOS.
struct LtShape {
  int dev, ta, tb;
  int64_t m, n, k, lda, ldb, ldd;
  bool operator==(const LtShape& o) const {
    return dev == o.dev && ta == o.ta && tb == o.tb && m == o.m && n == o.n && k == o.k && lda == o.lda &&
           ldb == o.ldb && ldd == o.ldd;
  }
};
constexpr size_t LT_ALGOS = 64;
std::vector<std::pair<LtShape, hipblasLtMatmulAlgo_t>> lt_algos;   // guarded by lt_mu

hipError_t lt_handle(hipblasLtHandle_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(lt_mu);
  if (!lt_handles[dev] && hipblasLtCreate(&lt_handles[dev]) != HIPBLAS_STATUS_SUCCESS) {
    lt_handles[dev] = nullptr;
    return hipErrorUnknown;
  }
  *out = lt_handles[dev];
  return hipSuccess;
}

// D (m x n, column-major, ld ldd) = op(A) op(B) in bf16 with fp32
// accumulation; A is stored (a_rows x a_cols, ld lda), B (b_rows x b_cols, ld ldb).
hipError_t lt_gemm(hipblasLtHandle_t handle, hipblasOperation_t ta, hipblasOperation_t tb, int64_t m, int64_t n,
                   int64_t k, const void* A, int64_t lda, const void* B, int64_t ldb, void* D, int64_t ldd,
                   hipStream_t stream) {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  hipError_t err = hipErrorUnknown;
  const int64_t a_rows = ta == HIPBLAS_OP_N ? m : k, a_cols = ta == HIPBLAS_OP_N ? k : m;
  const int64_t b_rows = tb == HIPBLAS_OP_N ? k : n, b_cols = tb == HIPBLAS_OP_N ? n : k;
  const float alpha = 1.f, beta = 0.f;
  hipblasLtMatmulHeuristicResult_t heur[1];
  int found = 0, dev = 0;
  bool cached = false;
  hipblasLtMatmulAlgo_t algo;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorUnknown;
  const LtShape key{dev, (int)ta, (int)tb, m, n, k, lda, ldb, ldd};
  if (hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) goto done;
  if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) != HIPBLAS_STATUS_SUCCESS)
    goto done;
  if (hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, a_rows, a_cols, lda) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, b_rows, b_cols, ldb) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&ld, HIP_R_16BF, m, n, ldd) != HIPBLAS_STATUS_SUCCESS)
    goto done;
  {
    std::lock_guard<std::mutex> lock(lt_mu);
    for (const auto& e : lt_algos)
      if (e.first == key) {
        algo = e.second;
        cached = true;
        break;
      }
  }
  if (!cached) {
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) goto done;
    if (hipblasLtMatmulAlgoGetHeuristic(handle, desc, la, lb, ld, ld, pref, 1, heur, &found) !=
            HIPBLAS_STATUS_SUCCESS ||
        found < 1)
      goto done;
    algo = heur[0].algo;
    std::lock_guard<std::mutex> lock(lt_mu);
    if (lt_algos.size() >= LT_ALGOS) lt_algos.erase(lt_algos.begin());
    lt_algos.emplace_back(key, algo);
  }
  if (hipblasLtMatmul(handle, desc, &alpha, A, la, B, lb, &beta, D, ld, D, ld, &algo, nullptr, 0, stream) ==
      HIPBLAS_STATUS_SUCCESS)
    err = hipSuccess;
done:
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ld) hipblasLtMatrixLayoutDestroy(ld);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (desc) hipblasLtMatmulDescDestroy(desc);
  return err;
}

}  // namespace

hipError_t launch_prefill_expanded(const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                                   const uint16_t* pool, int64_t num_blocks, const int32_t* block_table,
                                   int32_t max_blocks, const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H,
                                   int32_t max_len, const uint16_t* w_uk, const uint16_t* w_uv,
                                   float softmax_scale, double rope_base, uint16_t* o, float* lse,
                                   void* workspace, hipStream_t stream) {
  const ExpandedLayout w = expanded_layout(B, H, max_len);
  char* ws = (char*)workspace;
  uint16_t* cg = (uint16_t*)(ws + w.c_off);
  uint16_t* krg = (uint16_t*)(ws + w.kr_off);
  uint16_t* kx = (uint16_t*)(ws + w.k_off);
  uint16_t* vt = (uint16_t*)(ws + w.vt_off);
  const int64_t HD = (int64_t)H * D_NOPE;

  const dim3 ggrid((unsigned)(((int64_t)w.Lpad * ROW_CHUNKS + 255) / 256), (unsigned)B);
  hipLaunchKernelGGL(latent_gather_kernel, ggrid, dim3(256), 0, stream, pool, num_blocks, block_table, max_blocks,
                     seq_lens, w.Lpad, cg, krg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  hipblasLtHandle_t handle;
  e = lt_handle(&handle);
  if (e != hipSuccess) return e;
  for (int b = 0; b < B; ++b) {
    const uint16_t* c = cg + (int64_t)b * w.Lpad * D_C;
    // K_b [Lpad][HD] row-major = (HD x Lpad) column-major = W_UK (HD x 512) c_b^T (512 x Lpad)
    e = lt_gemm(handle, HIPBLAS_OP_T, HIPBLAS_OP_N, HD, w.Lpad, D_C, w_uk, D_C, c, D_C,
                kx + (int64_t)b * w.Lpad * HD, HD, stream);
    if (e != hipSuccess) return e;
    // V^T_b [HD][Lpad] row-major = (Lpad x HD) column-major = c_b (Lpad x 512) W_UV^T (512 x HD)
    e = lt_gemm(handle, HIPBLAS_OP_T, HIPBLAS_OP_N, w.Lpad, HD, D_C, c, D_C, w_uv, D_C,
                vt + (int64_t)b * HD * w.Lpad, w.Lpad, stream);
    if (e != hipSuccess) return e;
  }

  MhaArgs a;
  a.q_nope = q_nope;
  a.q_pe = q_pe;
  a.pos = pos;
  a.k = kx;
  a.kr = krg;
  a.vt = vt;
  a.seq_lens = seq_lens;
  a.o = o;
  a.lse = lse;
  a.Lq = Lq;
  a.H = H;
  a.Lpad = w.Lpad;
  a.max_len = max_len;
  a.scale_log2 = softmax_scale * 1.44269504088896340736f;
  a.fr = rope_freqs(rope_base);
  const int32_t nqb = (Lq + XQ - 1) / XQ;
  hipLaunchKernelGGL(mha_prefill_kernel, dim3((unsigned)(nqb * H), (unsigned)B), dim3(XTHREADS), 0, stream, a, nqb);
  return hipGetLastError();
}

}  // namespace mla
