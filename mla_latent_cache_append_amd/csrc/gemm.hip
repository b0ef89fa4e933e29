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
#include "append.h"

namespace mla {

constexpr int AQ_COLS = 128;                 // latent columns per absorb workgroup
constexpr int AQ_CHUNKS = D_C / AQ_COLS;     // 4 workgroups per head

// The [128 j][128 c] slice of W_UK[h] sits in LDS row-major (256 bytes per
// row) with 16-byte chunk k of row j stored at k ^ aq_swz(j): the 32 lanes of
// one transposing read cycle (rows 4i .. 4i+3 and 4i+8 .. 4i+11, two chunks
// each) then hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int aq_swz(int j) { return 2 * (j & 3) + 8 * ((j >> 3) & 1); }

// Each workgroup computes a [tokens x 128] column slice of q_lat for one
// head and rotates 64 (token, head) rows of q_pe, so the rotation spreads
// over the whole grid.
// W_UK[h] is stored [128 j][512 c] (rows of nn.Linear(d_c, H*d_nope).weight)
// and the contraction runs over j, its row index: the MFMA A operand
// (8 consecutive j of one column c) comes from two transposing LDS reads
// (ds_read_b64_tr_b16) of the row-major slice.
constexpr int AQ_LDS = D_NOPE * AQ_COLS * 2;   // 32 KiB weight slice
// Tokens per absorb workgroup: one workgroup per (head, column slice) takes
// a decode batch whole; a prefill-sized batch is split into runs of this many
// tokens, each on its own workgroups (grid H * 4 * ceil(N / AQ_TPW)).
constexpr int AQ_TPW = 256;
__host__ __device__ constexpr int aq_runs(int N) { return (N + AQ_TPW - 1) / AQ_TPW; }
// Within a run, wave w takes tokens 64 p + 16 w .. +15 in pass p: the four
// waves read disjoint query rows, and each keeps the whole 128-column weight
// slice in registers.
constexpr int AQ_WT = 16;
constexpr int AQ_PASSES = AQ_TPW / (4 * AQ_WT);
// A pass's outputs (16 tokens x 128 columns) go through this wave's own
// region of the LDS so that 16 lanes store one token's 256 contiguous bytes;
// rows padded to 272 bytes.
constexpr int AQ_OSTRIDE = AQ_COLS * 2 + 16;
static_assert(4 * AQ_WT * AQ_OSTRIDE <= AQ_LDS, "output staging fits in the weight slice's LDS");

__device__ __forceinline__ void absorb_q_block(
    int blk, char* wl, const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const int32_t* __restrict__ pos, const uint16_t* __restrict__ w_uk,
    uint16_t* __restrict__ q_out, int N, int H, const RopeFreqs& fr) {
  // Workgroups are dealt to the 8 XCDs round-robin by id. The four column
  // slices of one (token run, head) read the same query rows: give them ids
  // 8 apart, so they share an XCD and its L2 (when the count allows).
  int chunk, item;
  if (((H * aq_runs(N)) & 7) == 0) {
    chunk = (blk >> 3) & 3;
    item = ((blk >> 5) << 3) | (blk & 7);
  } else {
    chunk = blk % AQ_CHUNKS;
    item = blk / AQ_CHUNKS;
  }
  const int run = item / H;
  const int h = item - run * H;
  const int n_begin = run * AQ_TPW, n_end = min(N, n_begin + AQ_TPW);
  const int c0 = chunk * AQ_COLS;
  const uint16_t* w = w_uk + (int64_t)h * D_NOPE * D_C + c0;
  __attribute__((address_space(3))) char* wls = (__attribute__((address_space(3))) char*)wl;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  // Every load of the workgroup is issued before the first wait: the rope
  // pairs (with their positions and this lane's inverse frequency), the
  // weight slice and this wave's query rows of all its passes.
  //
  // Rope: the run's (token, head) rows, head fastest, are dealt 64 to each
  // of its 4H workgroups; thread (i = thread % 32, r = thread / 32) rotates
  // pair i of rows r + 8 m (m < 8) of its workgroup's. At 64 heads or more a
  // workgroup's rows are heads of one token, so each thread computes one
  // angle for its eight pairs. Rows past the run's last one wrap round to
  // its first rows and are stored again with the same values (every thread
  // stores: a store behind a branch would leave the vector memory counter
  // unknown to the compiler, whose next wait for a load would then also
  // wait for these stores to complete).
  constexpr int RP = AQ_TPW * (D_ROPE / 2) / (AQ_CHUNKS * 256);
  const int ri = (int)threadIdx.x & (D_ROPE / 2 - 1);
  const int rows = (n_end - n_begin) * H;
  const int r0 = 64 * (h * AQ_CHUNKS + chunk) + ((int)threadIdx.x >> 5);
  const double inv_freq = fr.f[ri];
  uint32_t x[RP];
  int ps[RP], rn[RP], rrow[RP];
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    int R = r0 + 8 * u;
    if (R >= rows) R %= rows;
    const int t = R / H;
    rn[u] = n_begin + t;
    rrow[u] = (n_begin + t) * H + (R - t * H);   // (token, head) row of q_pe and q_out
    x[u] = *(const uint32_t*)(q_pe + (int64_t)rrow[u] * D_ROPE + 2 * ri);
    ps[u] = pos[rn[u]];
  }
  // the weight slice: 2048 chunks of 16 bytes, eight per thread
  constexpr int PER = D_NOPE * (AQ_COLS / 8) / 256;
  u32x4 v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int k = u * 256 + threadIdx.x, j = k >> 4, ch = k & 15;
    v[u] = *(const u32x4*)(w + (int64_t)j * D_C + ch * 8);
  }
  // B = q_nope^T[K = j][N = token]: lane (g, c) holds token n0 + c, rows
  // 32 ks + 8 g .. +7. Lanes past the last token load a valid row; their
  // columns are stored over that token's with the same values.
  bf16x8 bq[AQ_PASSES][D_NOPE / 32];
#pragma unroll
  for (int p = 0; p < AQ_PASSES; ++p) {
    if (n_begin + 64 * p + 16 * wave >= n_end) break;   // wave-uniform: no tokens from this pass on
    const int n = min(n_begin + 64 * p + 16 * wave + c, n_end - 1);
    const uint16_t* src = q_nope + ((int64_t)n * H + h) * D_NOPE + 8 * g;
#pragma unroll
    for (int ks = 0; ks < D_NOPE / 32; ++ks) bq[p][ks] = as_bf16x8(*(const u32x4*)(src + 32 * ks));
  }
  __builtin_amdgcn_sched_barrier(0);
  {
    int n_prev = -1;
    double cs = 1.0, sn = 0.0;
#pragma unroll
    for (int u = 0; u < RP; ++u) {
      if (rn[u] != n_prev) {   // a new token: its angle
        rope_cos_sin(ps[u], inv_freq, cs, sn);
        n_prev = rn[u];
      }
      *(uint32_t*)(q_out + (int64_t)rrow[u] * D_K + D_C + 2 * ri) = rope_rotate_bf16(x[u], cs, sn);
    }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int k = u * 256 + threadIdx.x, j = k >> 4, ch = k & 15;
    *(__attribute__((address_space(3))) u32x4*)(wls + j * 256 + ((ch ^ aq_swz(j)) << 4)) = v[u];
  }
  __syncthreads();

  // A = W^T[M = column][K = j]: the eight 16-column blocks of the slice
  // (c0 + 16 cb + c), k-step ks covers j = 32 ks .. +31 and lane group g its
  // rows 32 ks + 8 g .. +7.
  bf16x8 af[AQ_COLS / 16][D_NOPE / 32];
#pragma unroll
  for (int cb = 0; cb < AQ_COLS / 16; ++cb) {
    const int col = 16 * cb + 4 * (c & 3);   // first column of this lane's 8-byte piece
    const int ch = col >> 3, half = (col >> 2) & 1;
#pragma unroll
    for (int ks = 0; ks < D_NOPE / 32; ++ks) {
      const int r0 = 32 * ks + 8 * g + (c >> 2), r1 = r0 + 4;
      const i16x4 v0 = lds_read_tr16_b64(wls, r0 * 256 + ((ch ^ aq_swz(r0)) << 4) + 8 * half);
      const i16x4 v1 = lds_read_tr16_b64(wls, r1 * 256 + ((ch ^ aq_swz(r1)) << 4) + 8 * half);
      af[cb][ks] = join_tr(v0, v1);
    }
  }
  __syncthreads();   // every wave holds its fragments: the slice's LDS becomes the output staging
  __attribute__((address_space(3))) char* ols = wls + wave * (AQ_WT * AQ_OSTRIDE);
#pragma unroll
  for (int p = 0; p < AQ_PASSES; ++p) {
    const int n0 = n_begin + 64 * p + 16 * wave;
    if (n0 >= n_end) break;   // wave-uniform
    f32x4 acc[AQ_COLS / 16] = {};
#pragma unroll
    for (int ks = 0; ks < D_NOPE / 32; ++ks)
#pragma unroll
      for (int cb = 0; cb < AQ_COLS / 16; ++cb) acc[cb] = mfma16x16x32(af[cb][ks], bq[p][ks], acc[cb]);
    // lane holds columns 16 cb + 4 g + i (i = 0..3) of token n0 + c
#pragma unroll
    for (int cb = 0; cb < AQ_COLS / 16; ++cb)
      *(__attribute__((address_space(3))) u32x2*)(ols + c * AQ_OSTRIDE + (16 * cb + 4 * g) * 2) =
          u32x2{pack_bf16x2(acc[cb][0], acc[cb][1]), pack_bf16x2(acc[cb][2], acc[cb][3])};
    // The LDS executes one wave's accesses in order: the reads below see the
    // writes above, and the next pass's writes follow these reads.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 16 tokens x 16 chunks of 16 bytes, four per lane: lanes 16 r .. 16 r + 15 store token 4 u + r
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = 4 * u + g;
      const int n = min(n0 + t, n_end - 1);
      *(u32x4*)(q_out + ((int64_t)n * H + h) * D_K + c0 + 8 * c) =
          *(const __attribute__((address_space(3))) u32x4*)(ols + t * AQ_OSTRIDE + 16 * c);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

__global__ __launch_bounds__(256) void absorb_q_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const int32_t* __restrict__ pos, const uint16_t* __restrict__ w_uk,
    uint16_t* __restrict__ q_out, int N, int H, RopeFreqs fr) {
  __shared__ __attribute__((aligned(16))) char wl[AQ_LDS];
  absorb_q_block(blockIdx.x, wl, q_nope, q_pe, pos, w_uk, q_out, N, H, fr);
}

// The step's first two calls in one launch: workgroups 0 .. H*4-1 absorb the
// N queries (as absorb_q_kernel), the rest append the same N new tokens to
// the cache, one wave per token (as the append kernels). Both read only their
// inputs and write disjoint outputs, so they share a launch; the attention
// that needs both follows on the stream.
template <bool FP8>
__global__ __launch_bounds__(256) void append_absorb_kernel(
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const int64_t* __restrict__ slot_mapping, void* __restrict__ pool, float* __restrict__ pool_scale,
    int64_t num_slots, const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const int32_t* __restrict__ pos, const uint16_t* __restrict__ w_uk, uint16_t* __restrict__ q_out,
    int N, int H, RopeFreqs fr) {
  __shared__ __attribute__((aligned(16))) char wl[AQ_LDS];
  const int n_absorb = H * AQ_CHUNKS * aq_runs(N);
  if ((int)blockIdx.x < n_absorb) {
    absorb_q_block(blockIdx.x, wl, q_nope, q_pe, pos, w_uk, q_out, N, H, fr);
  } else {
    const int j = ((int)blockIdx.x - n_absorb) * 4 + (int)(threadIdx.x >> 6);
    if constexpr (FP8)
      append_token_fp8(j, c_kv, k_pe, pos, slot_mapping, (uint8_t*)pool, pool_scale, num_slots, N, fr);
    else
      append_token(j, c_kv, k_pe, pos, slot_mapping, (uint16_t*)pool, num_slots, N, fr);
  }
}

hipError_t launch_append_absorb(const uint16_t* c_kv, const uint16_t* k_pe, const int64_t* slot_mapping,
                                void* pool, float* pool_scale, int64_t num_blocks, const uint16_t* q_nope,
                                const uint16_t* q_pe, const int32_t* pos, const uint16_t* w_uk,
                                uint16_t* q_out, int32_t N, int32_t H, double rope_base, hipStream_t stream) {
  const dim3 grid(H * AQ_CHUNKS * aq_runs(N) + (N + 3) / 4);
  if (pool_scale)
    hipLaunchKernelGGL(append_absorb_kernel<true>, grid, dim3(256), 0, stream, c_kv, k_pe, slot_mapping, pool,
                       pool_scale, num_blocks * BLOCK, q_nope, q_pe, pos, w_uk, q_out, N, H, rope_freqs(rope_base));
  else
    hipLaunchKernelGGL(append_absorb_kernel<false>, grid, dim3(256), 0, stream, c_kv, k_pe, slot_mapping, pool,
                       pool_scale, num_blocks * BLOCK, q_nope, q_pe, pos, w_uk, q_out, N, H, rope_freqs(rope_base));
  return hipGetLastError();
}

// The same for the two-buffer cache: the append part writes token j to
// [seq_idx[j]][pos[j]] of kv_cache and pe_cache (as the two-buffer append
// kernel), the absorb part is unchanged.
__global__ __launch_bounds__(256) void append_absorb_kvpe_kernel(
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe, const int32_t* __restrict__ seq_idx,
    uint16_t* __restrict__ kv_cache, uint16_t* __restrict__ pe_cache, int B, int max_seq,
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe, const int32_t* __restrict__ pos,
    const uint16_t* __restrict__ w_uk, uint16_t* __restrict__ q_out, int N, int H, RopeFreqs fr) {
  __shared__ __attribute__((aligned(16))) char wl[AQ_LDS];
  const int n_absorb = H * AQ_CHUNKS * aq_runs(N);
  if ((int)blockIdx.x < n_absorb)
    absorb_q_block(blockIdx.x, wl, q_nope, q_pe, pos, w_uk, q_out, N, H, fr);
  else
    append_token_kvpe(((int)blockIdx.x - n_absorb) * 4 + (int)(threadIdx.x >> 6), c_kv, k_pe, pos, seq_idx,
                      kv_cache, pe_cache, B, max_seq, N, fr);
}

hipError_t launch_append_absorb_kvpe(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* seq_idx,
                                     uint16_t* kv_cache, uint16_t* pe_cache, int32_t B, int32_t max_seq,
                                     const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                                     const uint16_t* w_uk, uint16_t* q_out, int32_t N, int32_t H, double rope_base,
                                     hipStream_t stream) {
  const dim3 grid(H * AQ_CHUNKS * aq_runs(N) + (N + 3) / 4);
  hipLaunchKernelGGL(append_absorb_kvpe_kernel, grid, dim3(256), 0, stream, c_kv, k_pe, seq_idx, kv_cache, pe_cache,
                     B, max_seq, q_nope, q_pe, pos, w_uk, q_out, N, H, rope_freqs(rope_base));
  return hipGetLastError();
}

constexpr int OU_TOK = 32;                  // tokens per pass (two 16-token MFMA blocks)
constexpr int OU_TPW = 256;                 // tokens per workgroup (runs of a prefill-sized batch)
__host__ __device__ constexpr int ou_runs(int N) { return (N + OU_TPW - 1) / OU_TPW; }

// W_UV[h] is stored [128 j][512 c] and the contraction runs over c, the
// contiguous axis of both W_UV and o_lat. Each wave keeps its 16 rows of
// W_UV (64 VGPRs, 16-byte global loads) and sweeps the tokens; the o_lat rows
// of a pass are staged once per workgroup in LDS (32 rows x 1 KiB, 16-byte
// chunk q of row t at slot q ^ (t & 15), so the 16 rows one fragment read
// covers hit 16 distinct bank groups) instead of being loaded by every wave.
// A workgroup takes OU_ROWS output rows (features) of one head: 64 (two
// workgroups per head, four waves) when one workgroup per (run, head) would
// not fill the 256 CUs, as at a decode step; else 128 (eight waves), so the
// o_lat rows are staged once per head.
template <int OU_ROWS>
__global__ __launch_bounds__(4 * OU_ROWS) void out_up_kernel(const uint16_t* __restrict__ o_lat,
                                                             const uint16_t* __restrict__ w_uv,
                                                             uint16_t* __restrict__ o, int N, int H) {
  constexpr int OU_CHUNKS = D_V / OU_ROWS;
  constexpr int THREADS = 4 * OU_ROWS;
  // o_lat rows of a pass, then its outputs (32 tokens x OU_ROWS features,
  // rows padded by 16 bytes) on their way to whole-line stores
  constexpr int OSTRIDE = OU_ROWS * 2 + 16;
  __shared__ __attribute__((aligned(16))) char ol[OU_TOK * D_C * 2 + OU_TOK * OSTRIDE];
  typedef __attribute__((address_space(3))) char lchar;
  lchar* ols = (lchar*)ol;
  lchar* ost = ols + OU_TOK * D_C * 2;
  // workgroup = (token run, head, part of the head's 128 output rows); the
  // two halves of 64 rows read the same o_lat rows: ids 8 apart put them on
  // one XCD (workgroups are dealt to the 8 XCDs round-robin) when the count
  // allows
  const int x = blockIdx.x;
  int half, item;
  if (OU_CHUNKS == 1) {
    half = 0;
    item = x;
  } else if (((H * ou_runs(N)) & 7) == 0) {
    half = (x >> 3) & 1;
    item = ((x >> 4) << 3) | (x & 7);
  } else {
    half = x % OU_CHUNKS;
    item = x / OU_CHUNKS;
  }
  const int run = item / H;
  const int h = item - run * H;
  const int hc = h * OU_CHUNKS + half;
  const int n_begin = run * OU_TPW, n_end = min(N, n_begin + OU_TPW);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int j0 = (hc % OU_CHUNKS) * OU_ROWS + 16 * wave;
  const uint16_t* w = w_uv + ((int64_t)h * D_V + j0 + c) * D_C;
  // 2048 chunks of 16 bytes per pass, eight per thread; rows past the last
  // token repeat a valid row (their outputs are not stored)
  constexpr int PER = OU_TOK * (D_C / 8) / THREADS;
  u32x4 v[PER];
  auto load_rows = [&](int n0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int k = u * THREADS + threadIdx.x, t = k >> 6, q = k & 63;
      const int n = min(n0 + t, n_end - 1);
      v[u] = *(const u32x4*)(o_lat + ((int64_t)n * H + h) * D_C + 8 * q);
    }
  };
  load_rows(n_begin);
  bf16x8 af[D_C / 32];
#pragma unroll
  for (int ks = 0; ks < D_C / 32; ++ks) af[ks] = as_bf16x8(*(const u32x4*)(w + 32 * ks + 8 * g));
  for (int n0 = n_begin; n0 < n_end; n0 += OU_TOK) {
    if (n0 > n_begin) __syncthreads();          // the previous pass has read its rows and stored its outputs
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int k = u * THREADS + threadIdx.x, t = k >> 6, q = k & 63;
      *(__attribute__((address_space(3))) u32x4*)(ols + t * 1024 + ((q ^ (t & 15)) << 4)) = v[u];
    }
    __syncthreads();
    if (n0 + OU_TOK < n_end) load_rows(n0 + OU_TOK);   // the next pass's rows, under this pass's products
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int t = 16 * tb + c;
      bf16x8 bv[D_C / 32];   // B = o_lat^T[K = c][N = token]: chunk 4 ks + g of row t
#pragma unroll
      for (int ks = 0; ks < D_C / 32; ++ks)
        bv[ks] = as_bf16x8(lds_read_b128(ols, t * 1024 + (((4 * ks + g) ^ (t & 15)) << 4)));
      // four independent accumulator chains keep the MFMA pipe busy
      f32x4 acc4[4] = {};
#pragma unroll
      for (int ks = 0; ks < D_C / 32; ++ks) acc4[ks & 3] = mfma16x16x32(af[ks], bv[ks], acc4[ks & 3]);
      const f32x4 acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
      // lane holds features j0 + 4 g + i (i = 0..3) of token t of the pass
      *(__attribute__((address_space(3))) u32x2*)(ost + t * OSTRIDE + (16 * wave + 4 * g) * 2) =
          u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    }
    __syncthreads();
    {
      // 32 tokens x OU_ROWS / 8 chunks of 16 bytes, one per thread: OU_ROWS / 8
      // lanes store a token's 2 * OU_ROWS bytes (rows past the last token hold
      // that token's outputs and are stored over it with the same values, so
      // the store is unconditional)
      const int t = (int)threadIdx.x / (OU_ROWS / 8), piece = (int)threadIdx.x % (OU_ROWS / 8);
      const int n = min(n0 + t, n_end - 1);
      *(u32x4*)(o + ((int64_t)n * H + h) * D_V + (hc % OU_CHUNKS) * OU_ROWS + 8 * piece) =
          *(const __attribute__((address_space(3))) u32x4*)(ost + t * OSTRIDE + 16 * piece);
    }
  }
}

hipError_t launch_absorb_q(const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                           const uint16_t* w_uk, uint16_t* q_out, int32_t N, int32_t H,
                           double rope_base, hipStream_t stream) {
  hipLaunchKernelGGL(absorb_q_kernel, dim3(H * AQ_CHUNKS * aq_runs(N)), dim3(256), 0, stream, q_nope, q_pe,
                     pos, w_uk, q_out, N, H, rope_freqs(rope_base));
  return hipGetLastError();
}

hipError_t launch_out_up(const uint16_t* o_lat, const uint16_t* w_uv, uint16_t* o, int32_t N,
                         int32_t H, hipStream_t stream) {
  if (H * ou_runs(N) >= 256)
    hipLaunchKernelGGL(out_up_kernel<128>, dim3(H * ou_runs(N)), dim3(512), 0, stream, o_lat, w_uv, o, N, H);
  else
    hipLaunchKernelGGL(out_up_kernel<64>, dim3(H * 2 * ou_runs(N)), dim3(256), 0, stream, o_lat, w_uv, o, N, H);
  return hipGetLastError();
}

}  // namespace mla
