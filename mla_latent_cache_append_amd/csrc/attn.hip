// mla_decode_attn: split-KV flash-decode over the paged 576-wide latent cache.
//
// What is computed ([AUDIT] = llm-atlas page "DeepSeek MLA 吸收式缓存：真实权重
// 执行与 FlashMLA 架构边界", §2.2-2.3; [MLA80] = CSDN page "80 行 PyTorch 从零写
// DeepSeek 的 MLA", §5): for each query row (absorbed content query q_lat and
// rotated rope query q_r, packed as 576 bf16) and the cache rows C_t =
// [c_kv | k_r] of its sequence,
//   s_t = scale * (q . C_t)              over all 576 features,
//   o_lat = sum_t softmax(s)_t C_t[:512]
// with causal visibility t <= position of the query.
//
// Design for gfx950:
//  * One cache block (64 tokens x 1,152 B = 72 KiB, contiguous in HBM) is the
//    tile. It is copied global -> LDS with direct 16-byte loads (no VGPR
//    staging), double-buffered (144 KiB of the 160 KiB LDS), 1 KiB per wave
//    instruction, fully coalesced.
//  * Every query row that shares the sequence reuses each tile: the tile is the
//    shared K (all 576 columns) and V (first 512 columns), one latent for all
//    heads ([AUDIT] §2.4; [MLA80] §5 "共享 k_r 广播到各 head").
//  * Scores are computed transposed, S^T = K Q^T, with the K tile as the MFMA A
//    operand (8 consecutive features of one token: one 16-byte LDS read) and
//    Q in registers. The S^T accumulator leaves each lane holding scores of
//    one query row, so the softmax row statistics need only two cross-lane
//    steps and the probabilities feed the PV product straight from registers.
//  * The context is accumulated transposed, O^T = V^T P^T, with V^T read by
//    ds_read_b64_tr_b16 from the same row-major tile, and the K dimension of
//    the PV product permuted to match the token order the S^T layout gives.
//  * LDS tile layout: row-major 72 chunks of 16 B per token, chunk index XOR
//    ((token >> 1) & 7). Both the K reads and the transposed V reads are then
//    free of bank conflicts.
//  * Split-KV is stream-K style: the tiles of all sequences form one line that
//    is cut into `width` equal ranges, one per workgroup, so ragged batches are
//    balanced exactly. A range that covers a whole sequence writes the final
//    o_lat; otherwise it writes (m, l, acc) partials that the combine kernel
//    merges in a fixed order (deterministic, no atomics).
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "own_asm.inc"

namespace mla {

// ------------------------------------------------------------------ plan

__device__ __forceinline__ int tiles_of(int L, int max_blocks) {
  L = max(L, 0);
  L = min(L, max_blocks * BLOCK);
  return (L + BLOCK - 1) / BLOCK;
}

// Wave-uniform values made explicit (SGPRs, scalar branches).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

// Total tiles over all sequences (wave-uniform).
__device__ int64_t plan_total_tiles(const int32_t* seq_lens, int B, int max_blocks) {
  const int lane = threadIdx.x & 63;
  int64_t total = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    total += wave_sum_i(b < B ? tiles_of(seq_lens[b], max_blocks) : 0);
  }
  return uni64(total);
}

// First sequence b whose tile range [S_b, S_b + tiles_b) contains tile x.
// Returns b (or B if none) and S_b (wave-uniform).
__device__ void plan_find(const int32_t* seq_lens, int B, int max_blocks, int64_t x, int& b_out,
                          int64_t& start_out) {
  const int lane = threadIdx.x & 63;
  int64_t base_sum = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    const int t = b < B ? tiles_of(seq_lens[b], max_blocks) : 0;
    int incl = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const uint64_t hit = __ballot(b < B && base_sum + incl > x);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      const int incl_src = __shfl(incl, src);
      const int t_src = __shfl(t, src);
      b_out = uni(base + src);
      start_out = uni64(base_sum + incl_src - t_src);
      return;
    }
    base_sum += uni(__shfl(incl, 63));
  }
  b_out = B;
  start_out = uni64(base_sum);
}

// Workgroup of range w (0..width-1) that holds tile x of the line of T tiles,
// where range w is [floor(w T / width), floor((w+1) T / width)).
__device__ __forceinline__ int plan_owner(int64_t x, int64_t T, int width) {
  return (int)(((x + 1) * (int64_t)width - 1) / T);
}

// ------------------------------------------------------------------ kernel

struct AttnArgs {
  const uint16_t* q;            // [B*rows][576]   (row (b, r) = b*rows + r)
  const uint16_t* pool;         // [num_blocks][64][576] bf16 (FP8 pool: [num_blocks][64][576] E4M3 codes)
  const float* pool_scale;      // FP8 pool only: [num_blocks][64] fp32 scale of each token's row
  const int32_t* block_table;   // [B][max_blocks]
  const int32_t* seq_lens;      // [B]
  uint16_t* o_lat;              // [B*rows][512]
  float* lse;                   // [B*rows] or null
  float* ws_ml;                 // [slots][rows][2]: (m, l) of each partial, fp32
  uint16_t* ws_acc;             // [slots][rows][512]: partial o_lat normalized by its l, bf16
  const uint16_t* pe;           // two-buffer layout: pe_cache [B][max_seq][64] (pool = kv_cache
                                //   [B][max_seq][512]); null for the paged pool
  int64_t num_blocks;
  int max_blocks;               // tiles a sequence may span (two-buffer layout: ceil(max_seq / 64))
  int max_keys;                 // keys a sequence may hold: max_blocks * 64, or max_seq
  int B, Lq, H, rows;
  int n_rg, width;
  float scale_log2;             // softmax scale * log2(e)
};

constexpr int TILE_BYTES = BLOCK_BYTES;          // 73,728
constexpr int TILE_CHUNKS = BLOCK * ROW_CHUNKS;  // 4,608 sixteen-byte chunks
constexpr int KSTEPS = D_K / 32;                 // 18 MFMA k-steps over 576 features
constexpr float LN2 = 0.69314718055994530942f;

typedef __attribute__((address_space(3))) char lds_char;

// LDS tile layout (blocked): chunks of 16 B ordered [tg 8][cg 9][tl 8][cl 8] for
// token t = 8 tg + tl and feature chunk c = 8 cg + cl (8 bf16 features), with
// cl stored XOR swz(t). One 1-KiB direct-load instruction fills one
// (tg, cg) block: 8 tokens x one 128-byte line each. swz spreads the 16 tokens
// a 16-lane group reads over all 16 bank groups, so both the K reads and the
// transposed V reads are conflict-free.
__device__ __forceinline__ int swz(int t) { return ((t & 7) >> 1) | (((t >> 3) & 1) << 2); }

__device__ __forceinline__ uint32_t lds_chunk_off(int t, int c) {
  return (uint32_t)((((t >> 3) * 9 + (c >> 3)) * 64 + (t & 7) * 8 + ((c & 7) ^ swz(t))) * 16);
}

// Where the rows of a run of tokens of one sequence come from. Paged pool:
// one 1,152-byte row per token inside a 64-token block. Two-buffer layout
// ([AUDIT] §0 and §4.2: V3's absorbed decode keeps kv_cache [B][max_seq][512]
// and pe_cache [B][max_seq][64]): a 1,024-byte latent row and a 128-byte rope
// row per token, in two arrays. The descriptors cover only the run's first
// n_valid tokens: rows past the end of the sequence (never written, arbitrary
// bits) arrive as zeros, so a masked probability of 0 never meets a NaN in
// the PV product.
struct TileSrc {
  sgpr_x4 main;   // pool rows, or the latent rows
  sgpr_x4 pe;     // rope rows (two-buffer layout)
  int stride;     // bytes per token of `main`
};

__device__ __forceinline__ TileSrc tile_src(const AttnArgs& a, int b, int blk, int tok0, int n_valid) {
  TileSrc s;
  if (a.pe) {
    const int64_t row = (int64_t)b * a.max_keys + tok0;
    s.main = buffer_rsrc((const char*)a.pool + row * (D_C * 2), n_valid * (D_C * 2));
    s.pe = buffer_rsrc((const char*)a.pe + row * (D_ROPE * 2), n_valid * (D_ROPE * 2));
    s.stride = D_C * 2;
  } else {
    s.main = buffer_rsrc((const char*)a.pool + (int64_t)blk * TILE_BYTES + (tok0 % BLOCK) * ROW_BYTES,
                         n_valid * ROW_BYTES);
    s.pe = s.main;
    s.stride = ROW_BYTES;
  }
  return s;
}

// One 1-KiB line: the 128-byte column group cg (features 64 cg .. +63; cg = 8
// is the rope part) of the 8 tokens tok .. tok + 7 of a tile source. Lane l
// reads token tok + l / 8, 16-byte chunk `chunk` of the group (the swizzled
// chunk the LDS slot l expects); the line lands at LDS address dst.
__device__ __forceinline__ void copy_line(const TileSrc& s, bool two_buf, int lane, uint32_t chunk, int tok,
                                          int cg, uint32_t dst) {
  const int tl = lane >> 3;
  if (two_buf && cg == 8)
    buffer_load_lds_16(s.pe, (uint32_t)(tl * (D_ROPE * 2)) + chunk, (uint32_t)(tok * (D_ROPE * 2)), dst);
  else
    buffer_load_lds_16(s.main, (uint32_t)(tl * s.stride) + chunk, (uint32_t)(tok * s.stride + cg * 128), dst);
}

// Copy one 64-token tile into an LDS tile buffer; wave w issues the 72 / NW
// line copies j = w*72/NW .. (w+1)*72/NW - 1. Buffer loads with an LDS
// destination: the per-lane offset is a VGPR, the per-instruction offset an
// SGPR, and the hardware bound-checks every lane against the descriptor's size.
template <int NW>
__device__ __forceinline__ void load_tile(const TileSrc& src, bool two_buf, lds_char* dst, int wave, int lane) {
  constexpr int PER_WAVE = (BLOCK / 8) * 9 / NW;
#pragma unroll
  for (int jj = 0; jj < PER_WAVE; ++jj) {
    const int j = wave * PER_WAVE + jj;
    const int tg = j / 9, cg = j - 9 * (j / 9);
    const uint32_t chunk = (uint32_t)(((lane & 7) ^ (((lane >> 3) >> 1) | ((tg & 1) << 2))) * 16);
    copy_line(src, two_buf, lane, chunk, tg * 8, cg, lds_addr(dst + j * 1024));
  }
}

// Rows are rescaled only when their running max grows by more than this many
// log2 units, so probabilities stay below 2^8 (exact range for bf16 and fp32)
// and the accumulators are touched outside the MFMAs only on rare tiles.
constexpr float RESCALE_LOG2 = 8.f;

// Online-softmax update of RB row blocks from this tile's scores, given as the
// 16 (NK = 2 k-blocks x 8) values per lane in PV k-slot order. Returns the
// packed bf16 probabilities. NCB accumulators per row block are rescaled only
// when some lane's max moved by more than RESCALE_LOG2.
//
// PMUL (FP8 cache): the probability of key j is multiplied by pmul[kb][j],
// its token's dequantization scale, before the bf16 rounding that feeds PV;
// the row sum takes the unscaled probability.
template <int RB, int NCB, bool PMUL = false>
__device__ __forceinline__ void softmax_update(float (&pv)[RB][2][8], float (&m_run)[RB],
                                               float (&l_run)[RB], f32x4 (&o)[RB][NCB],
                                               bf16x8 (&pf)[RB][2],
                                               const float (*pmul)[8] = nullptr) {
  float mx[RB];
  bool need = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float v = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) v = fmaxf(v, pv[rb][kb][j]);
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    mx[rb] = v;
    need |= v > m_run[rb] + RESCALE_LOG2;
  }
  if (__any(need)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (mx[rb] > m_run[rb] + RESCALE_LOG2) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - mx[rb]);  // 0 when m_run = -inf
        l_run[rb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o[rb][cb] *= alpha;
        m_run[rb] = mx[rb];
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float m_ref = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 pk;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(pv[rb][kb][j] - m_ref);
        psum += p;
        if constexpr (PMUL) pk[j] = (__bf16)(p * pmul[kb][j]);
        else pk[j] = (__bf16)p;
      }
      pf[rb][kb] = pk;
    }
    l_run[rb] += psum;
  }
}

// O^T[col][row] += V^T[col][token] P^T[token][row] over the 64 tokens of the
// tile for the column blocks cb0 .. cb0 + NCB - 1.
template <int RB, int NCB>
__device__ __forceinline__ void pv_product(lds_char* cur, const uint32_t (&vbase)[4], int cb0,
                                           const bf16x8 (&pf)[RB][2], f32x4 (&o)[RB][NCB]) {
  auto read_v = [&](int cbg, int kb) -> bf16x8 {
    lds_char* vrow = cur + vbase[cbg & 3];
    const i16x4 v0 = lds_read_tr16_b64(vrow, kb * 36864 + (cbg >> 2) * 1024);
    const i16x4 v1 = lds_read_tr16_b64(vrow, kb * 36864 + 18432 + (cbg >> 2) * 1024);
    return join_tr(v0, v1);
  };
  bf16x8 vn[2] = {read_v(cb0, 0), read_v(cb0, 1)};
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const bf16x8 vc[2] = {vn[0], vn[1]};
    if (cb + 1 < NCB) {
      vn[0] = read_v(cb0 + cb + 1, 0);
      vn[1] = read_v(cb0 + cb + 1, 1);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][cb] = mfma16x16x32(vc[kb], pf[rb][kb], o[rb][cb]);
    __builtin_amdgcn_sched_barrier(0);  // one column block of fragments in flight
  }
}

// Scale scores to log2 units and, on tiles that reach past the first query's
// position, mask keys beyond each row's limit. Score (rb, tb, i) belongs to
// token 16 tok_block(tb) + 4g + i of the tile.
template <int RB, int NTB, bool MASK>
__device__ __forceinline__ void scale_mask(f32x4 (&s)[RB][NTB], float scale_log2, int key0,
                                           int tok_block0, int g, const int (&lim)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = s[rb][tb][i] * scale_log2;
        if (MASK && key0 + 16 * (tok_block0 + tb) + 4 * g + i > lim[rb]) v = -INFINITY;
        s[rb][tb][i] = v;
      }
}

// Column split, one tile: wave w scores tokens 16w..16w+15 for all RB*16 rows,
// shares the scores through LDS, and accumulates columns 128w..128w+127.
//
// FP8: the tile holds the E4M3 codes converted exactly to bf16 and tsc (LDS)
// the 64 token scales; score t is multiplied by tsc[t] before the softmax
// scale and probability t by tsc[t] before PV.
template <int RB, bool MASK, bool FP8 = false>
__device__ __forceinline__ void cols_tile(lds_char* cur, __attribute__((address_space(3))) float* sbuf,
                                          const __attribute__((address_space(3))) float* tsc,
                                          const bf16x8 (&qf)[RB][KSTEPS], f32x4 (&o)[RB][8],
                                          float (&m_run)[RB], float (&l_run)[RB],
                                          const int (&lim)[RB], int key0, float scale_log2,
                                          const uint32_t (&kbase)[2], const uint32_t (&vbase)[4],
                                          int wave, int g, int c16) {
  constexpr int SB = 68;  // padded score-buffer row (floats)
  f32x4 s[RB][1];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) s[rb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 kn = lds_read_b128(cur + kbase[0], 0);
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const u32x4 kc = kn;
    if (ks + 1 < KSTEPS) kn = lds_read_b128(cur + kbase[(ks + 1) & 1], ((ks + 1) >> 1) * 1024);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s[rb][0] = mfma16x16x32(as_bf16x8(kc), qf[rb][ks], s[rb][0]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (FP8) {
    const f32x4 ts = *(const __attribute__((address_space(3))) f32x4*)(tsc + 16 * wave + 4 * g);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s[rb][0] *= ts;
  }
  scale_mask<RB, 1, MASK>(s, scale_log2, key0, wave, g, lim);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    *(__attribute__((address_space(3))) f32x4*)(sbuf + (rb * 16 + c16) * SB + 16 * wave + 4 * g) = s[rb][0];
  if constexpr (FP8) lds_barrier();  // tile copies in flight in registers stay in flight
  else __syncthreads();
  float pv[RB][2][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const f32x4 v = *(const __attribute__((address_space(3))) f32x4*)(
            sbuf + (rb * 16 + c16) * SB + 32 * kb + 16 * h2 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[rb][kb][4 * h2 + i] = v[i];
      }
  bf16x8 pf[RB][2];
  if constexpr (FP8) {
    // scales of the keys in PV k-slot order: token 32 kb + 16 h2 + 4 g + i
    float pm[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const f32x4 v = *(const __attribute__((address_space(3))) f32x4*)(tsc + 32 * kb + 16 * h2 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) pm[kb][4 * h2 + i] = v[i];
      }
    softmax_update<RB, 8, true>(pv, m_run, l_run, o, pf, pm);
  } else {
    softmax_update<RB, 8>(pv, m_run, l_run, o, pf);
  }
  pv_product<RB, 8>(cur, vbase, 8 * wave, pf, o);
}

// ------------------------------------------------------------- FP8 tiles
//
// FP8 pool: [num_blocks][64][576] E4M3 codes (one byte per element, a block
// is 36,864 contiguous bytes) and [num_blocks][64] fp32 token scales. A tile
// is copied into registers (nine 16-byte loads per thread, consecutive threads
// on consecutive 16 bytes), converted to bf16 exactly (every E4M3 value is a
// bf16 value) by v_cvt_scalef32_pk_bf16_fp8 with scale 1, and written to an
// LDS tile in the same swizzled bf16 layout the bf16 kernels read. The token
// scales are applied in fp32 to the scores and probabilities instead.
constexpr int TILE_BYTES8 = BLOCK * D_K;               // 36,864
constexpr int FP8_LOADS = TILE_BYTES8 / 16 / 256;      // 9 per thread
constexpr int ROW_CHUNKS8 = D_K / 16;                  // 36 sixteen-byte chunks per row

struct Fp8Stage {
  u32x4 v[FP8_LOADS];
  f32x4 sc;
  int n_valid;
};

// Codes and scales of tile `blk`. The whole block lies inside the pool, so
// every load is in bounds; tokens at or past n_valid (never written, any
// bits) become zero codes and zero scales only when the tile is stored, so
// that nothing waits for the loads before then.
__device__ __forceinline__ void fp8_tile_load(const uint8_t* pool8, const float* scales, int blk,
                                              int n_valid, int tid, Fp8Stage& st) {
  const uint8_t* base = pool8 + (int64_t)blk * TILE_BYTES8;
#pragma unroll
  for (int i = 0; i < FP8_LOADS; ++i)   // read once per call: non-temporal
    st.v[i] = __builtin_nontemporal_load((const u32x4*)(base + 16 * (tid + 256 * i)));
  st.sc = *(const f32x4*)(scales + (int64_t)blk * BLOCK + 4 * (tid & (BLOCK / 4 - 1)));
  st.n_valid = n_valid;
}

// Four E4M3 codes (bytes 0..3 of w) -> four bf16, exact.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);  // bytes 0, 1
  const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);   // bytes 2, 3
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Converted tile into the LDS tile at dst (bf16 chunks 2c and 2c+1 of token t
// for the 16 codes of fp8 chunk c) and its scales into sdst[64].
__device__ __forceinline__ void fp8_tile_store(const Fp8Stage& st, lds_char* dst,
                                               __attribute__((address_space(3))) float* sdst, int tid) {
#pragma unroll
  for (int i = 0; i < FP8_LOADS; ++i) {
    const int j = tid + 256 * i;
    const int t = j / ROW_CHUNKS8, c = j - ROW_CHUNKS8 * t;
    const u32x4 v = t < st.n_valid ? st.v[i] : u32x4{0u, 0u, 0u, 0u};
    const u32x2 a = fp8x4_to_bf16x4(v[0]), b = fp8x4_to_bf16x4(v[1]);
    const u32x2 e = fp8x4_to_bf16x4(v[2]), f = fp8x4_to_bf16x4(v[3]);
    *(__attribute__((address_space(3))) u32x4*)(dst + lds_chunk_off(t, 2 * c)) = u32x4{a[0], a[1], b[0], b[1]};
    *(__attribute__((address_space(3))) u32x4*)(dst + lds_chunk_off(t, 2 * c + 1)) = u32x4{e[0], e[1], f[0], f[1]};
  }
  if (tid < BLOCK / 4) {
    f32x4 sc;
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[e] = 4 * tid + e < st.n_valid ? st.sc[e] : 0.f;
    *(__attribute__((address_space(3))) f32x4*)(sdst + 4 * tid) = sc;
  }
}

// Few rows per sequence (16 or 32, e.g. 16 heads): the 4 waves of a
// workgroup share the same RB*16 rows (RB = 16-row MFMA blocks); see cols_tile.
//
// FP8 = true reads the FP8 pool (codes + token scales): tiles are staged
// through registers (see fp8_tile_load), one tile in flight while the
// previous one is computed; with more rows than one workgroup takes, several
// row groups share each key range (n_rg > 1).
template <int RB, bool FP8 = false>
__global__ __launch_bounds__(256, 1) void attn_cols_kernel(AttnArgs a) {
  constexpr bool CS = true;
  constexpr int NW = 4;
  constexpr int RG = RB * 16;   // rows per workgroup
  constexpr int NCB = 8;        // 16-column blocks per wave
  constexpr int SB_BYTES = RB * 16 * 68 * 4;
  constexpr int SC_BYTES = FP8 ? 2 * BLOCK * 4 : 0;   // token scales of the two tiles

  __shared__ __attribute__((aligned(1024))) char smem[2 * TILE_BYTES + SB_BYTES + SC_BYTES];
  lds_char* tiles = (lds_char*)smem;
  __attribute__((address_space(3))) float* sbuf =
      (__attribute__((address_space(3))) float*)(tiles + 2 * TILE_BYTES);
  __attribute__((address_space(3))) float* tscale =
      (__attribute__((address_space(3))) float*)(tiles + 2 * TILE_BYTES + SB_BYTES);
  const uint8_t* pool8 = (const uint8_t*)a.pool;

  const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;

  // ---- which (row group, range) this workgroup owns
  int unit = blockIdx.x;
  if (a.n_rg > 1) {
    // Put the row groups of one range on one XCD (workgroup ids are dealt to
    // the 8 XCDs round-robin) so their reads of the same tiles share its L2.
    const int full = (int)(gridDim.x / 64) * 64;
    if (unit < full) {
      const int loc = unit & 63;
      unit = (unit & ~63) + (loc & 7) * 8 + (loc >> 3);
    }
  }
  const int w = unit / a.n_rg;
  const int rg = unit - w * a.n_rg;

  const int64_t T = plan_total_tiles(a.seq_lens, a.B, a.max_blocks);
  if (T == 0) return;
  const int64_t x_begin = (int64_t)w * T / a.width;
  const int64_t x_end = (int64_t)(w + 1) * T / a.width;
  if (x_begin >= x_end) return;

  int b;
  int64_t seq_start;
  plan_find(a.seq_lens, a.B, a.max_blocks, x_begin, b, seq_start);

  const int row_base = rg * RG + (CS ? 0 : wave * RB * 16);  // first row of this wave

  const bool two_buf = a.pe != nullptr;   // kv_cache + pe_cache instead of the paged pool
  // K fragment (token 16 tb + c16, chunk 4 ks + g) = kbase[ks & 1] + tb*18432 + (ks >> 1)*1024
  const int ktok = c16 + (CS ? 16 * wave : 0);
  const uint32_t kbase[2] = {lds_chunk_off(ktok, g), lds_chunk_off(ktok, 4 + g)};
  // V^T fragment (token 32 kb + 16 h + 4g + c16/4, column 16 cb + 4 (c16 % 4)) =
  //   vbase[cb & 3] + kb*36864 + h*18432 + (cb >> 2)*1024
  uint32_t vbase[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
    vbase[q4] = lds_chunk_off(4 * g + (c16 >> 2), 2 * q4 + ((c16 & 3) >> 1)) + 8 * (c16 & 1);

  int64_t x = x_begin;
  while (x < x_end && b < a.B) {
    const int L = uni(a.seq_lens[b]);
    const int ntiles = tiles_of(L, a.max_blocks);
    const int64_t seg_end = min(x_end, seq_start + ntiles);
    const int k_first = (int)(x - seq_start);
    const int k_last = (int)(seg_end - seq_start);  // exclusive
    const bool whole = (x == seq_start) && (seg_end == seq_start + ntiles);
    bool bad = L > a.max_keys;
    const int Lc = min(L, a.max_keys);             // keys that exist in the cache
    // scalar loads (lgkmcnt): reading a block id never waits on the tile loads
    const __attribute__((address_space(4))) int32_t* bt =
        (const __attribute__((address_space(4))) int32_t*)(a.block_table + (int64_t)b * a.max_blocks);
    auto blk_at = [&](int k) { return two_buf ? 0 : (int)bt[k]; };
    auto blk_bad = [&](int blk) { return !two_buf && (blk < 0 || blk >= a.num_blocks); };
    Fp8Stage stage;
    {
      const int blk = blk_at(k_first);
      const int nv = min(BLOCK, Lc - k_first * BLOCK);
      if (blk_bad(blk)) bad = true;
      else if constexpr (FP8) fp8_tile_load(pool8, a.pool_scale, blk, nv, threadIdx.x, stage);
      else load_tile<NW>(tile_src(a, b, blk, k_first * BLOCK, nv), two_buf, tiles, wave, lane);
    }

    // ---- query fragments: B operand of S^T (lane: row c16, features 32ks + 8g .. +7)
    bf16x8 qf[RB][KSTEPS];
    int lim[RB];
    float m_run[RB], l_run[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = row_base + rb * 16 + c16;
      const bool valid = r < a.rows;
      const uint16_t* qrow = a.q + ((int64_t)b * a.rows + (valid ? r : 0)) * D_K + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        u32x4 v = *(const u32x4*)(qrow + 32 * ks);
        if (!valid) v = u32x4{0u, 0u, 0u, 0u};
        qf[rb][ks] = as_bf16x8(v);
      }
      // query i of this row sits at position L - Lq + i and sees keys <= it
      lim[rb] = valid ? L - a.Lq + r / a.H : -1;
      m_run[rb] = -INFINITY;
      l_run[rb] = 0.f;
    }
    f32x4 o[RB][NCB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) o[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Tiles [k_first, k_mask) hold only keys every row may see; later tiles
    // need the causal / length mask. Two loops keep the mask out of the main one.
    const int k_mask = max(k_first, min(k_last, max(0, L - a.Lq + 1) / BLOCK));
    auto step = [&](int k) -> lds_char* {
      wait_vmem();
      lds_barrier();
      if (k + 1 < k_last) {
        const int blk = blk_at(k + 1);
        if (blk_bad(blk)) bad = true;
        else
          load_tile<NW>(tile_src(a, b, blk, (k + 1) * BLOCK, min(BLOCK, Lc - (k + 1) * BLOCK)), two_buf,
                        tiles + ((k + 1 - k_first) & 1) * TILE_BYTES, wave, lane);
      }
      return tiles + ((k - k_first) & 1) * TILE_BYTES;
    };
    if constexpr (FP8) {
      // tile k is in LDS at the barrier; tile k + 1 travels in registers
      // while k is computed and is converted into the other buffer after it
      if (!bad) fp8_tile_store(stage, tiles, tscale, threadIdx.x);
      auto fp8_tile = [&](int k, auto mask) {
        lds_barrier();
        const int nb = (k + 1 - k_first) & 1;
        bool more = k + 1 < k_last;
        if (more) {
          const int blk = blk_at(k + 1);
          if (blk_bad(blk)) { bad = true; more = false; }
          else fp8_tile_load(pool8, a.pool_scale, blk, min(BLOCK, Lc - (k + 1) * BLOCK), threadIdx.x, stage);
        }
        const int cb = (k - k_first) & 1;
        cols_tile<RB, decltype(mask)::value, true>(tiles + cb * TILE_BYTES, sbuf, tscale + cb * BLOCK, qf, o,
                                                   m_run, l_run, lim, k * BLOCK, a.scale_log2, kbase, vbase,
                                                   wave, g, c16);
        if (more) fp8_tile_store(stage, tiles + nb * TILE_BYTES, tscale + nb * BLOCK, threadIdx.x);
      };
      for (int k = k_first; k < k_mask; ++k) fp8_tile(k, std::false_type{});
      for (int k = k_mask; k < k_last; ++k) fp8_tile(k, std::true_type{});
    } else {
      for (int k = k_first; k < k_mask; ++k) {
        lds_char* cur = step(k);
        cols_tile<RB, false>(cur, sbuf, nullptr, qf, o, m_run, l_run, lim, k * BLOCK, a.scale_log2, kbase, vbase, wave, g, c16);
      }
      for (int k = k_mask; k < k_last; ++k) {
        lds_char* cur = step(k);
        cols_tile<RB, true>(cur, sbuf, nullptr, qf, o, m_run, l_run, lim, k * BLOCK, a.scale_log2, kbase, vbase, wave, g, c16);
      }
    }

    // ---- finish the segment: row sums across the 4 lanes of each row
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l_run[rb] += __shfl_xor(l_run[rb], 16);
      l_run[rb] += __shfl_xor(l_run[rb], 32);
    }
    const int slot = w + b;
    const int cb0 = CS ? wave * NCB : 0;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = row_base + rb * 16 + c16;
      if (r >= a.rows) continue;
      const int64_t orow = (int64_t)b * a.rows + r;
      if (whole) {
        const float inv = l_run[rb] > 0.f ? 1.f / l_run[rb] : 0.f;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          f32x4 v = o[rb][cb] * inv;
          if (bad) v = f32x4{NAN, NAN, NAN, NAN};
          const u32x2 out = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *(u32x2*)(a.o_lat + orow * D_C + 16 * (cb0 + cb) + 4 * g) = out;
        }
        if (a.lse && g == 0 && (!CS || wave == 0)) {
          float lv = l_run[rb] > 0.f ? (m_run[rb] + __log2f(l_run[rb])) * LN2 : -INFINITY;
          if (bad) lv = NAN;
          a.lse[orow] = lv;
        }
      } else {
        const int64_t prow = (int64_t)slot * a.rows + r;
        const float inv = l_run[rb] > 0.f ? 1.f / l_run[rb] : 0.f;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          f32x4 v = o[rb][cb] * inv;
          if (bad) v = f32x4{NAN, NAN, NAN, NAN};
          const u32x2 out = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *(u32x2*)(a.ws_acc + prow * D_C + 16 * (cb0 + cb) + 4 * g) = out;
        }
        if (g == 0 && (!CS || wave == 0)) {
          a.ws_ml[prow * 2 + 0] = bad ? NAN : m_run[rb];
          a.ws_ml[prow * 2 + 1] = bad ? NAN : l_run[rb];
        }
      }
    }

    // ---- next sequence with tiles
    x = seg_end;
    seq_start += ntiles;
    ++b;
    while (b < a.B && tiles_of(uni(a.seq_lens[b]), a.max_blocks) == 0) ++b;
    __syncthreads();  // every wave is done with the tile buffers and sbuf
  }
}


// ================================================================== rows kernel
//
// Rows >= 48 per sequence (e.g. 128 heads): a workgroup owns 64 * NH query
// rows of one key range, as NH halves of 4 waves. In half hw, wave r (0..3)
//   * scores rows 64 hw + 16 r .. +15 against each 32-token half tile with
//     the full 576-wide query (S^T = K Q^T, Q in 72 VGPRs), runs their online
//     softmax, and writes the bf16 probabilities P^T to LDS;
//   * accumulates columns 128 r .. +127 of O for all 64 rows of its half
//     (O^T = V^T P^T, 128 AGPRs), reading the half's four P blocks from LDS.
// The whole key range's cache is read from HBM once per workgroup (all heads
// of the sequence on one CU), every wave stays within 256 registers (two
// waves per SIMD), and no score is computed twice. Iteration e scores half
// tile e+1 and accumulates half tile e, two independent MFMA streams; one
// barrier per half tile publishes both the next stage and the probabilities.
// Products use v_mfma_f32_16x16x32_bf16 (layout at mfma16x16x32).

constexpr int HT_TOK = 32;                      // tokens per half tile
constexpr int HT_BYTES = HT_TOK * ROW_BYTES;    // 36,864
constexpr int RSTAGE = 3;                       // LDS stages of half tiles

// Half-tile LDS layout: 16-byte chunks ordered [tg 4][cg 9][tl 8][cl 8] for
// token t = 8 tg + tl, feature chunk c = 8 cg + cl, cl stored XOR swz2(t).
// With 64 banks of 4 bytes (16 groups of 16 bytes), the 16 consecutive tokens
// of one chunk (a K read) land on 16 distinct groups, and so do the 4 tokens
// x 4 aligned chunks that 32 lanes of a transposed V read cover.
__device__ __forceinline__ int swz2(int t) {
  const int tl = t & 7;
  return (((tl >> 1) & 1) << 2) | ((tl >> 2) & 1) | (((t >> 3) & 1) << 1);
}
__device__ __forceinline__ uint32_t ht_off(int t, int c) {
  return (uint32_t)((((t >> 3) * 9 + (c >> 3)) * 64 + (t & 7) * 8 + ((c & 7) ^ swz2(t))) * 16);
}

template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int NH>
__global__ __launch_bounds__(256 * NH, 1) void attn_rows_kernel(AttnArgs a) {
  constexpr int NWAVE = 4 * NH;
  constexpr int PB_BYTES = NH * 4 * 64 * 16;       // P^T blocks of one half tile
  constexpr int QR_BYTES = NWAVE * 2 * 64 * 16;     // rope part of Q (2 k-steps) per wave
  __shared__ __attribute__((aligned(1024))) char smem[RSTAGE * HT_BYTES + 2 * PB_BYTES + QR_BYTES +
                                                       2 * NH * 64 * 4 * 2];
  lds_char* stages = (lds_char*)smem;
  lds_char* pbase = stages + RSTAGE * HT_BYTES;                       // [2][NH][4 rb][64 lanes] x 16 B
  lds_char* qrope = pbase + 2 * PB_BYTES;                               // [wave][2 ks][64 lanes] x 16 B
  __attribute__((address_space(3))) float* abase =
      (__attribute__((address_space(3))) float*)(qrope + QR_BYTES);      // [2][NH][64 rows] rescale factors
  __attribute__((address_space(3))) float* stat = abase + 2 * NH * 64;   // [NH][64 rows][2] (m, l)

  const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hw = wave >> 2, r4 = wave & 3;
  const int g = lane >> 4, c16 = lane & 15;

  int unit = blockIdx.x;
  if (a.n_rg > 1) {
    const int full = (int)(gridDim.x / 64) * 64;
    if (unit < full) {
      const int loc = unit & 63;
      unit = (unit & ~63) + (loc & 7) * 8 + (loc >> 3);
    }
  }
  const int w = unit / a.n_rg;
  const int rg = unit - w * a.n_rg;
  const int64_t T = plan_total_tiles(a.seq_lens, a.B, a.max_blocks);
  if (T == 0) return;
  const int64_t x_begin = (int64_t)w * T / a.width;
  const int64_t x_end = (int64_t)(w + 1) * T / a.width;
  if (x_begin >= x_end) return;
  int b;
  int64_t seq_start;
  plan_find(a.seq_lens, a.B, a.max_blocks, x_begin, b, seq_start);

  const int half_row0 = rg * 64 * NH + hw * 64;     // first row of this wave's half
  const int r_s = half_row0 + 16 * r4 + c16;        // row this lane scores
  // K fragment (token 16 tb + c16, chunk 4 ks + g) = kbase[ks & 1] + tb*18432 + (ks >> 1)*1024
  const uint32_t kbase[2] = {ht_off(c16, g), ht_off(c16, 4 + g)};
  // V^T fragment of column block cb (cols 128 r4 + 16 cb ..), first / second read:
  //   vbase[cb & 3] + (cb >> 2)*1024 (+ 18432 for tokens 16..31)
  uint32_t vbase[4];
  {
    const int t = 4 * g + (c16 >> 2);                // token of this lane's 4-element load
    const int e = (c16 & 3) >> 1;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      vbase[q] = ht_off(t, 16 * r4 + 2 * q + e) + 8 * (c16 & 1);   // chunk 16 r4 = column 128 r4
  }
  const uint32_t gchunk = (uint32_t)(((lane & 7) ^ swz2(8 * r4 + (lane >> 3))) * 16);
  const bool dma_wave = hw == 0;                    // half 0's four waves copy the tiles
  const bool two_buf = a.pe != nullptr;             // kv_cache + pe_cache instead of the paged pool

  int64_t x = x_begin;
  while (x < x_end && b < a.B) {
    const int L = uni(a.seq_lens[b]);
    const int ntiles = tiles_of(L, a.max_blocks);
    const int64_t seg_end = min(x_end, seq_start + ntiles);
    const int k_first = (int)(x - seq_start);
    const int k_last = (int)(seg_end - seq_start);
    const bool whole = (x == seq_start) && (seg_end == seq_start + ntiles);
    bool bad = L > a.max_keys;
    const int Lc = min(L, a.max_keys);              // keys that exist in the cache
    const int key_end = min(k_last * BLOCK, Lc);
    const int e0 = 2 * k_first, e1 = (key_end + HT_TOK - 1) / HT_TOK;

    // query fragments: B operand of S^T (lane: row r_s, features 32 ks + 8 g .. +7);
    // the 16 latent k-steps stay in registers, the 2 rope k-steps in LDS
    constexpr int KS_REG = D_C / 32;
    bf16x8 qf[KS_REG];
    lds_char* qr = qrope + wave * 2048 + lane * 16;
    {
      const bool valid = r_s < a.rows;
      const uint16_t* qrow = a.q + ((int64_t)b * a.rows + (valid ? r_s : 0)) * D_K + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        u32x4 v = *(const u32x4*)(qrow + 32 * ks);
        if (!valid) v = u32x4{0u, 0u, 0u, 0u};
        if (ks < KS_REG) qf[ks] = as_bf16x8(v);
        else *(__attribute__((address_space(3))) u32x4*)(qr + (ks - KS_REG) * 1024) = v;
      }
    }
    const int lim = r_s < a.rows ? L - a.Lq + r_s / a.H : -1;
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[4][8];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) o[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // block ids through scalar loads, one tile ahead
    const __attribute__((address_space(4))) int32_t* bt =
        (const __attribute__((address_space(4))) int32_t*)(a.block_table + (int64_t)b * a.max_blocks);
    auto blk_at = [&](int k) { return two_buf ? 0 : (k < ntiles ? (int)bt[k] : -1); };
    int kq = k_first;
    int blk_q = blk_at(kq);
    int blk_q1 = blk_at(kq + 1);
    auto issue = [&](int e) {
      const int k = e >> 1;
      if (k != kq) {
        kq = k;
        blk_q = blk_q1;
        blk_q1 = blk_at(kq + 1);
      }
      const int blk = blk_q;
      if (!two_buf && (blk < 0 || blk >= a.num_blocks)) {
        bad = true;
        return;
      }
      if (!dma_wave) return;
      const TileSrc src = tile_src(a, b, blk, e * HT_TOK, min(HT_TOK, Lc - e * HT_TOK));
      const uint32_t dst = lds_addr(stages + (e % RSTAGE) * HT_BYTES + r4 * 9 * 1024);
#pragma unroll
      for (int cg = 0; cg < 9; ++cg) copy_line(src, two_buf, lane, gchunk, 8 * r4, cg, dst + cg * 1024);
    };

    // Scores of half tile e for this wave's 16 rows, online softmax, and P^T /
    // rescale factors into buffer (e & 1). Scores value i of token block tb is
    // token 16 tb + 4 g + i of the half tile.
    auto scores = [&](int e) {
      lds_char* st = stages + (e % RSTAGE) * HT_BYTES;
      f32x4 s[2] = {};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        // no register prefetch: the other wave on the SIMD covers LDS latency
        u32x4 kc[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) kc[tb] = lds_read_b128(st + kbase[ks & 1], tb * 18432 + (ks >> 1) * 1024);
        const bf16x8 qk = ks < KS_REG ? qf[ks < KS_REG ? ks : 0]
                                      : as_bf16x8(lds_read_b128(qr, (ks - KS_REG) * 1024));
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) s[tb] = mfma16x16x32(as_bf16x8(kc[tb]), qk, s[tb]);
      }
      const int key0 = e * HT_TOK;
      if (key0 + HT_TOK - 1 > L - a.Lq) {       // some key past some row's position
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key0 + 16 * tb + 4 * g + i > lim) s[tb][i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[tb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mx *= a.scale_log2;                        // scale > 0: max commutes with it
      float alpha = 1.f;
      if (mx > m_run + RESCALE_LOG2) {           // rare: the running max moved a lot
        alpha = __builtin_amdgcn_exp2f(m_run - mx);   // 0 when m_run = -inf
        l_run *= alpha;
        m_run = mx;
      }
      __attribute__((address_space(3))) float* ab = abase + ((e & 1) * NH + hw) * 64;
      if (g == 0) ab[16 * r4 + c16] = alpha;
      const float m_ref = m_run == -INFINITY ? 0.f : m_run;
      bf16x8 pk;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tb][i], a.scale_log2, -m_ref));
          l_run += p;
          pk[4 * tb + i] = (__bf16)p;
        }
      *(__attribute__((address_space(3))) u32x4*)(pbase + (((e & 1) * NH + hw) * 4 + r4) * 1024 + lane * 16) =
          as_u32x4(pk);
    };

    // O^T[col][row] += V^T[col][token] P^T[token][row] over half tile e for
    // columns 128 r4 .. +127 and the half's 64 rows, after applying the
    // rows' rescale factors published with P.
    auto accumulate = [&](int e) {
      const __attribute__((address_space(3))) float* ab = abase + ((e & 1) * NH + hw) * 64;
      float al[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) al[rb] = ab[16 * rb + c16];
      bool any = false;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) any |= al[rb] != 1.f;
      if (__any(any)) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) o[rb][cb] *= al[rb];
      }
      lds_char* st = stages + (e % RSTAGE) * HT_BYTES;
      const lds_char* pb = pbase + ((e & 1) * NH + hw) * 4 * 1024 + lane * 16;
      bf16x8 pf[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) pf[rb] = as_bf16x8(lds_read_b128(pb, rb * 1024));
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const i16x4 v0 = lds_read_tr16_b64(st + vbase[cb & 3], (cb >> 2) * 1024);
        const i16x4 v1 = lds_read_tr16_b64(st + vbase[cb & 3], 18432 + (cb >> 2) * 1024);
        const bf16x8 vf = join_tr(v0, v1);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) o[rb][cb] = mfma16x16x32(vf, pf[rb], o[rb][cb]);
      }
    };

    // ---- pipeline: prologue loads e0, e0+1; stage e+2 is loaded during iteration e
    for (int e = e0; e < min(e1, e0 + 2); ++e) issue(e);
    if (dma_wave) {
      if (e1 - e0 >= 2) wait_vmem_n<9>();
      else wait_vmem_n<0>();
    }
    lds_barrier();
    scores(e0);
    for (int e = e0; e < e1; ++e) {
      // stage e+1 complete (only e+2, not yet issued, would be newer)
      if (dma_wave) wait_vmem_n<0>();
      lds_barrier();                 // stage e+1 and P / factors of e visible
      if (e + 2 < e1) issue(e + 2);  // into the stage of e-1, free after the barrier
      if (e + 1 < e1) scores(e + 1);
      accumulate(e);
    }

    // ---- finish the segment: row sums; publish (m, l) for the column owners
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    lds_barrier();
    if (g == 0) {
      stat[(hw * 64 + 16 * r4 + c16) * 2 + 0] = m_run;
      stat[(hw * 64 + 16 * r4 + c16) * 2 + 1] = l_run;
    }
    lds_barrier();
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = half_row0 + 16 * rb + c16;       // row of o[rb][*] in this lane
      if (r >= a.rows) continue;
      const float mr = stat[(hw * 64 + 16 * rb + c16) * 2 + 0];
      const float lr = stat[(hw * 64 + 16 * rb + c16) * 2 + 1];
      const int64_t orow = (int64_t)b * a.rows + r;
      if (whole) {
        const float inv = lr > 0.f ? 1.f / lr : 0.f;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          f32x4 v = o[rb][cb] * inv;
          if (bad) v = f32x4{NAN, NAN, NAN, NAN};
          const u32x2 out = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *(u32x2*)(a.o_lat + orow * D_C + 128 * r4 + 16 * cb + 4 * g) = out;
        }
        if (a.lse && r4 == 0 && g == 0) {
          const float lv = lr > 0.f ? (mr + __log2f(lr)) * LN2 : -INFINITY;
          a.lse[orow] = bad ? NAN : lv;
        }
      } else {
        const int64_t prow = (int64_t)(w + b) * a.rows + r;
        const float inv = lr > 0.f ? 1.f / lr : 0.f;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          f32x4 v = o[rb][cb] * inv;
          if (bad) v = f32x4{NAN, NAN, NAN, NAN};
          const u32x2 out = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *(u32x2*)(a.ws_acc + prow * D_C + 128 * r4 + 16 * cb + 4 * g) = out;
        }
        if (r4 == 0 && g == 0) {
          a.ws_ml[prow * 2 + 0] = bad ? NAN : mr;
          a.ws_ml[prow * 2 + 1] = bad ? NAN : lr;
        }
      }
    }
    x = seg_end;
    seq_start += ntiles;
    ++b;
    while (b < a.B && tiles_of(uni(a.seq_lens[b]), a.max_blocks) == 0) ++b;
    lds_barrier();
  }
}

// =================================================================== own kernel
//
// Rows >= 96 per sequence (e.g. 128 heads): a workgroup owns 128 query rows
// of one key range with one wave per SIMD, and wave w owns rows 32 w .. +31
// end to end. It holds their whole query (576 features, 144 VGPRs) and their
// whole output accumulator (O^T, 512 columns, 256 AGPRs), forms the scores
// S^T = K Q^T, runs the online softmax in registers and accumulates
// O^T += V^T P^T with the probabilities taken straight from the score
// registers. Waves share only the half tiles in LDS: one barrier per half
// tile. Iteration e accumulates half tile e and scores half tile e+1 in one
// branch-free region (two independent MFMA streams, the softmax VALU work
// under them). Products are v_mfma_f32_32x32x16_bf16:
//   A (32x16): a[j] = A[l % 32][8 (l / 32) + j]
//   B (16x32): b[j] = B[8 (l / 32) + j][l % 32]
//   D (32x32): d[i] = D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32]
// so score value i of lane l is token 8 (i / 4) + 4 (l / 32) + i % 4 of the
// half tile for row l % 32, and values 8 kk .. 8 kk + 7 are exactly the PV
// B operand of token block kk (k-slot 8 (l / 32) + u <-> token 16 kk +
// 8 (u / 4) + 4 (l / 32) + u % 4), with V^T read in the same token order.

typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Maximum over lanes l and l ^ 32 by the gfx950 lane-swap instruction (VALU,
// no LDS round trip). With both operands equal, the two results hold the
// wave's two halves in opposite order, so their maximum is the same either way.
__device__ __forceinline__ float max_xor32(float v) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
}

constexpr int OSTAGE = 4;                 // LDS stages: two read per iteration, two in flight
constexpr int OUT_STRIDE = 1040;          // bytes per output row staged in LDS (1 KiB + 16: fewer bank conflicts)
constexpr int KSTEPS16 = D_K / 16;        // k-steps of 16 features

// Scale an accumulator held in AGPRs. The empty asm statements pin the value
// to the AGPR class on both sides of the multiply, so that this rarely taken
// path does not lead the register allocator to move every accumulator of the
// kernel into VGPRs.
__device__ __forceinline__ void scale_acc(f32x16& acc, float f) {
  f32x16 t = acc;
  asm volatile("" : "+a"(t));
  t *= f;
  acc = t;
  asm volatile("" : "+a"(acc));
}

template <bool PE>
__global__ __launch_bounds__(256, 1) void attn_own_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[OSTAGE * HT_BYTES];
  lds_char* stages = (lds_char*)smem;

  const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c32 = lane & 31, h = lane >> 5;

  // Workgroups are dealt to the 8 XCDs round-robin by id; give each XCD a
  // contiguous run of work units, so the ranges of one sequence (and its query
  // rows, which all of them load) share that XCD's L2.
  int unit = blockIdx.x;
  if ((gridDim.x & 7) == 0) unit = (unit & 7) * (int)(gridDim.x >> 3) + (unit >> 3);
  const int w = unit / a.n_rg;
  const int rg = unit - w * a.n_rg;
  const int64_t T = plan_total_tiles(a.seq_lens, a.B, a.max_blocks);
  if (T == 0) return;
  const int64_t x_begin = (int64_t)w * T / a.width;
  const int64_t x_end = (int64_t)(w + 1) * T / a.width;
  if (x_begin >= x_end) return;
  int b;
  int64_t seq_start;
  plan_find(a.seq_lens, a.B, a.max_blocks, x_begin, b, seq_start);

  const int r = rg * 128 + 32 * wave + c32;   // this lane's query row within the sequence
  // K fragment of k-step ks (token c32, chunk 2 ks + h) sits at
  // (stage + kbase) ^ ((ks & 3) << 5), plus (ks >> 2) * 1024: within a group
  // of 8 chunks the chunk index only enters the swizzled slot bits 5..6, and
  // stage bases are multiples of 128 bytes.
  const uint32_t kbase = ht_off(c32, h);
  // V^T fragment of column block cb (columns 32 cb .. +31) and token block kk:
  //   tr(((stage + vbase) ^ ((cb & 1) << 6)) + kk * 18432 + (cb >> 1) * 1024)               tokens 16 kk + 4 h .. +3
  //   tr(((stage + vbase) ^ 32 ^ ((cb & 1) << 6)) + kk * 18432 + 9216 + (cb >> 1) * 1024)   tokens 16 kk + 8 + 4 h .. +3
  // (tokens 8 apart share the slot layout up to bit 1 of the swizzle, i.e.
  // byte bit 5; vbase < 1024 and stage bases are multiples of 1024)
  uint32_t vbase;
  {
    const int i16 = lane & 15, q = lane >> 4;
    const int tl = 4 * (q >> 1) + (i16 >> 2);
    const int e = 2 * (q & 1) + ((i16 & 3) >> 1);
    vbase = ht_off(tl, e) + 8 * (i16 & 1);
  }
  // Copy operands of a line: lane l reads token l / 8 of the wave's 8, at the
  // swizzled 16-byte chunk the LDS slot expects; the pool's rows are 1,152
  // bytes, the two-buffer cache's latent rows 1,024 (columns 0..1,023 as in
  // the pool) and its rope rows 128, in their own array (PE)
  constexpr int KV_ROW = PE ? D_C * 2 : ROW_BYTES;
  const uint32_t gchunk = (uint32_t)(((lane & 7) ^ swz2(8 * wave + (lane >> 3))) * 16);
  const uint32_t goff = (uint32_t)((lane >> 3) * KV_ROW) + gchunk;
  const uint32_t so = (uint32_t)uni(wave * 8 * KV_ROW);   // buffer offset of this wave's 8 tokens
  const uint32_t gpoff = (uint32_t)((lane >> 3) * (D_ROPE * 2)) + gchunk;   // rope rows (PE)
  const uint32_t sp = (uint32_t)uni(wave * 8 * (D_ROPE * 2));
  // the pool base as descriptor words, and its size as a 32-bit bound
  const uint32_t pool_lo = (uint32_t)uni((int)(uint32_t)(uintptr_t)a.pool);
  const uint32_t pool_hi = (uint32_t)uni((int)((uint32_t)((uintptr_t)a.pool >> 32) & 0xffffu));
  const uint32_t nblk = (uint32_t)uni((int)min(a.num_blocks, (int64_t)0x7fffffff));

  int64_t x = x_begin;
  while (x < x_end && b < a.B) {
    const int L = uni(a.seq_lens[b]);
    const int ntiles = tiles_of(L, a.max_blocks);
    const int64_t seg_end = min(x_end, seq_start + ntiles);
    const int k_first = (int)(x - seq_start);
    const int k_last = (int)(seg_end - seq_start);
    const bool whole = (x == seq_start) && (seg_end == seq_start + ntiles);
    bool bad = L > a.max_keys;
    const int key_end = min(k_last * BLOCK, L);
    const int e0 = 2 * k_first, e1 = (key_end + HT_TOK - 1) / HT_TOK;
    // two-buffer cache: the sequence's rows, and the keys that exist in them
    const int Lc = uni(min(L, a.max_keys));
    const uint16_t* kv_seq = PE ? (const uint16_t*)uni64((int64_t)(uintptr_t)(a.pool + (int64_t)b * a.max_keys * D_C))
                                : nullptr;
    const uint16_t* pe_seq = PE ? (const uint16_t*)uni64((int64_t)(uintptr_t)(a.pe + (int64_t)b * a.max_keys * D_ROPE))
                                : nullptr;

    const int lim = r < a.rows ? L - a.Lq + r / a.H : -1;   // last key row r sees
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[16];   // set by the first half tile's PV MFMAs (zero accumulator input)

    // Block ids come through scalar loads (lgkmcnt, not vmcnt, so reading one
    // never drains the tile copies in flight). In the loop the id of the
    // half tile copied at the end of an iteration is requested right after
    // its barrier, so the load is long complete when it is used.
    const __attribute__((address_space(4))) int32_t* bt =
        (const __attribute__((address_space(4))) int32_t*)(PE ? nullptr : a.block_table + (int64_t)b * a.max_blocks);
    auto blk_of = [&](int e) { return PE ? 0 : (e >> 1) < ntiles ? bt[e >> 1] : -1; };
    // Copy of half tile e (cache block blk) into its stage: descriptor rs and
    // this wave's LDS base mb (wave w copies tokens 8 w .. 8 w + 7, nine
    // 1-KiB lines). Past the segment's last half tile the descriptor covers
    // zero bytes, so the copy only writes zeros into a stage that is not read
    // again; every iteration then has exactly nine copies per wave in flight.
    // Two-buffer cache: the latent lines come through rs, the rope line
    // through rp, both at half tile e of the sequence's rows.
    auto prep = [&](int e, int blk, sgpr_x4& rs, sgpr_x4& rp, uint32_t& mb) {
      mb = lds_addr(stages + (e % OSTAGE) * HT_BYTES + wave * 9 * 1024);
      if constexpr (PE) {
        const int nv = e < e1 ? max(0, min(HT_TOK, Lc - e * HT_TOK)) : 0;
        rs = buffer_rsrc(kv_seq + (int64_t)e * HT_TOK * D_C, nv * (D_C * 2));
        rp = buffer_rsrc(pe_seq + (int64_t)e * HT_TOK * D_ROPE, nv * (D_ROPE * 2));
#pragma unroll
        for (int k = 0; k < 4; ++k) {   // uniform: keep them in SGPRs
          rs[k] = (uint32_t)uni((int)rs[k]);
          rp[k] = (uint32_t)uni((int)rp[k]);
        }
        return;
      }
      rs = buffer_rsrc(a.pool, 0);
      rp = rs;
      if (e >= e1) return;
      if (blk < 0 || blk >= a.num_blocks) {
        bad = true;
        return;
      }
      const int n_valid = min(HT_TOK, L - e * HT_TOK);
      rs = buffer_rsrc((const char*)a.pool + (int64_t)blk * TILE_BYTES + (e & 1) * HT_BYTES, n_valid * ROW_BYTES);
    };
    // LDS addresses of the K fragments (stage of half tile e) and of the V^T
    // fragments (stage of half tile e), as the instruction sequences take them
    uint32_t ka[4], va[4];
    auto k_addr = [&](int e) {
      const uint32_t sb = lds_addr(stages + (e % OSTAGE) * HT_BYTES) + kbase;
#pragma unroll
      for (int q = 0; q < 4; ++q) ka[q] = sb ^ (uint32_t)(q << 5);
    };
    auto v_addr = [&](int e) {
      const uint32_t sb = lds_addr(stages + (e % OSTAGE) * HT_BYTES) + vbase;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int c1 = 0; c1 < 2; ++c1) va[c1 + 2 * rr] = sb ^ (uint32_t)((c1 << 6) | (rr << 5));
    };

    // ---- pipeline: iteration e reads stage e (V) and e+1 (K); e+2 and e+3 in flight.
    // One instruction sequence per iteration (own_asm.inc):
    //   phase S: the score MFMAs of half tile e+1 under the probability half
    //            of the softmax of half tile e (2^(s scale - mref), l, P);
    //   phase P: the PV MFMAs of e, O^T[col][row] += V^T[col][token] P^T[token][row],
    //            under the max half of the softmax of e+1 (mask, row max,
    //            alpha, running max, mref, masked scores into s).
    // Between iterations the accumulators are rescaled by alpha (rarely: the
    // running max moves only in steps above 8 in log2 units). On the last
    // half tile the scores rerun on stage e: their max never exceeds the
    // running max, so the state is left as it is.
    // Start of the segment, in one instruction sequence: the copies of half
    // tile e0, the query fragments (B operand of S^T: row r, features
    // 16 ks + 8 h .. +7) loaded straight into registers, then the copies of
    // e0+1 and e0+2; it returns once e0 and the fragments have arrived, so
    // the query loads overlap the first copies' trip to memory. A fragment
    // load reads 32 bytes of each of 32 query rows; the rows are shared by
    // the workgroups of the sequence and come from L2. Rows past the last
    // query row read as zeros (the descriptor ends there).
    u32x4 qf[KSTEPS16];
    {
      const int nv = max(0, min(128, a.rows - rg * 128));
      sgpr_x4 qr = buffer_rsrc(a.q + ((int64_t)b * a.rows + rg * 128) * D_K, nv * ROW_BYTES);
#pragma unroll
      for (int k = 0; k < 4; ++k) qr[k] = (uint32_t)uni((int)qr[k]);   // uniform: keep it in SGPRs
      const uint32_t qv = (uint32_t)((32 * wave + c32) * ROW_BYTES + 16 * h);
      sgpr_x4 rs0, rs1, rs2, rp0, rp1, rp2;
      uint32_t mb0, mb1, mb2;
      prep(e0, blk_of(e0), rs0, rp0, mb0);
      prep(e0 + 1, blk_of(e0 + 1), rs1, rp1, mb1);
      prep(e0 + 2, blk_of(e0 + 2), rs2, rp2, mb2);
      if constexpr (PE)
        asm volatile(OWNP_ASM_QLOAD
                     : OWN_OPS_Q_OUT
                     : [qv] "v"(qv), [qr] "s"(qr), [mb0] "s"(mb0), [rs0] "s"(rs0), [mb1] "s"(mb1), [rs1] "s"(rs1),
                       [mb2] "s"(mb2), [rs2] "s"(rs2), [rp0] "s"(rp0), [rp1] "s"(rp1), [rp2] "s"(rp2),
                       [go] "v"(goff), OWN_OPS_SO, OWNP_OPS_SP
                     : "m0", "scc", "memory");
      else
        asm volatile(OWN_ASM_QLOAD
                     : OWN_OPS_Q_OUT
                     : [qv] "v"(qv), [qr] "s"(qr), [mb0] "s"(mb0), [rs0] "s"(rs0), [mb1] "s"(mb1), [rs1] "s"(rs1),
                       [mb2] "s"(mb2), [rs2] "s"(rs2), [go] "v"(goff), OWN_OPS_SO
                     : "m0", "scc", "memory");
    }
    lds_barrier();                         // every wave's copies of e0 are in the LDS
    k_addr(e0);
    float s[16];          // masked scores of the half tile whose PV comes next
    float alpha, mref;    // its rescale factor and probability reference
    {
      const int lr = lim - (e0 * HT_TOK + 4 * h);
      asm volatile(OWN_ASM_PRO
                   : OWN_OPS_S_OUT, [mrun] "+v"(m_run), [alpha] "=&v"(alpha), [mref] "=&v"(mref)
                   : OWN_OPS_Q, OWN_OPS_KA, [lr] "v"(lr), [scale] "s"(a.scale_log2)
                   : OWN_CLOB, "vcc", "scc", "memory");
    }
    // Half tile e+3 goes into the stage of e-1; its nine copies are spread
    // over the iteration's instruction sequence, which keeps the vector
    // memory queue from stalling the wave. The same sequence loads the block
    // id of half tile e+4 (a scalar load issued before its first LDS read)
    // and forms the descriptor of the next iteration's copies from it under
    // its last PV MFMAs, so that nothing but the loop test, the copy wait
    // and the barrier runs between the sequences (a lone wave issues about
    // one instruction per four cycles, and the MFMA pipe idles meanwhile);
    // the K / V^T addresses and the mask limit move on inside the sequences
    // too. Descriptor: base = pool + blk * 73,728 + (ep & 1) * 36,864 (bits
    // 47..32 in its second word), bytes = 1,152 * min(32, L - 32 ep), or 0
    // past the segment or for a block id outside the pool; such an id inside
    // the segment sets badacc.
    static_assert(TILE_BYTES == 0x12000 && HT_BYTES == 0x9000 && ROW_BYTES == 0x480 && HT_TOK == 32 &&
                      OSTAGE == 4, "constants of the descriptor sequence");
    sgpr_x4 rs, rp;
    uint32_t mb;
    prep(e0 + OSTAGE - 1, blk_of(e0 + OSTAGE - 1), rs, rp, mb);
    k_addr(e0 + 1 < e1 ? e0 + 1 : e0);
    v_addr(e0);
    const uint32_t mb0 = (uint32_t)uni((int)lds_addr(stages + wave * 9 * 1024));
    const int64_t bt_u = uni64((int64_t)(uintptr_t)bt);   // the sequence's block-table row, in SGPRs
    // two-buffer cache: the sequence's latent and rope rows, as descriptor words
    const uint32_t kv_lo = (uint32_t)uni((int)(uint32_t)(uintptr_t)kv_seq);
    const uint32_t kv_hi = (uint32_t)uni((int)((uint32_t)((uintptr_t)kv_seq >> 32) & 0xffffu));
    const uint32_t pe_lo = (uint32_t)uni((int)(uint32_t)(uintptr_t)pe_seq);
    const uint32_t pe_hi = (uint32_t)uni((int)((uint32_t)((uintptr_t)pe_seq >> 32) & 0xffffu));
    const int nt1 = uni(ntiles - 1);
    mb = (uint32_t)uni((int)mb);
    uint32_t badacc = 0;
    // half tiles below e_open hold only keys every row may see (no key mask)
    const int e_open = max(0, L - a.Lq + 1) / HT_TOK;
    int lr = lim - ((e0 + 1) * HT_TOK + 4 * h);   // mask limit of the scores of e0+1 (the sequence moves it on)
    // one iteration; the first half tile of the segment (FIRST) starts the
    // PV accumulators from zero and is peeled off the loop
    auto step = [&](const int e, auto first) {
      constexpr bool FIRST = decltype(first)::value;
      const bool more = e + 1 < e1;
      wait_vmem_n<9>();          // stage e+1 complete; the copies of e+2 may be in flight
      // stage e+1 visible; stage e-1 free. The sequence ends with every LDS
      // read done, so the barrier needs no lgkmcnt wait.
      asm volatile("s_barrier" ::: "memory");
      int t0, t1, t2;
      uint32_t r0, r1, r2, r3, r4, r5, r6, r7, blkv;
#define OWNP_ITER(NAME, OPS_O)                                                                        \
  asm volatile(NAME                                                                                   \
               : OPS_O, OWN_OPS_S, [mrun] "+v"(m_run), [lrun] "+v"(l_run), [alpha] "+v"(alpha),       \
                 [mref] "+v"(mref), [lr] "+v"(lr), OWN_OPS_KA_IO, OWN_OPS_VA_IO, OWN_OPS_BOOK_OUT,    \
                 OWNP_OPS_PREP_OUT                                                                    \
               : OWN_OPS_Q, [scale] "s"(a.scale_log2), [rs] "s"(rs), [rp] "s"(rp), [go] "v"(goff),    \
                 OWN_OPS_SO, OWNP_OPS_SP, OWN_OPS_BOOK_IN, OWNP_OPS_PREP_IN                           \
               : OWN_CLOB, "vcc", "m0", "scc", "memory")
#define OWN_ITER(NAME, OPS_O)                                                                         \
  asm volatile(NAME                                                                                   \
               : OPS_O, OWN_OPS_S, [mrun] "+v"(m_run), [lrun] "+v"(l_run), [alpha] "+v"(alpha),       \
                 [mref] "+v"(mref), [lr] "+v"(lr), OWN_OPS_KA_IO, OWN_OPS_VA_IO, OWN_OPS_BOOK_OUT,    \
                 OWN_OPS_PREP_OUT                                                                     \
               : OWN_OPS_Q, [scale] "s"(a.scale_log2), [rs] "s"(rs), [go] "v"(goff), OWN_OPS_SO,      \
                 OWN_OPS_BOOK_IN, OWN_OPS_PREP_IN                                                     \
               : OWN_CLOB, "vcc", "m0", "scc", "memory")
      if constexpr (PE) {
        if constexpr (FIRST)
          OWNP_ITER(OWNP_ASM_IT_FIRST, OWN_OPS_O_OUT);
        else
          OWNP_ITER(OWNP_ASM_IT, OWN_OPS_O);
        rp = sgpr_x4{(uint32_t)uni((int)r4), (uint32_t)uni((int)r5), (uint32_t)uni((int)r6), (uint32_t)uni((int)r7)};
      } else {
        if constexpr (FIRST)
          OWN_ITER(OWN_ASM_IT_FIRST, OWN_OPS_O_OUT);
        else
          OWN_ITER(OWN_ASM_IT, OWN_OPS_O);
      }
#undef OWN_ITER
#undef OWNP_ITER
      // the copies of half tile e+4, issued by the next sequence. The values
      // are in SGPRs, but an asm statement with vector outputs counts as
      // divergent to the compiler: readfirstlane marks them uniform, so that
      // the loop carries them in SGPRs.
      rs = sgpr_x4{(uint32_t)uni((int)r0), (uint32_t)uni((int)r1), (uint32_t)uni((int)r2), (uint32_t)uni((int)r3)};
      mb = (uint32_t)uni((int)mb);
      badacc = (uint32_t)uni((int)badacc);
      // alpha belongs to half tile e+1, whose PV runs in the next iteration
      if (more && __any(alpha != 1.f)) {
        // the sequence's last PV MFMAs may still be writing the accumulators
        asm volatile(OWN_ASM_GUARD ::: "memory");
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) scale_acc(o[cb], alpha);
      }
    };
    step(e0, std::true_type{});
    for (int e = e0 + 1; e < e1; ++e) step(e, std::false_type{});
    asm volatile(OWN_ASM_GUARD ::: "memory");   // PV results settle before the epilogue reads them
    if (badacc) bad = true;

    // ---- finish the segment. Both outputs hold o / l in bf16 (the final
    // o_lat, or a partial for the merge): each wave writes its 32 rows into
    // LDS (the stages are free now), then every wave stores whole 1 KiB rows,
    // one row per instruction.
    l_run += __shfl_xor(l_run, 32);
    {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      // the copies issued past the segment's end (zero-byte descriptors) still
      // write zeros into their stages: let them land before the staging
      wait_vmem_n<0>();
      lds_barrier();                       // every wave is done with the stages
      lds_char* orow_l = stages + (32 * wave + c32) * OUT_STRIDE + 8 * h;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v0 = o[cb][4 * j] * inv, v1 = o[cb][4 * j + 1] * inv;
          float v2 = o[cb][4 * j + 2] * inv, v3 = o[cb][4 * j + 3] * inv;
          if (bad) v0 = v1 = v2 = v3 = NAN;
          *(__attribute__((address_space(3))) u32x2*)(orow_l + (32 * cb + 8 * j) * 2) =
              u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        }
      lds_barrier();
      uint16_t* dst = whole ? a.o_lat + (int64_t)b * a.rows * D_C
                            : a.ws_acc + (int64_t)(w + b) * a.rows * D_C;
#pragma unroll 4
      for (int i = 0; i < 32; ++i) {
        const int rl = 32 * wave + i;            // row within the group
        const int rr = rg * 128 + rl;            // row within the sequence
        if (rr >= a.rows) break;
        const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(stages + rl * OUT_STRIDE + 16 * lane);
        *(u32x4*)(dst + (int64_t)rr * D_C + 8 * lane) = v;
      }
      if (r < a.rows && h == 0) {
        if (whole) {
          if (a.lse) {
            const float lv = l_run > 0.f ? (m_run + __log2f(l_run)) * LN2 : -INFINITY;
            a.lse[(int64_t)b * a.rows + r] = bad ? NAN : lv;
          }
        } else {
          const int64_t prow = (int64_t)(w + b) * a.rows + r;
          a.ws_ml[prow * 2 + 0] = bad ? NAN : m_run;
          a.ws_ml[prow * 2 + 1] = bad ? NAN : l_run;
        }
      }
    }
    x = seg_end;
    seq_start += ntiles;
    ++b;
    while (b < a.B && tiles_of(uni(a.seq_lens[b]), a.max_blocks) == 0) ++b;
    lds_barrier();
  }
}

// Merge the partials of each query row in range order. One wave per row,
// 8 output columns per lane. The lengths are read once; the (m, l) pairs of
// the first 64 ranges and the first 8 partial rows are requested together,
// so a row with up to 8 partials costs two memory round trips.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rb = (a.rows + 3) >> 2;           // workgroups per sequence, four rows each
  // Workgroups are dealt to the 8 XCDs round-robin by id. The split kernels
  // give each XCD a contiguous run of ranges (so the partials of one
  // sequence sit in that XCD's L2); give each XCD the same contiguous run of
  // (sequence, rows) items here, so that the merge reads them from there.
  unsigned item = blockIdx.x;
  if ((gridDim.x & 7) == 0) item = (item & 7) * (gridDim.x >> 3) + (item >> 3);
  const int b = (int)(item / (unsigned)rb);
  const int r = (int)(item - (unsigned)b * (unsigned)rb) * 4 + wave;
  if (r >= a.rows) return;
  // total tiles T, first tile of sequence b, and its tile count
  int64_t T = 0, start = 0;
  int ntiles = 0;
  for (int base = 0; base < a.B; base += 64) {
    const int bb = base + lane;
    const int t = bb < a.B ? tiles_of(a.seq_lens[bb], a.max_blocks) : 0;
    T += wave_sum_i(t);
    start += wave_sum_i(bb < b ? t : 0);
    if (b >= base && b < base + 64) ntiles = __shfl(t, b - base);
  }
  const int64_t orow = (int64_t)b * a.rows + r;
  uint16_t* out = a.o_lat + orow * D_C + 8 * lane;
  if (ntiles == 0) {
    *(u32x4*)out = u32x4{0u, 0u, 0u, 0u};
    if (a.lse && lane == 0) a.lse[orow] = -INFINITY;
    return;
  }
  const int w_lo = plan_owner(start, T, a.width);
  const int w_hi = plan_owner(start + ntiles - 1, T, a.width);
  if (w_lo == w_hi) return;  // one range held the whole sequence and wrote it

  // Ranges between w_lo and w_hi all lie inside sequence b, except empty ones
  // (more workgroups than tiles), which wrote nothing and get weight 0. They
  // are taken 64 at a time: lane k holds (m, l) of range c + k; the partial
  // rows are loaded eight at a time.
  auto empty = [&](int w) { return (int64_t)w * T / a.width == (int64_t)(w + 1) * T / a.width; };
  auto load_ml = [&](int c) -> float2 {
    const int w = c + lane;
    if (w > w_hi || empty(w)) return float2{-INFINITY, 0.f};
    return *(const float2*)(a.ws_ml + ((int64_t)(w + b) * a.rows + r) * 2);
  };
  auto load_rows = [&](int c, int cnt, int k0, u32x4 (&v)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // ranges past the last one read row c (in bounds); their weight is 0
      const int k = k0 + u < cnt ? k0 + u : 0;
      v[u] = *(const u32x4*)(a.ws_acc + ((int64_t)(c + k + b) * a.rows + r) * D_C + 8 * lane);
    }
  };
  const int cnt0 = min(64, w_hi - w_lo + 1);
  const float2 ml0 = load_ml(w_lo);
  u32x4 v[8];
  load_rows(w_lo, cnt0, 0, v);
  float M = wave_max_f(ml0.x);
  for (int c = w_lo + 64; c <= w_hi; c += 64) M = fmaxf(M, wave_max_f(load_ml(c).x));
  const float Mref = M == -INFINITY ? 0.f : M;
  // partial k holds o_k / l_k: weight it by l_k 2^(m_k - M)
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  for (int c = w_lo; c <= w_hi; c += 64) {
    const float2 ml = c == w_lo ? ml0 : load_ml(c);
    const float wt = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - Mref) * ml.y;
    l += wave_sum_f(wt);
    const int cnt = min(64, w_hi - c + 1);
    for (int k0 = 0; k0 < cnt; k0 += 8) {
      if (c != w_lo || k0 != 0) load_rows(c, cnt, k0, v);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wk = k0 + u < cnt ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), k0 + u)) : 0.f;
        if (wk != 0.f) {   // empty ranges hold no data
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += wk * bf16_to_f32((uint16_t)(v[u][i] & 0xffffu));
            acc[2 * i + 1] += wk * bf16_to_f32((uint16_t)(v[u][i] >> 16));
          }
        }
      }
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *(u32x4*)out = o;
  if (a.lse && lane == 0) a.lse[orow] = l > 0.f ? (M + __log2f(l)) * LN2 : (l != l ? NAN : -INFINITY);
}

// ------------------------------------------------------ 128 rows, FP8 pool
//
// attn_own_kernel over the FP8 pool (E4M3 codes [num_blocks][64][576] and
// power-of-two token scales [num_blocks][64]). Each wave copies its 8 tokens'
// codes (4,608 bytes, as five 1-KiB copies) and their scales into a staging
// slot of its own and widens them, the scale folded into the conversion,
// into the bf16 half-tile stages the same products read: code x 2^k is a
// bf16 value, so the stage holds the row exactly and everything after it is
// the bf16 kernel's arithmetic. Three stages (V of e, K of e+1, e+2 being
// widened) and two staging slots per wave (e+2 being widened, e+3 in flight;
// e+4 is copied into e+2's slot once it has been read). The widening and the
// copies are part of the iteration sequences (OWN8_ASM_*, own_asm.inc).
constexpr int FSTAGE = 3;
constexpr int F8_STG = 5376;                  // staging slot: 5,120 bytes of codes, 256 of scales
constexpr int F8_SC_OFF = 5120;
constexpr int HT_BYTES8 = HT_TOK * D_K;       // 18,432 code bytes per half tile
constexpr int TILE_BYTES8_ = BLOCK * D_K;     // 36,864 code bytes per block
static_assert(OUT_STRIDE * 128 <= FSTAGE * HT_BYTES + 8 * F8_STG, "output staging fits the FP8 kernel's LDS");

// Widen half tile e's codes from this wave's staging slot src into the bf16
// stage dst (this wave's 8 tokens, the layout of ht_off); the slot holds the
// 64 scales of e's block. A token at or past nv (past the sequence, codes
// zero-filled) takes scale 1.
__device__ __forceinline__ void widen8(const lds_char* src, lds_char* dst, int e, int wave, int lane, int nv) {
  const int tl = lane >> 3;
  float sc = *(const __attribute__((address_space(3))) float*)(src + F8_SC_OFF + 4 * (32 * (e & 1) + 8 * wave + tl));
  if (8 * wave + tl >= nv) sc = 1.f;
  const uint32_t rd = (uint32_t)(tl * D_K + 8 * ((lane & 7) ^ swz2(8 * wave + tl)));
  const uint32_t wr = (uint32_t)(wave * 9 * 1024 + lane * 16);
#pragma unroll
  for (int c = 0; c < 9; ++c) {
    const u32x2 v = *(const __attribute__((address_space(3))) u32x2*)(src + rd + 64 * c);
    u32x4 w4;
    w4[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], sc, false));
    w4[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], sc, true));
    w4[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], sc, false));
    w4[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], sc, true));
    *(__attribute__((address_space(3))) u32x4*)(dst + wr + 1024 * c) = w4;
  }
}

__global__ __launch_bounds__(256, 1) void attn_own8_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[FSTAGE * HT_BYTES + 8 * F8_STG];
  lds_char* stages = (lds_char*)smem;

  const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c32 = lane & 31, h = lane >> 5;
  lds_char* stg = stages + FSTAGE * HT_BYTES + wave * 2 * F8_STG;   // this wave's two staging slots

  int unit = blockIdx.x;
  if ((gridDim.x & 7) == 0) unit = (unit & 7) * (int)(gridDim.x >> 3) + (unit >> 3);
  const int w = unit / a.n_rg;
  const int rg = unit - w * a.n_rg;
  const int64_t T = plan_total_tiles(a.seq_lens, a.B, a.max_blocks);
  if (T == 0) return;
  const int64_t x_begin = (int64_t)w * T / a.width;
  const int64_t x_end = (int64_t)(w + 1) * T / a.width;
  if (x_begin >= x_end) return;
  int b;
  int64_t seq_start;
  plan_find(a.seq_lens, a.B, a.max_blocks, x_begin, b, seq_start);

  const int r = rg * 128 + 32 * wave + c32;
  const uint32_t kbase = ht_off(c32, h);       // as in attn_own_kernel
  uint32_t vbase;
  {
    const int i16 = lane & 15, q = lane >> 4;
    const int tl = 4 * (q >> 1) + (i16 >> 2);
    const int e = 2 * (q & 1) + ((i16 & 3) >> 1);
    vbase = ht_off(tl, e) + 8 * (i16 & 1);
  }
  // copies: lane l moves bytes 16 l (+ 1,024 c) of the wave's 4,608 and
  // scale l of the half tile's block (the sequences derive both offsets
  // from go8 = 16 l)
  const uint32_t go8 = (uint32_t)(lane * 16);
  const uint32_t so8 = (uint32_t)uni(wave * 8 * D_K);
  // widening: the lane's token within the half tile, and the staging offset
  // of its chunk (codes of chunk group c at staging + rdo + 64 c; the bf16
  // chunk goes to stage + 9,216 wave + go8 + 1,024 c)
  const uint32_t tlw = (uint32_t)(8 * wave + (lane >> 3));
  const uint32_t rdo = (uint32_t)((lane >> 3) * D_K + 8 * ((lane & 7) ^ swz2(8 * wave + (lane >> 3))));
  const uint8_t* pool8 = (const uint8_t*)a.pool;
  const uint32_t pool_lo = (uint32_t)uni((int)(uint32_t)(uintptr_t)pool8);
  const uint32_t pool_hi = (uint32_t)uni((int)((uint32_t)((uintptr_t)pool8 >> 32) & 0xffffu));
  const uint32_t nblk = (uint32_t)uni((int)min(a.num_blocks, (int64_t)0x7fffffff));
  const uint32_t stg_lds = (uint32_t)uni((int)lds_addr(stg));

  int64_t x = x_begin;
  while (x < x_end && b < a.B) {
    const int L = uni(a.seq_lens[b]);
    const int ntiles = tiles_of(L, a.max_blocks);
    const int64_t seg_end = min(x_end, seq_start + ntiles);
    const int k_first = (int)(x - seq_start);
    const int k_last = (int)(seg_end - seq_start);
    const bool whole = (x == seq_start) && (seg_end == seq_start + ntiles);
    bool bad = L > a.max_keys;
    const int key_end = min(k_last * BLOCK, L);
    const int e0 = 2 * k_first, e1 = (key_end + HT_TOK - 1) / HT_TOK;

    const int lim = r < a.rows ? L - a.Lq + r / a.H : -1;
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[16];

    const __attribute__((address_space(4))) int32_t* bt =
        (const __attribute__((address_space(4))) int32_t*)(a.block_table + (int64_t)b * a.max_blocks);
    // valid tokens of half tile e (0 past the segment)
    auto nv_of = [&](int e) { return e < e1 ? min(HT_TOK, L - e * HT_TOK) : 0; };
    // copies of half tile e from block blk: codes at pool8 + blk * 36,864 +
    // (e & 1) * 18,432 (nv * 576 bytes; none past the segment or for a block
    // id outside the pool), the block's 64 scales at pool_scale + blk * 64
    // (the pool's first 64, a safe address, when there are no codes)
    auto prep8 = [&](int e, int blk, sgpr_x4& rs, uint64_t& sb) {
      const bool in_seg = e < e1;
      const bool ok = (uint32_t)blk < nblk;
      if (in_seg && !ok) bad = true;
      const bool use = in_seg && ok;
      const uint64_t base = ((uint64_t)pool_hi << 32 | pool_lo) + (uint64_t)(uint32_t)blk * TILE_BYTES8_ +
                            (uint32_t)(e & 1) * HT_BYTES8;
      const uint32_t bytes = use ? (uint32_t)nv_of(e) * D_K : 0u;
      rs = use ? sgpr_x4{(uint32_t)base, (uint32_t)(base >> 32) & 0xffffu, bytes, 0x00020000u}
               : sgpr_x4{pool_lo, pool_hi, 0u, 0x00020000u};
      const uint64_t sc0 = (uint64_t)(uintptr_t)a.pool_scale;
      sb = use ? sc0 + (uint64_t)(uint32_t)blk * BLOCK * 4 : sc0;
    };
    auto blk_of = [&](int e) { return bt[min(e >> 1, ntiles - 1)]; };
    uint32_t ka[4], va[4];
    auto k_addr = [&](int e) {
      const uint32_t sbk = lds_addr(stages + (e % FSTAGE) * HT_BYTES) + kbase;
#pragma unroll
      for (int q = 0; q < 4; ++q) ka[q] = sbk ^ (uint32_t)(q << 5);
    };
    auto v_addr = [&](int e) {
      const uint32_t sbv = lds_addr(stages + (e % FSTAGE) * HT_BYTES) + vbase;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int c1 = 0; c1 < 2; ++c1) va[c1 + 2 * rr] = sbv ^ (uint32_t)((c1 << 6) | (rr << 5));
    };

    // ---- segment start: half tiles e0 and e0+1 copied (with the query
    // fragments between them) and widened, then e0+2 and e0+3 copied
    u32x4 qf[KSTEPS16];
    {
      const int nv = max(0, min(128, a.rows - rg * 128));
      sgpr_x4 qr = buffer_rsrc(a.q + ((int64_t)b * a.rows + rg * 128) * D_K, nv * ROW_BYTES);
#pragma unroll
      for (int k = 0; k < 4; ++k) qr[k] = (uint32_t)uni((int)qr[k]);
      const uint32_t qv = (uint32_t)((32 * wave + c32) * ROW_BYTES + 16 * h);
      sgpr_x4 rs0, rs1;
      uint64_t sb0, sb1;
      prep8(e0, blk_of(e0), rs0, sb0);
      prep8(e0 + 1, blk_of(e0 + 1), rs1, sb1);
      const uint32_t mb0 = stg_lds + (uint32_t)(e0 & 1) * F8_STG, mb1 = stg_lds + (uint32_t)((e0 + 1) & 1) * F8_STG;
      const uint32_t go8b = go8 + 4096, soff = go8 >> 2;
      asm volatile(OWN8_ASM_QLOAD
                   : OWN_OPS_Q_OUT
                   : [qv] "v"(qv), [qr] "s"(qr), [mb0] "s"(mb0), [rs0] "s"(rs0), [sb0] "s"(sb0), [mb1] "s"(mb1),
                     [rs1] "s"(rs1), [sb1] "s"(sb1), [go8] "v"(go8), [go8b] "v"(go8b), [so8] "s"(so8),
                     [soff] "v"(soff)
                   : "m0", "scc", "memory");
      widen8(stg + (e0 & 1) * F8_STG, stages + (e0 % FSTAGE) * HT_BYTES, e0, wave, lane, nv_of(e0));
      widen8(stg + ((e0 + 1) & 1) * F8_STG, stages + ((e0 + 1) % FSTAGE) * HT_BYTES, e0 + 1, wave, lane,
             nv_of(e0 + 1));
      prep8(e0 + 2, blk_of(e0 + 2), rs0, sb0);
      prep8(e0 + 3, blk_of(e0 + 3), rs1, sb1);
      asm volatile(OWN8_ASM_COPY
                   :
                   : [mb0] "s"(mb0), [rs0] "s"(rs0), [sb0] "s"(sb0), [mb1] "s"(mb1), [rs1] "s"(rs1), [sb1] "s"(sb1),
                     [go8] "v"(go8), [go8b] "v"(go8b), [so8] "s"(so8), [soff] "v"(soff)
                   : "m0", "scc", "memory");
    }
    lds_barrier();                         // every wave's e0 and e0+1 are widened
    k_addr(e0);
    float s[16];
    float alpha, mref;
    {
      const int lr = lim - (e0 * HT_TOK + 4 * h);
      asm volatile(OWN8_ASM_PRO
                   : OWN_OPS_S_OUT, [mrun] "+v"(m_run), [alpha] "=&v"(alpha), [mref] "=&v"(mref)
                   : OWN_OPS_Q, OWN_OPS_KA, [lr] "v"(lr), [scale] "s"(a.scale_log2)
                   : OWN8_CLOB, "vcc", "scc", "memory");
    }
    // iteration e widens e+2 and copies e+4 (prepared at the end of e-1)
    sgpr_x4 rs;
    uint64_t sb;
    prep8(e0 + 4, blk_of(e0 + 4), rs, sb);
    uint32_t mb8 = stg_lds + (uint32_t)(e0 & 1) * F8_STG;           // staging slot of e+2 and e+4
    int nv2 = nv_of(e0 + 2);
    int r3 = e0 % FSTAGE;
    // stage of e+2 plus this wave's 9 lines: where the widening writes
    const uint32_t stage0 = (uint32_t)uni((int)lds_addr(stages)) + (uint32_t)(wave * 9 * 1024);
    auto cwb_of = [&](int r) { return stage0 + (uint32_t)((r + 2) % FSTAGE) * HT_BYTES; };
    uint32_t cwb = cwb_of(r3);
    k_addr(e0 + 1 < e1 ? e0 + 1 : e0);
    v_addr(e0);
    const int e_open = max(0, L - a.Lq + 1) / HT_TOK;
    int lr = lim - ((e0 + 1) * HT_TOK + 4 * h);
    auto step = [&](const int e, auto first) {
      constexpr bool FIRST = decltype(first)::value;
      const bool more = e + 1 < e1;
      wait_vmem_n<6>();        // e+2's codes and scales are in this wave's staging; e+3 may be in flight
      asm volatile("s_barrier" ::: "memory");   // stage e+1 widened by every wave; stage of e-1 free
      const int blk_next = blk_of(e + 5);
      int t0, t1, t2;
#define OWN8_ITER(NAME, OPS_O)                                                                         \
  asm volatile(NAME                                                                                    \
               : OPS_O, OWN_OPS_S, [mrun] "+v"(m_run), [lrun] "+v"(l_run), [alpha] "+v"(alpha),        \
                 [mref] "+v"(mref), [lr] "+v"(lr), OWN_OPS_KA_IO, OWN_OPS_VA_IO, OWN_OPS_BOOK_OUT      \
               : OWN_OPS_Q, [scale] "s"(a.scale_log2), [rs] "s"(rs), [sb] "s"(sb), [so8] "s"(so8),     \
                 [go8] "v"(go8), [rdo] "v"(rdo), [tlw] "v"(tlw), [mb8] "s"(mb8), [cwb] "s"(cwb),       \
                 [nv2] "s"(nv2), [ep] "s"(e + 4), [eo] "s"(e_open), [e1] "s"(e1), [r3] "s"(r3)         \
               : OWN8_CLOB, "vcc", "m0", "scc", "memory")
      if constexpr (FIRST)
        OWN8_ITER(OWN8_ASM_IT_FIRST, OWN_OPS_O_OUT);
      else
        OWN8_ITER(OWN8_ASM_IT, OWN_OPS_O);
#undef OWN8_ITER
      if (more && __any(alpha != 1.f)) {
        asm volatile(OWN_ASM_GUARD ::: "memory");
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) scale_acc(o[cb], alpha);
        // The rescale borrows registers and may reload spilled values from
        // scratch; wait for them here (the compiler sees this wait), so
        // that the loop head needs none: a wait there would also drain the
        // copies in flight every iteration. Rescales are rare.
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      }
      prep8(e + 5, blk_next, rs, sb);
      mb8 = stg_lds + (uint32_t)((e + 1) & 1) * F8_STG;
      nv2 = nv_of(e + 3);
      r3 = r3 == FSTAGE - 1 ? 0 : r3 + 1;
      cwb = cwb_of(r3);
    };
    step(e0, std::true_type{});
    for (int e = e0 + 1; e < e1; ++e) step(e, std::false_type{});
    asm volatile(OWN_ASM_GUARD ::: "memory");

    l_run += __shfl_xor(l_run, 32);
    {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      wait_vmem_n<0>();                    // copies past the segment's end still write their slots
      lds_barrier();
      lds_char* orow_l = stages + (32 * wave + c32) * OUT_STRIDE + 8 * h;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v0 = o[cb][4 * j] * inv, v1 = o[cb][4 * j + 1] * inv;
          float v2 = o[cb][4 * j + 2] * inv, v3 = o[cb][4 * j + 3] * inv;
          if (bad) v0 = v1 = v2 = v3 = NAN;
          *(__attribute__((address_space(3))) u32x2*)(orow_l + (32 * cb + 8 * j) * 2) =
              u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        }
      lds_barrier();
      uint16_t* dst = whole ? a.o_lat + (int64_t)b * a.rows * D_C
                            : a.ws_acc + (int64_t)(w + b) * a.rows * D_C;
#pragma unroll 4
      for (int i = 0; i < 32; ++i) {
        const int rl = 32 * wave + i;
        const int rr = rg * 128 + rl;
        if (rr >= a.rows) break;
        const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(stages + rl * OUT_STRIDE + 16 * lane);
        *(u32x4*)(dst + (int64_t)rr * D_C + 8 * lane) = v;
      }
      if (r < a.rows && h == 0) {
        if (whole) {
          if (a.lse) {
            const float lv = l_run > 0.f ? (m_run + __log2f(l_run)) * LN2 : -INFINITY;
            a.lse[(int64_t)b * a.rows + r] = bad ? NAN : lv;
          }
        } else {
          const int64_t prow = (int64_t)(w + b) * a.rows + r;
          a.ws_ml[prow * 2 + 0] = bad ? NAN : m_run;
          a.ws_ml[prow * 2 + 1] = bad ? NAN : l_run;
        }
      }
    }
    x = seg_end;
    seq_start += ntiles;
    ++b;
    while (b < a.B && tiles_of(uni(a.seq_lens[b]), a.max_blocks) == 0) ++b;
    lds_barrier();
  }
}

// ------------------------------------------------------------------ host side

// pe != null: the two-buffer layout, pool = kv_cache, max_keys = max_seq
// (max_blocks = ceil(max_seq / 64), no block table); otherwise the paged pool
// (max_keys = max_blocks * 64).
static hipError_t launch_attention(const uint16_t* q, const void* pool, const uint16_t* pe,
                                   const float* pool_scale, int64_t num_blocks, const int32_t* block_table,
                                   int32_t max_blocks, int32_t max_keys, const int32_t* seq_lens, int32_t B,
                                   int32_t Lq, int32_t H, float softmax_scale, uint16_t* o_lat, float* lse,
                                   void* workspace, hipStream_t stream) {
  const bool fp8 = pool_scale != nullptr;
  const AttnPlan p = fp8 ? plan_attention_fp8(B, Lq, H) : pe ? plan_attention_kvpe(B, Lq, H) : plan_attention(B, Lq, H);
  AttnArgs a;
  a.q = q;
  a.pool = (const uint16_t*)pool;
  a.pool_scale = pool_scale;
  a.pe = pe;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.o_lat = o_lat;
  a.lse = lse;
  a.ws_ml = (float*)workspace;
  a.ws_acc = (uint16_t*)((char*)workspace + attention_ws_ml_bytes(B, Lq, H));
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  a.max_keys = max_keys;
  a.B = B;
  a.Lq = Lq;
  a.H = H;
  a.rows = Lq * H;
  a.n_rg = p.n_rg;
  a.width = p.width;
  a.scale_log2 = softmax_scale * 1.44269504088896340736f;
  const dim3 grid(p.width * p.n_rg);
  if (fp8) {
    if (p.variant == V_ROWS128) hipLaunchKernelGGL(attn_own8_kernel, grid, dim3(256), 0, stream, a);
    else if (p.variant == V_COLS16) hipLaunchKernelGGL((attn_cols_kernel<1, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((attn_cols_kernel<2, true>), grid, dim3(256), 0, stream, a);
  } else switch (p.variant) {
    case V_ROWS128:
      if (pe) hipLaunchKernelGGL(attn_own_kernel<true>, grid, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL(attn_own_kernel<false>, grid, dim3(256), 0, stream, a);
      break;
    case V_ROWS64:
      hipLaunchKernelGGL(attn_rows_kernel<1>, grid, dim3(256), 0, stream, a);
      break;
    case V_COLS32:
      hipLaunchKernelGGL((attn_cols_kernel<2>), grid, dim3(256), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((attn_cols_kernel<1>), grid, dim3(256), 0, stream, a);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)B * (unsigned)((a.rows + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_attn(const uint16_t* q, const uint16_t* pool, int64_t num_blocks,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H,
                              float softmax_scale, uint16_t* o_lat, float* lse, void* workspace,
                              hipStream_t stream) {
  return launch_attention(q, pool, nullptr, nullptr, num_blocks, block_table, max_blocks, max_blocks * BLOCK,
                          seq_lens, B, Lq, H, softmax_scale, o_lat, lse, workspace, stream);
}

hipError_t launch_decode_attn_kvpe(const uint16_t* q, const uint16_t* kv_cache, const uint16_t* pe_cache,
                                   int32_t max_seq, const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H,
                                   float softmax_scale, uint16_t* o_lat, float* lse, void* workspace,
                                   hipStream_t stream) {
  return launch_attention(q, kv_cache, pe_cache, nullptr, 0, nullptr, (max_seq + BLOCK - 1) / BLOCK, max_seq,
                          seq_lens, B, Lq, H, softmax_scale, o_lat, lse, workspace, stream);
}

hipError_t launch_decode_attn_fp8(const uint16_t* q, const uint8_t* pool8, const float* pool_scale,
                                  int64_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H,
                                  float softmax_scale, uint16_t* o_lat, float* lse, void* workspace,
                                  hipStream_t stream) {
  return launch_attention(q, pool8, nullptr, pool_scale, num_blocks, block_table, max_blocks, max_blocks * BLOCK,
                          seq_lens, B, Lq, H, softmax_scale, o_lat, lse, workspace, stream);
}

// ----------------------------------------------- without allocation
//
// For callers that cannot allocate (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc): the partials go to a fixed device
// array instead of a caller workspace. Each GPU the library runs on holds its
// own copy of the array until the process ends; every call on that GPU uses
// it, so calls that overlap in time on one GPU (other streams, other host
// threads) race. Nothing in it needs to start at a given value: each call
// writes every partial before its merge reads it.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
static std::mutex scratch_mu;
static void* scratch_dev[MAX_DEVICES];   // device address of `scratch` on each GPU

// Device address of this GPU's copy of `scratch`, looked up once per device
// with that device current. (In host code the array's name is only a
// stand-in: its address is not the device's.)
static hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return hipSuccess;
}

hipError_t launch_decode_attn_noalloc(const uint16_t* q, const uint16_t* pool, int64_t num_blocks,
                                      const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                                      int32_t B, int32_t Lq, int32_t H, float softmax_scale, uint16_t* o_lat,
                                      float* lse, hipStream_t stream) {
  if (attention_workspace_bytes(B, Lq, H) > NOALLOC_SCRATCH_BYTES) return hipErrorInvalidValue;
  if (stream) {
    int cur = -1, sdev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != cur) return hipErrorInvalidDevice;
  }
  void* ws = nullptr;
  const hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return e;
  return launch_attention(q, pool, nullptr, nullptr, num_blocks, block_table, max_blocks, max_blocks * BLOCK,
                          seq_lens, B, Lq, H, softmax_scale, o_lat, lse, ws, stream);
}

}  // namespace mla
