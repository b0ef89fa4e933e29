/*
 * libmla_absorb — weight-absorbed Multi-head Latent Attention (MLA) decode
 * over a paged latent cache (bf16 rows, or FP8 codes with a per-token scale),
 * for AMD MI355X (gfx950).
 *
 * Sources, cited by title and section:
 *   [AUDIT]  llm-atlas page "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界"
 *   [MLA80]  CSDN page "80 行 PyTorch 从零写 DeepSeek 的 MLA"
 *   [TRACE]  llm-atlas page "DeepSeek-V2-Lite 真实权重执行审计"
 *
 * One decode step of one attention layer is four calls on one stream:
 *   mla_cache_append  -> mla_absorb_q -> mla_decode_attn -> mla_out_up
 * (the first two may be one launch, mla_append_absorb; the _fp8 calls take
 * the FP8 cache in place of the bf16 pool).
 *
 * Conventions shared by every call
 *   - bf16 tensors are passed as uint16_t bit patterns; every tensor is dense
 *     row-major with the shape given at its argument.
 *   - Every pointer named "device" is caller-owned device memory. The library
 *     never allocates, frees or synchronises inside these calls; all work is
 *     enqueued on `stream` (a hipStream_t; NULL = the null stream) in call order.
 *   - Return value: MLA_OK (0) or a negative mla_status. Arguments are checked
 *     on the host before anything is enqueued; on an error nothing is enqueued.
 *     Device-resident values (positions, slots, block ids, lengths) cannot be
 *     checked on the host: the kernels bound-check them as stated per call so
 *     that a bad value never reads or writes outside the buffers.
 *   - Cache layout: pool[num_blocks][block_size=64][576] bf16, one 1,152-byte row
 *     per token: [c_kv (512) | RoPE(k_pe) (64)] ([AUDIT] §2.4 and §6.1 MQA mode
 *     head_dim_k = 576; [TRACE] §3.1 the [B,T,576] projection).
 *   - A token at absolute position p of sequence b lives at slot
 *     block_table[b][p / 64] * 64 + p % 64.
 *   - Alignment: the kernels move rows with 16-byte vector accesses. The
 *     append, absorb and up-projection calls (and their fused and _fp8 /
 *     _kvpe variants) return MLA_ERR_INVALID_ARG unless c_kv, the pool (or
 *     kv_cache, or the FP8 codes and scales), q_nope, W_UK, the absorbed
 *     queries, o_lat, W_UV and o are 16-byte aligned, k_pe, q_pe, pos,
 *     seq_idx and pe_cache 4-byte aligned and slot_mapping 8-byte aligned;
 *     the attention calls state theirs.
 */
#ifndef MLA_ABSORB_H
#define MLA_ABSORB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, bad dims value */
  MLA_ERR_UNSUPPORTED = -2,   /* a dims value outside what the kernels implement */
  MLA_ERR_WORKSPACE = -3,     /* workspace missing or smaller than mla_decode_workspace_size */
  MLA_ERR_LAUNCH = -4,        /* the HIP runtime reported an error at launch */
} mla_status;

/* Layer shape. The kernels implement d_c = 512, d_rope = 64, d_nope = 128,
 * d_v = 128, block_size = 64 (V2-Lite / V2 / V3 attention: [TRACE] §1.2,
 * [MLA80] §1) and 1 <= num_heads <= 128 with num_heads % 16 == 0 for the
 * attention call. softmax_scale is 1/sqrt(d_nope + d_rope): the naive path
 * attends over 192-wide heads with SDPA's default scale ([MLA80] §2
 * MLA.forward). rope_base is 10000 ([MLA80] appendix A build_rope). */
typedef struct mla_dims {
  int32_t num_heads;
  int32_t d_c;
  int32_t d_rope;
  int32_t d_nope;
  int32_t d_v;
  int32_t block_size;
  float softmax_scale;
  float rope_base;
} mla_dims;

/* Fills `d` with the defaults above for `num_heads` heads. */
void mla_dims_default(mla_dims* d, int32_t num_heads);

/* Human-readable name of a status code (static storage). */
const char* mla_status_str(int status);

/*
 * mla_cache_append — write T new tokens into the paged latent cache.
 * For each token j: row = [c_kv[j] | RoPE(k_pe[j], pos[j])], stored at
 * pool slot slot_mapping[j]. RoPE rotates interleaved pairs (2i, 2i+1) by
 * pos * rope_base^(-2i/64) ([MLA80] appendix A); the rope key is shared by all
 * heads and cached once per token ([MLA80] §2, [AUDIT] §2.4). It is rotated
 * once here instead of at every step ([MLA80] §2 rotates the cached k_R each
 * forward; the score is the same because the rotation depends only on the
 * key's own position).
 *   c_kv          device [T][512] bf16   latent of each new token
 *   k_pe          device [T][64]  bf16   un-rotated rope key of each new token
 *   pos           device [T]      int32  absolute position of each token
 *   slot_mapping  device [T]      int64  destination slot; a slot outside
 *                                        [0, num_blocks*64) is skipped (no write)
 *   pool          device [num_blocks][64][576] bf16, updated in place
 * The c_kv half is copied bit-exactly; the rope half is computed with an fp64
 * angle and rotation and rounded once to bf16 (nearest even).
 */
int mla_cache_append(const mla_dims* dims, const uint16_t* c_kv, const uint16_t* k_pe,
                     const int32_t* pos, const int64_t* slot_mapping, uint16_t* pool,
                     int64_t num_blocks, int32_t T, void* stream);

/*
 * mla_absorb_q — absorb W_UK into the query and rotate its rope part.
 * q[n][h] = [ W_UK[h]^T q_nope[n][h] (512) | RoPE(q_pe[n][h], pos[n]) (64) ]
 * ([AUDIT] §2.2: q^T (W_K c) = (W_K^T q)^T c; [MLA80] §4 Path B and §5).
 *   q_nope  device [N][H][128] bf16
 *   q_pe    device [N][H][64]  bf16 (un-rotated)
 *   pos     device [N] int32   absolute position of each query token
 *   w_uk    device [H][128][512] bf16  per-head [d_nope x d_c] up-projection
 *                               (the head's rows of nn.Linear(d_c, H*d_nope).weight)
 *   q_out   device [N][H][576] bf16
 * The 128-long contraction accumulates in fp32 (bf16 MFMA) and is rounded once
 * to bf16. N above 2^22 gives MLA_ERR_UNSUPPORTED (as for mla_append_absorb
 * and mla_out_up).
 */
int mla_absorb_q(const mla_dims* dims, const uint16_t* q_nope, const uint16_t* q_pe,
                 const int32_t* pos, const uint16_t* w_uk, uint16_t* q_out, int32_t N,
                 void* stream);

/*
 * mla_decode_workspace_size — bytes of device workspace mla_decode_attn needs
 * for B sequences of Lq queries each (partial results of the key-range splits).
 * Pure host arithmetic; depends only on its arguments. 0 for arguments the
 * attention calls reject (invalid dims, B or Lq <= 0, Lq*H above 2^20, or
 * B*ceil(Lq*H/4) above 2^31-1).
 */
size_t mla_decode_workspace_size(const mla_dims* dims, int32_t B, int32_t Lq);

/*
 * mla_decode_attn — latent attention over the paged cache, split over the
 * key range and merged.
 * For query row (b, i, h), at absolute position p = seq_lens[b] - Lq + i:
 *   s_t   = softmax_scale * (q[:512] . C_t[:512] + q[512:] . C_t[512:]),  t <= p
 *   o_lat = sum_t softmax(s)_t C_t[:512],   lse = log sum_t exp(s_t)
 * where C_t is cache row t of sequence b ([AUDIT] §2.2-2.3; [MLA80] §5:
 * content score against the shared latent, rope score against the shared
 * k_R broadcast to every head, context formed in the 512-wide latent).
 * seq_lens counts keys including this step's appended tokens (append precedes
 * attend: [MLA80] §2 concatenates the cache before attending), so query i sees
 * itself and the earlier new tokens (causal among the Lq new tokens).
 *   q            device [B*Lq][H][576] bf16 (row n = b*Lq + i; from mla_absorb_q)
 *   pool         device [num_blocks][64][576] bf16
 *   block_table  device [B][max_blocks_per_seq] int32
 *   seq_lens     device [B] int32
 *   o_lat        device [B*Lq][H][512] bf16
 *   lse          device [B*Lq][H] float32, or NULL
 *   workspace    device, at least mla_decode_workspace_size(dims, B, Lq) bytes
 * Lq may be a whole prefill chunk (many new tokens per sequence). q, pool,
 * o_lat and workspace must be 16-byte aligned and lse 4-byte aligned
 * (MLA_ERR_INVALID_ARG otherwise). Returns
 * MLA_ERR_UNSUPPORTED when H is not a multiple of 16, Lq*H exceeds 2^20, the
 * table spans more than 2^30 keys, or B*ceil(Lq*H/4) exceeds 2^31-1.
 * Device-value handling: a length above max_blocks_per_seq*64 or a block id
 * outside [0, num_blocks) makes that sequence's outputs NaN (never an
 * out-of-bounds access); a length <= 0 gives zero outputs and lse = -inf, as
 * does a row whose position is negative.
 * Deterministic: the split plan depends only on seq_lens, B, Lq and H, and
 * partials are merged in a fixed order without atomics.
 */
int mla_decode_attn(const mla_dims* dims, const uint16_t* q, const uint16_t* pool,
                    int64_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t B, int32_t Lq, uint16_t* o_lat, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Size of the fixed per-GPU array in which mla_decode_attn_noalloc keeps its
 * partial results (64 MiB; held by each GPU the library runs on until the
 * process ends). */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * mla_decode_attn_noalloc — mla_decode_attn without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that forbid
 * allocation. The partials of the key-range splits go to a fixed array of
 * MLA_NOALLOC_SCRATCH_BYTES bytes per GPU instead; the call allocates
 * nothing (no hipMalloc, no allocating library routine), and the first call
 * on a GPU looks up that GPU's copy of the array.
 * Arguments, layouts, results, device-value handling and determinism are
 * those of mla_decode_attn (same kernels; outputs bit-identical to it).
 * Limits and errors: MLA_ERR_WORKSPACE when the shape needs more than
 * MLA_NOALLOC_SCRATCH_BYTES (mla_decode_workspace_size(dims, B, Lq) above it),
 * checked on the host before anything is enqueued; MLA_ERR_INVALID_ARG when
 * `stream` belongs to another GPU than the current one; otherwise as
 * mla_decode_attn.
 * Concurrency: every call on one GPU shares that GPU's array, which keeps the
 * last call's contents. Calls that overlap in time on one GPU (other streams,
 * other host threads) race and give wrong results; calls in one stream are
 * ordered and safe.
 */
int mla_decode_attn_noalloc(const mla_dims* dims, const uint16_t* q, const uint16_t* pool,
                            int64_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t B, int32_t Lq, uint16_t* o_lat, float* lse,
                            void* stream);

/*
 * mla_append_absorb — mla_cache_append and mla_absorb_q of one decode step in
 * a single launch, for the usual case where the step's N new tokens are its N
 * queries: new token n (c_kv[n], k_pe[n]) sits at position pos[n] and goes
 * to slot_mapping[n], and query n (q_nope[n], q_pe[n]) is absorbed at the
 * same position. Results are bit-identical to the two separate calls;
 * arguments, layouts, slot handling and errors as there (T = N). Both parts
 * only read their inputs and write disjoint outputs.
 */
int mla_append_absorb(const mla_dims* dims, const uint16_t* c_kv, const uint16_t* k_pe,
                      const int64_t* slot_mapping, uint16_t* pool, int64_t num_blocks,
                      const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                      const uint16_t* w_uk, uint16_t* q_out, int32_t N, void* stream);

/*
 * FP8 latent cache ([AUDIT] §6.1: FlashMLA's support matrix pairs its
 * MQA-mode kernels with an FP8 KV cache; the pages name the format only).
 * Reading used here: the same 576-element row per token, stored as OCP FP8
 * E4M3 codes ("e4m3fn": exponent bias 7, 3 mantissa bits, largest finite 448,
 * 0x7f / 0xff NaN) of row / scale, with one fp32 scale per token, a power
 * of two: the smallest 2^k with max|row| / 2^k <= 448, k >= -124 (1 for an
 * all-zero row). E4M3 being floating point, a power-of-two scale loses
 * nothing against max|row| / 448, and every code times its scale is exactly
 * a bf16 value. Half the bytes of the bf16 pool per token (576 + 4 against
 * 1,152).
 *   pool8       device [num_blocks][64][576] uint8  E4M3 codes
 *   pool_scale  device [num_blocks][64]      fp32   scale of each slot's row
 */

/*
 * mla_cache_append_fp8 — mla_cache_append into the FP8 pool. The row
 * [c_kv | RoPE(k_pe, pos)] is formed in fp32 (the latent exactly, the rope
 * part with an fp64 angle and rotation, rounded once), its absmax taken, and
 * every element encoded as E4M3 of (element / scale) with IEEE fp32 division,
 * nearest value with ties to even. Arguments as mla_cache_append; a slot
 * outside [0, num_blocks*64) is skipped (neither codes nor scale written).
 * Non-finite inputs give unspecified codes.
 */
int mla_cache_append_fp8(const mla_dims* dims, const uint16_t* c_kv, const uint16_t* k_pe,
                         const int32_t* pos, const int64_t* slot_mapping, uint8_t* pool8,
                         float* pool_scale, int64_t num_blocks, int32_t T, void* stream);

/*
 * mla_append_absorb_fp8 — mla_append_absorb into the FP8 pool (the append
 * part as mla_cache_append_fp8).
 */
int mla_append_absorb_fp8(const mla_dims* dims, const uint16_t* c_kv, const uint16_t* k_pe,
                          const int64_t* slot_mapping, uint8_t* pool8, float* pool_scale,
                          int64_t num_blocks, const uint16_t* q_nope, const uint16_t* q_pe,
                          const int32_t* pos, const uint16_t* w_uk, uint16_t* q_out, int32_t N,
                          void* stream);

/*
 * mla_decode_attn_fp8 — mla_decode_attn over the FP8 pool: C_t is the row the
 * codes stand for, code value x pool_scale of its slot. The scale being a
 * power of two, code x scale is exactly a bf16 value, and the kernels use
 * that row in the bf16 products: the 128-row kernel (96 or more query rows
 * per sequence) widens code x scale to bf16 in the LDS; the column kernels
 * (fewer rows) form scores from the codes and multiply them by the scale in
 * fp32, and multiply probabilities by it before their bf16 rounding for the
 * weighted sum. Both give the same scores and terms, exactly, up to
 * summation order (scaling by a power of two commutes with rounding). pool8
 * and pool_scale must be 16-byte aligned. Every other argument, the
 * workspace (the same mla_decode_workspace_size), the alignment rules, the
 * error codes, the device-value handling and determinism are as for
 * mla_decode_attn.
 * Cost against the bf16 pool: with few query rows per sequence (16 heads)
 * the call is bound by memory and half the bytes make it faster (16 heads,
 * 4,096 keys: ~48 against ~60 us); at 128 heads both run on the 128-row
 * kernel, bound by its products, and take about the same time (16,384 keys:
 * ~152 against ~153-160 us), so FP8 there saves memory, not time.
 */
int mla_decode_attn_fp8(const mla_dims* dims, const uint16_t* q, const uint8_t* pool8,
                        const float* pool_scale, int64_t num_blocks, const int32_t* block_table,
                        int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B, int32_t Lq,
                        uint16_t* o_lat, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Expanded-form attention for long query chunks ([MLA80] §2: the model's
 * forward expands per-head keys and values from the latent, k_c[t,h] =
 * W_UK[h] c_kv[t] and v[t,h] = W_UV[h] c_kv[t], concatenates the shared RoPE
 * key and runs multi-head attention; [MLA80] §3 times prefill in that form).
 * It computes what mla_absorb_q + mla_decode_attn + mla_out_up compute
 * together, o[n,h] = sum_t softmax_t(q[n,h].k[t,h] scale) v[t,h] with
 * q = [q_nope | RoPE(q_pe, pos)], k = [k_c | k_r], over the same visible keys
 * (query token i of a sequence of L keys sits at L - Lq + i), by another
 * route: 2 L H 256 512 flops for the expansion plus 2 H Lq L (192 + 128) for
 * the attention, against 2 H Lq L (576 + 512) for the absorbed form, so it
 * pays once a chunk holds a few hundred query tokens per sequence.
 *   Steps, on `stream`: the sequence's cache rows are gathered into the
 *   workspace, W_UK and W_UV expand them in two bf16 GEMMs per sequence
 *   (hipBLASLt; fp32 accumulation, one rounding of k_c and v to bf16), and a
 *   causal attention kernel forms the scores in bf16 MFMAs, the softmax in
 *   fp32 and o in one rounding to bf16. The expansion runs over max_len rows
 *   (rounded up to 32) for every sequence. The first call on a device creates
 *   that device's hipBLASLt handle, kept until the process ends; the GEMMs
 *   are given no hipBLASLt workspace.
 *   q_nope [B*Lq][H][128] bf16, q_pe [B*Lq][H][64] bf16 (not rotated),
 *   pos [B*Lq] int32: the queries, as for mla_absorb_q (token n = b*Lq + i).
 *   pool, num_blocks, block_table, max_blocks_per_seq, seq_lens, B, Lq: as
 *   for mla_decode_attn (seq_lens include the chunk's own tokens).
 *   max_len: host bound on every seq_lens[b]; a sequence longer than max_len
 *   gets NaN outputs, one with a block id outside the pool NaN outputs.
 *   w_uk, w_uv [H][128][512] bf16 (nn.Linear rows, as for mla_absorb_q and
 *   mla_out_up).
 *   o [B*Lq][H][128] bf16 out; lse [B*Lq][H] fp32 out or NULL (natural log of
 *   the sum of exp of the scaled scores; -inf and o = 0 for a row that sees
 *   no key).
 *   workspace: device memory of mla_prefill_expanded_workspace_size bytes,
 *   256-byte aligned, contents ignored (the expanded K and V^T: 2 B max_len
 *   H 256 bytes plus the gathered rows).
 * Pointers 16-byte aligned (lse 4-byte). Errors: MLA_ERR_INVALID_ARG (null,
 * non-positive size, misalignment), MLA_ERR_UNSUPPORTED (B > 65,535, Lq or
 * max_len > 2^20, B*Lq > 2^30), MLA_ERR_WORKSPACE, MLA_ERR_LAUNCH (a launch
 * or a GEMM failed to enqueue), all before anything is enqueued except the
 * last.
 */
size_t mla_prefill_expanded_workspace_size(const mla_dims* dims, int32_t B, int32_t max_len);
int mla_prefill_expanded(const mla_dims* dims, const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                         const uint16_t* pool, int64_t num_blocks, const int32_t* block_table,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B, int32_t Lq,
                         int32_t max_len, const uint16_t* w_uk, const uint16_t* w_uv, uint16_t* o, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Two-buffer latent cache ([AUDIT] §0: the V3 reference's absorbed decode
 * keeps kv_cache [1,32,512] and pe_cache [1,32,64]; §4.2: a 32-slot buffer,
 * 32,768 + 4,096 = 36,864 bytes allocated for 26 active tokens). The same
 * 576-element row per token as the paged pool, split in two arrays indexed by
 * [sequence][position], with room for max_seq positions per sequence:
 *   kv_cache  device [B][max_seq][512] bf16   c_kv of each token
 *   pe_cache  device [B][max_seq][64]  bf16   RoPE(k_pe) of each token
 */

/*
 * mla_cache_append_kvpe — mla_cache_append into the two-buffer cache: token j
 * goes to [seq_idx[j]][pos[j]] of both arrays (c_kv[j] bit-exactly into
 * kv_cache, RoPE(k_pe[j], pos[j]) rounded once to bf16 into pe_cache). A
 * sequence index outside [0, B) or a position outside [0, max_seq) skips the
 * token (no write).
 *   seq_idx  device [T] int32  sequence of each new token
 * Other arguments as mla_cache_append. MLA_ERR_INVALID_ARG for a null
 * pointer or B, max_seq, T <= 0.
 */
int mla_cache_append_kvpe(const mla_dims* dims, const uint16_t* c_kv, const uint16_t* k_pe,
                          const int32_t* pos, const int32_t* seq_idx, uint16_t* kv_cache, uint16_t* pe_cache,
                          int32_t B, int32_t max_seq, int32_t T, void* stream);

/*
 * mla_append_absorb_kvpe — mla_cache_append_kvpe and mla_absorb_q of one
 * decode step in a single launch (as mla_append_absorb for the paged pool):
 * new token n (c_kv[n], k_pe[n]) goes to [seq_idx[n]][pos[n]] of both
 * arrays, and query n (q_nope[n], q_pe[n]) is absorbed at position pos[n].
 * Results are bit-identical to the two separate calls; arguments, layouts,
 * skipped tokens and errors as there (T = N; N above 2^22 gives
 * MLA_ERR_UNSUPPORTED). Both parts only read their inputs and write disjoint
 * outputs.
 */
int mla_append_absorb_kvpe(const mla_dims* dims, const uint16_t* c_kv, const uint16_t* k_pe,
                           const int32_t* seq_idx, uint16_t* kv_cache, uint16_t* pe_cache, int32_t B,
                           int32_t max_seq, const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                           const uint16_t* w_uk, uint16_t* q_out, int32_t N, void* stream);

/*
 * mla_decode_attn_kvpe — mla_decode_attn over the two-buffer cache: key t of
 * sequence b is C_t = [kv_cache[b][t] | pe_cache[b][t]] (the V3 reference
 * forms the score as the latent product plus the rope product, [AUDIT] §0).
 * No block table; seq_lens[b] <= max_seq (a longer sequence gets NaN
 * outputs, never a read past its rows). q, kv_cache, pe_cache, o_lat and
 * workspace 16-byte aligned, lse 4-byte aligned. The workspace size, the
 * other arguments, the error codes and determinism are as for
 * mla_decode_attn; MLA_ERR_UNSUPPORTED also when max_seq exceeds 2^30.
 */
int mla_decode_attn_kvpe(const mla_dims* dims, const uint16_t* q, const uint16_t* kv_cache,
                         const uint16_t* pe_cache, int32_t max_seq, const int32_t* seq_lens, int32_t B,
                         int32_t Lq, uint16_t* o_lat, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * mla_out_up — expand the latent context through W_UV per head.
 * o[n][h] = W_UV[h] o_lat[n][h]   ([AUDIT] §2.3: sum_t p_t (W_V c_t) = W_V (sum_t p_t c_t))
 *   o_lat  device [N][H][512] bf16
 *   w_uv   device [H][128][512] bf16  (the head's rows of nn.Linear(d_c, H*d_v).weight)
 *   o      device [N][H][128] bf16
 * fp32 accumulation (bf16 MFMA), one rounding to bf16. N at most 2^22.
 */
int mla_out_up(const mla_dims* dims, const uint16_t* o_lat, const uint16_t* w_uv, uint16_t* o,
               int32_t N, void* stream);

/*
 * mla_linear_workspace_size — bytes of fp32 device workspace with which
 * mla_linear splits the contraction of an [N][K] -> [N][M] map over several
 * workgroups (maps with few output tiles, e.g. K = 7168 -> M = 512 at 32
 * tokens). 0 when the map is never split, or the sizes are not supported.
 */
size_t mla_linear_workspace_size(int32_t N, int32_t K, int32_t M);

/*
 * mla_linear — a bias-free linear map, for the projections around the
 * attention ([MLA80] §2: Wdq, Wuq, Wqr, Wdkv, Wkr and the output projection
 * Wo are nn.Linear(bias=False) maps of the layer).
 * y[n] = W x[n] (+ residual[n])
 *   x          device [N][K] bf16
 *   w          device [M][K] bf16 (nn.Linear weight layout: [out][in])
 *   residual   device [N][M] bf16, or NULL; may be the same buffer as y
 *   y          device [N][M] bf16
 *   workspace  device, 16-byte aligned, or NULL; caller-owned; overlaps none
 *              of the other buffers, and calls that may run at the same
 *              time (other streams) each need their own
 *   workspace_bytes  its size; when it is at least
 *              mla_linear_workspace_size(N, K, M) (and that is > 0) the
 *              contraction is split and the fp32 partial sums are added
 *              in a fixed order by a second kernel; otherwise the call runs
 *              unsplit and leaves the workspace untouched
 * fp32 accumulation (bf16 MFMA), the residual added in fp32, one rounding to
 * bf16. K must be a multiple of 32 and M of 4, K and M at most 2^30, N at
 * most 2,097,120 (MLA_ERR_UNSUPPORTED otherwise); null pointers, sizes <= 0 or a misaligned
 * workspace give MLA_ERR_INVALID_ARG. Deterministic: calls with the same
 * sizes and the same choice (split or not) give the same bits; split and
 * unsplit results differ only in fp32 summation order.
 */
int mla_linear(const uint16_t* x, const uint16_t* w, const uint16_t* residual, uint16_t* y,
               int32_t N, int32_t K, int32_t M, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ABSORB_H */
