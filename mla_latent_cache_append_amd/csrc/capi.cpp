// C ABI of libmla_absorb: argument checks on the host, then kernel launches on
// the caller's stream. Declarations and their contracts: include/mla_absorb.h.
#include <initializer_list>
#include "mla_absorb.h"

#include <math.h>

#include "kernels.h"

namespace {

int check_dims(const mla_dims* d) {
  if (!d) return MLA_ERR_INVALID_ARG;
  if (d->num_heads <= 0 || !(d->softmax_scale > 0.f) || !isfinite(d->softmax_scale) ||
      !(d->rope_base > 1.f) || !isfinite(d->rope_base))
    return MLA_ERR_INVALID_ARG;
  if (d->d_c != mla::D_C || d->d_rope != mla::D_ROPE || d->d_nope != mla::D_NOPE ||
      d->d_v != mla::D_V || d->block_size != mla::BLOCK || d->num_heads > 128)
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

// Tokens of one absorb / out_up call: their grids (a workgroup per 256-token
// run, head and column slice, plus one per four appended tokens) stay within
// the 2^32 work-items a launch dimension holds.
constexpr int32_t MAX_TOKENS = 1 << 22;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Attention shapes the kernels index with 32-bit arithmetic: the rows of one
// sequence (Lq * H <= 2^20) and the merge's grid (one workgroup per four
// query rows of every sequence).
bool attn_shape_ok(int32_t B, int32_t Lq, int32_t H) {
  const int64_t rows = (int64_t)Lq * H;
  return rows <= (1 << 20) && (int64_t)B * ((rows + 3) / 4) <= 0x7fffffff;
}

// Linear maps: K a multiple of 32, M of 4, both at most 2^30; at most 65,535
// workgroup rows of 32 tokens.
int linear_shape(int32_t N, int32_t K, int32_t M) {
  if (K % 32 != 0 || M % 4 != 0 || N > 65535 * 32 || K > (1 << 30) || M > (1 << 30)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// The attention kernels move 16 bytes per lane through q, the cache, o_lat
// and the workspace, and read token scales four at a time.
bool attn_aligned(const void* q, const void* pool, const void* pool_scale, const void* o_lat,
                  const float* lse, const void* workspace) {
  return aligned(q, 16) && aligned(pool, 16) && aligned(pool_scale, 16) && aligned(o_lat, 16) &&
         aligned(lse, 4) && aligned(workspace, 16);
}

// The append, absorb and up-projection kernels move bf16 rows (and FP8 code
// rows) with 16-byte vector accesses, rope pairs and int32 indices with 4-byte
// ones and slot numbers with 8-byte ones.
bool rows_aligned(std::initializer_list<const void*> p16, std::initializer_list<const void*> p4,
                  const void* p8 = nullptr) {
  for (const void* p : p16)
    if (!aligned(p, 16)) return false;
  for (const void* p : p4)
    if (!aligned(p, 4)) return false;
  return aligned(p8, 8);
}

}  // namespace

extern "C" {

void mla_dims_default(mla_dims* d, int32_t num_heads) {
  if (!d) return;
  d->num_heads = num_heads;
  d->d_c = mla::D_C;
  d->d_rope = mla::D_ROPE;
  d->d_nope = mla::D_NOPE;
  d->d_v = mla::D_V;
  d->block_size = mla::BLOCK;
  d->softmax_scale = (float)(1.0 / sqrt((double)(mla::D_NOPE + mla::D_ROPE)));
  d->rope_base = 10000.f;
}

const char* mla_status_str(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported dimensions";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int mla_cache_append(const mla_dims* dims, const uint16_t* c_kv, const uint16_t* k_pe,
                     const int32_t* pos, const int64_t* slot_mapping, uint16_t* pool,
                     int64_t num_blocks, int32_t T, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!c_kv || !k_pe || !pos || !slot_mapping || !pool || num_blocks <= 0 || T <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!rows_aligned({c_kv, pool}, {k_pe, pos}, slot_mapping)) return MLA_ERR_INVALID_ARG;
  return launch_status(mla::launch_cache_append(c_kv, k_pe, pos, slot_mapping, pool, num_blocks, T,
                                                (double)dims->rope_base, (hipStream_t)stream));
}

int mla_absorb_q(const mla_dims* dims, const uint16_t* q_nope, const uint16_t* q_pe,
                 const int32_t* pos, const uint16_t* w_uk, uint16_t* q_out, int32_t N,
                 void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!q_nope || !q_pe || !pos || !w_uk || !q_out || N <= 0) return MLA_ERR_INVALID_ARG;
  if (!rows_aligned({q_nope, w_uk, q_out}, {q_pe, pos})) return MLA_ERR_INVALID_ARG;
  if (N > MAX_TOKENS) return MLA_ERR_UNSUPPORTED;
  return launch_status(mla::launch_absorb_q(q_nope, q_pe, pos, w_uk, q_out, N, dims->num_heads,
                                            (double)dims->rope_base, (hipStream_t)stream));
}

size_t mla_decode_workspace_size(const mla_dims* dims, int32_t B, int32_t Lq) {
  if (check_dims(dims) != MLA_OK || B <= 0 || Lq <= 0 || !attn_shape_ok(B, Lq, dims->num_heads)) return 0;
  return mla::attention_workspace_bytes(B, Lq, dims->num_heads);
}

int mla_decode_attn(const mla_dims* dims, const uint16_t* q, const uint16_t* pool,
                    int64_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t B, int32_t Lq, uint16_t* o_lat, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (dims->num_heads % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if (!q || !pool || !block_table || !seq_lens || !o_lat || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || B <= 0 || Lq <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!attn_aligned(q, pool, nullptr, o_lat, lse, workspace)) return MLA_ERR_INVALID_ARG;
  // rows of one sequence index 32-bit offsets inside the kernels
  if (!attn_shape_ok(B, Lq, dims->num_heads) || (int64_t)max_blocks_per_seq * mla::BLOCK > (1 << 30))
    return MLA_ERR_UNSUPPORTED;
  const size_t need = mla::attention_workspace_bytes(B, Lq, dims->num_heads);
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  return launch_status(mla::launch_decode_attn(q, pool, num_blocks, block_table, max_blocks_per_seq,
                                               seq_lens, B, Lq, dims->num_heads,
                                               dims->softmax_scale, o_lat, lse, workspace,
                                               (hipStream_t)stream));
}

size_t mla_prefill_expanded_workspace_size(const mla_dims* dims, int32_t B, int32_t max_len) {
  if (check_dims(dims) != MLA_OK || B <= 0 || B > 65535 || max_len <= 0 || max_len > (1 << 20)) return 0;
  return mla::expanded_layout(B, dims->num_heads, max_len).bytes;
}

int mla_prefill_expanded(const mla_dims* dims, const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                         const uint16_t* pool, int64_t num_blocks, const int32_t* block_table,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B, int32_t Lq,
                         int32_t max_len, const uint16_t* w_uk, const uint16_t* w_uv, uint16_t* o, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!q_nope || !q_pe || !pos || !pool || !block_table || !seq_lens || !w_uk || !w_uv || !o ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || B <= 0 || Lq <= 0 || max_len <= 0)
    return MLA_ERR_INVALID_ARG;
  // 16-byte loads of q, the cache and the weights; 8-byte stores of o
  if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(pool, 16) || !aligned(w_uk, 16) ||
      !aligned(w_uv, 16) || !aligned(o, 16) || !aligned(lse, 4) || !aligned(workspace, 256))
    return MLA_ERR_INVALID_ARG;
  // one launch dimension per sequence (65,535 at most); 2^20 keys and query tokens
  if (B > 65535 || max_len > (1 << 20) || Lq > (1 << 20) || (int64_t)B * Lq > (1 << 30) ||
      (int64_t)max_blocks_per_seq * mla::BLOCK > (1 << 30))
    return MLA_ERR_UNSUPPORTED;
  const size_t need = mla::expanded_layout(B, dims->num_heads, max_len).bytes;
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  return launch_status(mla::launch_prefill_expanded(
      q_nope, q_pe, pos, pool, num_blocks, block_table, max_blocks_per_seq, seq_lens, B, Lq, dims->num_heads,
      max_len, w_uk, w_uv, dims->softmax_scale, (double)dims->rope_base, o, lse, workspace, (hipStream_t)stream));
}

int mla_decode_attn_noalloc(const mla_dims* dims, const uint16_t* q, const uint16_t* pool,
                            int64_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t B, int32_t Lq, uint16_t* o_lat, float* lse,
                            void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (dims->num_heads % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if (!q || !pool || !block_table || !seq_lens || !o_lat || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || B <= 0 || Lq <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!attn_aligned(q, pool, nullptr, o_lat, lse, nullptr)) return MLA_ERR_INVALID_ARG;
  if (!attn_shape_ok(B, Lq, dims->num_heads) || (int64_t)max_blocks_per_seq * mla::BLOCK > (1 << 30))
    return MLA_ERR_UNSUPPORTED;
  if (mla::attention_workspace_bytes(B, Lq, dims->num_heads) > mla::NOALLOC_SCRATCH_BYTES)
    return MLA_ERR_WORKSPACE;
  const hipError_t e = mla::launch_decode_attn_noalloc(q, pool, num_blocks, block_table, max_blocks_per_seq,
                                                       seq_lens, B, Lq, dims->num_heads, dims->softmax_scale,
                                                       o_lat, lse, (hipStream_t)stream);
  return e == hipErrorInvalidDevice ? MLA_ERR_INVALID_ARG : launch_status(e);
}

int mla_append_absorb(const mla_dims* dims, const uint16_t* c_kv, const uint16_t* k_pe,
                      const int64_t* slot_mapping, uint16_t* pool, int64_t num_blocks,
                      const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                      const uint16_t* w_uk, uint16_t* q_out, int32_t N, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!c_kv || !k_pe || !slot_mapping || !pool || num_blocks <= 0 || !q_nope || !q_pe || !pos || !w_uk ||
      !q_out || N <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!rows_aligned({c_kv, pool, q_nope, w_uk, q_out}, {k_pe, q_pe, pos}, slot_mapping)) return MLA_ERR_INVALID_ARG;
  if (N > MAX_TOKENS) return MLA_ERR_UNSUPPORTED;
  return launch_status(mla::launch_append_absorb(c_kv, k_pe, slot_mapping, pool, nullptr, num_blocks, q_nope,
                                                 q_pe, pos, w_uk, q_out, N, dims->num_heads,
                                                 (double)dims->rope_base, (hipStream_t)stream));
}

int mla_append_absorb_fp8(const mla_dims* dims, const uint16_t* c_kv, const uint16_t* k_pe,
                          const int64_t* slot_mapping, uint8_t* pool8, float* pool_scale,
                          int64_t num_blocks, const uint16_t* q_nope, const uint16_t* q_pe,
                          const int32_t* pos, const uint16_t* w_uk, uint16_t* q_out, int32_t N,
                          void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!c_kv || !k_pe || !slot_mapping || !pool8 || !pool_scale || num_blocks <= 0 || !q_nope || !q_pe ||
      !pos || !w_uk || !q_out || N <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!rows_aligned({c_kv, pool8, pool_scale, q_nope, w_uk, q_out}, {k_pe, q_pe, pos}, slot_mapping))
    return MLA_ERR_INVALID_ARG;
  if (N > MAX_TOKENS) return MLA_ERR_UNSUPPORTED;
  return launch_status(mla::launch_append_absorb(c_kv, k_pe, slot_mapping, pool8, pool_scale, num_blocks,
                                                 q_nope, q_pe, pos, w_uk, q_out, N, dims->num_heads,
                                                 (double)dims->rope_base, (hipStream_t)stream));
}

int mla_cache_append_fp8(const mla_dims* dims, const uint16_t* c_kv, const uint16_t* k_pe,
                         const int32_t* pos, const int64_t* slot_mapping, uint8_t* pool8,
                         float* pool_scale, int64_t num_blocks, int32_t T, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!c_kv || !k_pe || !pos || !slot_mapping || !pool8 || !pool_scale || num_blocks <= 0 || T <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!rows_aligned({c_kv, pool8, pool_scale}, {k_pe, pos}, slot_mapping)) return MLA_ERR_INVALID_ARG;
  return launch_status(mla::launch_cache_append_fp8(c_kv, k_pe, pos, slot_mapping, pool8, pool_scale,
                                                    num_blocks, T, (double)dims->rope_base,
                                                    (hipStream_t)stream));
}

int mla_decode_attn_fp8(const mla_dims* dims, const uint16_t* q, const uint8_t* pool8,
                        const float* pool_scale, int64_t num_blocks, const int32_t* block_table,
                        int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B, int32_t Lq,
                        uint16_t* o_lat, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (dims->num_heads % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if (!q || !pool8 || !pool_scale || !block_table || !seq_lens || !o_lat || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || B <= 0 || Lq <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!attn_aligned(q, pool8, pool_scale, o_lat, lse, workspace)) return MLA_ERR_INVALID_ARG;
  if (!attn_shape_ok(B, Lq, dims->num_heads) || (int64_t)max_blocks_per_seq * mla::BLOCK > (1 << 30))
    return MLA_ERR_UNSUPPORTED;
  const size_t need = mla::attention_workspace_bytes(B, Lq, dims->num_heads);
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  return launch_status(mla::launch_decode_attn_fp8(q, pool8, pool_scale, num_blocks, block_table,
                                                   max_blocks_per_seq, seq_lens, B, Lq,
                                                   dims->num_heads, dims->softmax_scale, o_lat, lse,
                                                   workspace, (hipStream_t)stream));
}

int mla_cache_append_kvpe(const mla_dims* dims, const uint16_t* c_kv, const uint16_t* k_pe,
                          const int32_t* pos, const int32_t* seq_idx, uint16_t* kv_cache, uint16_t* pe_cache,
                          int32_t B, int32_t max_seq, int32_t T, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!c_kv || !k_pe || !pos || !seq_idx || !kv_cache || !pe_cache || B <= 0 || max_seq <= 0 || T <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!rows_aligned({c_kv, kv_cache}, {k_pe, pos, seq_idx, pe_cache})) return MLA_ERR_INVALID_ARG;
  return launch_status(mla::launch_cache_append_kvpe(c_kv, k_pe, pos, seq_idx, kv_cache, pe_cache, B, max_seq, T,
                                                     (double)dims->rope_base, (hipStream_t)stream));
}

int mla_append_absorb_kvpe(const mla_dims* dims, const uint16_t* c_kv, const uint16_t* k_pe,
                           const int32_t* seq_idx, uint16_t* kv_cache, uint16_t* pe_cache, int32_t B,
                           int32_t max_seq, const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                           const uint16_t* w_uk, uint16_t* q_out, int32_t N, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!c_kv || !k_pe || !seq_idx || !kv_cache || !pe_cache || B <= 0 || max_seq <= 0 || !q_nope || !q_pe ||
      !pos || !w_uk || !q_out || N <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!rows_aligned({c_kv, kv_cache, q_nope, w_uk, q_out}, {k_pe, pos, seq_idx, pe_cache, q_pe}))
    return MLA_ERR_INVALID_ARG;
  if (N > MAX_TOKENS) return MLA_ERR_UNSUPPORTED;
  return launch_status(mla::launch_append_absorb_kvpe(c_kv, k_pe, seq_idx, kv_cache, pe_cache, B, max_seq, q_nope,
                                                      q_pe, pos, w_uk, q_out, N, dims->num_heads,
                                                      (double)dims->rope_base, (hipStream_t)stream));
}

int mla_decode_attn_kvpe(const mla_dims* dims, const uint16_t* q, const uint16_t* kv_cache,
                         const uint16_t* pe_cache, int32_t max_seq, const int32_t* seq_lens, int32_t B,
                         int32_t Lq, uint16_t* o_lat, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (dims->num_heads % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if (!q || !kv_cache || !pe_cache || !seq_lens || !o_lat || max_seq <= 0 || B <= 0 || Lq <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!attn_aligned(q, kv_cache, pe_cache, o_lat, lse, workspace)) return MLA_ERR_INVALID_ARG;
  if (!attn_shape_ok(B, Lq, dims->num_heads) || max_seq > (1 << 30)) return MLA_ERR_UNSUPPORTED;
  const size_t need = mla::attention_workspace_bytes(B, Lq, dims->num_heads);
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  return launch_status(mla::launch_decode_attn_kvpe(q, kv_cache, pe_cache, max_seq, seq_lens, B, Lq,
                                                    dims->num_heads, dims->softmax_scale, o_lat, lse, workspace,
                                                    (hipStream_t)stream));
}

int mla_out_up(const mla_dims* dims, const uint16_t* o_lat, const uint16_t* w_uv, uint16_t* o,
               int32_t N, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!o_lat || !w_uv || !o || N <= 0) return MLA_ERR_INVALID_ARG;
  if (!rows_aligned({o_lat, w_uv, o}, {})) return MLA_ERR_INVALID_ARG;
  if (N > MAX_TOKENS) return MLA_ERR_UNSUPPORTED;
  return launch_status(
      mla::launch_out_up(o_lat, w_uv, o, N, dims->num_heads, (hipStream_t)stream));
}

size_t mla_linear_workspace_size(int32_t N, int32_t K, int32_t M) {
  if (N <= 0 || K <= 0 || M <= 0 || linear_shape(N, K, M) != MLA_OK) return 0;
  return mla::plan_linear(N, K, M, true).ws_bytes;
}

int mla_linear(const uint16_t* x, const uint16_t* w, const uint16_t* residual, uint16_t* y,
               int32_t N, int32_t K, int32_t M, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !w || !y || N <= 0 || K <= 0 || M <= 0) return MLA_ERR_INVALID_ARG;
  if (workspace && ((uintptr_t)workspace % 16 != 0)) return MLA_ERR_INVALID_ARG;
  if (linear_shape(N, K, M) != MLA_OK) return MLA_ERR_UNSUPPORTED;
  return launch_status(mla::launch_linear(x, w, residual, y, workspace, workspace ? workspace_bytes : 0, N, K, M,
                                          (hipStream_t)stream));
}

}  // extern "C"
