// Host stand-ins for the kernel launchers, for the sanitizer build of the C
// ABI (capi.cpp + plan.cpp, compiled for the CPU alone). Each one reads and
// writes, on host memory, every element the real kernels read or write for
// the same arguments, as the layouts in mla_absorb.h define them; the test
// driver hands the C ABI host buffers of exactly the documented sizes, so an
// argument check that lets a too-small buffer through, or a plan whose
// workspace arithmetic undercounts, shows up as an AddressSanitizer report.
#include <string.h>

#include <vector>

#include "kernels.h"

namespace {

volatile uint32_t g_sink;  // keeps the reads from being optimised away

template <class T>
void touch_read(const T* p, size_t n) {
  uint32_t s = 0;
  const unsigned char* b = (const unsigned char*)p;
  for (size_t i = 0; i < n * sizeof(T); ++i) s += b[i];
  g_sink = g_sink + s;
}
template <class T>
void touch_write(T* p, size_t n) {
  memset((void*)p, 0, n * sizeof(T));
}

// Cache rows the append kernels write: slot s in [0, num_blocks*64) gets row s.
void append_rows(const int64_t* slot_mapping, int32_t T, int64_t num_blocks, void* pool, size_t row_bytes,
                 float* pool_scale) {
  touch_read(slot_mapping, (size_t)T);
  for (int32_t t = 0; t < T; ++t) {
    const int64_t s = slot_mapping[t];
    if (s < 0 || s >= num_blocks * mla::BLOCK) continue;
    touch_write((unsigned char*)pool + (size_t)s * row_bytes, row_bytes);
    if (pool_scale) touch_write(pool_scale + s, 1);
  }
}

// The split-KV attention: queries, lengths, the blocks each length covers,
// the outputs, and the workspace slots of the plan the launcher dispatches.
void attention(const mla::AttnPlan& p, const uint16_t* q, const void* pool, size_t block_bytes,
               const float* pool_scale, const uint16_t* pe, int64_t num_blocks, const int32_t* block_table,
               int32_t max_blocks, int32_t max_keys, const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H,
               uint16_t* o_lat, float* lse, void* workspace) {
  const size_t rows = (size_t)Lq * (size_t)H;
  touch_read(q, (size_t)B * rows * mla::D_K);
  touch_read(seq_lens, (size_t)B);
  for (int32_t b = 0; b < B; ++b) {
    const int32_t L = seq_lens[b];
    if (L <= 0) continue;
    const int32_t Lc = L < max_keys ? L : max_keys;
    const int32_t nt = (Lc + mla::BLOCK - 1) / mla::BLOCK;
    if (block_table) {
      touch_read(block_table + (size_t)b * max_blocks, (size_t)nt);
      for (int32_t k = 0; k < nt; ++k) {
        const int32_t blk = block_table[(size_t)b * max_blocks + k];
        if (blk < 0 || blk >= num_blocks) continue;
        touch_read((const unsigned char*)pool + (size_t)blk * block_bytes, block_bytes);
        if (pool_scale) touch_read(pool_scale + (size_t)blk * mla::BLOCK, (size_t)mla::BLOCK);
      }
    } else {  // two-buffer layout: Lc rows of sequence b in each buffer
      touch_read((const uint16_t*)pool + (size_t)b * max_keys * mla::D_C, (size_t)Lc * mla::D_C);
      touch_read(pe + (size_t)b * max_keys * mla::D_ROPE, (size_t)Lc * mla::D_ROPE);
    }
  }
  touch_write(o_lat, (size_t)B * rows * mla::D_C);
  if (lse) touch_write(lse, (size_t)B * rows);
  // partial slot k of the plan: (m, l) at ws_ml + 2 (k rows + r), the bf16
  // partial row at ws_acc + (k rows + r) 512, for k < width + B
  const size_t slots = (size_t)p.width + (size_t)B;
  float* ws_ml = (float*)workspace;
  uint16_t* ws_acc = (uint16_t*)((char*)workspace + mla::attention_ws_ml_bytes(B, Lq, H));
  touch_write(ws_ml, slots * rows * 2);
  touch_write(ws_acc, slots * rows * mla::D_C);
}

std::vector<unsigned char>& noalloc_scratch() {
  static std::vector<unsigned char> s(mla::NOALLOC_SCRATCH_BYTES);
  return s;
}

}  // namespace

namespace mla {

hipError_t launch_cache_append(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* pos,
                               const int64_t* slot_mapping, uint16_t* pool, int64_t num_blocks, int32_t T,
                               double, hipStream_t) {
  touch_read(c_kv, (size_t)T * D_C);
  touch_read(k_pe, (size_t)T * D_ROPE);
  touch_read(pos, (size_t)T);
  append_rows(slot_mapping, T, num_blocks, pool, ROW_BYTES, nullptr);
  return hipSuccess;
}

hipError_t launch_absorb_q(const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos, const uint16_t* w_uk,
                           uint16_t* q_out, int32_t N, int32_t H, double, hipStream_t) {
  touch_read(q_nope, (size_t)N * H * D_NOPE);
  touch_read(q_pe, (size_t)N * H * D_ROPE);
  touch_read(pos, (size_t)N);
  touch_read(w_uk, (size_t)H * D_NOPE * D_C);
  touch_write(q_out, (size_t)N * H * D_K);
  return hipSuccess;
}

hipError_t launch_append_absorb(const uint16_t* c_kv, const uint16_t* k_pe, const int64_t* slot_mapping, void* pool,
                                float* pool_scale, int64_t num_blocks, const uint16_t* q_nope,
                                const uint16_t* q_pe, const int32_t* pos, const uint16_t* w_uk, uint16_t* q_out,
                                int32_t N, int32_t H, double rope_base, hipStream_t stream) {
  touch_read(c_kv, (size_t)N * D_C);
  touch_read(k_pe, (size_t)N * D_ROPE);
  append_rows(slot_mapping, N, num_blocks, pool, pool_scale ? (size_t)D_K : (size_t)ROW_BYTES, pool_scale);
  return launch_absorb_q(q_nope, q_pe, pos, w_uk, q_out, N, H, rope_base, stream);
}

hipError_t launch_append_absorb_kvpe(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* seq_idx,
                                     uint16_t* kv_cache, uint16_t* pe_cache, int32_t B, int32_t max_seq,
                                     const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                                     const uint16_t* w_uk, uint16_t* q_out, int32_t N, int32_t H, double rope_base,
                                     hipStream_t stream) {
  const hipError_t e = launch_cache_append_kvpe(c_kv, k_pe, pos, seq_idx, kv_cache, pe_cache, B, max_seq, N,
                                                rope_base, stream);
  if (e != hipSuccess) return e;
  return launch_absorb_q(q_nope, q_pe, pos, w_uk, q_out, N, H, rope_base, stream);
}

hipError_t launch_out_up(const uint16_t* o_lat, const uint16_t* w_uv, uint16_t* o, int32_t N, int32_t H,
                         hipStream_t) {
  touch_read(o_lat, (size_t)N * H * D_C);
  touch_read(w_uv, (size_t)H * D_V * D_C);
  touch_write(o, (size_t)N * H * D_V);
  return hipSuccess;
}

hipError_t launch_linear(const uint16_t* x, const uint16_t* w, const uint16_t* r, uint16_t* y, void* workspace,
                         size_t workspace_bytes, int32_t N, int32_t K, int32_t M, hipStream_t) {
  touch_read(x, (size_t)N * K);
  touch_read(w, (size_t)M * K);
  if (r) touch_read(r, (size_t)N * M);
  LinearPlan p = plan_linear(N, K, M, true);
  if (p.ks > 1 && (workspace == nullptr || workspace_bytes < p.ws_bytes)) p = plan_linear(N, K, M, false);
  if (p.ks > 1) touch_write((unsigned char*)workspace, p.ws_bytes);
  touch_write(y, (size_t)N * M);
  return hipSuccess;
}

hipError_t launch_decode_attn(const uint16_t* q, const uint16_t* pool, int64_t num_blocks, const int32_t* block_table,
                              int32_t max_blocks, const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H, float,
                              uint16_t* o_lat, float* lse, void* workspace, hipStream_t) {
  attention(plan_attention(B, Lq, H), q, pool, (size_t)BLOCK_BYTES, nullptr, nullptr, num_blocks, block_table,
            max_blocks, max_blocks * BLOCK, seq_lens, B, Lq, H, o_lat, lse, workspace);
  return hipSuccess;
}

hipError_t launch_decode_attn_noalloc(const uint16_t* q, const uint16_t* pool, int64_t num_blocks,
                                      const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                                      int32_t B, int32_t Lq, int32_t H, float scale, uint16_t* o_lat, float* lse,
                                      hipStream_t stream) {
  if (attention_workspace_bytes(B, Lq, H) > NOALLOC_SCRATCH_BYTES) return hipErrorInvalidValue;
  return launch_decode_attn(q, pool, num_blocks, block_table, max_blocks, seq_lens, B, Lq, H, scale, o_lat, lse,
                            noalloc_scratch().data(), stream);
}

hipError_t launch_cache_append_kvpe(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* pos,
                                    const int32_t* seq_idx, uint16_t* kv_cache, uint16_t* pe_cache, int32_t B,
                                    int32_t max_seq, int32_t T, double, hipStream_t) {
  touch_read(c_kv, (size_t)T * D_C);
  touch_read(k_pe, (size_t)T * D_ROPE);
  touch_read(pos, (size_t)T);
  touch_read(seq_idx, (size_t)T);
  for (int32_t t = 0; t < T; ++t) {
    if (seq_idx[t] < 0 || seq_idx[t] >= B || pos[t] < 0 || pos[t] >= max_seq) continue;
    const size_t row = (size_t)seq_idx[t] * max_seq + pos[t];
    touch_write(kv_cache + row * D_C, (size_t)D_C);
    touch_write(pe_cache + row * D_ROPE, (size_t)D_ROPE);
  }
  return hipSuccess;
}

hipError_t launch_decode_attn_kvpe(const uint16_t* q, const uint16_t* kv_cache, const uint16_t* pe_cache,
                                   int32_t max_seq, const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H, float,
                                   uint16_t* o_lat, float* lse, void* workspace, hipStream_t) {
  attention(plan_attention_kvpe(B, Lq, H), q, kv_cache, 0, nullptr, pe_cache, 0, nullptr,
            (max_seq + BLOCK - 1) / BLOCK, max_seq, seq_lens, B, Lq, H, o_lat, lse, workspace);
  return hipSuccess;
}

hipError_t launch_cache_append_fp8(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* pos,
                                   const int64_t* slot_mapping, uint8_t* pool8, float* pool_scale, int64_t num_blocks,
                                   int32_t T, double, hipStream_t) {
  touch_read(c_kv, (size_t)T * D_C);
  touch_read(k_pe, (size_t)T * D_ROPE);
  touch_read(pos, (size_t)T);
  append_rows(slot_mapping, T, num_blocks, pool8, (size_t)D_K, pool_scale);
  return hipSuccess;
}

hipError_t launch_prefill_expanded(const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                                   const uint16_t* pool, int64_t num_blocks, const int32_t* block_table,
                                   int32_t max_blocks, const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H,
                                   int32_t max_len, const uint16_t* w_uk, const uint16_t* w_uv, float, double,
                                   uint16_t* o, float* lse, void* workspace, hipStream_t) {
  const size_t N = (size_t)B * Lq;
  touch_read(q_nope, N * H * D_NOPE);
  touch_read(q_pe, N * H * D_ROPE);
  touch_read(pos, N);
  touch_read(seq_lens, (size_t)B);
  touch_read(w_uk, (size_t)H * D_NOPE * D_C);
  touch_read(w_uv, (size_t)H * D_V * D_C);
  const ExpandedLayout w = expanded_layout(B, H, max_len);
  for (int32_t b = 0; b < B; ++b) {   // the gather reads the rows of keys below min(L, max_len)
    const int32_t L = seq_lens[b] < max_len ? seq_lens[b] : max_len;
    const int32_t nt = L > 0 ? (L + BLOCK - 1) / BLOCK : 0;
    const int32_t nk = nt < max_blocks ? nt : max_blocks;
    touch_read(block_table + (size_t)b * max_blocks, (size_t)nk);
    for (int32_t k = 0; k < nk; ++k) {
      const int32_t blk = block_table[(size_t)b * max_blocks + k];
      if (blk >= 0 && blk < num_blocks) touch_read(pool + (size_t)blk * BLOCK * D_K, (size_t)BLOCK * D_K);
    }
  }
  char* ws = (char*)workspace;
  const size_t rows = (size_t)B * w.Lpad;
  touch_write((uint16_t*)(ws + w.c_off), rows * D_C);
  touch_write((uint16_t*)(ws + w.kr_off), rows * D_ROPE);
  touch_write((uint16_t*)(ws + w.k_off), rows * H * D_NOPE);
  touch_write((uint16_t*)(ws + w.vt_off), rows * H * D_NOPE);
  touch_write(o, N * H * D_V);
  if (lse) touch_write(lse, N * H);
  return hipSuccess;
}

hipError_t launch_decode_attn_fp8(const uint16_t* q, const uint8_t* pool8, const float* pool_scale,
                                  int64_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H, float, uint16_t* o_lat,
                                  float* lse, void* workspace, hipStream_t) {
  attention(plan_attention_fp8(B, Lq, H), q, pool8, (size_t)BLOCK * D_K, pool_scale, nullptr, num_blocks,
            block_table, max_blocks, max_blocks * BLOCK, seq_lens, B, Lq, H, o_lat, lse, workspace);
  return hipSuccess;
}

}  // namespace mla
