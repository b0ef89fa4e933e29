// Host-side launch entry points of the libmla_absorb kernels. Each function
// enqueues its kernel(s) on `stream` and returns hipGetLastError(); the C ABI
// (capi.cpp) validates arguments before calling them.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Fixed layer dimensions the kernels implement (V2-Lite / V2 / V3 attention).
constexpr int D_C = 512;           // KV latent width
constexpr int D_ROPE = 64;         // decoupled rope key width
constexpr int D_K = D_C + D_ROPE;  // 576: one cache row
constexpr int D_NOPE = 128;
constexpr int D_V = 128;
constexpr int BLOCK = 64;          // tokens per cache block
constexpr int ROW_BYTES = D_K * 2;              // 1,152
constexpr int BLOCK_BYTES = BLOCK * ROW_BYTES;  // 73,728
constexpr int ROW_CHUNKS = ROW_BYTES / 16;      // 72 sixteen-byte chunks per row

// Launch shapes, shared by the host plans (plan.cpp) and the kernels.
constexpr int TARGET_WGS = 256;  // attention: one workgroup per CU on a 256-CU MI355X
constexpr int LIN_N = 32;        // linear: tokens per workgroup (two 16-token MFMA tiles)
constexpr int LIN_WAVES = 16;    // linear: waves per workgroup, each a slice of the contraction

hipError_t launch_cache_append(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* pos,
                               const int64_t* slot_mapping, uint16_t* pool, int64_t num_blocks,
                               int32_t T, double rope_base, hipStream_t stream);

hipError_t launch_absorb_q(const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                           const uint16_t* w_uk, uint16_t* q_out, int32_t N, int32_t H,
                           double rope_base, hipStream_t stream);

// append (bf16 pool, or FP8 codes when pool_scale is non-null) and absorb in one launch;
// new token n sits at pos[n] and is also query n
hipError_t launch_append_absorb(const uint16_t* c_kv, const uint16_t* k_pe, const int64_t* slot_mapping,
                                void* pool, float* pool_scale, int64_t num_blocks, const uint16_t* q_nope,
                                const uint16_t* q_pe, const int32_t* pos, const uint16_t* w_uk,
                                uint16_t* q_out, int32_t N, int32_t H, double rope_base, hipStream_t stream);

// the same into the two-buffer cache: new token n goes to [seq_idx[n]][pos[n]]
hipError_t launch_append_absorb_kvpe(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* seq_idx,
                                     uint16_t* kv_cache, uint16_t* pe_cache, int32_t B, int32_t max_seq,
                                     const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                                     const uint16_t* w_uk, uint16_t* q_out, int32_t N, int32_t H, double rope_base,
                                     hipStream_t stream);

hipError_t launch_out_up(const uint16_t* o_lat, const uint16_t* w_uv, uint16_t* o, int32_t N,
                         int32_t H, hipStream_t stream);

// Shape of a linear map's launch: step width, features per workgroup, and
// the number of contraction slices (ks > 1 needs ws_bytes of fp32 workspace).
struct LinearPlan {
  bool wide;        // 128-wide contraction steps (K % 128 == 0, K <= 8192)
  int mt;           // 16-feature tiles per workgroup (1, 2 or 4)
  int u;            // 32-wide steps per wave with loads in flight together
  int ks;           // contraction slices, each its own workgroups
  size_t ws_bytes;  // ks * N * M * 4 when ks > 1, else 0
};
// can_split = false: the best plan with ks = 1 (no workspace).
LinearPlan plan_linear(int32_t N, int32_t K, int32_t M, bool can_split);

// Splits only when workspace holds at least plan_linear(..., true).ws_bytes;
// otherwise runs plan_linear(..., false).
hipError_t launch_linear(const uint16_t* x, const uint16_t* w, const uint16_t* r, uint16_t* y, void* workspace,
                         size_t workspace_bytes, int32_t N, int32_t K, int32_t M, hipStream_t stream);

// Split-KV plan shared by the host (workspace sizing, grid) and the kernels.
// Kernel shapes: the 128-row and 64-row kernels, the 32- and 16-row column kernels.
enum { V_ROWS128 = 0, V_ROWS64 = 1, V_COLS32 = 2, V_COLS16 = 3 };
struct AttnPlan {
  int variant;    // kernel shape, see attn.hip
  int rg_rows;    // query rows per workgroup (row group)
  int n_rg;       // row groups per sequence
  int width;      // workgroups per row group (stream-K width)
};

AttnPlan plan_attention(int32_t B, int32_t Lq, int32_t H);
AttnPlan plan_attention_fp8(int32_t B, int32_t Lq, int32_t H);
AttnPlan plan_attention_kvpe(int32_t B, int32_t Lq, int32_t H);

// Workspace of the expanded-form attention (expand.hip): the gathered latent
// rows c [B][Lpad][512] and rope keys [B][Lpad][64], the expanded content keys
// K [B][Lpad][H 128] and the transposed values V^T [B][H 128][Lpad], each
// region on a 256-byte boundary; Lpad = max_len rounded up to 32.
struct ExpandedLayout {
  int32_t Lpad;
  size_t c_off, kr_off, k_off, vt_off, bytes;
};
ExpandedLayout expanded_layout(int32_t B, int32_t H, int32_t max_len);

// Expanded-form attention of Lq query tokens per sequence: gather, the two
// expansion GEMMs per sequence, the attention kernel (expand.hip).
hipError_t launch_prefill_expanded(const uint16_t* q_nope, const uint16_t* q_pe, const int32_t* pos,
                                   const uint16_t* pool, int64_t num_blocks, const int32_t* block_table,
                                   int32_t max_blocks, const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H,
                                   int32_t max_len, const uint16_t* w_uk, const uint16_t* w_uv,
                                   float softmax_scale, double rope_base, uint16_t* o, float* lse,
                                   void* workspace, hipStream_t stream);

// Partial-result slots of one call: width + B (one per (workgroup, sequence) pair).
size_t attention_workspace_bytes(int32_t B, int32_t Lq, int32_t H);
// Bytes of the workspace's (m, l) part; the bf16 partials start there.
size_t attention_ws_ml_bytes(int32_t B, int32_t Lq, int32_t H);

hipError_t launch_decode_attn(const uint16_t* q, const uint16_t* pool, int64_t num_blocks,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H,
                              float softmax_scale, uint16_t* o_lat, float* lse, void* workspace,
                              hipStream_t stream);

// mla_decode_attn with its partials in a fixed per-device array of this many
// bytes instead of a caller workspace (see attn.hip); a shape whose workspace
// exceeds it returns hipErrorInvalidValue before anything is enqueued, and a
// stream of another device than the current one hipErrorInvalidDevice.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
hipError_t launch_decode_attn_noalloc(const uint16_t* q, const uint16_t* pool, int64_t num_blocks,
                                      const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                                      int32_t B, int32_t Lq, int32_t H, float softmax_scale, uint16_t* o_lat,
                                      float* lse, hipStream_t stream);

// Two-buffer latent cache: kv_cache [B][max_seq][512] and pe_cache [B][max_seq][64] bf16.
hipError_t launch_cache_append_kvpe(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* pos,
                                    const int32_t* seq_idx, uint16_t* kv_cache, uint16_t* pe_cache, int32_t B,
                                    int32_t max_seq, int32_t T, double rope_base, hipStream_t stream);

hipError_t launch_decode_attn_kvpe(const uint16_t* q, const uint16_t* kv_cache, const uint16_t* pe_cache,
                                   int32_t max_seq, const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H,
                                   float softmax_scale, uint16_t* o_lat, float* lse, void* workspace,
                                   hipStream_t stream);

// FP8 latent cache: codes [num_blocks][64][576] E4M3, scales [num_blocks][64] fp32.
hipError_t launch_cache_append_fp8(const uint16_t* c_kv, const uint16_t* k_pe, const int32_t* pos,
                                   const int64_t* slot_mapping, uint8_t* pool8, float* pool_scale,
                                   int64_t num_blocks, int32_t T, double rope_base, hipStream_t stream);

hipError_t launch_decode_attn_fp8(const uint16_t* q, const uint8_t* pool8, const float* pool_scale,
                                  int64_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* seq_lens, int32_t B, int32_t Lq, int32_t H,
                                  float softmax_scale, uint16_t* o_lat, float* lse, void* workspace,
                                  hipStream_t stream);

}  // namespace mla
