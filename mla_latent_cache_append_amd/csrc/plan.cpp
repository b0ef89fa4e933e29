// Host-side launch plans: the split-KV shape of an attention call, the size
// of its workspace, and the shape of a linear map's launch. Plain C++ with no
// device code, so that the argument checks of the C ABI and this arithmetic
// also build for the CPU alone (the sanitizer test in tests/asan/).
#include <algorithm>

#include "kernels.h"

namespace mla {

AttnPlan plan_attention(int32_t B, int32_t Lq, int32_t H) {
  (void)B;
  AttnPlan p;
  const int rows = Lq * H;
  if (rows >= 96) { p.variant = V_ROWS128; p.rg_rows = 128; }
  else if (rows >= 48) { p.variant = V_ROWS64; p.rg_rows = 64; }
  else if (rows >= 32) { p.variant = V_COLS32; p.rg_rows = 32; }
  else { p.variant = V_COLS16; p.rg_rows = 16; }
  p.n_rg = (rows + p.rg_rows - 1) / p.rg_rows;
  p.width = (TARGET_WGS + p.n_rg - 1) / p.n_rg;
  return p;
}

// FP8 pool: the 128-row kernel from 96 rows per sequence (codes widened in
// the LDS), the column kernel below, 16 or 32 rows per row group.
AttnPlan plan_attention_fp8(int32_t B, int32_t Lq, int32_t H) {
  (void)B;
  AttnPlan p;
  const int rows = Lq * H;
  if (rows >= 96) { p.variant = V_ROWS128; p.rg_rows = 128; }
  else if (rows <= 16) { p.variant = V_COLS16; p.rg_rows = 16; }
  else { p.variant = V_COLS32; p.rg_rows = 32; }
  p.n_rg = (rows + p.rg_rows - 1) / p.rg_rows;
  p.width = (TARGET_WGS + p.n_rg - 1) / p.n_rg;
  return p;
}

// Two-buffer layout (kv_cache + pe_cache): the same kernels as the paged
// pool (the 128-row kernel reads the rope rows through a second descriptor).
AttnPlan plan_attention_kvpe(int32_t B, int32_t Lq, int32_t H) { return plan_attention(B, Lq, H); }

// Workspace: (m, l) of every partial in fp32, then the partials themselves
// in bf16, normalized by their l, starting on a 256-byte boundary. Sized for
// the widest of the plans, so one workspace serves every cache format and layout.
static size_t ws_slots(int32_t B, int32_t Lq, int32_t H) {
  const int w = std::max(std::max(plan_attention(B, Lq, H).width, plan_attention_fp8(B, Lq, H).width),
                         plan_attention_kvpe(B, Lq, H).width);
  return (size_t)w + (size_t)B;
}
size_t attention_ws_ml_bytes(int32_t B, int32_t Lq, int32_t H) {
  const size_t bytes = ws_slots(B, Lq, H) * (size_t)Lq * (size_t)H * 2 * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

size_t attention_workspace_bytes(int32_t B, int32_t Lq, int32_t H) {
  return attention_ws_ml_bytes(B, Lq, H) + ws_slots(B, Lq, H) * (size_t)Lq * (size_t)H * D_C * sizeof(uint16_t);
}

ExpandedLayout expanded_layout(int32_t B, int32_t H, int32_t max_len) {
  auto r256 = [](size_t n) { return (n + 255) & ~(size_t)255; };
  ExpandedLayout w;
  w.Lpad = (max_len + 31) / 32 * 32;
  const size_t rows = (size_t)B * (size_t)w.Lpad;
  const size_t hd = (size_t)H * D_NOPE;
  w.c_off = 0;
  w.kr_off = w.c_off + r256(rows * D_C * sizeof(uint16_t));
  w.k_off = w.kr_off + r256(rows * D_ROPE * sizeof(uint16_t));
  w.vt_off = w.k_off + r256(rows * hd * sizeof(uint16_t));
  w.bytes = w.vt_off + r256(rows * hd * sizeof(uint16_t));
  return w;
}

LinearPlan plan_linear(int32_t N, int32_t K, int32_t M, bool can_split) {
  LinearPlan p;
  const int64_t ny = (N + LIN_N - 1) / LIN_N;
  auto wgs = [&](int mt) { return ((int64_t)M + 16 * mt - 1) / (16 * mt) * ny; };
  p.ks = 1;
  if (wgs(4) >= 224) {
    // wide outputs: 64 features per workgroup halve the activation bytes
    // each workgroup streams per weight byte; all of a wave's steps in one
    // batch of loads when they fit three
    p.wide = false;
    p.mt = 4;
    p.u = K / 32 <= 3 * LIN_WAVES ? 3 : 2;
  } else if (K % 128 != 0 || K > 8192) {
    p.wide = false;
    if (can_split && K >= 8192 && 2 * wgs(4) >= 224) {
      p.mt = 4;     // long contraction: 64 features, halves of it on their own workgroups
      p.ks = 2;
      p.u = 2;
    } else {
      p.mt = wgs(2) >= 128 ? 2 : 1;
      p.u = 4;
    }
  } else {
    p.wide = true;
    p.mt = M >= 1024 ? 2 : 1;
    p.u = 1;
    if (can_split && wgs(p.mt) < 128) {
      // about 192 workgroups, each slice keeping at least three steps
      const int64_t want = (192 + wgs(p.mt) - 1) / wgs(p.mt), most = (K / 128) / 3;
      p.ks = (int)std::max<int64_t>(1, std::min(want, most));
    }
  }
  p.ws_bytes = p.ks > 1 ? (size_t)p.ks * (size_t)N * (size_t)M * sizeof(float) : 0;
  return p;
}

}  // namespace mla
