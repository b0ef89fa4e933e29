// Drives every entry point of the C ABI (capi.cpp) against the host launcher
// stand-ins (stub_launch.cpp) with buffers of exactly the sizes mla_absorb.h
// documents: valid calls must return MLA_OK and stay inside those buffers,
// invalid ones must return their error code before touching anything. Built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py, which also builds it once with
// -DPLANT_SHORT_WORKSPACE (a workspace 256 bytes shorter than the size the
// call is told) to show that an overrun is caught.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "mla_absorb.h"

static int g_fail = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                             \
    }                                                                       \
  } while (0)

template <class T>
struct Buf {  // heap array of exactly n elements (operator new: 16-byte aligned)
  std::vector<T> v;
  explicit Buf(size_t n) : v(n) {}
  T* p() { return v.data(); }
};

static mla_dims dims_for(int h) {
  mla_dims d;
  mla_dims_default(&d, h);
  return d;
}

static void test_dims() {
  Buf<uint16_t> q(16 * 576), o(16 * 512);
  mla_dims d = dims_for(16);
  d.num_heads = 0;
  EXPECT(mla_out_up(&d, o.p(), o.p(), o.p(), 1, nullptr) == MLA_ERR_INVALID_ARG);
  d = dims_for(16);
  d.softmax_scale = NAN;
  EXPECT(mla_out_up(&d, o.p(), o.p(), o.p(), 1, nullptr) == MLA_ERR_INVALID_ARG);
  d = dims_for(16);
  d.rope_base = INFINITY;
  EXPECT(mla_out_up(&d, o.p(), o.p(), o.p(), 1, nullptr) == MLA_ERR_INVALID_ARG);
  d = dims_for(16);
  d.d_c = 256;
  EXPECT(mla_out_up(&d, o.p(), o.p(), o.p(), 1, nullptr) == MLA_ERR_UNSUPPORTED);
  d = dims_for(256);
  EXPECT(mla_out_up(&d, o.p(), o.p(), o.p(), 1, nullptr) == MLA_ERR_UNSUPPORTED);
  EXPECT(mla_out_up(nullptr, o.p(), o.p(), o.p(), 1, nullptr) == MLA_ERR_INVALID_ARG);
  mla_dims_default(nullptr, 16);
  for (int s = -1; s <= 4; ++s) EXPECT(mla_status_str(s) != nullptr);
}

static void test_append_absorb_out_up() {
  for (int H : {16, 128}) {
    const mla_dims d = dims_for(H);
    const int T = 7;
    const int64_t nb = 2;
    Buf<uint16_t> ckv(T * 512), kpe(T * 64), pool(nb * 64 * 576), qn(T * H * 128), qp(T * H * 64),
        wuk(H * 128 * 512), qo(T * H * 576), ol(T * H * 512), o(T * H * 128);
    Buf<int32_t> pos(T);
    Buf<int64_t> slot(T);
    Buf<uint8_t> pool8(nb * 64 * 576);
    Buf<float> sc(nb * 64);
    const int64_t slots[T] = {0, 5, 127, 128, -1, 64, 1000000};  // three outside [0, 128)
    for (int t = 0; t < T; ++t) slot.p()[t] = slots[t], pos.p()[t] = t;
    EXPECT(mla_cache_append(&d, ckv.p(), kpe.p(), pos.p(), slot.p(), pool.p(), nb, T, nullptr) == MLA_OK);
    EXPECT(mla_cache_append(&d, ckv.p(), kpe.p(), pos.p(), slot.p(), pool.p(), 0, T, nullptr) == MLA_ERR_INVALID_ARG);
    EXPECT(mla_cache_append(&d, ckv.p(), kpe.p(), pos.p(), slot.p(), pool.p(), nb, 0, nullptr) == MLA_ERR_INVALID_ARG);
    EXPECT(mla_cache_append(&d, nullptr, kpe.p(), pos.p(), slot.p(), pool.p(), nb, T, nullptr) == MLA_ERR_INVALID_ARG);
    EXPECT(mla_cache_append_fp8(&d, ckv.p(), kpe.p(), pos.p(), slot.p(), pool8.p(), sc.p(), nb, T, nullptr) == MLA_OK);
    EXPECT(mla_cache_append_fp8(&d, ckv.p(), kpe.p(), pos.p(), slot.p(), pool8.p(), nullptr, nb, T, nullptr) ==
           MLA_ERR_INVALID_ARG);
    EXPECT(mla_absorb_q(&d, qn.p(), qp.p(), pos.p(), wuk.p(), qo.p(), T, nullptr) == MLA_OK);
    EXPECT(mla_absorb_q(&d, qn.p(), qp.p(), pos.p(), wuk.p(), qo.p(), -3, nullptr) == MLA_ERR_INVALID_ARG);
    EXPECT(mla_append_absorb(&d, ckv.p(), kpe.p(), slot.p(), pool.p(), nb, qn.p(), qp.p(), pos.p(), wuk.p(), qo.p(), T,
                             nullptr) == MLA_OK);
    EXPECT(mla_append_absorb_fp8(&d, ckv.p(), kpe.p(), slot.p(), pool8.p(), sc.p(), nb, qn.p(), qp.p(), pos.p(),
                                 wuk.p(), qo.p(), T, nullptr) == MLA_OK);
    EXPECT(mla_out_up(&d, ol.p(), wuk.p(), o.p(), T, nullptr) == MLA_OK);
    EXPECT(mla_out_up(&d, ol.p(), wuk.p(), nullptr, T, nullptr) == MLA_ERR_INVALID_ARG);
    EXPECT(mla_out_up(&d, ol.p(), wuk.p(), o.p(), (1 << 22) + 1, nullptr) == MLA_ERR_UNSUPPORTED);
    EXPECT(mla_absorb_q(&d, qn.p(), qp.p(), pos.p(), wuk.p(), qo.p(), (1 << 22) + 1, nullptr) == MLA_ERR_UNSUPPORTED);
  }
}

static void test_linear() {
  struct S { int N, K, M; } shapes[] = {{5, 64, 12}, {1, 8192, 64}, {33, 1024, 4096}, {2, 16384, 512}, {70, 96, 8}};
  for (const S& s : shapes) {
    Buf<uint16_t> x((size_t)s.N * s.K), w((size_t)s.M * s.K), r((size_t)s.N * s.M), y((size_t)s.N * s.M);
    const size_t ws = mla_linear_workspace_size(s.N, s.K, s.M);
    Buf<unsigned char> work(ws ? ws : 1);
    EXPECT(mla_linear(x.p(), w.p(), r.p(), y.p(), s.N, s.K, s.M, ws ? work.p() : nullptr, ws, nullptr) == MLA_OK);
    EXPECT(mla_linear(x.p(), w.p(), nullptr, y.p(), s.N, s.K, s.M, nullptr, 0, nullptr) == MLA_OK);
    if (ws > 16)  // a short workspace runs the unsplit plan and leaves it alone
      EXPECT(mla_linear(x.p(), w.p(), r.p(), y.p(), s.N, s.K, s.M, work.p(), ws - 16, nullptr) == MLA_OK);
  }
  Buf<uint16_t> a(64 * 64);
  Buf<unsigned char> work(64);
  EXPECT(mla_linear(a.p(), a.p(), nullptr, a.p(), 1, 48, 4, nullptr, 0, nullptr) == MLA_ERR_UNSUPPORTED);
  EXPECT(mla_linear(a.p(), a.p(), nullptr, a.p(), 1, 64, 6, nullptr, 0, nullptr) == MLA_ERR_UNSUPPORTED);
  EXPECT(mla_linear(a.p(), a.p(), nullptr, a.p(), 1, 64, 4, work.p() + 4, 32, nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_linear(a.p(), a.p(), nullptr, a.p(), 0, 64, 4, nullptr, 0, nullptr) == MLA_ERR_INVALID_ARG);
  // sizes at the ends of the int32 range: rejected or sized without overflow
  EXPECT(mla_linear_workspace_size(1, 32, 0x7ffffffc) == 0);
  EXPECT(mla_linear_workspace_size(65535 * 32, 0x7fffffe0, 4) == 0);
  EXPECT(mla_linear_workspace_size(65535 * 32 + 1, 32, 4) == 0);
  EXPECT(mla_linear(a.p(), a.p(), nullptr, a.p(), 1, 32, 0x7ffffffc, nullptr, 0, nullptr) == MLA_ERR_UNSUPPORTED);
}

// One paged-pool attention case: blocks handed out in a scrambled order,
// some table entries out of range, lengths including 0, a partial block and
// one above the table's reach.
static void attn_case(int B, int Lq, int H, bool fp8) {
  const mla_dims d = dims_for(H);
  const int max_blocks = 5;
  const int64_t nb = (int64_t)B * max_blocks;
  const size_t rows = (size_t)Lq * H;
  Buf<uint16_t> q(B * rows * 576), pool(fp8 ? 16 : nb * 64 * 576), o(B * rows * 512);
  Buf<uint8_t> pool8(fp8 ? nb * 64 * 576 : 16);
  Buf<float> sc(fp8 ? nb * 64 : 4), lse(B * rows);
  Buf<int32_t> table((size_t)B * max_blocks), lens(B);
  for (int i = 0; i < B * max_blocks; ++i) table.p()[i] = (int32_t)((i * 7 + 3) % nb);
  table.p()[1] = -1;
  if (B > 1) table.p()[max_blocks + 2] = (int32_t)nb;
  const int32_t lens_pat[] = {1, 0, 64 * max_blocks, 65, 64 * max_blocks + 1, 200, 7};
  for (int b = 0; b < B; ++b) lens.p()[b] = lens_pat[b % 7] + (b % 7 == 0 ? Lq - 1 : 0);
  const size_t need = mla_decode_workspace_size(&d, B, Lq);
  EXPECT(need > 0 && need % 256 == 0);
#ifdef PLANT_SHORT_WORKSPACE
  Buf<unsigned char> ws(need - 256);
#else
  Buf<unsigned char> ws(need);
#endif
  auto call = [&](uint16_t* qq, void* w, size_t wb, float* l) {
    return fp8 ? mla_decode_attn_fp8(&d, qq, pool8.p(), sc.p(), nb, table.p(), max_blocks, lens.p(), B, Lq, o.p(), l,
                                     w, wb, nullptr)
               : mla_decode_attn(&d, qq, pool.p(), nb, table.p(), max_blocks, lens.p(), B, Lq, o.p(), l, w, wb,
                                 nullptr);
  };
  EXPECT(call(q.p(), ws.p(), need, lse.p()) == MLA_OK);
  EXPECT(call(q.p(), ws.p(), need, nullptr) == MLA_OK);
  EXPECT(call(q.p(), ws.p(), need - 16, lse.p()) == MLA_ERR_WORKSPACE);
  EXPECT(call(q.p(), nullptr, need, lse.p()) == MLA_ERR_WORKSPACE);
  EXPECT(call(q.p() + 1, ws.p(), need, lse.p()) == MLA_ERR_INVALID_ARG);
  EXPECT(call(q.p(), ws.p() + 8, need, lse.p()) == MLA_ERR_INVALID_ARG);
  EXPECT(call(q.p(), ws.p(), need, (float*)((char*)lse.p() + 2)) == MLA_ERR_INVALID_ARG);
  if (!fp8 && need <= MLA_NOALLOC_SCRATCH_BYTES)
    EXPECT(mla_decode_attn_noalloc(&d, q.p(), pool.p(), nb, table.p(), max_blocks, lens.p(), B, Lq, o.p(), lse.p(),
                                   nullptr) == MLA_OK);
}

static void test_attention() {
  const int cases[][3] = {{1, 1, 16}, {3, 1, 16}, {7, 1, 32}, {2, 1, 64}, {5, 1, 128}, {2, 3, 128},
                          {3, 8, 128}, {1, 64, 16}, {2, 203, 128}, {9, 2, 48}};
  for (auto& c : cases) {
    attn_case(c[0], c[1], c[2], false);
    attn_case(c[0], c[1], c[2], true);
  }
  const mla_dims d = dims_for(128), d20 = dims_for(20);
  Buf<uint16_t> a(16);
  Buf<int32_t> t(16);
  Buf<unsigned char> w(1 << 16);
  EXPECT(mla_decode_attn(&d20, a.p(), a.p(), 1, t.p(), 1, t.p(), 1, 1, a.p(), nullptr, w.p(), 1 << 16, nullptr) ==
         MLA_ERR_UNSUPPORTED);
  EXPECT(mla_decode_attn(&d, a.p(), a.p(), 1, t.p(), 1, t.p(), 1, 8193, a.p(), nullptr, w.p(), 1 << 16, nullptr) ==
         MLA_ERR_UNSUPPORTED);
  EXPECT(mla_decode_attn(&d, a.p(), a.p(), 1, t.p(), 1 << 25, t.p(), 1, 1, a.p(), nullptr, w.p(), 1 << 16, nullptr) ==
         MLA_ERR_UNSUPPORTED);
  EXPECT(mla_decode_attn(&d, a.p(), a.p(), 0, t.p(), 1, t.p(), 1, 1, a.p(), nullptr, w.p(), 1 << 16, nullptr) ==
         MLA_ERR_INVALID_ARG);
  // workspace sizes at the ends of the int32 range: 0 (unsupported) rather than overflow
  EXPECT(mla_decode_workspace_size(&d, 1, 1 << 30) == 0);
  EXPECT(mla_decode_workspace_size(&d, 0x7fffffff, 8192) == 0);
  EXPECT(mla_decode_workspace_size(&d, 67108863, 1) > 0);    // B * ceil(128 / 4) = 2^31 - 32
  EXPECT(mla_decode_workspace_size(&d, 67108864, 1) == 0);   // one sequence more: 2^31
  EXPECT(mla_decode_workspace_size(&d, 1, 0) == 0);
  // no-alloc: a shape whose partials exceed the fixed array is refused
  EXPECT(mla_decode_attn_noalloc(&d, a.p(), a.p(), 1, t.p(), 1, t.p(), 64, 512, a.p(), nullptr, nullptr) ==
         MLA_ERR_WORKSPACE);
}

static void test_kvpe() {
  for (int H : {16, 128}) {
    const mla_dims d = dims_for(H);
    const int B = 3, max_seq = 100, T = 6, Lq = 2;
    const size_t rows = (size_t)Lq * H;
    Buf<uint16_t> ckv(T * 512), kpe(T * 64), kv((size_t)B * max_seq * 512), pe((size_t)B * max_seq * 64),
        q(B * rows * 576), o(B * rows * 512);
    Buf<int32_t> pos(T), sidx(T), lens(B);
    const int32_t P[T] = {0, 99, 100, -1, 50, 3}, S[T] = {0, 2, 1, 1, 3, -1};
    for (int t = 0; t < T; ++t) pos.p()[t] = P[t], sidx.p()[t] = S[t];
    EXPECT(mla_cache_append_kvpe(&d, ckv.p(), kpe.p(), pos.p(), sidx.p(), kv.p(), pe.p(), B, max_seq, T, nullptr) ==
           MLA_OK);
    EXPECT(mla_cache_append_kvpe(&d, ckv.p(), kpe.p(), pos.p(), sidx.p(), kv.p(), pe.p(), 0, max_seq, T, nullptr) ==
           MLA_ERR_INVALID_ARG);
    {
      Buf<uint16_t> qn((size_t)T * H * 128), qp((size_t)T * H * 64), wuk((size_t)H * 128 * 512), qo((size_t)T * H * 576);
      EXPECT(mla_append_absorb_kvpe(&d, ckv.p(), kpe.p(), sidx.p(), kv.p(), pe.p(), B, max_seq, qn.p(), qp.p(), pos.p(),
                                    wuk.p(), qo.p(), T, nullptr) == MLA_OK);
      EXPECT(mla_append_absorb_kvpe(&d, ckv.p(), kpe.p(), sidx.p(), kv.p(), nullptr, B, max_seq, qn.p(), qp.p(),
                                    pos.p(), wuk.p(), qo.p(), T, nullptr) == MLA_ERR_INVALID_ARG);
    }
    const int32_t L[B] = {100, 0, 250};  // the last one above max_seq
    for (int b = 0; b < B; ++b) lens.p()[b] = L[b];
    const size_t need = mla_decode_workspace_size(&d, B, Lq);
    Buf<unsigned char> ws(need);
    Buf<float> lse(B * rows);
    EXPECT(mla_decode_attn_kvpe(&d, q.p(), kv.p(), pe.p(), max_seq, lens.p(), B, Lq, o.p(), lse.p(), ws.p(), need,
                                nullptr) == MLA_OK);
    EXPECT(mla_decode_attn_kvpe(&d, q.p(), kv.p(), pe.p(), max_seq, lens.p(), B, Lq, o.p(), lse.p(), ws.p(), need - 16,
                                nullptr) == MLA_ERR_WORKSPACE);
    EXPECT(mla_decode_attn_kvpe(&d, q.p(), kv.p(), pe.p() + 1, max_seq, lens.p(), B, Lq, o.p(), lse.p(), ws.p(), need,
                                nullptr) == MLA_ERR_INVALID_ARG);
    EXPECT(mla_decode_attn_kvpe(&d, q.p(), kv.p(), pe.p(), (1 << 30) + 1, lens.p(), B, Lq, o.p(), lse.p(), ws.p(),
                                need, nullptr) == MLA_ERR_UNSUPPORTED);
  }
}

// The expanded-form prefill: gathered rows, expanded K and V^T in a workspace
// on a 256-byte boundary, one length above max_len, one 0, block ids out of
// the pool.
static void test_expanded() {
  for (int H : {16, 128}) {
    const mla_dims d = dims_for(H);
    const int B = 3, Lq = 4, max_len = 200, max_blocks = 4;
    const int64_t nb = (int64_t)B * max_blocks;
    const size_t N = (size_t)B * Lq;
    Buf<uint16_t> qn(N * H * 128), qp(N * H * 64), pool(nb * 64 * 576), wuk((size_t)H * 128 * 512),
        wuv((size_t)H * 128 * 512), o(N * H * 128);
    Buf<int32_t> pos(N), table((size_t)B * max_blocks), lens(B);
    Buf<float> lse(N * H);
    for (int i = 0; i < B * max_blocks; ++i) table.p()[i] = (int32_t)((i * 5 + 1) % nb);
    table.p()[2] = -1;
    table.p()[max_blocks + 1] = (int32_t)nb;
    const int32_t L[B] = {200, 0, 250};   // the last one above max_len
    for (int b = 0; b < B; ++b) lens.p()[b] = L[b];
    const size_t need = mla_prefill_expanded_workspace_size(&d, B, max_len);
    EXPECT(need > 0 && need % 256 == 0);
#ifdef PLANT_SHORT_WORKSPACE
    const size_t have = need - 256;
#else
    const size_t have = need;
#endif
    void* ws = aligned_alloc(256, have);
    auto call = [&](uint16_t* q, void* w, size_t wb, float* l, int lq, int ml) {
      return mla_prefill_expanded(&d, q, qp.p(), pos.p(), pool.p(), nb, table.p(), max_blocks, lens.p(), B, lq, ml,
                                  wuk.p(), wuv.p(), o.p(), l, w, wb, nullptr);
    };
    EXPECT(call(qn.p(), ws, need, lse.p(), Lq, max_len) == MLA_OK);
    EXPECT(call(qn.p(), ws, need, nullptr, Lq, max_len) == MLA_OK);
    EXPECT(call(qn.p(), ws, need - 16, lse.p(), Lq, max_len) == MLA_ERR_WORKSPACE);
    EXPECT(call(qn.p(), nullptr, need, lse.p(), Lq, max_len) == MLA_ERR_WORKSPACE);
    EXPECT(call(qn.p() + 1, ws, need, lse.p(), Lq, max_len) == MLA_ERR_INVALID_ARG);
    EXPECT(call(qn.p(), (char*)ws + 16, need, lse.p(), Lq, max_len) == MLA_ERR_INVALID_ARG);
    EXPECT(call(qn.p(), ws, need, (float*)((char*)lse.p() + 2), Lq, max_len) == MLA_ERR_INVALID_ARG);
    EXPECT(call(qn.p(), ws, need, lse.p(), 0, max_len) == MLA_ERR_INVALID_ARG);
    EXPECT(call(qn.p(), ws, need, lse.p(), Lq, (1 << 20) + 1) == MLA_ERR_UNSUPPORTED);
    free(ws);
  }
  const mla_dims d = dims_for(128);
  EXPECT(mla_prefill_expanded_workspace_size(&d, 0, 10) == 0);
  EXPECT(mla_prefill_expanded_workspace_size(&d, 65536, 10) == 0);
  EXPECT(mla_prefill_expanded_workspace_size(&d, 1, 0) == 0);
  EXPECT(mla_prefill_expanded_workspace_size(&d, 65535, 1 << 20) > 0);   // sized in 64 bits
}

int main() {
  test_dims();
  test_append_absorb_out_up();
  test_linear();
  test_attention();
  test_kvpe();
  test_expanded();
  if (g_fail) {
    fprintf(stderr, "sanitizer driver: %d expectation(s) failed\n", g_fail);
    return 1;
  }
  printf("sanitizer driver: all entry points checked\n");
  return 0;
}
