"""Host-only checks of the C ABI library: it loads, exports every symbol the
header declares, and its host-side argument checks return the documented
status codes without touching a device (no kernel is launched here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_absorb.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(mla_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def nat():
    from mla_latent_cache_append_amd import native
    if not os.path.exists(native.LIB_PATH):
        from mla_latent_cache_append_amd import build
        build.build()
    native.lib()
    return native


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("mla_cache_append", "mla_absorb_q", "mla_decode_attn", "mla_out_up", "mla_linear",
              "mla_linear_workspace_size", "mla_decode_workspace_size", "mla_status_str", "mla_dims_default"):
        assert n in names


def test_library_exports_every_declared_symbol(nat):
    lib = nat.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings_and_defaults(nat):
    assert nat.mla_status_str(0) == "ok"
    assert nat.mla_status_str(-3).startswith("workspace")
    d = nat.mla_dims_default(128)
    assert (d.num_heads, d.d_c, d.d_rope, d.d_nope, d.d_v, d.block_size) == (128, 512, 64, 128, 128, 64)
    assert abs(d.softmax_scale - 192 ** -0.5) < 1e-7 and d.rope_base == 10000.0


def test_workspace_size_is_host_arithmetic(nat):
    d = nat.mla_dims_default(128)
    s1 = nat.mla_decode_workspace_size(d, 32, 1)
    s8 = nat.mla_decode_workspace_size(d, 16, 8)
    assert s1 > 0 and s8 > 0 and s1 % 4 == 0
    # (range slots + sequences) x rows x ((m, l) in fp32 + 512 bf16 partials),
    # the bf16 part starting on a 256-byte boundary
    slots = s1 // (128 * (8 + 1024))
    assert s1 == ((slots * 128 * 8 + 255) // 256) * 256 + slots * 128 * 1024
    bad = nat.mla_dims_default(128)
    bad.d_c = 256
    assert nat.mla_decode_workspace_size(bad, 32, 1) == 0


def test_invalid_arguments_return_status(nat):
    lib = nat.lib()
    d = nat.mla_dims_default(16)
    P = ctypes.c_void_p
    fake = P(0x1000)   # never dereferenced: the host checks fail first
    null = P(0)
    assert lib.mla_cache_append(ctypes.byref(d), null, fake, fake, fake, fake, 4, 1, null) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_append(ctypes.byref(d), fake, fake, fake, fake, fake, 4, 0, null) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(ctypes.byref(d), fake, fake, fake, fake, null, 3, null) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_out_up(ctypes.byref(d), fake, fake, fake, -1, null) == nat.MLA_ERR_INVALID_ARG
    # workspace smaller than required
    assert lib.mla_decode_attn(ctypes.byref(d), fake, fake, 4, fake, 2, fake, 2, 1, fake, null,
                               fake, 16, null) == nat.MLA_ERR_WORKSPACE
    assert lib.mla_decode_attn(ctypes.byref(d), fake, fake, 4, fake, 2, fake, 2, 1, fake, null,
                               null, 1 << 30, null) == nat.MLA_ERR_WORKSPACE
    # unsupported shapes
    d24 = nat.mla_dims_default(24)
    assert lib.mla_decode_attn(ctypes.byref(d24), fake, fake, 4, fake, 2, fake, 2, 1, fake, null,
                               fake, 1 << 30, null) == nat.MLA_ERR_UNSUPPORTED
    d.block_size = 32
    assert lib.mla_cache_append(ctypes.byref(d), fake, fake, fake, fake, fake, 4, 1, null) == nat.MLA_ERR_UNSUPPORTED
    d = nat.mla_dims_default(16)
    d.softmax_scale = 0.0
    assert lib.mla_out_up(ctypes.byref(d), fake, fake, fake, 1, null) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_append(None, fake, fake, fake, fake, fake, 4, 1, null) == nat.MLA_ERR_INVALID_ARG


def split_slices(N, K, M):
    """The documented split rule, restated: 64 features per workgroup alone
    when that gives >= 224 workgroups (unsplit); a contraction that is not a
    multiple of 128 or longer than 8192 splits in two when K >= 8192 and two
    halves of 64-feature workgroups reach 224; otherwise 128-wide steps with
    32 features when M >= 1024 (else 16), cut into ceil(192 / workgroups)
    slices, at most a third of the 128-wide steps, when fewer than 128
    workgroups remain."""
    ny = -(-N // 32)
    wgs = lambda mt: -(-M // (16 * mt)) * ny
    if wgs(4) >= 224:
        return 1
    if K % 128 or K > 8192:
        return 2 if K >= 8192 and 2 * wgs(4) >= 224 else 1
    mt = 2 if M >= 1024 else 1
    if wgs(mt) >= 128:
        return 1
    return max(1, min(-(-192 // wgs(mt)), (K // 128) // 3))


@pytest.mark.parametrize("N,K,M", [(32, 7168, 512), (32, 7168, 64), (32, 7168, 1536), (32, 1536, 16384),
                                   (32, 16384, 7168), (1, 2048, 2048), (200, 512, 64), (33, 1536, 2048),
                                   (7, 96, 12), (32, 2048, 512), (90, 8224, 2420), (64, 1536, 7168),
                                   (3, 16384, 1024), (32, 8192, 7168)])
def test_linear_workspace_size_is_the_split_rule(nat, N, K, M):
    ks = split_slices(N, K, M)
    assert nat.mla_linear_workspace_size(N, K, M) == (ks * N * M * 4 if ks > 1 else 0)


def test_linear_layer_maps_split_as_measured(nat):
    # the 128-head layer's maps at 32 tokens: Wdkv 6 slices, Wkr 18, Wdq 4, Wo 2; Wuq and Wqr unsplit
    assert nat.mla_linear_workspace_size(32, 7168, 512) == 6 * 32 * 512 * 4
    assert nat.mla_linear_workspace_size(32, 7168, 64) == 18 * 32 * 64 * 4
    assert nat.mla_linear_workspace_size(32, 7168, 1536) == 4 * 32 * 1536 * 4
    assert nat.mla_linear_workspace_size(32, 16384, 7168) == 2 * 32 * 7168 * 4
    for K, M in ((1536, 16384), (1536, 8192)):
        assert nat.mla_linear_workspace_size(32, K, M) == 0
    # unsupported sizes report no workspace
    for N, K, M in ((0, 7168, 512), (32, 48, 512), (32, 7168, 6), (65535 * 32 + 1, 128, 4)):
        assert nat.mla_linear_workspace_size(N, K, M) == 0


def test_linear_checks_arguments_on_the_host(nat):
    lib = nat.lib()
    P = ctypes.c_void_p
    fake, null = P(0x1000), P(0)
    call = lambda x, y, N, K, M, ws, wsb: lib.mla_linear(x, fake, null, y, N, K, M, ws, wsb, null)
    assert call(null, fake, 32, 7168, 512, null, 0) == nat.MLA_ERR_INVALID_ARG
    assert call(fake, null, 32, 7168, 512, null, 0) == nat.MLA_ERR_INVALID_ARG
    assert call(fake, fake, 0, 7168, 512, null, 0) == nat.MLA_ERR_INVALID_ARG
    assert call(fake, fake, 32, 7168, 512, P(0x1008), 1 << 20) == nat.MLA_ERR_INVALID_ARG   # misaligned
    assert call(fake, fake, 32, 48, 512, null, 0) == nat.MLA_ERR_UNSUPPORTED
    assert call(fake, fake, 32, 7168, 6, null, 0) == nat.MLA_ERR_UNSUPPORTED
    assert call(fake, fake, 65535 * 32 + 1, 7168, 512, null, 0) == nat.MLA_ERR_UNSUPPORTED


def test_size_limits_return_unsupported(nat):
    # rows of one sequence (Lq * H) above 2^20, a block table spanning more than
    # 2^30 keys, and more merge workgroups than a grid holds: refused on the host
    lib = nat.lib()
    d = nat.mla_dims_default(16)
    P = ctypes.c_void_p
    fake, null = P(0x1000), P(0)
    for fn in (lib.mla_decode_attn, ):
        assert fn(ctypes.byref(d), fake, fake, 4, fake, 2, fake, 1, (1 << 16) + 1, fake, null, fake, 1 << 40,
                  null) == nat.MLA_ERR_UNSUPPORTED
        assert fn(ctypes.byref(d), fake, fake, 4, fake, (1 << 24) + 1, fake, 1, 1, fake, null, fake, 1 << 40,
                  null) == nat.MLA_ERR_UNSUPPORTED
        assert fn(ctypes.byref(d), fake, fake, 4, fake, 2, fake, 1 << 30, 1 << 16, fake, null, fake, 1 << 40,
                  null) == nat.MLA_ERR_UNSUPPORTED
    assert lib.mla_decode_attn_fp8(ctypes.byref(d), fake, fake, fake, 4, fake, 2, fake, 1, (1 << 16) + 1, fake,
                                   null, fake, 1 << 40, null) == nat.MLA_ERR_UNSUPPORTED
    assert lib.mla_decode_attn_fp8(ctypes.byref(d), fake, fake, fake, 4, fake, (1 << 24) + 1, fake, 1, 1, fake,
                                   null, fake, 1 << 40, null) == nat.MLA_ERR_UNSUPPORTED
    # heads above 128
    d200 = nat.mla_dims_default(144)
    assert lib.mla_decode_attn(ctypes.byref(d200), fake, fake, 4, fake, 2, fake, 1, 1, fake, null, fake, 1 << 40,
                               null) == nat.MLA_ERR_UNSUPPORTED


def test_row_calls_reject_misaligned_pointers(nat):
    """The append, absorb and up-projection calls move rows with 16-byte
    vector accesses: a misaligned row pointer is refused before any launch."""
    lib = nat.lib()
    d = nat.mla_dims_default(16)
    P = ctypes.c_void_p
    a, m2, m4 = P(0x1000), P(0x1002), P(0x1004)
    assert lib.mla_cache_append(ctypes.byref(d), m4, a, a, a, a, 4, 2, None) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_append(ctypes.byref(d), a, m2, a, a, a, 4, 2, None) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_append(ctypes.byref(d), a, a, a, m4, a, 4, 2, None) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(ctypes.byref(d), a, a, a, a, m4, 2, None) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_out_up(ctypes.byref(d), a, m4, a, 2, None) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_append_absorb(ctypes.byref(d), a, a, a, a, 4, m4, a, a, a, a, 2,
                                 None) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_append_absorb_kvpe(ctypes.byref(d), a, a, a, a, m2, 2, 8, a, a, a, a, a, 2,
                                      None) == nat.MLA_ERR_INVALID_ARG


def test_fused_append_absorb_checks_arguments_on_the_host(nat):
    lib = nat.lib()
    d = nat.mla_dims_default(16)
    P = ctypes.c_void_p
    fake, null = P(0x1000), P(0)
    assert lib.mla_append_absorb(ctypes.byref(d), fake, fake, fake, fake, 4, fake, fake, fake, fake, null, 2,
                                 null) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_append_absorb(ctypes.byref(d), fake, fake, fake, fake, 4, fake, fake, fake, fake, fake, 0,
                                 null) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_append_absorb_fp8(ctypes.byref(d), fake, fake, fake, fake, null, 4, fake, fake, fake, fake,
                                     fake, 2, null) == nat.MLA_ERR_INVALID_ARG
    # two-buffer cache: null pe_cache, B = 0, N beyond 2^22
    assert lib.mla_append_absorb_kvpe(ctypes.byref(d), fake, fake, fake, fake, null, 2, 8, fake, fake, fake, fake,
                                      fake, 2, null) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_append_absorb_kvpe(ctypes.byref(d), fake, fake, fake, fake, fake, 0, 8, fake, fake, fake, fake,
                                      fake, 2, null) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_append_absorb_kvpe(ctypes.byref(d), fake, fake, fake, fake, fake, 2, 8, fake, fake, fake, fake,
                                      fake, (1 << 22) + 1, null) == nat.MLA_ERR_UNSUPPORTED
    d.block_size = 32
    assert lib.mla_append_absorb(ctypes.byref(d), fake, fake, fake, fake, 4, fake, fake, fake, fake, fake, 2,
                                 null) == nat.MLA_ERR_UNSUPPORTED


def test_fp8_calls_check_arguments_on_the_host(nat):
    lib = nat.lib()
    d = nat.mla_dims_default(16)
    P = ctypes.c_void_p
    fake, null = P(0x1000), P(0)
    # missing scale array, zero tokens
    assert lib.mla_cache_append_fp8(ctypes.byref(d), fake, fake, fake, fake, fake, null, 4, 1,
                                    null) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_append_fp8(ctypes.byref(d), fake, fake, fake, fake, fake, fake, 4, 0,
                                    null) == nat.MLA_ERR_INVALID_ARG
    # missing scale array; workspace too small; heads not a multiple of 16
    assert lib.mla_decode_attn_fp8(ctypes.byref(d), fake, fake, null, 4, fake, 2, fake, 2, 1, fake, null,
                                   fake, 1 << 30, null) == nat.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_attn_fp8(ctypes.byref(d), fake, fake, fake, 4, fake, 2, fake, 2, 1, fake, null,
                                   fake, 16, null) == nat.MLA_ERR_WORKSPACE
    d24 = nat.mla_dims_default(24)
    assert lib.mla_decode_attn_fp8(ctypes.byref(d24), fake, fake, fake, 4, fake, 2, fake, 2, 1, fake, null,
                                   fake, 1 << 30, null) == nat.MLA_ERR_UNSUPPORTED
    d.block_size = 32
    assert lib.mla_cache_append_fp8(ctypes.byref(d), fake, fake, fake, fake, fake, fake, 4, 1,
                                    null) == nat.MLA_ERR_UNSUPPORTED


def test_probe_library_exports_its_two_probes(nat):
    # the stream-read and MFMA-loop probes bench.py reports as achievable peaks
    from mla_latent_cache_append_amd import build
    if not os.path.exists(build.PROBE_LIB):
        build.build()
    lib = ctypes.CDLL(build.PROBE_LIB)
    for n in ("mla_probe_stream_read", "mla_probe_mfma"):
        assert hasattr(lib, n), n


def test_attention_calls_reject_misaligned_buffers(nat):
    """q, pool, o_lat and the workspace carry 16-byte accesses in the kernels
    (pool_scale too for the FP8 call), lse 4-byte ones: a misaligned pointer is
    an invalid argument, caught on the host before any launch."""
    lib = nat.lib()
    d = nat.mla_dims_default(16)
    P = ctypes.c_void_p
    ok, odd, null = P(0x1000), P(0x1008), P(0)
    big = 1 << 30

    def attn(q=ok, pool=ok, o=ok, lse=null, ws=ok):
        return lib.mla_decode_attn(ctypes.byref(d), q, pool, 4, ok, 2, ok, 2, 1, o, lse, ws, big, null)

    def attn8(q=ok, pool=ok, sc=ok, o=ok, lse=null, ws=ok):
        return lib.mla_decode_attn_fp8(ctypes.byref(d), q, pool, sc, 4, ok, 2, ok, 2, 1, o, lse, ws, big, null)

    for kw in ({"q": odd}, {"pool": odd}, {"o": odd}, {"ws": odd}, {"lse": P(0x1002)}):
        assert attn(**kw) == nat.MLA_ERR_INVALID_ARG, kw
        assert attn8(**kw) == nat.MLA_ERR_INVALID_ARG, kw
    assert attn8(sc=odd) == nat.MLA_ERR_INVALID_ARG


def test_no_alloc_attention_rejects_shapes_beyond_its_array(nat):
    """The workspace of a 512-token prefill chunk of 4 sequences at 128 heads
    (~338 MB) exceeds the fixed 64 MiB array: refused on the host (no device
    is touched)."""
    lib = nat.lib()
    d = nat.mla_dims_default(128)
    P = ctypes.c_void_p
    ok, null = P(0x1000), P(0)
    assert nat.mla_decode_workspace_size(d, 4, 512) > 64 << 20
    assert lib.mla_decode_attn_noalloc(ctypes.byref(d), ok, ok, 4, ok, 2, ok, 4, 512, ok, null,
                                       null) == nat.MLA_ERR_WORKSPACE
    assert lib.mla_decode_attn_noalloc(ctypes.byref(d), null, ok, 4, ok, 2, ok, 1, 1, ok, null,
                                       null) == nat.MLA_ERR_INVALID_ARG


def test_expanded_workspace_size_is_its_layout(nat):
    """Gathered latent and rope rows, then the expanded K and V^T, each region
    on a 256-byte boundary, for max_len rounded up to 32 rows per sequence."""
    d = nat.mla_dims_default(128)
    r256 = lambda n: (n + 255) // 256 * 256
    for B, max_len in [(4, 1000), (1, 1), (3, 32), (2, 33), (7, 16896)]:
        rows = B * ((max_len + 31) // 32 * 32)
        want = r256(rows * 512 * 2) + r256(rows * 64 * 2) + 2 * r256(rows * 128 * 128 * 2)
        assert nat.mla_prefill_expanded_workspace_size(d, B, max_len) == want, (B, max_len)
    for B, max_len in [(0, 10), (65536, 10), (1, 0), (1, (1 << 20) + 1)]:
        assert nat.mla_prefill_expanded_workspace_size(d, B, max_len) == 0, (B, max_len)


def test_expanded_checks_arguments_on_the_host(nat):
    lib = nat.lib()
    d = nat.mla_dims_default(128)
    P = ctypes.c_void_p
    fake, null = P(0x1000), P(0)   # never dereferenced: the host checks fail first
    need = nat.mla_prefill_expanded_workspace_size(d, 4, 1000)

    def call(dims=d, q=fake, pool=fake, nb=16, mb=16, B=4, Lq=8, max_len=1000, o=fake, lse=null, ws=fake,
             wsb=need):
        return lib.mla_prefill_expanded(ctypes.byref(dims), q, fake, fake, pool, nb, fake, mb, fake, B, Lq, max_len,
                                        fake, fake, o, lse, ws, wsb, null)

    for kw in (dict(q=null), dict(pool=null), dict(o=null), dict(B=0), dict(Lq=0), dict(max_len=0), dict(nb=0),
               dict(mb=0), dict(q=P(0x1008)), dict(o=P(0x1004)), dict(lse=P(0x1002)), dict(ws=P(0x1010))):
        assert call(**kw) == nat.MLA_ERR_INVALID_ARG, kw
    for kw in (dict(B=65536), dict(max_len=(1 << 20) + 1), dict(Lq=(1 << 20) + 1), dict(mb=(1 << 24) + 1)):
        assert call(**kw) == nat.MLA_ERR_UNSUPPORTED, kw
    assert call(wsb=need - 1) == nat.MLA_ERR_WORKSPACE
    assert call(ws=null) == nat.MLA_ERR_WORKSPACE
    bad = nat.mla_dims_default(128)
    bad.d_c = 256
    assert call(dims=bad) == nat.MLA_ERR_UNSUPPORTED


def test_prefill_form_follows_the_measured_crossover():
    """The step's form choice (host logic): the expanded form from the
    measured crossover's query-token count on, over the paged bf16 pool only."""
    from mla_latent_cache_append_amd import step
    assert step.prefill_form(1) == "absorbed"
    assert step.prefill_form(step.EXPANDED_FROM_LQ - 1) == "absorbed"
    assert step.prefill_form(step.EXPANDED_FROM_LQ) == "expanded"
    assert step.prefill_form(2048) == "expanded"
    assert step.prefill_form(2048, "fp8") == "absorbed"
    assert step.prefill_form(2048, "kvpe") == "absorbed"
    assert 256 < step.EXPANDED_FROM_LQ < 512   # between the sweep's last absorbed-faster and first expanded-faster sizes
