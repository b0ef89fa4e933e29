"""Thin ctypes binding of libmla_absorb (include/mla_absorb.h).

Same names as the C ABI. Each function checks tensor devices, dtypes, shapes
and contiguity, then passes raw device pointers and torch's current HIP stream
to the library; every step of the computation runs in the library's kernels.
If the library is missing the functions raise: there is no fallback path.

bf16 tensors are torch.bfloat16 (their storage is the bf16 bit pattern the C
ABI takes as uint16_t).
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_absorb.so")

D_C, D_ROPE, D_NOPE, D_V, BLOCK = 512, 64, 128, 128, 64
D_K = D_C + D_ROPE

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_LAUNCH = 0, -1, -2, -3, -4


class MlaDims(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("d_c", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("d_nope", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("rope_base", ctypes.c_float),
    ]


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {mla_status_str(status)} (status {status})")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SIG = {
    "mla_dims_default": (None, [ctypes.POINTER(MlaDims), _I32]),
    "mla_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_cache_append": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _P, _I64, _I32, _P]),
    "mla_absorb_q": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _P, _I32, _P]),
    "mla_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MlaDims), _I32, _I32]),
    "mla_decode_attn": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _I64, _P, _I32, _P, _I32, _I32,
                                       _P, _P, _P, ctypes.c_size_t, _P]),
    "mla_decode_attn_noalloc": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _I64, _P, _I32, _P, _I32, _I32,
                                               _P, _P, _P]),
    "mla_append_absorb": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _I64, _P, _P, _P, _P, _P,
                                         _I32, _P]),
    "mla_append_absorb_fp8": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _P, _I64, _P, _P, _P, _P,
                                             _P, _I32, _P]),
    "mla_cache_append_fp8": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _P, _P, _I64, _I32, _P]),
    "mla_decode_attn_fp8": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _P, _I64, _P, _I32, _P, _I32,
                                           _I32, _P, _P, _P, ctypes.c_size_t, _P]),
    "mla_cache_append_kvpe": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                             _P]),
    "mla_append_absorb_kvpe": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _P, _I32, _I32, _P, _P, _P,
                                              _P, _P, _I32, _P]),
    "mla_decode_attn_kvpe": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _P, _I32, _P, _I32, _I32, _P, _P,
                                            _P, ctypes.c_size_t, _P]),
    "mla_out_up": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _P, _I32, _P]),
    "mla_prefill_expanded_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MlaDims), _I32, _I32]),
    "mla_prefill_expanded": (ctypes.c_int, [ctypes.POINTER(MlaDims), _P, _P, _P, _P, _I64, _P, _I32, _P, _I32,
                                            _I32, _I32, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "mla_linear_workspace_size": (ctypes.c_size_t, [_I32, _I32, _I32]),
    "mla_linear": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _P, ctypes.c_size_t, _P]),
}


def lib() -> ctypes.CDLL:
    """Load libmla_absorb.so (built by ``mla_latent_cache_append_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def mla_status_str(status: int) -> str:
    return lib().mla_status_str(int(status)).decode()


def mla_dims_default(num_heads: int) -> MlaDims:
    d = MlaDims()
    lib().mla_dims_default(ctypes.byref(d), int(num_heads))
    return d


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _check(name: str, t: torch.Tensor, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _ok(fn: str, status: int):
    if status != MLA_OK:
        raise MlaError(fn, status)


def mla_cache_append(dims: MlaDims, c_kv, k_pe, pos, slot_mapping, pool, stream=None):
    """Write [c_kv | RoPE(k_pe, pos)] rows into ``pool`` at ``slot_mapping``."""
    T = c_kv.shape[0]
    _check("c_kv", c_kv, torch.bfloat16, (T, D_C))
    _check("k_pe", k_pe, torch.bfloat16, (T, D_ROPE))
    _check("pos", pos, torch.int32, (T,))
    _check("slot_mapping", slot_mapping, torch.int64, (T,))
    _check("pool", pool, torch.bfloat16)
    if pool.dim() != 3 or tuple(pool.shape[1:]) != (BLOCK, D_K):
        raise ValueError("pool must be [num_blocks, 64, 576]")
    _ok("mla_cache_append", lib().mla_cache_append(
        ctypes.byref(dims), _ptr(c_kv), _ptr(k_pe), _ptr(pos), _ptr(slot_mapping), _ptr(pool),
        pool.shape[0], T, _stream(stream)))


def mla_absorb_q(dims: MlaDims, q_nope, q_pe, pos, w_uk, q_out, stream=None):
    """q_out[n,h] = [W_UK[h]^T q_nope[n,h] | RoPE(q_pe[n,h], pos[n])]."""
    N, H = q_nope.shape[0], dims.num_heads
    _check("q_nope", q_nope, torch.bfloat16, (N, H, D_NOPE))
    _check("q_pe", q_pe, torch.bfloat16, (N, H, D_ROPE))
    _check("pos", pos, torch.int32, (N,))
    _check("w_uk", w_uk, torch.bfloat16, (H, D_NOPE, D_C))
    _check("q_out", q_out, torch.bfloat16, (N, H, D_K))
    _ok("mla_absorb_q", lib().mla_absorb_q(
        ctypes.byref(dims), _ptr(q_nope), _ptr(q_pe), _ptr(pos), _ptr(w_uk), _ptr(q_out), N,
        _stream(stream)))


def mla_decode_workspace_size(dims: MlaDims, B: int, Lq: int) -> int:
    return int(lib().mla_decode_workspace_size(ctypes.byref(dims), int(B), int(Lq)))


def mla_decode_attn(dims: MlaDims, q, pool, block_table, seq_lens, Lq: int, o_lat, lse=None,
                    workspace=None, stream=None):
    """Latent attention of ``q`` [B*Lq, H, 576] over the paged cache."""
    H = dims.num_heads
    B = seq_lens.shape[0]
    _check("q", q, torch.bfloat16, (B * Lq, H, D_K))
    _check("pool", pool, torch.bfloat16)
    _check("block_table", block_table, torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _check("seq_lens", seq_lens, torch.int32, (B,))
    _check("o_lat", o_lat, torch.bfloat16, (B * Lq, H, D_C))
    if lse is not None:
        _check("lse", lse, torch.float32, (B * Lq, H))
    if workspace is None:
        raise ValueError("workspace is required (mla_decode_workspace_size bytes, uint8)")
    _check("workspace", workspace, torch.uint8)
    _ok("mla_decode_attn", lib().mla_decode_attn(
        ctypes.byref(dims), _ptr(q), _ptr(pool), pool.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), B, Lq, _ptr(o_lat), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(stream)))


def mla_prefill_expanded_workspace_size(dims: MlaDims, B: int, max_len: int) -> int:
    return int(lib().mla_prefill_expanded_workspace_size(ctypes.byref(dims), int(B), int(max_len)))


def mla_prefill_expanded(dims: MlaDims, q_nope, q_pe, pos, pool, block_table, seq_lens, Lq: int, max_len: int,
                         w_uk, w_uv, o, lse=None, workspace=None, stream=None):
    """Expanded-form attention of ``Lq`` query tokens per sequence: o [B*Lq, H, 128]
    straight from q_nope, q_pe (not rotated) and pos, through per-head keys and
    values expanded from the cache (``max_len`` bounds every length)."""
    H = dims.num_heads
    B = seq_lens.shape[0]
    N = B * Lq
    _check("q_nope", q_nope, torch.bfloat16, (N, H, D_NOPE))
    _check("q_pe", q_pe, torch.bfloat16, (N, H, D_ROPE))
    _check("pos", pos, torch.int32, (N,))
    _check("pool", pool, torch.bfloat16)
    _check("block_table", block_table, torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _check("seq_lens", seq_lens, torch.int32, (B,))
    _check("w_uk", w_uk, torch.bfloat16, (H, D_NOPE, D_C))
    _check("w_uv", w_uv, torch.bfloat16, (H, D_V, D_C))
    _check("o", o, torch.bfloat16, (N, H, D_V))
    if lse is not None:
        _check("lse", lse, torch.float32, (N, H))
    if workspace is None:
        raise ValueError("workspace is required (mla_prefill_expanded_workspace_size bytes, uint8)")
    _check("workspace", workspace, torch.uint8)
    _ok("mla_prefill_expanded", lib().mla_prefill_expanded(
        ctypes.byref(dims), _ptr(q_nope), _ptr(q_pe), _ptr(pos), _ptr(pool), pool.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), B, Lq, int(max_len), _ptr(w_uk), _ptr(w_uv), _ptr(o), _ptr(lse),
        _ptr(workspace), workspace.numel(), _stream(stream)))


def mla_decode_attn_noalloc(dims: MlaDims, q, pool, block_table, seq_lens, Lq: int, o_lat, lse=None, stream=None):
    """mla_decode_attn with its partials in the library's fixed per-GPU array
    (no workspace; calls overlapping in time on one GPU race)."""
    H = dims.num_heads
    B = seq_lens.shape[0]
    _check("q", q, torch.bfloat16, (B * Lq, H, D_K))
    _check("pool", pool, torch.bfloat16)
    _check("block_table", block_table, torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _check("seq_lens", seq_lens, torch.int32, (B,))
    _check("o_lat", o_lat, torch.bfloat16, (B * Lq, H, D_C))
    if lse is not None:
        _check("lse", lse, torch.float32, (B * Lq, H))
    _ok("mla_decode_attn_noalloc", lib().mla_decode_attn_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(pool), pool.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), B, Lq, _ptr(o_lat), _ptr(lse), _stream(stream)))


def mla_append_absorb(dims: MlaDims, c_kv, k_pe, slot_mapping, pool, q_nope, q_pe, pos, w_uk, q_out,
                      pool_scale=None, stream=None):
    """Append the N new tokens and absorb the N queries of the same tokens in one
    launch (FP8 pool when ``pool_scale`` is given)."""
    N, H = q_nope.shape[0], dims.num_heads
    _check("c_kv", c_kv, torch.bfloat16, (N, D_C))
    _check("k_pe", k_pe, torch.bfloat16, (N, D_ROPE))
    _check("slot_mapping", slot_mapping, torch.int64, (N,))
    _check("q_nope", q_nope, torch.bfloat16, (N, H, D_NOPE))
    _check("q_pe", q_pe, torch.bfloat16, (N, H, D_ROPE))
    _check("pos", pos, torch.int32, (N,))
    _check("w_uk", w_uk, torch.bfloat16, (H, D_NOPE, D_C))
    _check("q_out", q_out, torch.bfloat16, (N, H, D_K))
    if pool_scale is None:
        _check("pool", pool, torch.bfloat16)
        if pool.dim() != 3 or tuple(pool.shape[1:]) != (BLOCK, D_K):
            raise ValueError("pool must be [num_blocks, 64, 576]")
        _ok("mla_append_absorb", lib().mla_append_absorb(
            ctypes.byref(dims), _ptr(c_kv), _ptr(k_pe), _ptr(slot_mapping), _ptr(pool), pool.shape[0],
            _ptr(q_nope), _ptr(q_pe), _ptr(pos), _ptr(w_uk), _ptr(q_out), N, _stream(stream)))
    else:
        _check_fp8_pool(pool, pool_scale)
        _ok("mla_append_absorb_fp8", lib().mla_append_absorb_fp8(
            ctypes.byref(dims), _ptr(c_kv), _ptr(k_pe), _ptr(slot_mapping), _ptr(pool), _ptr(pool_scale),
            pool.shape[0], _ptr(q_nope), _ptr(q_pe), _ptr(pos), _ptr(w_uk), _ptr(q_out), N, _stream(stream)))


def _check_fp8_pool(pool8, pool_scale):
    _check("pool8", pool8, torch.uint8)
    if pool8.dim() != 3 or tuple(pool8.shape[1:]) != (BLOCK, D_K):
        raise ValueError("pool8 must be [num_blocks, 64, 576] uint8")
    _check("pool_scale", pool_scale, torch.float32, (pool8.shape[0], BLOCK))


def mla_cache_append_fp8(dims: MlaDims, c_kv, k_pe, pos, slot_mapping, pool8, pool_scale, stream=None):
    """Write E4M3 codes of [c_kv | RoPE(k_pe, pos)] / scale into ``pool8`` and
    each token's scale into ``pool_scale`` at ``slot_mapping``."""
    T = c_kv.shape[0]
    _check("c_kv", c_kv, torch.bfloat16, (T, D_C))
    _check("k_pe", k_pe, torch.bfloat16, (T, D_ROPE))
    _check("pos", pos, torch.int32, (T,))
    _check("slot_mapping", slot_mapping, torch.int64, (T,))
    _check_fp8_pool(pool8, pool_scale)
    _ok("mla_cache_append_fp8", lib().mla_cache_append_fp8(
        ctypes.byref(dims), _ptr(c_kv), _ptr(k_pe), _ptr(pos), _ptr(slot_mapping), _ptr(pool8),
        _ptr(pool_scale), pool8.shape[0], T, _stream(stream)))


def mla_decode_attn_fp8(dims: MlaDims, q, pool8, pool_scale, block_table, seq_lens, Lq: int, o_lat,
                        lse=None, workspace=None, stream=None):
    """Latent attention of ``q`` [B*Lq, H, 576] over the FP8 paged cache."""
    H = dims.num_heads
    B = seq_lens.shape[0]
    _check("q", q, torch.bfloat16, (B * Lq, H, D_K))
    _check_fp8_pool(pool8, pool_scale)
    _check("block_table", block_table, torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _check("seq_lens", seq_lens, torch.int32, (B,))
    _check("o_lat", o_lat, torch.bfloat16, (B * Lq, H, D_C))
    if lse is not None:
        _check("lse", lse, torch.float32, (B * Lq, H))
    if workspace is None:
        raise ValueError("workspace is required (mla_decode_workspace_size bytes, uint8)")
    _check("workspace", workspace, torch.uint8)
    _ok("mla_decode_attn_fp8", lib().mla_decode_attn_fp8(
        ctypes.byref(dims), _ptr(q), _ptr(pool8), _ptr(pool_scale), pool8.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), B, Lq, _ptr(o_lat), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(stream)))


def _check_kvpe(kv_cache, pe_cache):
    _check("kv_cache", kv_cache, torch.bfloat16)
    if kv_cache.dim() != 3 or kv_cache.shape[2] != D_C:
        raise ValueError("kv_cache must be [B, max_seq, 512]")
    _check("pe_cache", pe_cache, torch.bfloat16, (kv_cache.shape[0], kv_cache.shape[1], D_ROPE))


def mla_cache_append_kvpe(dims: MlaDims, c_kv, k_pe, pos, seq_idx, kv_cache, pe_cache, stream=None):
    """Write c_kv into ``kv_cache[seq_idx, pos]`` and RoPE(k_pe, pos) into
    ``pe_cache[seq_idx, pos]`` (the two-buffer cache)."""
    T = c_kv.shape[0]
    _check("c_kv", c_kv, torch.bfloat16, (T, D_C))
    _check("k_pe", k_pe, torch.bfloat16, (T, D_ROPE))
    _check("pos", pos, torch.int32, (T,))
    _check("seq_idx", seq_idx, torch.int32, (T,))
    _check_kvpe(kv_cache, pe_cache)
    _ok("mla_cache_append_kvpe", lib().mla_cache_append_kvpe(
        ctypes.byref(dims), _ptr(c_kv), _ptr(k_pe), _ptr(pos), _ptr(seq_idx), _ptr(kv_cache), _ptr(pe_cache),
        kv_cache.shape[0], kv_cache.shape[1], T, _stream(stream)))


def mla_append_absorb_kvpe(dims: MlaDims, c_kv, k_pe, seq_idx, kv_cache, pe_cache, q_nope, q_pe, pos, w_uk,
                           q_out, stream=None):
    """Append the N new tokens into the two-buffer cache and absorb the N
    queries of the same tokens in one launch."""
    N, H = q_nope.shape[0], dims.num_heads
    _check("c_kv", c_kv, torch.bfloat16, (N, D_C))
    _check("k_pe", k_pe, torch.bfloat16, (N, D_ROPE))
    _check("seq_idx", seq_idx, torch.int32, (N,))
    _check("q_nope", q_nope, torch.bfloat16, (N, H, D_NOPE))
    _check("q_pe", q_pe, torch.bfloat16, (N, H, D_ROPE))
    _check("pos", pos, torch.int32, (N,))
    _check("w_uk", w_uk, torch.bfloat16, (H, D_NOPE, D_C))
    _check("q_out", q_out, torch.bfloat16, (N, H, D_K))
    _check_kvpe(kv_cache, pe_cache)
    _ok("mla_append_absorb_kvpe", lib().mla_append_absorb_kvpe(
        ctypes.byref(dims), _ptr(c_kv), _ptr(k_pe), _ptr(seq_idx), _ptr(kv_cache), _ptr(pe_cache),
        kv_cache.shape[0], kv_cache.shape[1], _ptr(q_nope), _ptr(q_pe), _ptr(pos), _ptr(w_uk), _ptr(q_out), N,
        _stream(stream)))


def mla_decode_attn_kvpe(dims: MlaDims, q, kv_cache, pe_cache, seq_lens, Lq: int, o_lat, lse=None,
                         workspace=None, stream=None):
    """Latent attention of ``q`` [B*Lq, H, 576] over the two-buffer cache
    (kv_cache [B, max_seq, 512], pe_cache [B, max_seq, 64])."""
    H = dims.num_heads
    B = seq_lens.shape[0]
    _check("q", q, torch.bfloat16, (B * Lq, H, D_K))
    _check_kvpe(kv_cache, pe_cache)
    if kv_cache.shape[0] != B:
        raise ValueError("kv_cache must hold B sequences")
    _check("seq_lens", seq_lens, torch.int32, (B,))
    _check("o_lat", o_lat, torch.bfloat16, (B * Lq, H, D_C))
    if lse is not None:
        _check("lse", lse, torch.float32, (B * Lq, H))
    if workspace is None:
        raise ValueError("workspace is required (mla_decode_workspace_size bytes, uint8)")
    _check("workspace", workspace, torch.uint8)
    _ok("mla_decode_attn_kvpe", lib().mla_decode_attn_kvpe(
        ctypes.byref(dims), _ptr(q), _ptr(kv_cache), _ptr(pe_cache), kv_cache.shape[1], _ptr(seq_lens), B, Lq,
        _ptr(o_lat), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))


def mla_out_up(dims: MlaDims, o_lat, w_uv, o, stream=None):
    """o[n,h] = W_UV[h] o_lat[n,h]."""
    N, H = o_lat.shape[0], dims.num_heads
    _check("o_lat", o_lat, torch.bfloat16, (N, H, D_C))
    _check("w_uv", w_uv, torch.bfloat16, (H, D_V, D_C))
    _check("o", o, torch.bfloat16, (N, H, D_V))
    _ok("mla_out_up", lib().mla_out_up(
        ctypes.byref(dims), _ptr(o_lat), _ptr(w_uv), _ptr(o), N, _stream(stream)))


def mla_linear_workspace_size(N: int, K: int, M: int) -> int:
    return int(lib().mla_linear_workspace_size(int(N), int(K), int(M)))


def mla_linear(x, w, y, residual=None, workspace=None, stream=None):
    """y[n] = W x[n] (+ residual[n]); x [N, K], w [M, K], y [N, M] bf16.
    ``workspace`` (uint8, optional): with mla_linear_workspace_size(N, K, M)
    bytes or more the contraction is split over more workgroups."""
    N, K = x.shape
    M = w.shape[0]
    _check("x", x, torch.bfloat16, (N, K))
    _check("w", w, torch.bfloat16, (M, K))
    _check("y", y, torch.bfloat16, (N, M))
    if residual is not None:
        _check("residual", residual, torch.bfloat16, (N, M))
    if workspace is not None:
        _check("workspace", workspace, torch.uint8)
    _ok("mla_linear", lib().mla_linear(_ptr(x), _ptr(w), _ptr(residual), _ptr(y), N, K, M, _ptr(workspace),
                                       workspace.numel() if workspace is not None else 0, _stream(stream)))
