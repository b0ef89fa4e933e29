"""One absorbed-MLA decode step over a paged latent cache, as four library calls.

append (new tokens' [c_kv | RoPE(k_pe)] rows) -> absorb_q -> decode_attn -> out_up,
all on the current stream, into buffers allocated once here. ``LayerStep``
wraps a step in the layer's projections (bias-free linear maps, [MLA80] §2 of
the CSDN page "80 行 PyTorch 从零写 DeepSeek 的 MLA") and a residual output
projection, for stacks of layers.
"""

from __future__ import annotations

import torch

from . import native as nat

# Query tokens per sequence from which the expanded form (mla_prefill_expanded)
# is faster than the absorbed calls: measured crossover ~295-340 at 16,384
# cached tokens and 128 heads on MI355X. Both forms' costs grow with the keys
# and the heads alike (expansion 2 L H 256 512 flops, attention 2 H Lq L 320,
# against 2 H Lq L 1088 absorbed), so the crossover depends mostly on Lq.
EXPANDED_FROM_LQ = 320


def prefill_form(Lq: int, cache: str = "bf16") -> str:
    """"expanded" for chunks of at least EXPANDED_FROM_LQ query tokens per
    sequence over the paged bf16 pool, else "absorbed" (decode steps, short
    chunks, and the FP8 and two-buffer caches, which only the absorbed calls
    read)."""
    return "expanded" if cache == "bf16" and Lq >= EXPANDED_FROM_LQ else "absorbed"


class DecodeStep:
    """Buffers and arguments of one decode step for B sequences of Lq new tokens.

    ``pool`` [num_blocks, 64, 576] bf16, ``block_table`` [B, max_blocks] int32 and
    ``seq_lens`` [B] int32 (keys including the new tokens) stay owned by the
    caller; the step writes the new tokens' cache rows before attending.
    With ``pool_scale`` ([num_blocks, 64] fp32) the pool is the FP8 cache
    ([num_blocks, 64, 576] uint8 E4M3 codes) and the step uses the FP8 calls.
    With ``pe_cache`` ([B, max_seq, 64] bf16) the cache is the two-buffer
    layout: ``pool`` is kv_cache [B, max_seq, 512], there is no block table,
    and the ``slots`` argument of ``append`` / ``__call__`` is each new
    token's sequence index (int32) instead of its pool slot.

    ``form`` selects how the step attends: "absorbed" (absorb_q,
    decode_attn, out_up), "expanded" (mla_prefill_expanded: per-head K and V
    expanded from the cache, then multi-head attention; paged bf16 pool
    only, sequences of at most ``max_len`` keys, a workspace allocated here)
    or "auto" (``prefill_form(Lq)``). Both fill ``o`` and ``lse``; the
    expanded form leaves ``q`` and ``o_lat`` unwritten.
    """

    def __init__(self, H: int, B: int, Lq: int, pool, block_table, seq_lens, w_uk, w_uv,
                 device="cuda", pool_scale=None, pe_cache=None, form: str = "absorbed", max_len: int = 0):
        self.dims = nat.mla_dims_default(H)
        self.H, self.B, self.Lq, self.N = H, B, Lq, B * Lq
        self.pool, self.block_table, self.seq_lens = pool, block_table, seq_lens
        self.pool_scale = pool_scale
        self.pe_cache = pe_cache
        self.w_uk, self.w_uv = w_uk, w_uv
        N = self.N
        self.q = torch.empty(N, H, nat.D_K, dtype=torch.bfloat16, device=device)
        self.o_lat = torch.empty(N, H, nat.D_C, dtype=torch.bfloat16, device=device)
        self.lse = torch.empty(N, H, dtype=torch.float32, device=device)
        self.o = torch.empty(N, H, nat.D_V, dtype=torch.bfloat16, device=device)
        ws = nat.mla_decode_workspace_size(self.dims, B, Lq)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        cache = "fp8" if pool_scale is not None else "kvpe" if pe_cache is not None else "bf16"
        self.form = prefill_form(Lq, cache) if form == "auto" else form
        if self.form not in ("absorbed", "expanded"):
            raise ValueError(f"form must be 'absorbed', 'expanded' or 'auto', not {form!r}")
        self.max_len = int(max_len)
        self.expanded_ws = None
        if self.form == "expanded":
            if cache != "bf16":
                raise ValueError("the expanded form reads the paged bf16 pool only")
            if self.max_len <= 0:
                raise ValueError("the expanded form needs max_len (the longest sequence, in keys)")
            xs = nat.mla_prefill_expanded_workspace_size(self.dims, B, self.max_len)
            if xs == 0:
                raise ValueError("shape not supported by the expanded form")
            self.expanded_ws = torch.empty(xs, dtype=torch.uint8, device=device)

    def append(self, c_kv, k_pe, pos, slots):
        if self.pe_cache is not None:
            nat.mla_cache_append_kvpe(self.dims, c_kv, k_pe, pos, slots, self.pool, self.pe_cache)
        elif self.pool_scale is None:
            nat.mla_cache_append(self.dims, c_kv, k_pe, pos, slots, self.pool)
        else:
            nat.mla_cache_append_fp8(self.dims, c_kv, k_pe, pos, slots, self.pool, self.pool_scale)

    def decode_attn(self):
        """The attention call alone, over the absorbed queries in ``self.q``."""
        if self.pe_cache is not None:
            nat.mla_decode_attn_kvpe(self.dims, self.q, self.pool, self.pe_cache, self.seq_lens, self.Lq,
                                     self.o_lat, self.lse, self.workspace)
        elif self.pool_scale is None:
            nat.mla_decode_attn(self.dims, self.q, self.pool, self.block_table, self.seq_lens, self.Lq,
                                self.o_lat, self.lse, self.workspace)
        else:
            nat.mla_decode_attn_fp8(self.dims, self.q, self.pool, self.pool_scale, self.block_table,
                                    self.seq_lens, self.Lq, self.o_lat, self.lse, self.workspace)

    def attend_expanded(self, q_nope, q_pe, q_pos):
        """The expanded form over the cache as it stands: o and lse."""
        nat.mla_prefill_expanded(self.dims, q_nope, q_pe, q_pos, self.pool, self.block_table, self.seq_lens,
                                 self.Lq, self.max_len, self.w_uk, self.w_uv, self.o, self.lse, self.expanded_ws)

    def attend(self, q_nope, q_pe, q_pos):
        if self.form == "expanded":
            self.attend_expanded(q_nope, q_pe, q_pos)
            return
        nat.mla_absorb_q(self.dims, q_nope, q_pe, q_pos, self.w_uk, self.q)
        self.decode_attn()
        nat.mla_out_up(self.dims, self.o_lat, self.w_uv, self.o)

    def __call__(self, c_kv, k_pe, q_nope, q_pe, q_pos, slots):
        """Append the N new tokens (row n = b*Lq + i at position q_pos[n]), then
        attend: append and absorb share one launch, then attention and out_up."""
        if self.form == "expanded":
            self.append(c_kv, k_pe, q_pos, slots)
            self.attend(q_nope, q_pe, q_pos)
            return self.o
        if self.pe_cache is not None:
            nat.mla_append_absorb_kvpe(self.dims, c_kv, k_pe, slots, self.pool, self.pe_cache, q_nope, q_pe, q_pos,
                                       self.w_uk, self.q)
        else:
            nat.mla_append_absorb(self.dims, c_kv, k_pe, slots, self.pool, q_nope, q_pe, q_pos, self.w_uk, self.q,
                                  pool_scale=self.pool_scale)
        self.decode_attn()
        nat.mla_out_up(self.dims, self.o_lat, self.w_uv, self.o)
        return self.o

    def capture(self, c_kv, k_pe, q_nope, q_pe, q_pos, slots, reps: int = 1):
        """Record ``reps`` whole steps in a row (four kernels each, no
        allocation, no memset) as one HIP graph over these input tensors;
        returns the graph, whose replay() reruns them on whatever the tensors
        then hold. Several steps per graph amortise the graph launch, as a
        decode loop captured ahead of time does."""
        return _capture(self, c_kv, k_pe, q_nope, q_pe, q_pos, slots, reps=reps)


def _capture(fn, *args, reps: int = 1):
    """HIP graph of ``reps`` calls fn(*args) in a row, after one eager call on
    a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # one eager run initialises the stream state
        fn(*args)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn(*args)
    return g


class LayerStep:
    """One attention layer for the new tokens of B sequences, around a
    ``DecodeStep`` (which owns the layer's cache, W_UK and W_UV):

        c_kv = Wdkv h, k_pe = Wkr h, qz = Wdq h, q_nope = Wuq qz, q_pe = Wqr qz
        o = decode(c_kv, k_pe, q_nope, q_pe)
        h_out = h + Wo [o_0 | ... | o_{H-1}]

    Weights are [out, in] bf16 device tensors; every product runs in
    ``mla_linear`` (the residual add is fused into the last one); each map
    has its own slice of one workspace, so maps with few output tiles split
    their contraction over more workgroups. Wdkv and Wkr run one after the
    other on a side stream beside Wdq, Wqr and Wuq (the decode waits for
    both streams); measured against three side streams (Wdkv, Wkr, Wqr each
    on its own) and against one stream, this is ~5 us per layer faster at
    128 heads."""

    def __init__(self, decode: DecodeStep, w_dq, w_uq, w_qr, w_dkv, w_kr, w_o, device="cuda"):
        self.decode = decode
        self.w_dq, self.w_uq, self.w_qr, self.w_dkv, self.w_kr, self.w_o = w_dq, w_uq, w_qr, w_dkv, w_kr, w_o
        N, H = decode.N, decode.H
        d_model, d_cq = w_dq.shape[1], w_dq.shape[0]
        if tuple(w_uq.shape) != (H * nat.D_NOPE, d_cq) or tuple(w_qr.shape) != (H * nat.D_ROPE, d_cq):
            raise ValueError("query up-projections do not match the heads or the query latent width")
        if tuple(w_dkv.shape) != (nat.D_C, d_model) or tuple(w_kr.shape) != (nat.D_ROPE, d_model):
            raise ValueError("KV down-projections do not match the latent widths or d_model")
        if tuple(w_o.shape) != (d_model, H * nat.D_V):
            raise ValueError("output projection does not match the heads or d_model")
        bf = dict(dtype=torch.bfloat16, device=device)
        self.qz = torch.empty(N, d_cq, **bf)
        self.q_nope = torch.empty(N, H, nat.D_NOPE, **bf)
        self.q_pe = torch.empty(N, H, nat.D_ROPE, **bf)
        self.c_kv = torch.empty(N, nat.D_C, **bf)
        self.k_pe = torch.empty(N, nat.D_ROPE, **bf)
        self.out = torch.empty(N, d_model, **bf)
        # one workspace, a 256-byte-aligned slice per map: maps on different
        # streams run at the same time and must not share partial sums
        shapes = {"dkv": (d_model, nat.D_C), "kr": (d_model, nat.D_ROPE), "dq": (d_model, d_cq),
                  "uq": (d_cq, H * nat.D_NOPE), "qr": (d_cq, H * nat.D_ROPE), "o": (H * nat.D_V, d_model)}
        sizes = {k: nat.mla_linear_workspace_size(N, K, M) for k, (K, M) in shapes.items()}
        offs, total = {}, 0
        for k, sz in sizes.items():
            offs[k] = total
            total += (sz + 255) // 256 * 256
        self.workspace = torch.empty(max(total, 1), dtype=torch.uint8, device=device)
        self.ws = {k: (self.workspace[offs[k]:offs[k] + sz] if sz else None) for k, sz in sizes.items()}
        # side stream at the default priority
        self.side_kv = torch.cuda.Stream(device=device)

    def __call__(self, h, q_pos, slots):
        N = self.decode.N
        main = torch.cuda.current_stream()
        self.side_kv.wait_stream(main)
        with torch.cuda.stream(self.side_kv):
            nat.mla_linear(h, self.w_dkv, self.c_kv, workspace=self.ws["dkv"])
            nat.mla_linear(h, self.w_kr, self.k_pe, workspace=self.ws["kr"])
        nat.mla_linear(h, self.w_dq, self.qz, workspace=self.ws["dq"])
        nat.mla_linear(self.qz, self.w_qr, self.q_pe.view(N, -1), workspace=self.ws["qr"])
        nat.mla_linear(self.qz, self.w_uq, self.q_nope.view(N, -1), workspace=self.ws["uq"])
        main.wait_stream(self.side_kv)
        self.decode(self.c_kv, self.k_pe, self.q_nope, self.q_pe, q_pos, slots)
        nat.mla_linear(self.decode.o.view(N, -1), self.w_o, self.out, residual=h, workspace=self.ws["o"])
        return self.out

    def capture(self, h, q_pos, slots, reps: int = 1):
        """Record ``reps`` whole layers in a row as one HIP graph over these
        input tensors; replay() reruns them on whatever they then hold (the
        layer rewrites the same cache rows and outputs, so a repeat gives
        the same result)."""
        return _capture(self, h, q_pos, slots, reps=reps)
