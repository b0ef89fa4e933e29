"""One absorbed-MLA decode step over a paged latent cache, as four library calls.

append (new tokens' [c_kv | RoPE(k_pe)] rows) -> absorb_q -> decode_attn -> out_up,
all on the current stream, into buffers allocated once here.
"""

from __future__ import annotations

import torch

from . import native as nat


class DecodeStep:
    """Buffers and arguments of one decode step for B sequences of Lq new tokens.

    ``pool`` [num_blocks, 64, 576] bf16, ``block_table`` [B, max_blocks] int32 and
    ``seq_lens`` [B] int32 (keys including the new tokens) stay owned by the
    caller; the step writes the new tokens' cache rows before attending.
    """

    def __init__(self, H: int, B: int, Lq: int, pool, block_table, seq_lens, w_uk, w_uv,
                 device="cuda"):
        self.dims = nat.mla_dims_default(H)
        self.H, self.B, self.Lq, self.N = H, B, Lq, B * Lq
        self.pool, self.block_table, self.seq_lens = pool, block_table, seq_lens
        self.w_uk, self.w_uv = w_uk, w_uv
        N = self.N
        self.q = torch.empty(N, H, nat.D_K, dtype=torch.bfloat16, device=device)
        self.o_lat = torch.empty(N, H, nat.D_C, dtype=torch.bfloat16, device=device)
        self.lse = torch.empty(N, H, dtype=torch.float32, device=device)
        self.o = torch.empty(N, H, nat.D_V, dtype=torch.bfloat16, device=device)
        ws = nat.mla_decode_workspace_size(self.dims, B, Lq)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)

    def append(self, c_kv, k_pe, pos, slots):
        nat.mla_cache_append(self.dims, c_kv, k_pe, pos, slots, self.pool)

    def attend(self, q_nope, q_pe, q_pos):
        nat.mla_absorb_q(self.dims, q_nope, q_pe, q_pos, self.w_uk, self.q)
        nat.mla_decode_attn(self.dims, self.q, self.pool, self.block_table, self.seq_lens, self.Lq,
                            self.o_lat, self.lse, self.workspace)
        nat.mla_out_up(self.dims, self.o_lat, self.w_uv, self.o)

    def __call__(self, c_kv, k_pe, q_nope, q_pe, q_pos, slots):
        """Append the N new tokens (row n = b*Lq + i at position q_pos[n]), then attend."""
        self.append(c_kv, k_pe, q_pos, slots)
        self.attend(q_nope, q_pe, q_pos)
        return self.o

    def capture(self, c_kv, k_pe, q_nope, q_pe, q_pos, slots):
        """Record one whole step (five kernels, no allocation, no memset) as a
        HIP graph over these input tensors; returns the graph, whose replay()
        reruns the step on whatever the tensors then hold."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):       # one eager run initialises the stream state
            self(c_kv, k_pe, q_nope, q_pe, q_pos, slots)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self(c_kv, k_pe, q_nope, q_pe, q_pos, slots)
        return g
