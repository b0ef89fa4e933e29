"""Seeded synthetic inputs for absorbed-MLA decode, shared by tests and bench.

This module holds no arithmetic of the method. It only names the workloads,
draws seeded random values (rounded to bf16 bit patterns), draws sequence
lengths, builds block tables and lists cache slots. The oracle and the HIP
path both receive exactly these arrays; neither side produces inputs for the
other.

Values: c_kv, k_pe, q_nope, q_pe ~ N(0, 1); W_UK, W_UV ~ N(0, 1/512), each
drawn in float32 and rounded to bf16 (round to nearest even). Every tensor has
its own counter-keyed stream ``(seed, tag, index)`` so one sequence's cache
can be regenerated without drawing the others.
"""

from __future__ import annotations

import dataclasses

import numpy as np

TAG_CKV, TAG_KPE, TAG_QNOPE, TAG_QPE, TAG_WUK, TAG_WUV, TAG_LENS, TAG_TABLE = range(1, 9)
TAG_LAYER, TAG_HIDDEN = 9, 10

BLOCK = 64
D_C, D_ROPE, D_NOPE, D_V = 512, 64, 128, 128


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def normal_bf16(key, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of N(0, std^2) draws from the stream ``key``."""
    rng = np.random.default_rng(list(key))
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


@dataclasses.dataclass
class Workload:
    """One decode step: B sequences, Lq new query tokens each, lens[b] keys
    (keys include the Lq new tokens, which are appended before attending)."""

    name: str
    B: int
    H: int
    Lq: int
    lens: np.ndarray            # [B] int64, keys per sequence incl. the new tokens
    table_kind: str             # "contiguous" | "permuted"
    seed: int
    block_table: np.ndarray = None   # [B, max_blocks] int32, -1 past a sequence's end
    num_blocks: int = 0

    def __post_init__(self):
        self.lens = np.asarray(self.lens, dtype=np.int64)
        nblk = -(-self.lens // BLOCK)
        total = int(nblk.sum())
        self.num_blocks = max(total, 1)
        max_blocks = max(int(nblk.max()), 1)
        if self.table_kind == "contiguous":
            order = np.arange(total, dtype=np.int64)
        elif self.table_kind == "permuted":
            order = np.random.default_rng([self.seed, TAG_TABLE]).permutation(total)
        else:
            raise ValueError(self.table_kind)
        bt = np.full((self.B, max_blocks), -1, dtype=np.int32)
        off = 0
        for b in range(self.B):
            n = int(nblk[b])
            bt[b, :n] = order[off:off + n]
            off += n
        self.block_table = bt

    # ---- sizes
    @property
    def N(self) -> int:
        return self.B * self.Lq

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]

    def cache_bytes(self) -> int:
        """Latent-cache bytes one decode step reads: sum_b lens[b] * 576 * 2."""
        return int(self.lens.sum()) * (D_C + D_ROPE) * 2

    # ---- cache slots
    def slots(self, b: int, positions) -> np.ndarray:
        """Pool slot of each position of sequence b: block_table[b][p // 64] * 64 + p % 64."""
        p = np.asarray(positions, dtype=np.int64)
        return self.block_table[b, p // BLOCK].astype(np.int64) * BLOCK + p % BLOCK

    # ---- values
    def seq_cache(self, b: int, L: int | None = None):
        """(c_kv [L,512], k_pe [L,64]) bf16 bits of sequence b, positions 0..L-1."""
        L = int(self.lens[b]) if L is None else L
        return (normal_bf16((self.seed, TAG_CKV, b), (L, D_C)),
                normal_bf16((self.seed, TAG_KPE, b), (L, D_ROPE)))

    def queries(self, step: int = 0):
        """(q_nope [N,H,128], q_pe [N,H,64]) bf16 bits; row n = b * Lq + i."""
        return (normal_bf16((self.seed, TAG_QNOPE, step), (self.N, self.H, D_NOPE)),
                normal_bf16((self.seed, TAG_QPE, step), (self.N, self.H, D_ROPE)))

    def weights(self):
        """(W_UK, W_UV), each [H, 128, 512] bf16 bits, N(0, 1/512)."""
        std = 1.0 / np.sqrt(512.0)
        return (normal_bf16((self.seed, TAG_WUK), (self.H, D_NOPE, D_C), std),
                normal_bf16((self.seed, TAG_WUV), (self.H, D_V, D_C), std))

    def query_positions(self) -> np.ndarray:
        """[N] int32 absolute position of each query row: lens[b] - Lq + i."""
        i = np.arange(self.Lq)
        return (self.lens[:, None] - self.Lq + i[None, :]).reshape(-1).astype(np.int32)


def make(name: str, seed: int = 0, B: int | None = None, L: int | None = None,
         lens=None) -> Workload:
    """Build a named workload; ``B``/``L``/``lens`` shrink it for fast tests."""
    if name == "v2lite_tiny_b1_h16_l26":
        # 25-token prefill + 1-token decode at V2-Lite attention shape
        return Workload(name, 1, 16, 1, [26] if lens is None else lens, "contiguous", seed)
    if name == "v2lite_b64_h16_l4096":
        B = 64 if B is None else B
        L = 4096 if L is None else L
        return Workload(name, B, 16, 1, [L] * B if lens is None else lens, "contiguous", seed)
    if name == "v3_b32_h128_l16384":
        B = 32 if B is None else B
        L = 16384 if L is None else L
        return Workload(name, B, 128, 1, [L] * B if lens is None else lens, "permuted", seed)
    if name == "v3share8_b32_h128_l2048":
        # one GPU's share of the 128-head 16k batch when each sequence's keys
        # are split over 8 GPUs: 2,048 keys per sequence
        B = 32 if B is None else B
        L = 2048 if L is None else L
        return Workload(name, B, 128, 1, [L] * B if lens is None else lens, "permuted", seed)
    if name == "ragged_b128_h128_l1to32768":
        B = 128 if B is None else B
        hi = 32768 if L is None else L
        if lens is None:
            lens = np.random.default_rng([seed, TAG_LENS]).integers(1, hi, size=B, endpoint=True)
        return Workload(name, B, 128, 1, lens, "permuted", seed)
    if name == "causal8_b16_h128_l65544":
        B = 16 if B is None else B
        L = 65536 + 8 if L is None else L
        return Workload(name, B, 128, 8, [L] * B if lens is None else lens, "permuted", seed)
    if name == "chunk512_b4_h128_l16896":
        # chunked prefill: a 512-token chunk appended to 16,384 cached tokens
        B = 4 if B is None else B
        L = 16384 + 512 if L is None else L
        return Workload(name, B, 128, 512, [L] * B if lens is None else lens, "permuted", seed)
    raise KeyError(name)


FULL_WORKLOADS = (
    "v2lite_tiny_b1_h16_l26",
    "v2lite_b64_h16_l4096",
    "v3_b32_h128_l16384",
    "ragged_b128_h128_l1to32768",
    "causal8_b16_h128_l65544",
)

def layer_weights(seed: int, layer: int, H: int, d_model: int, d_cq: int) -> dict:
    """bf16 bits of one layer's projection weights in nn.Linear layout
    ([out, in]), each N(0, 1/in): Wdq [d_cq, d_model], Wuq [H*128, d_cq],
    Wqr [H*64, d_cq], Wdkv [512, d_model], Wkr [64, d_model],
    Wo [d_model, H*128]. (W_UK and W_UV come from the layer's Workload.)"""
    shapes = dict(w_dq=(d_cq, d_model), w_uq=(H * D_NOPE, d_cq), w_qr=(H * D_ROPE, d_cq),
                  w_dkv=(D_C, d_model), w_kr=(D_ROPE, d_model), w_o=(d_model, H * D_V))
    return {k: normal_bf16((seed, TAG_LAYER, layer, i), shp, 1.0 / np.sqrt(shp[1]))
            for i, (k, shp) in enumerate(shapes.items())}


def hidden_states(seed: int, N: int, d_model: int) -> np.ndarray:
    """bf16 bits of the new tokens' hidden states entering the first layer, N(0, 1)."""
    return normal_bf16((seed, TAG_HIDDEN), (N, d_model))


# chunked prefill over the latent: many query tokens per sequence
PREFILL_WORKLOADS = ("chunk512_b4_h128_l16896",)
