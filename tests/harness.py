"""Shared helpers of the GPU parity tests: run one decode step of a workload
through the C ABI, run the fp64 oracle on chosen sequences, compare.

Error metrics follow the vocabulary of [AUDIT] ("DeepSeek MLA 吸收式缓存：真实
权重执行与 FlashMLA 架构边界") §5: max / mean / p99 absolute error and the exact
fraction, plus the relative bars the parity tests use:
max|d| <= 2e-2 * max|ref| and mean|d| / mean|ref| <= 5e-3.
"""

from __future__ import annotations

import numpy as np
import torch

import workloads
from oracle import mla as orc

MAX_REL = 2e-2
MEAN_REL = 5e-3


# ----------------------------------------------------------------- conversions


def to_dev(bits) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def f64_of(t: torch.Tensor) -> np.ndarray:
    return orc.bf16_bits_to_f64(bits_of(t))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 of float64 values (via float32 is exact only when no
    double rounding occurs; used only for the reported exact fraction)."""
    return orc.bf16_bits_to_f64(workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


# ----------------------------------------------------------------- metrics


def metrics(gpu: np.ndarray, ref: np.ndarray) -> dict:
    gpu = np.asarray(gpu, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    d = np.abs(gpu - ref)
    return dict(
        max_abs=float(d.max()), mean_abs=float(d.mean()), p99_abs=float(np.percentile(d, 99)),
        exact=float(np.mean(gpu == bf16_round(ref))),
        max_rel=float(d.max() / max(np.abs(ref).max(), 1e-300)),
        mean_rel=float(d.mean() / max(np.abs(ref).mean(), 1e-300)),
        n=int(d.size))


def assert_parity(name: str, gpu, ref, max_rel=MAX_REL, mean_rel=MEAN_REL) -> dict:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(gpu), fin), f"{name}: finiteness differs"
    assert np.array_equal(gpu[~fin], ref[~fin]), f"{name}: non-finite values differ"
    m = metrics(gpu[fin], ref[fin]) if fin.any() else dict(max_rel=0.0, mean_rel=0.0)
    print(f"  {name}: " + ", ".join(f"{k}={v:.3g}" for k, v in m.items()), flush=True)
    assert m["max_rel"] <= max_rel, f"{name}: max rel {m['max_rel']:.3g} > {max_rel}"
    assert m["mean_rel"] <= mean_rel, f"{name}: mean rel {m['mean_rel']:.3g} > {mean_rel}"
    return m


# ----------------------------------------------------------------- GPU side


class DeviceRun:
    """Fill the paged pool with every sequence's history through
    mla_cache_append, then run one decode step (append the Lq new tokens,
    absorb, attend, up-project) through the C ABI."""

    def __init__(self, w: workloads.Workload, step: int = 0, append_chunk: int = 32768, fp8: bool = False):
        from mla_latent_cache_append_amd.step import DecodeStep
        self.w = w
        H, B, Lq = w.H, w.B, w.Lq
        dev = torch.device("cuda")
        self.fp8 = fp8
        if fp8:
            # never-written slots hold NaN codes and NaN scales
            self.pool = torch.full((w.num_blocks, 64, 576), 0x7F, dtype=torch.uint8, device=dev)
            self.pool_scale = torch.full((w.num_blocks, 64), float("nan"), dtype=torch.float32, device=dev)
        else:
            self.pool = torch.full((w.num_blocks, 64, 576), float("nan"), dtype=torch.bfloat16, device=dev)
            self.pool_scale = None
        self.block_table = torch.from_numpy(w.block_table).to(dev)
        self.seq_lens = torch.from_numpy(w.lens.astype(np.int32)).to(dev)
        wuk, wuv = w.weights()
        self.w_uk_bits, self.w_uv_bits = wuk, wuv
        self.step = DecodeStep(H, B, Lq, self.pool, self.block_table, self.seq_lens, to_dev(wuk), to_dev(wuv),
                               pool_scale=self.pool_scale)
        new_ckv = np.zeros((w.N, 512), np.uint16)
        new_kpe = np.zeros((w.N, 64), np.uint16)
        new_slot = np.full(w.N, -1, np.int64)
        qpos = w.query_positions()
        for b in range(B):
            L = int(w.lens[b])
            if B >= 16 and b % 16 == 0:
                print(f"  filling cache: sequence {b}/{B}", flush=True)
            if L <= 0:
                continue
            ckv, kpe = w.seq_cache(b)
            hist = max(L - Lq, 0)
            for s0 in range(0, hist, append_chunk):
                s1 = min(hist, s0 + append_chunk)
                p = np.arange(s0, s1)
                self.step.append(to_dev(ckv[s0:s1]), to_dev(kpe[s0:s1]),
                                 torch.from_numpy(p.astype(np.int32)).to(dev),
                                 torch.from_numpy(w.slots(b, p)).to(dev))
            for i in range(Lq):
                p = L - Lq + i
                if p >= 0:
                    n = b * Lq + i
                    new_ckv[n], new_kpe[n] = ckv[p], kpe[p]
                    new_slot[n] = w.slots(b, [p])[0]
        self.q_nope, self.q_pe = w.queries(step)
        self.new = (to_dev(new_ckv), to_dev(new_kpe), torch.from_numpy(qpos).to(dev),
                    torch.from_numpy(new_slot).to(dev))
        self.qpos = qpos

    def run(self):
        ckv, kpe, qpos, slot = self.new
        self.step(ckv, kpe, to_dev(self.q_nope), to_dev(self.q_pe), qpos, slot)
        torch.cuda.synchronize()
        s = self.step
        return dict(q=bits_of(s.q), o_lat=bits_of(s.o_lat), lse=s.lse.cpu().numpy().astype(np.float64),
                    o=bits_of(s.o))

    def pool_rows(self, b: int, L: int) -> np.ndarray:
        """bf16 bits of sequence b's cache rows 0..L-1, read through the block table."""
        slots = self.w.slots(b, np.arange(L))
        flat = self.pool.view(-1, 576)
        return bits_of(flat[torch.from_numpy(slots).cuda()])

    def pool_rows_fp8(self, b: int, L: int) -> tuple[np.ndarray, np.ndarray]:
        """E4M3 codes [L, 576] and scales [L] of sequence b's FP8 cache rows 0..L-1."""
        idx = torch.from_numpy(self.w.slots(b, np.arange(L))).cuda()
        return (self.pool.view(-1, 576)[idx].cpu().numpy(),
                self.pool_scale.view(-1)[idx].cpu().numpy())


# ----------------------------------------------------------------- oracle side


def oracle_seq(w: workloads.Workload, b: int, step: int = 0, q_nope=None, q_pe=None) -> dict:
    """fp64 oracle outputs of sequence b (absorbed path) from the seeded inputs."""
    Lq = w.Lq
    if q_nope is None:
        q_nope, q_pe = w.queries(step)
    f = orc.bf16_bits_to_f64
    L = int(w.lens[b])
    ckv, kpe = w.seq_cache(b) if L > 0 else (np.zeros((0, 512), np.uint16), np.zeros((0, 64), np.uint16))
    wuk, wuv = w.weights()
    sl = slice(b * Lq, (b + 1) * Lq)
    return orc.absorbed_decode(f(q_nope[sl]), f(q_pe[sl]), f(ckv), f(kpe), f(wuk), f(wuv))


def oracle_seq_fp8(w: workloads.Workload, b: int, step: int = 0) -> dict:
    """fp64 oracle outputs of sequence b over its FP8 cache: the oracle's own
    quantization of the seeded rows, then the absorbed decode on the values
    the codes stand for. Also returns the codes and scales."""
    Lq = w.Lq
    q_nope, q_pe = w.queries(step)
    f = orc.bf16_bits_to_f64
    L = int(w.lens[b])
    ckv, kpe = w.seq_cache(b)
    codes, scale = orc.cache_rows_fp8(f(ckv), f(kpe), np.arange(L))
    wuk, wuv = w.weights()
    sl = slice(b * Lq, (b + 1) * Lq)
    out = orc.absorbed_decode_fp8(f(q_nope[sl]), f(q_pe[sl]), codes, scale, f(wuk), f(wuv))
    out.update(codes=codes, scale=scale)
    return out


def oracle_queries(w: workloads.Workload, b: int, idx, step: int = 0) -> dict:
    """fp64 oracle outputs of query tokens idx (indices into the Lq new
    tokens) of sequence b only, at their absolute positions: the oracle's
    steps on a subset of rows, for sequences too long to take whole."""
    Lq = w.Lq
    q_nope, q_pe = w.queries(step)
    f = orc.bf16_bits_to_f64
    L = int(w.lens[b])
    ckv, kpe = w.seq_cache(b)
    wuk, wuv = w.weights()
    rows = b * Lq + np.asarray(idx)
    q_pos = L - Lq + np.asarray(idx, dtype=np.int64)
    c_kv = f(ckv)
    k_r = orc.rope(f(kpe), np.arange(L))
    q_lat, q_r = orc.absorb_q(f(q_nope[rows]), f(q_pe[rows]), q_pos, f(wuk))
    o_lat, lse = orc.latent_attention(q_lat, q_r, c_kv, k_r, q_pos, orc.default_scale())
    return dict(q_lat=q_lat, q_r=q_r, o_lat=o_lat, lse=lse, o=orc.out_up(o_lat, f(wuv)))


def check_queries(name: str, w, out: dict, b: int, idx) -> None:
    """Compare the GPU outputs of query tokens idx of sequence b with the oracle."""
    ref = oracle_queries(w, b, idx)
    rows = b * w.Lq + np.asarray(idx)
    q = orc.bf16_bits_to_f64(out["q"][rows])
    assert_parity(f"{name} b={b} q_lat", q[..., :512], ref["q_lat"])
    assert_parity(f"{name} b={b} q_r", q[..., 512:], ref["q_r"])
    assert_parity(f"{name} b={b} o_lat", orc.bf16_bits_to_f64(out["o_lat"][rows]), ref["o_lat"])
    assert_parity(f"{name} b={b} lse", out["lse"][rows], ref["lse"], max_rel=2e-2, mean_rel=5e-3)
    assert_parity(f"{name} b={b} o", orc.bf16_bits_to_f64(out["o"][rows]), ref["o"])


def check_seq(name: str, w, out: dict, b: int, ref: dict | None = None) -> None:
    """Compare the GPU outputs of sequence b with the oracle, stage by stage."""
    ref = oracle_seq(w, b) if ref is None else ref
    Lq, H = w.Lq, w.H
    sl = slice(b * Lq, (b + 1) * Lq)
    q = orc.bf16_bits_to_f64(out["q"][sl])
    L = int(w.lens[b])
    valid = np.arange(L - Lq, L) >= 0
    assert_parity(f"{name} b={b} q_lat", q[..., :512], ref["q_lat"])
    assert_parity(f"{name} b={b} q_r", q[..., 512:], ref["q_r"])
    assert_parity(f"{name} b={b} o_lat", orc.bf16_bits_to_f64(out["o_lat"][sl])[valid], ref["o_lat"][valid])
    assert_parity(f"{name} b={b} lse", out["lse"][sl][valid], ref["lse"][valid], max_rel=2e-2, mean_rel=5e-3)
    assert_parity(f"{name} b={b} o", orc.bf16_bits_to_f64(out["o"][sl])[valid], ref["o"][valid])
    # rows without any visible key: zero output, lse = -inf
    if (~valid).any():
        assert np.all(orc.bf16_bits_to_f64(out["o_lat"][sl])[~valid] == 0)
        assert np.all(out["lse"][sl][~valid] == -np.inf)
