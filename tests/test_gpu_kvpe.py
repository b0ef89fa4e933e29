"""GPU parity of the two-buffer latent cache (kv_cache [B][max_seq][512] +
pe_cache [B][max_seq][64], the layout of the V3 reference's absorbed decode:
[AUDIT] "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界" §0 and §4.2)
against the fp64 oracle, through the C ABI.

The cases: the V2-Lite tiny case in a 32-slot buffer (26 of 32 slots written,
36,864 bytes allocated, the figures of §4.2), the 16-head 4k batch at full
size (sampled sequences against the oracle, every sequence bit for bit
against the paged pool), 128 heads, several query tokens, a max_seq that is
not a multiple of the 64-token tile, a length beyond max_seq, and appends
outside the buffers.
"""

import json
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import mla as orc
from tests import harness as hz

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "cache_accounting.json")


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_latent_cache_append_amd import native
    native.lib()


class KvpeRun:
    """Fill kv_cache / pe_cache with every sequence's history through
    mla_cache_append_kvpe (never-written slots hold NaN), then one decode
    step: append the Lq new tokens, absorb, attend, up-project."""

    def __init__(self, w: workloads.Workload, max_seq: int, lens_dev=None, chunk: int = 32768):
        from mla_latent_cache_append_amd import native as nat
        self.nat, self.w, self.max_seq = nat, w, max_seq
        B, H, Lq = w.B, w.H, w.Lq
        self.dims = nat.mla_dims_default(H)
        self.kv = torch.full((B, max_seq, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.pe = torch.full((B, max_seq, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            L = min(int(w.lens[b]), max_seq)
            hist = max(L - Lq, 0)
            ckv, kpe = w.seq_cache(b, L)
            for s0 in range(0, hist, chunk):
                s1 = min(hist, s0 + chunk)
                self.append(ckv[s0:s1], kpe[s0:s1], np.arange(s0, s1), np.full(s1 - s0, b))
        self.seq_lens = torch.from_numpy(np.asarray(w.lens if lens_dev is None else lens_dev,
                                                    dtype=np.int32)).cuda()
        wuk, wuv = w.weights()
        self.w_uk, self.w_uv = hz.to_dev(wuk), hz.to_dev(wuv)
        N = w.N
        self.q = torch.empty(N, H, 576, dtype=torch.bfloat16, device="cuda")
        self.o_lat = torch.empty(N, H, 512, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(N, H, dtype=torch.float32, device="cuda")
        self.o = torch.empty(N, H, 128, dtype=torch.bfloat16, device="cuda")
        self.ws = torch.empty(nat.mla_decode_workspace_size(self.dims, B, Lq), dtype=torch.uint8, device="cuda")

    def append(self, ckv_bits, kpe_bits, pos, seq):
        self.nat.mla_cache_append_kvpe(self.dims, hz.to_dev(ckv_bits), hz.to_dev(kpe_bits),
                                       torch.from_numpy(np.asarray(pos, np.int32)).cuda(),
                                       torch.from_numpy(np.asarray(seq, np.int32)).cuda(), self.kv, self.pe)

    def step(self):
        """Append the new tokens (positions L - Lq .. L - 1), then attend."""
        w, nat = self.w, self.nat
        ckv_n = np.zeros((w.N, 512), np.uint16)
        kpe_n = np.zeros((w.N, 64), np.uint16)
        pos_n = w.query_positions()
        seq_n = np.repeat(np.arange(w.B), w.Lq)
        for b in range(w.B):
            L = int(w.lens[b])
            if L > self.max_seq:
                continue
            ckv, kpe = w.seq_cache(b)
            for i in range(w.Lq):
                p = L - w.Lq + i
                if p >= 0:
                    ckv_n[b * w.Lq + i], kpe_n[b * w.Lq + i] = ckv[p], kpe[p]
        self.append(ckv_n, kpe_n, pos_n, np.where(w.lens[seq_n] <= self.max_seq, seq_n, -1))
        q_nope, q_pe = w.queries(0)
        qpos = torch.from_numpy(pos_n).cuda()
        nat.mla_absorb_q(self.dims, hz.to_dev(q_nope), hz.to_dev(q_pe), qpos, self.w_uk, self.q)
        nat.mla_decode_attn_kvpe(self.dims, self.q, self.kv, self.pe, self.seq_lens, w.Lq, self.o_lat, self.lse,
                                 self.ws)
        nat.mla_out_up(self.dims, self.o_lat, self.w_uv, self.o)
        torch.cuda.synchronize()
        return dict(q=hz.bits_of(self.q), o_lat=hz.bits_of(self.o_lat),
                    lse=self.lse.cpu().numpy().astype(np.float64), o=hz.bits_of(self.o))


def test_v2lite_tiny_in_32_slot_buffer():
    """25-token prefill + 1 decode in a 32-slot buffer ([AUDIT] §0, §4.2):
    26 slots written (latent bit-exact, rope within 1 bf16 ulp), 6 untouched,
    36,864 bytes allocated for 29,952 active, outputs at the oracle's bar."""
    w = workloads.make("v2lite_tiny_b1_h16_l26", seed=0)
    _say("kvpe v2lite tiny: B=1 H=16 L=26 in 32 slots")
    run = KvpeRun(w, 32)
    out = run.step()
    hz.check_seq("kvpe tiny", w, out, 0)
    ckv, kpe = w.seq_cache(0)
    kv, pe = hz.bits_of(run.kv), hz.bits_of(run.pe)
    assert np.array_equal(kv[0, :26], ckv)
    ref_r = orc.cache_rows(orc.bf16_bits_to_f64(ckv), orc.bf16_bits_to_f64(kpe), np.arange(26))[:, 512:]
    assert np.all(np.abs(orc.bf16_bits_to_f64(pe[0, :26]) - ref_r) <= hz.bf16_ulp(ref_r))
    assert np.all(np.isnan(orc.bf16_bits_to_f64(kv[0, 26:]))) and np.all(np.isnan(orc.bf16_bits_to_f64(pe[0, 26:])))
    gold = json.load(open(GOLDEN))
    want_alloc = next(g["value"] for g in gold["allocated_bytes_bf16_32_slots"] if g["kind"] == "latent")
    want_active = next(g["value"] for g in gold["active_bytes_bf16"] if g.get("kind") == "latent")
    allocated = run.kv.numel() * run.kv.element_size() + run.pe.numel() * run.pe.element_size()
    written = (~torch.isnan(run.kv.float()).all(dim=2)).sum().item()
    active = written * (run.kv.shape[2] + run.pe.shape[2]) * run.kv.element_size()
    assert (allocated, active) == (want_alloc, want_active)
    print(f"  allocated {allocated} B, active {active} B (the page's 36,864 and 29,952)", flush=True)


def test_v2lite_4k_full_size_matches_oracle_and_paged_pool():
    """The 16-head 4k batch (B=64, L=4096) at full size: sampled sequences
    against the oracle; every output bit for bit equal to the paged pool's
    (the same kernel over the same rows, read from other addresses)."""
    w = workloads.make("v2lite_b64_h16_l4096", seed=0)
    _say("kvpe v2lite_b64_h16_l4096 full size")
    out = KvpeRun(w, 4096).step()
    for b in (0, 37, 63):
        hz.check_seq("kvpe v2lite 4k", w, out, b)
    paged = hz.DeviceRun(w).run()
    for k in ("q", "o_lat", "o"):
        assert np.array_equal(out[k], paged[k]), k
    assert np.array_equal(out["lse"], paged["lse"])
    print("  bitwise equal to the paged pool", flush=True)


@pytest.mark.parametrize("H,Lq,lens,max_seq", [
    (128, 1, [1000, 3001], 3072),          # 128 heads: the 128-row kernel, rope rows through their own descriptor
    (128, 2, [37, 100, 1, 64], 100),       # two 128-row groups, max_seq not a multiple of 64
    (48, 2, [700, 1, 129], 700),           # 96 rows: the 128-row kernel with its last wave all padding
    (32, 2, [300, 65], 320),               # 64 rows: the 64-row kernel
    (16, 3, [5, 64, 130, 200], 256),       # several new tokens, causal among themselves
    (32, 1, [1, 64, 65, 100], 100),        # max_seq not a multiple of 64, tails of 1..36
    (64, 2, [700, 1, 129], 700),
])
def test_small_cases(H, Lq, lens, max_seq):
    w = workloads.Workload(f"kvpe_h{H}_lq{Lq}", len(lens), H, Lq, lens, "contiguous", seed=11)
    _say(f"kvpe H={H} Lq={Lq} lens={lens} max_seq={max_seq}")
    out = KvpeRun(w, max_seq).step()
    for b in range(w.B):
        hz.check_seq(f"kvpe H={H}", w, out, b)


def test_length_beyond_max_seq_gives_nan_and_spares_the_others():
    """A length above max_seq makes that sequence's outputs NaN (its rows are
    never read past the buffer); the other sequences are unaffected."""
    w = workloads.Workload("kvpe_bad", 3, 16, 1, [90, 128, 40], "contiguous", seed=5)
    _say("kvpe lens [90, 128 (> max_seq 100), 40]")
    run = KvpeRun(w, 100)
    out = run.step()
    for b in (0, 2):
        hz.check_seq("kvpe bad-neighbour", w, out, b)
    assert np.all(np.isnan(orc.bf16_bits_to_f64(out["o_lat"][1])))
    assert np.all(np.isnan(out["lse"][1]))


def test_length_beyond_max_seq_128_heads():
    """The same through the 128-row kernel, with the long sequence last: its
    length lies between max_seq and the next multiple of 64, so only the
    clamp of the copies to max_seq keeps them inside the buffers."""
    w = workloads.Workload("kvpe_bad128", 3, 128, 1, [90, 40, 128], "contiguous", seed=6)
    _say("kvpe H=128 lens [90, 40, 128 (> max_seq 100)]")
    out = KvpeRun(w, 100).step()
    for b in (0, 1):
        hz.check_seq("kvpe bad-last 128", w, out, b)
    assert np.all(np.isnan(orc.bf16_bits_to_f64(out["o_lat"][2])))
    assert np.all(np.isnan(out["lse"][2]))


def test_v3_16k_full_size_matches_paged_pool():
    """The 128-head 16k batch (B=32, L=16384) at full size: two sequences
    against the oracle, every output bit for bit equal to the paged pool's
    (the 128-row kernel over the same rows, read through two descriptors)."""
    w = workloads.make("v3_b32_h128_l16384", seed=0)
    _say("kvpe v3_b32_h128_l16384 full size")
    out = KvpeRun(w, 16384).step()
    for b in (0, 31):
        hz.check_seq("kvpe v3 16k", w, out, b)
    paged = hz.DeviceRun(w).run()
    for k in ("q", "o_lat", "o"):
        assert np.array_equal(out[k], paged[k]), k
    assert np.array_equal(out["lse"], paged["lse"])
    print("  bitwise equal to the paged pool", flush=True)


def test_append_skips_outside_the_buffers():
    from mla_latent_cache_append_amd import native as nat
    _say("kvpe append with sequence -1, 2 (B=2), position -1 and max_seq")
    dims = nat.mla_dims_default(16)
    kv = torch.zeros(2, 8, 512, dtype=torch.bfloat16, device="cuda")
    pe = torch.zeros(2, 8, 64, dtype=torch.bfloat16, device="cuda")
    T = 5
    ckv = torch.ones(T, 512, dtype=torch.bfloat16, device="cuda")
    kpe = torch.ones(T, 64, dtype=torch.bfloat16, device="cuda")
    pos = torch.tensor([0, 1, -1, 8, 3], dtype=torch.int32, device="cuda")
    seq = torch.tensor([-1, 2, 0, 1, 1], dtype=torch.int32, device="cuda")
    nat.mla_cache_append_kvpe(dims, ckv, kpe, pos, seq, kv, pe)
    torch.cuda.synchronize()
    written = (kv != 0).any(dim=2)
    assert written.sum().item() == 1 and bool(written[1, 3])
    assert bool((pe != 0).any(dim=2)[1, 3]) and (pe != 0).any(dim=2).sum().item() == 1


@pytest.mark.parametrize("H,lens,max_seq", [(128, [700, 33, 1500, 64], 1600), (16, [300, 1, 129, 64, 65], 320)],
                         ids=lambda v: str(v))
def test_fused_append_absorb_equals_separate_calls(H, lens, max_seq):
    """mla_append_absorb_kvpe (append into both arrays and absorb in one
    launch) against mla_cache_append_kvpe + mla_absorb_q from the same
    starting cache: both arrays and the absorbed queries bit-identical, with
    one token outside the sequences and one at a position past max_seq
    (skipped by both)."""
    from mla_latent_cache_append_amd import native as nat
    w = workloads.Workload("kvpe_fused", len(lens), H, 1, lens, "contiguous", seed=23)
    _say(f"two-buffer fused append+absorb: H={H} lens={lens} max_seq={max_seq}")
    run = KvpeRun(w, max_seq)
    ckv_n = np.zeros((w.N, 512), np.uint16)
    kpe_n = np.zeros((w.N, 64), np.uint16)
    for b in range(w.B):
        ckv, kpe = w.seq_cache(b)
        ckv_n[b], kpe_n[b] = ckv[-1], kpe[-1]
    pos_n = w.query_positions().copy()
    seq_n = np.arange(w.B, dtype=np.int32)
    seq_n[1] = -1               # outside the sequences: skipped
    pos_n[2] = max_seq          # past the buffers: skipped
    ckv_d, kpe_d = hz.to_dev(ckv_n), hz.to_dev(kpe_n)
    pos_d, seq_d = torch.from_numpy(pos_n.astype(np.int32)).cuda(), torch.from_numpy(seq_n).cuda()
    q_nope, q_pe = w.queries(0)
    qn, qp = hz.to_dev(q_nope), hz.to_dev(q_pe)
    kv0, pe0 = run.kv.clone(), run.pe.clone()
    nat.mla_cache_append_kvpe(run.dims, ckv_d, kpe_d, pos_d, seq_d, run.kv, run.pe)
    nat.mla_absorb_q(run.dims, qn, qp, pos_d, run.w_uk, run.q)
    torch.cuda.synchronize()
    sep_kv, sep_pe, sep_q = run.kv.clone(), run.pe.clone(), run.q.clone()
    run.kv.copy_(kv0)
    run.pe.copy_(pe0)
    run.q.fill_(float("nan"))
    nat.mla_append_absorb_kvpe(run.dims, ckv_d, kpe_d, seq_d, run.kv, run.pe, qn, qp, pos_d, run.w_uk, run.q)
    torch.cuda.synchronize()
    assert torch.equal(run.q.view(torch.int16), sep_q.view(torch.int16))
    assert torch.equal(run.kv.view(torch.int16), sep_kv.view(torch.int16))
    assert torch.equal(run.pe.view(torch.int16), sep_pe.view(torch.int16))
    # written rows: the valid new tokens' only
    changed = ((run.kv.view(torch.int16) != kv0.view(torch.int16)).any(dim=2)
               | (run.pe.view(torch.int16) != pe0.view(torch.int16)).any(dim=2)).nonzero().cpu().numpy()
    expect = {(b, int(pos_n[b])) for b in range(w.B) if b not in (1, 2)}
    assert {(int(b), int(p)) for b, p in changed} <= expect
    print("  both arrays and the queries bit-identical to the separate calls", flush=True)
