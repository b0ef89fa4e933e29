"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases span several 64-token tiles and ragged tails; full-size workloads
compare sampled sequences. Every test prints the case it runs before it runs.
"""

import hashlib

import numpy as np
import pytest
import torch

import workloads
from oracle import mla as orc
from tests import harness as hz

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_latent_cache_append_amd import native
    native.lib()


# ------------------------------------------------------------------ cache append


def test_append_latent_bit_exact_rope_within_ulp():
    w = workloads.make("ragged_b128_h128_l1to32768", seed=1, B=4, lens=[1, 70, 200, 1031])
    _say(f"append {w.name} lens={list(w.lens)}")
    run = hz.DeviceRun(w)
    run.run()
    for b in range(w.B):
        L = int(w.lens[b])
        rows = run.pool_rows(b, L)
        ckv, kpe = w.seq_cache(b)
        assert np.array_equal(rows[:, :512], ckv), f"latent bits differ in seq {b}"
        ref = orc.cache_rows(orc.bf16_bits_to_f64(ckv), orc.bf16_bits_to_f64(kpe), np.arange(L))[:, 512:]
        got = orc.bf16_bits_to_f64(rows[:, 512:])
        err = np.abs(got - ref)
        assert np.all(err <= hz.bf16_ulp(ref)), f"rope part beyond 1 bf16 ulp in seq {b}"
        print(f"  seq {b}: rope exactly rounded fraction {np.mean(err <= 0.5 * hz.bf16_ulp(ref) * (1 + 1e-9)):.6f}")


def test_append_skips_out_of_range_slots():
    from mla_latent_cache_append_amd import native as nat
    _say("append with slots -1 and num_blocks*64")
    dims = nat.mla_dims_default(16)
    pool = torch.zeros(2, 64, 576, dtype=torch.bfloat16, device="cuda")
    ckv = torch.ones(3, 512, dtype=torch.bfloat16, device="cuda")
    kpe = torch.ones(3, 64, dtype=torch.bfloat16, device="cuda")
    pos = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    slot = torch.tensor([-1, 128, 5], dtype=torch.int64, device="cuda")
    nat.mla_cache_append(dims, ckv, kpe, pos, slot, pool)
    torch.cuda.synchronize()
    flat = pool.view(-1, 576).float().cpu()
    assert torch.all(flat[5, :512] == 1)
    flat[5] = 0
    assert torch.all(flat == 0)


# ------------------------------------------------------------------ per-stage parity, small


@pytest.mark.parametrize("H,Lq,lens", [
    (16, 1, [1, 63, 64, 65, 129, 1000]),
    (32, 1, [5, 64, 300]),
    (64, 1, [2, 130, 517]),
    (128, 1, [1, 64, 65, 700]),
    (128, 8, [8, 9, 71, 200]),
    (16, 3, [3, 4, 64, 66, 190]),
    (32, 3, [3, 33, 96, 300]),       # 96 rows: the 128-row kernel's threshold, its fourth wave all padding
    # prefill chunks: many query tokens per sequence, causal among themselves
    (128, 64, [64, 100, 1000]),
    (16, 203, [203, 777]),
], ids=lambda v: str(v))
def test_decode_step_small(H, Lq, lens):
    name = {16: "v2lite_b64_h16_l4096", 32: "v2lite_b64_h16_l4096"}.get(H, "v3_b32_h128_l16384")
    w = workloads.Workload(f"small_h{H}_lq{Lq}", len(lens), H, Lq, lens,
                           "permuted" if H >= 64 else "contiguous", seed=H + Lq)
    _say(f"decode step H={H} Lq={Lq} lens={lens}")
    out = hz.DeviceRun(w).run()
    for b in range(w.B):
        hz.check_seq(w.name, w, out, b)


def test_many_short_sequences_multi_segment():
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 300, size=300)
    w = workloads.Workload("many_h16", 300, 16, 1, lens, "permuted", seed=5)
    _say(f"decode step B=300 H=16 lens 1..300 (ranges span many sequences)")
    out = hz.DeviceRun(w).run()
    for b in [0, 1, 2, 150, 298, 299, int(np.argmax(lens)), int(np.argmin(lens))]:
        hz.check_seq(w.name, w, out, b)


@pytest.mark.parametrize("H,Lq,lens", [
    (16, 4, [0, 3, 5, 64]),       # 64 rows: the 64-row kernel, merged by the merge launch
    (16, 1, [0, 3, 5, 64]),       # 16 rows: the column kernel, which merges its own partials
    (16, 2, [0, 70, 0, 3000]),    # 32 rows, empty sequences between split ones
    (16, 1, [0, 0, 0]),           # no keys at all
], ids=lambda v: str(v))
def test_zero_and_short_lengths(H, Lq, lens):
    w = workloads.Workload("short", len(lens), H, Lq, lens, "contiguous", seed=9)
    _say(f"lens {lens} with Lq={Lq}, H={H}: empty sequences (and positions below 0)")
    out = hz.DeviceRun(w).run()
    rows = Lq * H
    for b, L in enumerate(lens):
        if L == 0:
            o_lat = orc.bf16_bits_to_f64(out["o_lat"][b * Lq:(b + 1) * Lq])
            assert np.all(o_lat == 0) and np.all(out["lse"][b * Lq:(b + 1) * Lq] == -np.inf), b
        else:
            hz.check_seq(w.name, w, out, b)
    assert out["o_lat"].shape[0] * out["o_lat"].shape[1] == len(lens) * rows


# ------------------------------------------------------------------ tiny V2-Lite layer


def test_tiny_prefill_then_decode_matches_one_shot():
    """25-token prefill + 1-token decode at V2-Lite shape equals the 26-token
    one-shot forward ([MLA80] §2 cache-equivalence test); the cache holds
    26 x 1,152 = 29,952 active bytes ([AUDIT] §4.1)."""
    from mla_latent_cache_append_amd import native as nat
    from mla_latent_cache_append_amd.step import DecodeStep
    H, L = 16, 26
    w = workloads.make("v2lite_tiny_b1_h16_l26", seed=0)
    ckv, kpe = w.seq_cache(0)
    qn = workloads.normal_bf16((0, workloads.TAG_QNOPE, 99), (L, H, 128))
    qp = workloads.normal_bf16((0, workloads.TAG_QPE, 99), (L, H, 64))
    wuk, wuv = w.weights()
    f = orc.bf16_bits_to_f64
    one_shot = orc.absorbed_decode(f(qn), f(qp), f(ckv), f(kpe), f(wuk), f(wuv))
    _say("tiny V2-Lite: prefill 25 (Lq=25) then decode 1")
    pool = torch.full((1, 64, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    outs = []
    for lo, hi in ((0, 25), (25, 26)):
        lens = torch.tensor([hi], dtype=torch.int32, device="cuda")
        st = DecodeStep(H, 1, hi - lo, pool, bt, lens, hz.to_dev(wuk), hz.to_dev(wuv))
        pos = torch.arange(lo, hi, dtype=torch.int32, device="cuda")
        st(hz.to_dev(ckv[lo:hi]), hz.to_dev(kpe[lo:hi]), hz.to_dev(qn[lo:hi]), hz.to_dev(qp[lo:hi]),
           pos, pos.to(torch.int64))
        torch.cuda.synchronize()
        outs.append((hz.f64_of(st.o), st.lse.cpu().numpy().astype(np.float64), hz.f64_of(st.o_lat)))
    hz.assert_parity("prefill o", outs[0][0], one_shot["o"][:25])
    hz.assert_parity("prefill o_lat", outs[0][2], one_shot["o_lat"][:25])
    hz.assert_parity("prefill lse", outs[0][1], one_shot["lse"][:25])
    hz.assert_parity("decode o", outs[1][0], one_shot["o"][25:])
    hz.assert_parity("decode lse", outs[1][1], one_shot["lse"][25:])
    active = L * nat.D_K * 2
    assert active == 29952
    assert pool.numel() * 2 == 73728     # one 64-token block allocated
    assert not torch.isnan(pool[0, :L].float()).any() and torch.isnan(pool[0, L:].float()).all()


# ------------------------------------------------------------------ robustness


def test_determinism_bitwise():
    w = workloads.make("ragged_b128_h128_l1to32768", seed=3, B=6, L=3000)
    _say(f"determinism: two runs of {w.name} lens={list(w.lens)}")
    run = hz.DeviceRun(w)
    a = run.run()
    b = run.run()
    for k in ("q", "o_lat", "o"):
        assert hashlib.sha256(a[k].tobytes()).hexdigest() == hashlib.sha256(b[k].tobytes()).hexdigest(), k
    assert np.array_equal(a["lse"], b["lse"])


def test_bad_block_id_and_length_poison_only_their_sequence():
    w = workloads.Workload("poison", 3, 16, 1, [100, 100, 100], "contiguous", seed=4)
    _say("block id out of range in seq 1 and seq_len beyond the table in seq 2")
    run = hz.DeviceRun(w)
    run.block_table[1, 1] = w.num_blocks          # out of range
    run.seq_lens[2] = w.max_blocks * 64 + 1       # beyond the table
    out = run.run()
    o_lat = orc.bf16_bits_to_f64(out["o_lat"])
    assert np.all(np.isnan(o_lat[1])) and np.all(np.isnan(o_lat[2]))
    hz.check_seq("poison", w, out, 0)


# ------------------------------------------------------------------ full sizes, sampled


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", [
    "v2lite_b64_h16_l4096", "v3_b32_h128_l16384", "ragged_b128_h128_l1to32768", "causal8_b16_h128_l65544",
])
def test_full_size_sampled(name):
    w = workloads.make(name, seed=0)
    _say(f"full size {name}: B={w.B} H={w.H} Lq={w.Lq} total keys={int(w.lens.sum())}")
    out = hz.DeviceRun(w).run()
    picks = sorted({0, w.B - 1, int(np.argmax(w.lens)), int(np.argmin(w.lens)), w.B // 2})
    for b in picks:
        hz.check_seq(name, w, out, b)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", workloads.PREFILL_WORKLOADS)
def test_prefill_chunk_full_size_sampled(name):
    """A 512-token prefill chunk on a 16k context at 128 heads: 65,536 query
    rows per sequence. The oracle takes a few query tokens of each sequence
    (the first, the last and two between), the GPU computes all of them."""
    w = workloads.make(name, seed=0)
    _say(f"prefill chunk {name}: B={w.B} H={w.H} Lq={w.Lq} total keys={int(w.lens.sum())}")
    out = hz.DeviceRun(w).run()
    for b in (0, w.B - 1):
        hz.check_queries(name, w, out, b, [0, 1, w.Lq // 2 + 3, w.Lq - 1])
