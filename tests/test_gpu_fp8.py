"""GPU parity of the FP8 latent cache ([AUDIT] §6.1 lists an FP8 KV cache for
the 576-wide MQA-mode kernels; the format is the reading documented at
mla_cache_append_fp8): the append kernel's codes and scales against the
oracle's quantizer, and the FP8 attention through the C ABI against the fp64
oracle run on the values the oracle's codes stand for.

Bars: codes and scales equal the oracle's, except where the rope part's fp32
value (fp64 rotation with the kernel's own sin/cos against libm, one rounding)
lands on the other side of a rounding boundary: then a scale may differ by one
fp32 ulp and a code by one step, in at most 1e-4 of the values. Outputs take
the per-stage bar (max|d| <= 2e-2 max|ref|, mean|d|/mean|ref| <= 5e-3).
"""

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


def check_codes(name, run, w, b, ref_codes, ref_scale):
    L = int(w.lens[b])
    codes, scale = run.pool_rows_fp8(b, L)
    assert codes.shape == ref_codes.shape
    s_rel = np.abs(scale.astype(np.float64) - ref_scale) / ref_scale
    assert np.all(s_rel <= 2.0 ** -23), f"{name} b={b}: scale beyond one fp32 ulp"
    diff = codes != ref_codes
    step = np.abs(codes.astype(np.int64) - ref_codes.astype(np.int64))
    same_sign = (codes & 0x80) == (ref_codes & 0x80)
    assert np.all(~diff | (same_sign & (step == 1))), f"{name} b={b}: a code is off by more than one step"
    frac = diff.mean()
    print(f"  {name} b={b}: codes equal {1 - frac:.7f}, scales equal {np.mean(s_rel == 0):.6f}", flush=True)
    assert frac <= 1e-4, f"{name} b={b}: {frac:.3g} of the codes differ"


def check_outputs(name, w, out, b, ref):
    Lq = w.Lq
    sl = slice(b * Lq, (b + 1) * Lq)
    L = int(w.lens[b])
    valid = np.arange(L - Lq, L) >= 0
    hz.assert_parity(f"{name} b={b} o_lat", orc.bf16_bits_to_f64(out["o_lat"][sl])[valid], ref["o_lat"][valid])
    hz.assert_parity(f"{name} b={b} lse", out["lse"][sl][valid], ref["lse"][valid])
    hz.assert_parity(f"{name} b={b} o", orc.bf16_bits_to_f64(out["o"][sl])[valid], ref["o"][valid])
    if (~valid).any():
        assert np.all(orc.bf16_bits_to_f64(out["o_lat"][sl])[~valid] == 0)
        assert np.all(out["lse"][sl][~valid] == -np.inf)


# ------------------------------------------------------------------ append


def test_fp8_append_codes_and_scales():
    w = workloads.make("ragged_b128_h128_l1to32768", seed=11, B=4, lens=[1, 70, 200, 1031])
    _say(f"fp8 append {w.name} lens={list(w.lens)}")
    run = hz.DeviceRun(w, fp8=True)
    run.run()
    for b in range(w.B):
        ref = hz.oracle_seq_fp8(w, b)
        check_codes("fp8 append", run, w, b, ref["codes"], ref["scale"])


def test_fp8_append_skips_out_of_range_slots_and_zero_row():
    from mla_latent_cache_append_amd import native as nat
    _say("fp8 append: slots -1 and num_blocks*64, an all-zero row")
    dims = nat.mla_dims_default(16)
    pool = torch.zeros(2, 64, 576, dtype=torch.uint8, device="cuda")
    scale = torch.full((2, 64), -1.0, dtype=torch.float32, device="cuda")
    ckv = torch.ones(4, 512, dtype=torch.bfloat16, device="cuda")
    kpe = torch.ones(4, 64, dtype=torch.bfloat16, device="cuda")
    ckv[3] = 0
    kpe[3] = 0
    pos = torch.tensor([0, 1, 2, 3], dtype=torch.int32, device="cuda")
    slot = torch.tensor([-1, 128, 5, 6], dtype=torch.int64, device="cuda")
    nat.mla_cache_append_fp8(dims, ckv, kpe, pos, slot, pool, scale)
    torch.cuda.synchronize()
    codes = pool.view(-1, 576).cpu().numpy()
    sc = scale.view(-1).cpu().numpy()
    ref_codes, ref_scale = orc.cache_rows_fp8(np.ones((1, 512)), np.ones((1, 64)), np.array([2]))
    assert np.array_equal(codes[5], ref_codes[0]) and sc[5] == ref_scale[0]
    # an all-zero row: scale 1, zero codes (negative zeros from the rotation keep their sign bit)
    z_codes, z_scale = orc.cache_rows_fp8(np.zeros((1, 512)), np.zeros((1, 64)), np.array([3]))
    assert z_scale[0] == 1.0 and np.all(orc.e4m3_decode(z_codes) == 0)
    assert np.array_equal(codes[6], z_codes[0]) and sc[6] == 1.0
    others = np.ones(128, bool)
    others[[5, 6]] = False
    assert np.all(codes[others] == 0) and np.all(sc[others] == -1.0)


# ------------------------------------------------------------------ attention, small


@pytest.mark.parametrize("H,Lq,lens", [
    (16, 1, [1, 63, 64, 65, 129, 1000]),
    (32, 1, [5, 64, 300]),
    (64, 1, [2, 130, 517]),
    (128, 1, [1, 64, 65, 700]),
    (128, 8, [8, 9, 71, 200]),
    (16, 3, [3, 4, 64, 66, 190]),
    (32, 3, [3, 33, 96, 300]),       # 96 rows: the 128-row kernel's threshold, its fourth wave all padding
    # prefill chunks over the FP8 cache: many query tokens, causal among themselves
    (128, 64, [64, 100, 1000]),
    (16, 203, [203, 777]),
], ids=lambda v: str(v))
def test_fp8_decode_small(H, Lq, lens):
    w = workloads.Workload(f"fp8_h{H}_lq{Lq}", len(lens), H, Lq, lens,
                           "permuted" if H >= 64 else "contiguous", seed=100 + H + Lq)
    _say(f"fp8 decode step H={H} Lq={Lq} lens={lens}")
    run = hz.DeviceRun(w, fp8=True)
    out = run.run()
    for b in range(w.B):
        ref = hz.oracle_seq_fp8(w, b)
        check_codes(w.name, run, w, b, ref["codes"], ref["scale"])
        check_outputs(w.name, w, out, b, ref)


@pytest.mark.parametrize("H", [16, 128])
def test_fp8_zero_lengths_and_determinism(H):
    w = workloads.Workload("fp8_short", 4, H, 4, [0, 3, 5, 64], "contiguous", seed=19)
    _say(f"fp8 H={H} lens [0, 3, 5, 64] with Lq=4, run twice")
    run = hz.DeviceRun(w, fp8=True)
    out = run.run()
    again = run.run()
    for k in ("o_lat", "o"):
        assert np.array_equal(out[k], again[k]), k
    assert np.array_equal(out["lse"], again["lse"])
    assert np.all(orc.bf16_bits_to_f64(out["o_lat"][0:4]) == 0) and np.all(out["lse"][0:4] == -np.inf)
    for b in (1, 2, 3):
        check_outputs(w.name, w, out, b, hz.oracle_seq_fp8(w, b))


@pytest.mark.parametrize("H", [16, 128])   # the column kernel, the 128-row kernel
def test_fp8_bad_block_id_poisons_only_its_sequence(H):
    w = workloads.Workload("fp8_poison", 3, H, 1, [100, 100, 100], "contiguous", seed=14)
    _say(f"fp8 H={H}: block id out of range in seq 1 and seq_len beyond the table in seq 2")
    run = hz.DeviceRun(w, fp8=True)
    run.block_table[1, 1] = w.num_blocks
    run.seq_lens[2] = w.max_blocks * 64 + 1
    out = run.run()
    o_lat = orc.bf16_bits_to_f64(out["o_lat"])
    assert np.all(np.isnan(o_lat[1])) and np.all(np.isnan(o_lat[2]))
    check_outputs(w.name, w, out, 0, hz.oracle_seq_fp8(w, 0))


# ------------------------------------------------------------------ full sizes, sampled


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["v2lite_b64_h16_l4096", "v3_b32_h128_l16384", "ragged_b128_h128_l1to32768",
                                  "causal8_b16_h128_l65544"])
def test_fp8_full_size_sampled(name):
    w = workloads.make(name, seed=0)
    _say(f"fp8 full size {name}: B={w.B} H={w.H} Lq={w.Lq} total keys={int(w.lens.sum())}")
    run = hz.DeviceRun(w, fp8=True)
    out = run.run()
    for b in sorted({0, w.B // 2, w.B - 1, int(np.argmax(w.lens)), int(np.argmin(w.lens))}):
        ref = hz.oracle_seq_fp8(w, b)
        check_codes(name, run, w, b, ref["codes"], ref["scale"])
        check_outputs(name, w, out, b, ref)
