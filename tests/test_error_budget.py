"""Error budget of the GPU path, one rounding point at a time.

The GPU path differs from the fp64 oracle only where it rounds: the absorbed
query q_lat, the rotated query and key parts q_r and k_r (each once to
bf16), the probabilities before the PV product (bf16, the row sum keeps
them unrounded), the split partials o/l (bf16, one more rounding on rows
whose keys are split over several workgroups), o_lat (bf16) and o (bf16,
computed from the stored o_lat). The fp32 accumulations add errors near
2^-24 and are left out. This file applies each rounding alone, and all of
them together, to the oracle's own pipeline (nearest-even bf16 of the exact
fp64 value) and reports the mean relative error mean|d| / mean|ref| of o_lat
and o that it causes, on inputs drawn as the workloads draw them. It checks
that the sum stays inside the parity bar and that no single point costs more
than about one bf16 rounding of the output (mean relative error 1.41e-3); `python tests/test_error_budget.py
[L] [H]` prints the table for other sizes.
"""
import sys

import numpy as np
import pytest

import workloads
from oracle import mla as orc

POINTS = ("q_lat", "q_r", "k_r", "P", "partials", "o_lat", "o")


def bf16(x):
    """Nearest-even bf16 of float64 values (normal range), without a detour
    through float32 (which could round twice)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m 2^e, |m| in [0.5, 1)
    return np.ldexp(np.rint(m * 256.0), e - 8)   # 8 significant bits, ties to even


def decode(q_lat, q_r, c_kv, k_r, w_uv, on, splits):
    """o_lat and o of one decode query (Lq = 1) with the rounding points in `on`."""
    r = lambda name, x: bf16(x) if name in on else x
    q_lat, q_r, k_r = r("q_lat", q_lat), r("q_r", q_r), r("k_r", k_r)
    s = orc.latent_scores(q_lat, q_r, c_kv, k_r, orc.default_scale())[0]   # [H, L]
    L = c_kv.shape[0]
    bounds = np.linspace(0, L, splits + 1).astype(int)
    parts = []
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        m = s[:, t0:t1].max(axis=1, keepdims=True)
        p = np.exp(s[:, t0:t1] - m)
        l = p.sum(axis=1)                               # the row sum takes unrounded p
        acc = r("P", p) @ c_kv[t0:t1]
        ol = r("partials", acc / l[:, None]) if splits > 1 else acc / l[:, None]
        parts.append((m[:, 0], l, ol))
    M = np.max([p[0] for p in parts], axis=0)
    wts = [np.exp(p[0] - M) * p[1] for p in parts]
    o_lat = sum(w[:, None] * p[2] for w, p in zip(wts, parts)) / sum(wts)[:, None]
    o_lat = r("o_lat", o_lat)
    o = np.einsum("hjc,hc->hj", w_uv, o_lat)
    return o_lat, r("o", o)


def budget(L: int, H: int, splits: int, seed: int = 3):
    w = workloads.Workload("budget", 1, H, 1, [L], "contiguous", seed=seed)
    f = orc.bf16_bits_to_f64
    ckv, kpe = (f(x) for x in w.seq_cache(0))
    qn, qp = (f(x) for x in w.queries(0))
    wuk, wuv = (f(x) for x in w.weights())
    q_lat, q_r = orc.absorb_q(qn, qp, w.query_positions()[:1], wuk)
    k_r = orc.rope(kpe, np.arange(L))
    ref = decode(q_lat, q_r, ckv, k_r, wuv, (), splits)

    def rel(on):
        got = decode(q_lat, q_r, ckv, k_r, wuv, on, splits)
        return tuple(float(np.abs(g - r_).mean() / np.abs(r_).mean()) for g, r_ in zip(got, ref))

    rows = {p: rel((p,)) for p in POINTS}
    rows["all"] = rel(POINTS)
    return rows


def _table(L, H, splits):
    rows = budget(L, H, splits)
    print(f"L={L} H={H} ranges={splits}: mean relative error of o_lat / o")
    for k, (a, b) in rows.items():
        print(f"  {k:9s} {a:.2e} {b:.2e}")
    return rows


# One bf16 rounding of values spread over many binades: |error| is uniform up
# to half a unit of the 8th significant bit, so mean|d| / mean|x| is about
# 2^-9 * E[2^e / |x|] = 2^-9 * (1/2) / ln 2 = 1.41e-3.
ONE_ROUNDING = 2.0 ** -9 * 0.5 / np.log(2.0)


def test_bf16_helper_is_nearest_even():
    """The helper against the float32 route (exact for float32 inputs: no
    double rounding) and against the mean error of one rounding."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200_000).astype(np.float32)
    ref = orc.bf16_bits_to_f64(workloads.f32_to_bf16_bits(x))
    assert np.array_equal(bf16(x.astype(np.float64)), ref)
    rel = np.abs(ref - x).mean() / np.abs(x).mean()
    assert abs(rel / ONE_ROUNDING - 1.0) < 0.05, rel


@pytest.mark.parametrize("L,H,splits", [(26, 16, 1), (130, 16, 3), (4096, 128, 8)])
def test_error_budget(L, H, splits):
    rows = _table(L, H, splits)
    for p in POINTS:
        assert rows[p][1] < 1.5 * ONE_ROUNDING, (p, rows[p])
    assert rows["o"][1] > 0.7 * ONE_ROUNDING    # the last rounding acts on o itself
    total_o = rows["all"][1]
    # the points add roughly in quadrature; the sum stays inside the 5e-3 bar
    assert total_o < 4.5e-3, rows["all"]
    assert total_o <= 1.2 * np.sqrt(sum(rows[p][1] ** 2 for p in POINTS)) + 1e-4, rows


if __name__ == "__main__":
    L = int(sys.argv[1]) if len(sys.argv) > 1 else 16384
    H = int(sys.argv[2]) if len(sys.argv) > 2 else 128
    _table(L, H, 8)
