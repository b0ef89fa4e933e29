"""Pins of the fp64 oracle against what the pages and mathematics fix.

Every check is a function of the oracle module so that the planted-mistake
tests at the bottom can show each pin fails when a plausible slip (a dropped
term, a wrong sign, a wrong scale, a wrong causal alignment, the wrong weight,
a missing merge weight) is planted in the oracle on the CPU.

Tags: [AUDIT] llm-atlas "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界";
[MLA80] CSDN "80 行 PyTorch 从零写 DeepSeek 的 MLA".
"""

import cmath
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import mla


def rand_case(seed, H=4, Lq=1, L=37, scale_q=1.0):
    rng = np.random.default_rng(seed)
    return dict(
        q_nope=rng.standard_normal((Lq, H, 128)) * scale_q,
        q_pe=rng.standard_normal((Lq, H, 64)) * scale_q,
        c_kv=rng.standard_normal((L, 512)),
        k_pe=rng.standard_normal((L, 64)),
        w_uk=rng.standard_normal((H, 128, 512)) / math.sqrt(512),
        w_uv=rng.standard_normal((H, 128, 512)) / math.sqrt(512),
    )


def c1_case(seed=0):
    """The tiny V2-Lite-shape layer: H=16, 25-token prefill + 1 decode (L=26)."""
    w = workloads.make("v2lite_tiny_b1_h16_l26", seed)
    c_kv, k_pe = w.seq_cache(0)
    q_nope, q_pe = w.queries()
    w_uk, w_uv = w.weights()
    f = mla.bf16_bits_to_f64
    return dict(q_nope=f(q_nope), q_pe=f(q_pe), c_kv=f(c_kv), k_pe=f(k_pe), w_uk=f(w_uk), w_uv=f(w_uv))


def rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(1.0, float(np.max(np.abs(b)))))


# --------------------------------------------------------------------------- checks


def err_naive_vs_absorbed(m, case, dtype=np.float64):
    a = m.absorbed_decode(**case, dtype=dtype)
    n = m.naive_decode(**case, dtype=dtype)
    return max(rel(a["o"], n["o"]), rel(a["lse"], n["lse"]))


def err_sdpa(m, case):
    """The naive path's softmax, scale and mask vs torch SDPA (float64, CPU),
    called as [MLA80] §2 calls it: default scale, boolean mask."""
    n = m.naive_decode(**case)
    q = torch.from_numpy(np.ascontiguousarray(n["q"].transpose(1, 0, 2)))[None]
    k = torch.from_numpy(np.ascontiguousarray(n["k"].transpose(1, 0, 2)))[None]
    v = torch.from_numpy(np.ascontiguousarray(n["v"].transpose(1, 0, 2)))[None]
    L, Lq = case["c_kv"].shape[0], case["q_nope"].shape[0]
    mask = torch.from_numpy(np.arange(L)[None, :] <= np.arange(L - Lq, L)[:, None])
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    return rel(n["o"], o[0].numpy().transpose(1, 0, 2))


def err_expansion_vs_linear(m, case):
    """Per-head expansion k_c = W_UK[h] c as nn.Linear(d_c, n_h*d_h) computes it
    ([MLA80] §2: ``self.Wuk(c_kv).view(B, Lt, n_h, d_h)``)."""
    n = m.naive_decode(**case)
    H = case["w_uk"].shape[0]
    c = torch.from_numpy(case["c_kv"])
    kc = torch.nn.functional.linear(c, torch.from_numpy(case["w_uk"].reshape(H * 128, 512))).view(-1, H, 128)
    v = torch.nn.functional.linear(c, torch.from_numpy(case["w_uv"].reshape(H * 128, 512))).view(-1, H, 128)
    return max(rel(n["k"][..., :128], kc.numpy()), rel(n["v"], v.numpy()))


def err_rope_complex(m, seed=0):
    """RoPE of an interleaved pair is multiplication of x[2i] + i x[2i+1] by
    exp(i theta_i), theta_i = p * 10000^(-2i/64) ([MLA80] appendix A pairs
    x[::2] with x[1::2])."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((9, 64))
    pos = np.array([0, 1, 2, 7, 100, 4095, 16383, 32767, 65543])
    y = m.rope(x, pos)
    worst = 0.0
    for r in range(x.shape[0]):
        for i in range(32):
            th = pos[r] * 10000.0 ** (-2.0 * i / 64)
            z = complex(x[r, 2 * i], x[r, 2 * i + 1]) * cmath.exp(1j * th)
            worst = max(worst, abs(y[r, 2 * i] - z.real), abs(y[r, 2 * i + 1] - z.imag))
    return worst


def err_incremental(m, case):
    """25-token prefill + 1-token decode equals one 26-token causal forward
    ([MLA80] §2 cache equivalence test: prefill rows 0.00, decoded row 4.47e-8
    at fp32)."""
    L = case["c_kv"].shape[0]
    full = dict(case, q_nope=case["q_nope_all"], q_pe=case["q_pe_all"])
    full.pop("q_nope_all"); full.pop("q_pe_all")
    one_shot = m.absorbed_decode(**full)
    pre = dict(full, q_nope=full["q_nope"][:L - 1], q_pe=full["q_pe"][:L - 1],
               c_kv=full["c_kv"][:L - 1], k_pe=full["k_pe"][:L - 1])
    dec = dict(full, q_nope=full["q_nope"][L - 1:], q_pe=full["q_pe"][L - 1:])
    p = m.absorbed_decode(**pre)
    d = m.absorbed_decode(**dec)
    return max(rel(p["o"], one_shot["o"][:L - 1]), rel(d["o"], one_shot["o"][L - 1:]))


def err_multi_query(m, case):
    """Lq new tokens attending causally equal Lq one-token decodes, query i
    over the first L-Lq+i+1 keys."""
    Lq = case["q_nope"].shape[0]
    L = case["c_kv"].shape[0]
    a = m.absorbed_decode(**case)
    worst = 0.0
    for i in range(Lq):
        Li = L - Lq + i + 1
        d = m.absorbed_decode(**dict(case, q_nope=case["q_nope"][i:i + 1], q_pe=case["q_pe"][i:i + 1],
                                     c_kv=case["c_kv"][:Li], k_pe=case["k_pe"][:Li]))
        worst = max(worst, rel(d["o_lat"], a["o_lat"][i:i + 1]), rel(d["lse"], a["lse"][i:i + 1]))
    return worst


def err_partition(m, case, seed=0, trials=6):
    """Any partition of the key range, merged, equals the unsplit result."""
    L = case["c_kv"].shape[0]
    Lq = case["q_nope"].shape[0]
    q_pos = m.query_positions(L, Lq)
    k_r = m.rope(case["k_pe"], np.arange(L))
    q_lat, q_r = m.absorb_q(case["q_nope"], case["q_pe"], q_pos, case["w_uk"])
    ref, ref_lse = m.latent_attention(q_lat, q_r, case["c_kv"], k_r, q_pos, m.default_scale())
    rng = np.random.default_rng(seed)
    worst = 0.0
    for _ in range(trials):
        cuts = np.sort(rng.integers(0, L + 1, size=rng.integers(1, 6)))
        edges = [0] + list(cuts) + [L]
        parts = [m.partial_attention(q_lat, q_r, case["c_kv"], k_r, q_pos, m.default_scale(), a, b)
                 for a, b in zip(edges[:-1], edges[1:])]
        o, lse = m.merge_partials(parts)
        worst = max(worst, rel(o, ref), rel(lse, ref_lse))
    return worst


# --------------------------------------------------------------------------- brute force


def brute_force(case):
    """Scalar loops written from the definition (absorbed order), no NumPy math."""
    qn, qp, ckv, kpe, wuk, wuv = (case[k].tolist() for k in ("q_nope", "q_pe", "c_kv", "k_pe", "w_uk", "w_uv"))
    Lq, H, L = len(qn), len(qn[0]), len(ckv)
    scale = 1.0 / math.sqrt(192.0)

    def rot(x, p):
        y = list(x)
        for i in range(32):
            th = p / (10000.0 ** (2.0 * i / 64.0))
            c, s = math.cos(th), math.sin(th)
            y[2 * i] = x[2 * i] * c - x[2 * i + 1] * s
            y[2 * i + 1] = x[2 * i + 1] * c + x[2 * i] * s
        return y

    kr = [rot(kpe[t], t) for t in range(L)]
    out = [[None] * H for _ in range(Lq)]
    olat = [[None] * H for _ in range(Lq)]
    for i in range(Lq):
        p = L - Lq + i
        for h in range(H):
            ql = [sum(wuk[h][j][c] * qn[i][h][j] for j in range(128)) for c in range(512)]
            qr = rot(qp[i][h], p)
            s = []
            for t in range(p + 1):
                s.append(scale * (sum(ql[c] * ckv[t][c] for c in range(512)) +
                                  sum(qr[r] * kr[t][r] for r in range(64))))
            mx = max(s)
            e = [math.exp(v - mx) for v in s]
            z = sum(e)
            ol = [sum(e[t] * ckv[t][c] for t in range(p + 1)) / z for c in range(512)]
            olat[i][h] = ol
            out[i][h] = [sum(wuv[h][j][c] * ol[c] for c in range(512)) for j in range(128)]
    return np.array(olat), np.array(out)


# --------------------------------------------------------------------------- pins


@pytest.mark.parametrize("seed,H,Lq,L", [(0, 16, 1, 26), (1, 4, 1, 1), (2, 3, 4, 9), (3, 8, 8, 70), (4, 2, 1, 200)])
def test_naive_equals_absorbed_fp64(seed, H, Lq, L):
    # [AUDIT] §2.2-2.3: the two association orders are the same function
    assert err_naive_vs_absorbed(mla, rand_case(seed, H, Lq, L)) <= 1e-10


def test_naive_equals_absorbed_c1():
    assert err_naive_vs_absorbed(mla, c1_case()) <= 1e-10


def test_fp32_gap_is_rounding_level():
    """In float32 the two orders differ only by rounding ([AUDIT] §5.3 prints
    max 1.19e-7 on its outputs; [MLA80] §4 prints 2.38e-6 on scores)."""
    e = err_naive_vs_absorbed(mla, c1_case(), dtype=np.float32)
    assert 0.0 < e < 1e-4


@pytest.mark.parametrize("seed,H,Lq,L", [(0, 16, 1, 26), (5, 4, 3, 17), (6, 2, 26, 26)])
def test_naive_vs_torch_sdpa(seed, H, Lq, L):
    assert err_sdpa(mla, rand_case(seed, H, Lq, L)) <= 1e-12


def test_expansion_matches_linear_layout():
    assert err_expansion_vs_linear(mla, rand_case(7, 3, 1, 11)) <= 1e-12


def test_rope_is_complex_rotation():
    assert err_rope_complex(mla) <= 1e-9


def test_rope_identity_norm_relative():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 64))
    assert np.array_equal(mla.rope(x, np.zeros(5)), x)                       # R(0) = I
    y = mla.rope(x, np.array([1, 10, 1000, 30000, 65543]))
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    base = mla.rope(q, 40) @ mla.rope(k, 13)
    for d in (1, 77, 5000, 60000):                                            # only p - t matters
        assert abs(mla.rope(q, 40 + d) @ mla.rope(k, 13 + d) - base) <= 1e-9 * (1 + abs(base))


def test_incremental_equals_one_shot():
    case = rand_case(8, 16, 1, 26)
    rng = np.random.default_rng(9)
    case["q_nope_all"] = rng.standard_normal((26, 16, 128))
    case["q_pe_all"] = rng.standard_normal((26, 16, 64))
    assert err_incremental(mla, case) <= 1e-12


def test_multi_query_causal_equals_single_decodes():
    assert err_multi_query(mla, rand_case(10, 4, 8, 75)) <= 1e-12


def test_partition_merge():
    assert err_partition(mla, rand_case(11, 4, 1, 150)) <= 1e-12
    assert err_partition(mla, rand_case(12, 3, 8, 40), seed=1) <= 1e-12     # causal: empty ranges occur


def test_brute_force_tiny_full_dims():
    case = rand_case(13, H=2, Lq=2, L=5)
    ol, o = brute_force(case)
    a = mla.absorbed_decode(**case)
    assert rel(a["o_lat"], ol) <= 1e-12 and rel(a["o"], o) <= 1e-12


def test_special_cases():
    # one key: o_lat is that key exactly
    case = rand_case(14, 4, 1, 1)
    a = mla.absorbed_decode(**case)
    assert np.array_equal(a["o_lat"][0, :, :], np.broadcast_to(case["c_kv"][0], (4, 512)))
    assert np.allclose(a["lse"], mla.default_scale() * (
        np.einsum("hc,c->h", a["q_lat"][0], case["c_kv"][0]) + a["q_r"][0] @ a["k_r"][0]), rtol=1e-13)
    # zero query: uniform weights, o_lat = mean of the keys, lse = log L
    case = rand_case(15, 4, 1, 33, scale_q=0.0)
    a = mla.absorbed_decode(**case)
    assert rel(a["o_lat"][0], np.broadcast_to(case["c_kv"].mean(0), (4, 512))) <= 1e-13
    assert np.allclose(a["lse"], math.log(33), rtol=1e-14)
    # one dominant key: o_lat -> that key
    case = rand_case(16, 2, 1, 20)
    a0 = mla.absorbed_decode(**case)
    case["c_kv"][7] = 40.0 * a0["q_lat"][0, 0] / np.linalg.norm(a0["q_lat"][0, 0])
    a = mla.absorbed_decode(**case)
    assert rel(a["o_lat"][0, 0], case["c_kv"][7]) <= 1e-6


def check_large_L_tilting():
    """Gaussian exponential tilting: for keys c ~ N(0, I) the softmax-weighted
    mean sum_t p_t c_t with p_t proportional to exp(a . c_t) tends to a as L
    grows (E[c e^{a.c}] / E[e^{a.c}] = a). Here a = scale * q_lat, with the
    rope part of the score an independent Gaussian factor that cancels. At
    L = 50,000 and |a| = 1 the effective sample is ~L/e, so the projection of
    o_lat on a is 1 within ~0.01 and its angle to a small."""
    rng = np.random.default_rng(23)
    L = 50_000
    c_kv = rng.standard_normal((L, 512))
    k_r = rng.standard_normal((L, 64))
    scale = mla.default_scale()
    q_lat = rng.standard_normal((1, 1, 512))
    q_lat *= 1.0 / (scale * np.linalg.norm(q_lat))          # |scale * q_lat| = 1
    q_r = rng.standard_normal((1, 1, 64)) * 0.5 / (scale * 8.0)
    o_lat, _ = mla.latent_attention(q_lat, q_r, c_kv, k_r, np.array([L - 1]), scale)
    a = scale * q_lat[0, 0]
    o = o_lat[0, 0]
    proj = float(o @ a / (a @ a))
    cos = float(o @ a / (np.linalg.norm(o) * np.linalg.norm(a)))
    assert abs(proj - 1.0) < 0.03, proj
    assert cos > 0.95, cos
    return proj, cos


def test_large_L_tilting_limit():
    check_large_L_tilting()


def test_rope_on_content_breaks_absorption():
    """Negative control ([MLA80] §4: RoPE on K_C makes absorption diverge by
    1.03e+01): the checker must see an O(1) difference."""
    case = rand_case(17, 4, 1, 64)
    a = mla.absorbed_decode(**case)
    n = mla.naive_decode(**case, rope_on_content=True)
    assert rel(a["o"], n["o"]) > 1e-2


# --------------------------------------------------------------------------- planted mistakes


def test_planted_dropped_rope_term(monkeypatch):
    good = mla.latent_scores
    monkeypatch.setattr(mla, "latent_scores", lambda ql, qr, c, kr, sc, dtype=np.float64:
                        good(ql, qr * 0, c, kr, sc, dtype))
    assert err_naive_vs_absorbed(mla, rand_case(20, 4, 1, 30)) > 1e-3


def test_planted_rope_sign(monkeypatch):
    def bad(x, pos, base=10000.0, dtype=np.float64):
        return mla_rope_orig(x, -np.asarray(pos), base, dtype)
    mla_rope_orig = mla.rope
    monkeypatch.setattr(mla, "rope", bad)
    assert err_rope_complex(mla) > 1e-3


def test_planted_rope_pairing(monkeypatch):
    """Half-split pairing (x[i], x[i+32]) instead of interleaved pairs."""
    orig = mla.rope

    def bad(x, pos, base=10000.0, dtype=np.float64):
        x = np.asarray(x, dtype=dtype)
        h = x.shape[-1] // 2
        perm = np.stack([np.arange(h), np.arange(h) + h], -1).reshape(-1)
        y = orig(x[..., perm], pos, base, dtype)
        out = np.empty_like(y)
        out[..., perm] = y
        return out
    monkeypatch.setattr(mla, "rope", bad)
    assert err_rope_complex(mla) > 1e-3


def test_planted_wrong_scale(monkeypatch):
    monkeypatch.setattr(mla, "default_scale", lambda d_nope=128, d_rope=64: 1.0 / math.sqrt(576))
    assert err_sdpa(mla, rand_case(21, 4, 1, 30)) > 1e-3


def test_planted_top_left_causal(monkeypatch):
    monkeypatch.setattr(mla, "query_positions", lambda L, Lq: np.arange(Lq, dtype=np.int64))
    case = rand_case(22, 4, 1, 26)
    rng = np.random.default_rng(9)
    case["q_nope_all"] = rng.standard_normal((26, 4, 128))
    case["q_pe_all"] = rng.standard_normal((26, 4, 64))
    assert err_incremental(mla, case) > 1e-3


def test_planted_wrong_weight(monkeypatch):
    orig = mla.absorb_q
    monkeypatch.setattr(mla, "absorb_q", lambda qn, qp, pos, w, base=10000.0, dtype=np.float64:
                        orig(qn, qp, pos, np.ascontiguousarray(w[::-1]), base, dtype))
    assert err_naive_vs_absorbed(mla, rand_case(23, 4, 1, 30)) > 1e-3


def test_planted_merge_without_weights(monkeypatch):
    def bad(parts):
        l = sum(p[1] for p in parts)
        acc = sum(p[2] for p in parts)
        return acc / l[..., None], np.log(l)
    monkeypatch.setattr(mla, "merge_partials", bad)
    assert err_partition(mla, rand_case(24, 4, 1, 150)) > 1e-3


def test_planted_softmax_temperature(monkeypatch):
    """A softmax taken at the wrong temperature (scores halved inside the
    weights) fails the large-L tilting limit."""
    real = mla.masked_softmax
    monkeypatch.setattr(mla, "masked_softmax", lambda s_, mask: real(0.5 * s_, mask))
    with pytest.raises(AssertionError):
        check_large_L_tilting()
