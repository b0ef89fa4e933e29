"""Pins of the oracle's whole-layer functions (the projections around the
attention, [MLA80] §2 MLA.__init__ / forward) and of the layer stack.

Tags: [MLA80] CSDN "80 行 PyTorch 从零写 DeepSeek 的 MLA"; [AUDIT] llm-atlas
"DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界".
"""

import math

import numpy as np

from oracle import mla


def layer_weights(rng, d_model=40, d_cq=24, H=2):
    """Random weights in nn.Linear layout; d_cq != d_model so that a query
    computed from the wrong input fails on shapes."""
    g = lambda *s: rng.standard_normal(s) / math.sqrt(s[-1])
    w_uk = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    w_uv = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    return dict(w_dq=g(d_cq, d_model), w_uq=g(H * 128, d_cq), w_qr=g(H * 64, d_cq),
                w_dkv=g(512, d_model), w_kr=g(64, d_model), w_uk=w_uk, w_uv=w_uv,
                w_o=g(d_model, H * 128))


def test_linear_is_the_scalar_sum():
    # y[n][o] = sum_i x[n][i] w[o][i], by plain loops on a tiny case
    rng = np.random.default_rng(1)
    x, w = rng.standard_normal((3, 5)), rng.standard_normal((4, 5))
    y = mla.linear(x, w)
    for n in range(3):
        for o in range(4):
            assert abs(y[n, o] - sum(x[n, i] * w[o, i] for i in range(5))) < 1e-13


def test_layer_absorbed_equals_expanded():
    # the two definitions of the attention inside one layer ([MLA80] §2 vs §5)
    rng = np.random.default_rng(2)
    lw = layer_weights(rng)
    h = rng.standard_normal((3, 40))
    hc, hk = rng.standard_normal((20, 512)), rng.standard_normal((20, 64))
    a = mla.layer_decode(h, hc, hk, lw, path="absorbed")["y"]
    b = mla.layer_decode(h, hc, hk, lw, path="naive")["y"]
    assert np.max(np.abs(a - b)) <= 1e-10 * max(1.0, np.max(np.abs(b)))


def test_single_key_layer_is_linear_algebra():
    # no history and one new token: its only key gets weight 1, so
    # o_lat = c_kv = Wdkv h, o[h] = W_UV[h] o_lat and y = sum_h Wo[:, head h] o[h]
    rng = np.random.default_rng(3)
    lw = layer_weights(rng, H=3)
    h = rng.standard_normal((1, 40))
    y = mla.layer_decode(h, np.zeros((0, 512)), np.zeros((0, 64)), lw)["y"][0]
    c = lw["w_dkv"] @ h[0]
    want = sum(lw["w_o"][:, 128 * j:128 * (j + 1)] @ (lw["w_uv"][j] @ c) for j in range(3))
    assert np.max(np.abs(y - want)) < 1e-12


def test_zero_query_weights_give_the_mean_of_all_keys():
    # W_UK = 0 and Wqr = 0 make every score 0: uniform weights over the
    # history and the new tokens' own latents (appended before attending);
    # the last new token sees every key
    rng = np.random.default_rng(4)
    lw = layer_weights(rng)
    lw["w_uk"] = np.zeros_like(lw["w_uk"])
    lw["w_qr"] = np.zeros_like(lw["w_qr"])
    h = rng.standard_normal((2, 40))
    hc, hk = rng.standard_normal((7, 512)), rng.standard_normal((7, 64))
    r = mla.layer_decode(h, hc, hk, lw)
    keys = np.concatenate([hc, (lw["w_dkv"] @ h.T).T])
    mean_last = keys.mean(axis=0)              # 9 keys
    mean_first = keys[:8].mean(axis=0)         # the first new token sees 8
    for j in range(2):
        np.testing.assert_allclose(r["o"][1, j], lw["w_uv"][j] @ mean_last, atol=1e-12)
        np.testing.assert_allclose(r["o"][0, j], lw["w_uv"][j] @ mean_first, atol=1e-12)


def test_query_path_goes_through_the_compression():
    # scaling Wdq by a and Wuq, Wqr by 1/a leaves the layer unchanged only if
    # the queries are formed from qz = Wdq h
    rng = np.random.default_rng(5)
    lw = layer_weights(rng)
    h = rng.standard_normal((2, 40))
    hc, hk = rng.standard_normal((11, 512)), rng.standard_normal((11, 64))
    y0 = mla.layer_decode(h, hc, hk, lw)["y"]
    lw2 = dict(lw, w_dq=lw["w_dq"] * 3.0, w_uq=lw["w_uq"] / 3.0, w_qr=lw["w_qr"] / 3.0)
    assert np.max(np.abs(mla.layer_decode(h, hc, hk, lw2)["y"] - y0)) < 1e-12
    lw3 = dict(lw, w_uq=lw["w_uq"] * 3.0)      # the content scores alone change
    assert np.max(np.abs(mla.layer_decode(h, hc, hk, lw3)["y"] - y0)) > 1e-3


def test_stack_is_residual():
    rng = np.random.default_rng(6)
    layers = [layer_weights(rng) for _ in range(3)]
    hists = [(rng.standard_normal((5, 512)), rng.standard_normal((5, 64))) for _ in range(3)]
    h0 = rng.standard_normal((1, 40))
    hs = mla.stack_decode(h0, hists, layers)
    assert len(hs) == 3
    np.testing.assert_allclose(hs[0], h0 + mla.layer_decode(h0, *hists[0], layers[0])["y"], atol=1e-13)
    np.testing.assert_allclose(hs[2], hs[1] + mla.layer_decode(hs[1], *hists[2], layers[2])["y"], atol=1e-13)
    # a layer whose Wo is zero passes the stream through unchanged
    layers[1] = dict(layers[1], w_o=np.zeros_like(layers[1]["w_o"]))
    hs = mla.stack_decode(h0, hists, layers)
    np.testing.assert_array_equal(hs[1], hs[0])
