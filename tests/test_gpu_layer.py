"""The projections around the attention (mla_linear) and a stack of whole
layers on the GPU against the fp64 oracle: how the error of the bf16 path
grows from layer to layer ([AUDIT] §9 item 4 asks for exactly this;
[MLA80] §2 gives the layer: Wdq, Wuq, Wqr, Wdkv, Wkr around the attention,
Wo after it).
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import mla as orc
from tests import harness as hz

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_latent_cache_append_amd import native
    native.lib()


@pytest.mark.parametrize("N,K,M,resid", [
    (1, 2048, 2048, False), (32, 2048, 512, True), (33, 1536, 2048, True), (7, 96, 12, False),
    (1, 32, 4, True), (200, 512, 64, False),
    # wide maps take 32 features per workgroup (at least 128 workgroups): even and ragged M, ragged N
    (32, 1024, 8192, True), (40, 512, 4100, False),
    # the 128-head layer's narrow maps (contraction split over 6, 18 and 4 slices with a workspace),
    # a ragged token count, and a contraction past 8192 (32-wide steps)
    (32, 7168, 512, False), (32, 7168, 64, True), (32, 7168, 1536, True), (19, 4096, 256, True),
    (3, 16384, 1024, True),
    # 64 features per workgroup: unsplit with three (K = 1536) and two (K = 2048) steps in flight;
    # a long contraction not a multiple of 128 split in two (ragged M tile, three token tiles)
    (64, 1536, 7168, False), (64, 2048, 7168, True), (90, 8224, 2420, True),
], ids=lambda v: str(v))
def test_linear_matches_oracle(N, K, M, resid):
    """Unsplit (no workspace) and, where the map splits, split (workspace of
    mla_linear_workspace_size bytes, filled with 0xff first): both against
    the fp64 oracle; the split call repeated gives the same bits; a workspace
    one slice short gives the unsplit bits; in place (residual = output)
    gives the same bits as out of place."""
    from mla_latent_cache_append_amd import native as nat
    print(f"\n[case] linear N={N} K={K} M={M} residual={resid}", flush=True)
    x = workloads.normal_bf16((7, 1, N, K), (N, K))
    w = workloads.normal_bf16((7, 2, M, K), (M, K), 1.0 / np.sqrt(K))
    r = workloads.normal_bf16((7, 3, N, M), (N, M)) if resid else None
    f = orc.bf16_bits_to_f64
    ref = orc.linear(f(x), f(w)) + (f(r) if resid else 0.0)
    xd, wd = hz.to_dev(x), hz.to_dev(w)
    rd = hz.to_dev(r) if resid else None

    def run(ws=None, in_place=False):
        if in_place:
            out = rd.clone()
            nat.mla_linear(xd, wd, out, residual=out, workspace=ws)
        else:
            out = torch.full((N, M), float("nan"), dtype=torch.bfloat16, device="cuda")
            nat.mla_linear(xd, wd, out, residual=rd, workspace=ws)
        torch.cuda.synchronize()
        return out

    bits = lambda t: t.view(torch.int16)
    y = run()
    hz.assert_parity("linear", hz.f64_of(y), ref)
    if resid:
        assert torch.equal(bits(run(in_place=True)), bits(y))
    nbytes = nat.mla_linear_workspace_size(N, K, M)
    print(f"  split workspace: {nbytes} bytes", flush=True)
    if nbytes == 0:
        return
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    ys = run(ws)
    hz.assert_parity("linear split", hz.f64_of(ys), ref)
    assert torch.equal(bits(run(ws)), bits(ys))
    if resid:
        assert torch.equal(bits(run(ws, in_place=True)), bits(ys))
    short = ws[:nbytes - N * M * 4]
    assert torch.equal(bits(run(short)), bits(y))


def test_linear_rejects_unsupported_shapes():
    from mla_latent_cache_append_amd import native as nat
    x = torch.zeros(2, 48, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(8, 48, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(2, 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nat.MlaError):
        nat.mla_linear(x, w, y)      # K = 48 is not a multiple of 32


def test_layer_stack_error_growth():
    """Six layers (V2-Lite attention shape: H=16; d_model 2048, query latent
    1536), two sequences with 300 and 1000 cached tokens per layer plus the
    new token. Every layer's output h_l and its contribution y_l = h_l -
    h_{l-1} are compared with the oracle's fp64 stack started from the same
    bf16 inputs. (y_l on the GPU is Wo o of the layer taken again without
    the residual, so that it is not measured through the bf16 rounding of h.)

    Tolerance: h_l takes the per-stage bar (2e-2 max, 5e-3 mean relative).
    y_l is the end of a chain of about ten bf16 roundings inside the layer
    (qz, q_nope, q_pe, c_kv, k_pe, q_lat, P, o_lat, o, y), each of which alone
    gives a mean relative error of ~1.4e-3 (the single-rounding figure of the
    linear cases); independent errors add to ~4.5e-3 at the first layer and
    grow as earlier layers' errors reach the queries and keys, so y_l is held
    to 2e-2 max and 1e-2 mean relative."""
    from mla_latent_cache_append_amd import native as nat
    from mla_latent_cache_append_amd.step import LayerStep
    H, d_model, d_cq, n_layers = 16, 2048, 1536, 6
    lens = [301, 1001]
    B = len(lens)
    f = orc.bf16_bits_to_f64
    runs, steps, layers_f64, hists = [], [], [], []
    for l in range(n_layers):
        w = workloads.Workload(f"layer{l}", B, H, 1, lens, "permuted", seed=100 + l)
        run = hz.DeviceRun(w)
        lw = workloads.layer_weights(100, l, H, d_model, d_cq)
        steps.append(LayerStep(run.step, **{k: hz.to_dev(v) for k, v in lw.items()}))
        runs.append(run)
        wuk, wuv = w.weights()
        layers_f64.append(dict({k: f(v) for k, v in lw.items()}, w_uk=f(wuk), w_uv=f(wuv)))
        hists.append([tuple(f(a) for a in w.seq_cache(b, lens[b] - 1)) for b in range(B)])
    h0 = workloads.hidden_states(100, B, d_model)
    print(f"\n[case] layer stack: {n_layers} layers, H={H}, d_model={d_model}, lens={lens}", flush=True)
    h = hz.to_dev(h0)
    y = torch.empty(B, d_model, dtype=torch.bfloat16, device="cuda")
    gpu_h, gpu_y = [], []
    for l, st in enumerate(steps):
        _, _, qpos, slot = runs[l].new
        h = st(h, qpos, slot).clone()
        nat.mla_linear(st.decode.o.view(B, -1), st.w_o, y, workspace=st.ws["o"])
        gpu_h.append(hz.f64_of(h))
        gpu_y.append(hz.f64_of(y))
    torch.cuda.synchronize()
    ref_h = [np.stack([orc.stack_decode(f(h0[b:b + 1]), [hists[l][b] for l in range(n_layers)],
                                        layers_f64)[l][0] for b in range(B)]) for l in range(n_layers)]
    prev_r = f(h0)
    for l in range(n_layers):
        mh = hz.assert_parity(f"layer {l} h", gpu_h[l], ref_h[l])
        my = hz.assert_parity(f"layer {l} y", gpu_y[l], ref_h[l] - prev_r, max_rel=2e-2, mean_rel=1e-2)
        print(f"  layer {l}: h max_rel {mh['max_rel']:.2e} mean_rel {mh['mean_rel']:.2e} | "
              f"y max_rel {my['max_rel']:.2e} mean_rel {my['mean_rel']:.2e}", flush=True)
        prev_r = ref_h[l]


@pytest.mark.parametrize("reps", [1, 3])
def test_layer_graph_replays_match_eager(reps):
    """The whole layer (projections, two of them on a side stream, the split
    ones with their reduce kernels, decode step, residual output projection)
    recorded as one HIP graph (``reps`` layers in a row) replays bit for bit
    to the eager layer, with eager work that overwrites every buffer the
    layer writes between replays."""
    from mla_latent_cache_append_amd.step import LayerStep
    H, d_model, d_cq = 16, 2048, 1536
    w = workloads.Workload("layer_graph", 3, H, 1, [70, 600, 1500], "permuted", seed=300)
    run = hz.DeviceRun(w)
    lw = workloads.layer_weights(300, 0, H, d_model, d_cq)
    st = LayerStep(run.step, **{k: hz.to_dev(v) for k, v in lw.items()})
    h = hz.to_dev(workloads.hidden_states(300, w.B, d_model))
    _, _, qpos, slot = run.new
    print(f"\n[case] layer graph: H=16, lens [70, 600, 1500], layers per graph {reps}", flush=True)
    eager = st(h, qpos, slot).clone()
    torch.cuda.synchronize()
    g = st.capture(h, qpos, slot, reps=reps)
    torch.cuda.synchronize()
    for rep in range(3):
        # every buffer the layer writes, the side stream's projections' included
        for buf in (st.out, st.decode.o, st.c_kv, st.k_pe, st.qz, st.q_nope, st.q_pe):
            buf.fill_(float("nan"))
        st.workspace.fill_(0xFF)    # the split maps' fp32 partial sums
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.out.view(torch.int16), eager.view(torch.int16)), rep
        print(f"  replay {rep}: bitwise equal to the eager layer", flush=True)
