"""absorb_q and out_up at prefill-sized token counts: the tokens are cut into
256-token runs, each on its own workgroups (absorb: each wave on its own
16-token passes, the rope rows of a run dealt 64 to a workgroup; out_up:
64- or 128-row workgroups by grid size), the outputs staged through LDS.
Token counts that end inside a run and inside a pass check the tails, head
counts below and above 8 the rope dealing; sampled tokens at run and pass
edges are compared with the oracle (the per-head products of [AUDIT] §2.2
and §2.3), and every output element must have been written."""

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


# (300, 21) and (513, 7): heads x runs not a multiple of 8, the plain workgroup order (no XCD grouping);
# (513, 7): rope rows of a workgroup span several tokens; (1000, 24): four runs, the last one partial
@pytest.mark.parametrize("N,H", [(2085, 128), (257, 128), (256, 16), (300, 21), (513, 7), (1000, 24)])
def test_absorb_and_out_up_in_token_runs(N, H):
    from mla_latent_cache_append_amd import native as nat
    print(f"\n[case] absorb_q / out_up N={N} H={H}", flush=True)
    w = workloads.Workload("runs", 1, H, 1, [1], "contiguous", seed=N + H)
    wuk, wuv = w.weights()
    qn = workloads.normal_bf16((N, 901, H), (N, H, 128))
    qp = workloads.normal_bf16((N, 902, H), (N, H, 64))
    ol = workloads.normal_bf16((N, 903, H), (N, H, 512))
    pos = (16384 + np.arange(N)).astype(np.int32)
    dims = nat.mla_dims_default(H)
    dev = torch.device("cuda")
    q_out = torch.full((N, H, 576), float("nan"), dtype=torch.bfloat16, device=dev)
    o = torch.full((N, H, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    nat.mla_absorb_q(dims, hz.to_dev(qn), hz.to_dev(qp), torch.from_numpy(pos).to(dev), hz.to_dev(wuk), q_out)
    nat.mla_out_up(dims, hz.to_dev(ol), hz.to_dev(wuv), o)
    torch.cuda.synchronize()
    assert not torch.isnan(q_out).any() and not torch.isnan(o).any(), "an output element was not written"
    f = orc.bf16_bits_to_f64
    toks = sorted({t for t in (0, 1, 31, 32, 255, 256, 257, 1023, 2047, 2048, 2080, N - 2, N - 1) if 0 <= t < N})
    q_lat, q_r = orc.absorb_q(f(qn[toks]), f(qp[toks]), pos[toks], f(wuk))
    ref_o = orc.out_up(f(ol[toks]), f(wuv))
    got_q = hz.f64_of(q_out)[toks]
    got_o = hz.f64_of(o)[toks]
    hz.assert_parity(f"N={N} H={H} q_lat", got_q[..., :512], q_lat)
    hz.assert_parity(f"N={N} H={H} q_r", got_q[..., 512:], q_r)
    hz.assert_parity(f"N={N} H={H} o", got_o, ref_o)
    # fp32 accumulation and one rounding: nearly every element is the nearest bf16 of the exact value
    assert np.mean(got_q[..., :512] == hz.bf16_round(q_lat)) > 0.99
    assert np.mean(got_o == hz.bf16_round(ref_o)) > 0.99
