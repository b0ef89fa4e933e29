"""The fused first half of a decode step (mla_append_absorb: append of the N
new tokens and absorption of the N queries of the same tokens in one launch)
against the two separate calls: the cache bytes (bf16 rows, or FP8 codes and
scales) and the absorbed queries must be bit-identical. The separate calls are
themselves pinned to the oracle by the parity tests, and every decode step
those tests run goes through the fused call."""

import numpy as np
import pytest
import torch

import workloads
from tests import harness as hz

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_latent_cache_append_amd import native
    native.lib()


@pytest.mark.parametrize("H,lens,fp8", [(128, [700, 33, 1500, 64], False), (16, [300, 1, 129, 64, 65], False),
                                       (128, [700, 33, 1500, 64], True), (16, [300, 1, 129, 64, 65], True)])
def test_fused_append_absorb_equals_separate_calls(H, lens, fp8):
    from mla_latent_cache_append_amd import native as nat
    w = workloads.Workload("fused", len(lens), H, 1, lens, "permuted", seed=21)
    print(f"\n[case] fused append+absorb: H={H} lens={lens} fp8={fp8}", flush=True)
    run = hz.DeviceRun(w, fp8=fp8)
    ckv, kpe, qpos, slot = run.new
    qn, qp = hz.to_dev(run.q_nope), hz.to_dev(run.q_pe)
    st = run.step
    pool0 = run.pool.clone()
    scale0 = None if run.pool_scale is None else run.pool_scale.clone()
    # separate calls
    st.append(ckv, kpe, qpos, slot)
    nat.mla_absorb_q(st.dims, qn, qp, qpos, st.w_uk, st.q)
    torch.cuda.synchronize()
    sep_pool, sep_q = run.pool.clone(), st.q.clone()
    sep_scale = None if run.pool_scale is None else run.pool_scale.clone()
    # fused call from the same starting cache
    run.pool.copy_(pool0)
    if scale0 is not None:
        run.pool_scale.copy_(scale0)
    st.q.fill_(float("nan"))
    nat.mla_append_absorb(st.dims, ckv, kpe, slot, run.pool, qn, qp, qpos, st.w_uk, st.q, pool_scale=run.pool_scale)
    torch.cuda.synchronize()
    assert torch.equal(st.q.view(torch.int16), sep_q.view(torch.int16))
    if fp8:
        assert torch.equal(run.pool, sep_pool)
        assert torch.equal(run.pool_scale.view(torch.int32), sep_scale.view(torch.int32))
    else:
        assert torch.equal(run.pool.view(torch.int16), sep_pool.view(torch.int16))
    # the new tokens' rows were written (the pool differs from the starting one there only)
    bits = (lambda t: t) if fp8 else (lambda t: t.view(torch.int16))   # NaN rows compare by their bits
    changed = (bits(run.pool).view(-1, 576) != bits(pool0).view(-1, 576)).any(dim=1).nonzero().flatten().cpu().numpy()
    assert set(changed.tolist()) <= set(slot.cpu().numpy().tolist())
    print("  cache and queries bit-identical to the separate calls", flush=True)
