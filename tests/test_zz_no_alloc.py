"""mla_decode_attn_noalloc (partials in the library's fixed per-GPU array, no
workspace) against mla_decode_attn (caller workspace) through the C ABI:
two calls in a row, the second with a smaller input, each bit for bit equal
to the workspace entry point on the same inputs (same kernels, same plan)."""

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


def _compare(w: workloads.Workload):
    from mla_latent_cache_append_amd import native as nat
    run = hz.DeviceRun(w)
    ref = run.run()                                   # the step's attention: mla_decode_attn
    s = run.step
    o_lat = torch.full_like(s.o_lat, float("nan"))
    lse = torch.full_like(s.lse, float("nan"))
    nat.mla_decode_attn_noalloc(s.dims, s.q, run.pool, run.block_table, run.seq_lens, w.Lq, o_lat, lse)
    torch.cuda.synchronize()
    assert np.array_equal(hz.bits_of(o_lat), ref["o_lat"]), "o_lat differs from mla_decode_attn"
    assert np.array_equal(lse.cpu().numpy().astype(np.float64), ref["lse"]), "lse differs from mla_decode_attn"
    hz.check_seq(f"noalloc {w.name}", w, {**ref, "o_lat": hz.bits_of(o_lat)}, 0)


def test_no_alloc_matches_workspace_entry_point_twice():
    # 128 heads, ragged lengths: every sequence split over several ranges, so
    # the merge reads partials from the fixed array
    big = workloads.Workload("noalloc_big", 6, 128, 1, [5000, 1, 3000, 640, 4097, 2000], "permuted", seed=21)
    print(f"\n[case] noalloc call 1: B={big.B} H=128 lens={list(big.lens)}", flush=True)
    _compare(big)
    # smaller, other kernel (16 heads); the array still holds call 1's partials
    small = workloads.Workload("noalloc_small", 3, 16, 2, [26, 130, 700], "permuted", seed=22)
    print(f"[case] noalloc call 2: B={small.B} H=16 Lq=2 lens={list(small.lens)}", flush=True)
    _compare(small)
