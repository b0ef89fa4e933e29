"""A decode step recorded as a HIP graph replays to the eager result.

The step (append, absorb, split attention, combine, up-projection) is captured
once; each replay follows eager work that overwrites the outputs, and every
replay must reproduce the eager step bit for bit (the kernels are
deterministic and the graph holds no memset nodes). The eager step itself is
checked against the fp64 oracle on two sequences.
"""

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


@pytest.mark.parametrize("H,lens,fp8,reps", [(128, [700, 33, 1500, 64], False, 1), (16, [300, 1, 129], False, 1),
                                            (16, [300, 1, 129], True, 1), (128, [700, 33, 1500, 64], False, 3)])
def test_graph_replays_match_eager(H, lens, fp8, reps):
    """reps > 1: several whole steps in one graph (the step is idempotent: it
    rewrites the same cache rows and recomputes the same outputs)."""
    w = workloads.Workload("graph", len(lens), H, 1, lens, "permuted", seed=11)
    print(f"\n[case] graph replay: H={H} lens={lens} fp8={fp8} steps per graph={reps}", flush=True)
    run = hz.DeviceRun(w, fp8=fp8)
    ckv, kpe, qpos, slot = run.new
    qn, qp = hz.to_dev(run.q_nope), hz.to_dev(run.q_pe)
    step = run.step
    step(ckv, kpe, qn, qp, qpos, slot)
    torch.cuda.synchronize()
    eager = {k: getattr(step, k).clone() for k in ("q", "o_lat", "lse", "o")}
    out = dict(q=hz.bits_of(eager["q"]), o_lat=hz.bits_of(eager["o_lat"]),
               lse=eager["lse"].cpu().numpy().astype(np.float64), o=hz.bits_of(eager["o"]))
    for b in (0, len(lens) - 1):
        hz.check_seq("eager", w, out, b, ref=hz.oracle_seq_fp8(w, b) if fp8 else None)
    g = step.capture(ckv, kpe, qn, qp, qpos, slot, reps=reps)
    torch.cuda.synchronize()
    for rep in range(3):
        for k in ("q", "o_lat", "o"):
            getattr(step, k).fill_(float("nan"))
        step.lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, ref in eager.items():
            got = getattr(step, k)
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref), (rep, k)
        print(f"  replay {rep}: bitwise equal to the eager step", flush=True)
