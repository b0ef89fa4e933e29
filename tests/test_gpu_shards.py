"""A sequence's keys split into shards, as a context-parallel deployment
would split them over GPUs: each shard is attended to on its own (the same
mla_decode_attn call, the shard's slice of the block table, the full
sequence's query), and the shards' (o_lat, lse) pairs merge into the whole
sequence's attention with the log-sum-exp rule of the oracle's partial merge
(softmax over a union of disjoint key sets). Checked against the unsplit call
and the fp64 oracle, at the 128-head 16k shape split eight ways (2,048 keys
per shard, one GPU's share)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import mla as orc
from tests import harness as hz

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.mark.parametrize("shards", [8, 3])
def test_sharded_keys_merge_to_the_whole_sequence(shards):
    from mla_latent_cache_append_amd import native as nat
    w = workloads.make("v3_b32_h128_l16384", seed=0, B=1)
    L, H = int(w.lens[0]), w.H
    blocks = L // 64
    _say(f"one 16k sequence at 128 heads in {shards} key shards")
    run = hz.DeviceRun(w)
    full = run.run()
    # shard g takes whole 64-token blocks [cuts[g], cuts[g+1]) of the sequence's block table
    cuts = np.linspace(0, blocks, shards + 1).round().astype(int)
    per = np.diff(cuts)
    bt = np.zeros((shards, int(per.max())), np.int32)
    for g in range(shards):
        bt[g, :per[g]] = w.block_table[0, cuts[g]:cuts[g + 1]]
    dev = torch.device("cuda")
    lens = torch.from_numpy((per * 64).astype(np.int32)).to(dev)
    q = run.step.q.repeat(shards, 1, 1).contiguous()          # the full sequence's query in every shard
    o_lat = torch.empty(shards, H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(shards, H, dtype=torch.float32, device=dev)
    dims = nat.mla_dims_default(H)
    ws = torch.empty(nat.mla_decode_workspace_size(dims, shards, 1), dtype=torch.uint8, device=dev)
    nat.mla_decode_attn(dims, q, run.pool, torch.from_numpy(bt).to(dev), lens, 1, o_lat, lse, ws)
    torch.cuda.synchronize()
    o_g = orc.bf16_bits_to_f64(hz.bits_of(o_lat))
    lse_g = lse.cpu().numpy().astype(np.float64)
    # a normalised partial (o_g, lse_g) is (m, l, acc) = (lse_g, 1, o_g)
    o_m, lse_m = orc.merge_partials([(lse_g[g], np.ones(H), o_g[g]) for g in range(shards)])
    # against the unsplit call on the same cache and query
    hz.assert_parity("merged vs unsplit o_lat", o_m, orc.bf16_bits_to_f64(full["o_lat"][0]))
    hz.assert_parity("merged vs unsplit lse", lse_m, full["lse"][0], max_rel=2e-2, mean_rel=5e-3)
    # against the oracle
    ref = hz.oracle_queries(w, 0, [0])
    hz.assert_parity("merged vs oracle o_lat", o_m[None], ref["o_lat"])
    hz.assert_parity("merged vs oracle lse", lse_m[None], ref["lse"], max_rel=2e-2, mean_rel=5e-3)
