"""Host-side checks of the seeded input generator and the block tables."""

import numpy as np

import workloads


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-3], dtype=np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa wins (1.0)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2 ** -6 and back[3] == 1.0
    assert back[4] == -2.5
    assert abs(back[5] - 3.0e-3) <= 2 ** -8 * 3.0e-3      # half an ulp (2^-7 relative)


def test_streams_are_deterministic_and_keyed():
    w = workloads.make("v3_b32_h128_l16384", seed=3, B=3, L=100)
    a = w.seq_cache(1)
    b = w.seq_cache(1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(w.seq_cache(0)[0], a[0])
    # a shorter draw is a prefix of a longer one (same stream)
    assert np.array_equal(w.seq_cache(1, 40)[0], a[0][:40])


def test_block_tables_are_disjoint_and_cover_pool():
    for name in workloads.FULL_WORKLOADS:
        w = workloads.make(name, seed=0)
        used = []
        for b in range(w.B):
            n = -(-int(w.lens[b]) // 64)
            row = w.block_table[b]
            assert np.all(row[:n] >= 0) and np.all(row[n:] == -1)
            used.append(row[:n])
        used = np.concatenate(used)
        assert len(np.unique(used)) == len(used) == w.num_blocks
        assert used.min() == 0 and used.max() == w.num_blocks - 1


def test_ragged_lengths_in_range():
    w = workloads.make("ragged_b128_h128_l1to32768", seed=0)
    assert w.lens.min() >= 1 and w.lens.max() <= 32768
    assert abs(w.lens.mean() - 16384.5) < 3 * 32768 / np.sqrt(12 * 128)


def test_query_positions_and_slots():
    w = workloads.make("causal8_b16_h128_l65544", seed=0, B=2, L=100)
    qp = w.query_positions()
    assert list(qp[:8]) == list(range(92, 100))
    s = w.slots(1, np.arange(100))
    assert len(np.unique(s)) == 100
    assert np.all(s // 64 == np.repeat(w.block_table[1, :2], 64)[:100])


def test_context_share_workload_is_an_eighth_of_the_128_head_batch():
    """One GPU's share of the 128-head 16k batch when each sequence's keys are
    split over 8 GPUs: the same batch and heads, 2,048 keys per sequence, and
    a permuted block table that covers its pool."""
    full = workloads.make("v3_b32_h128_l16384", seed=0)
    share = workloads.make("v3share8_b32_h128_l2048", seed=0)
    assert (share.B, share.H, share.Lq) == (full.B, full.H, full.Lq)
    assert np.all(share.lens * 8 == full.lens)
    assert share.num_blocks * 8 == full.num_blocks
    used = share.block_table[share.block_table >= 0]
    assert sorted(used.tolist()) == list(range(share.num_blocks))


def test_prefill_chunk_workload_shape():
    w = workloads.make("chunk512_b4_h128_l16896", seed=0)
    assert (w.B, w.H, w.Lq, w.N) == (4, 128, 512, 2048)
    assert np.all(w.lens == 16896) and w.num_blocks == 4 * 264
    q = w.query_positions()
    assert q[0] == 16384 and q[511] == 16895 and q[512] == 16384


def test_query_subset_oracle_matches_whole_sequence():
    # the sampled check used at full size takes the oracle's steps on a
    # subset of query tokens; on a small case it must give the same rows
    from tests import harness as hz
    w = workloads.Workload("subset", 2, 16, 6, [6, 40], "permuted", seed=21)
    for b in (0, 1):
        full = hz.oracle_seq(w, b)
        idx = [0, 3, 5]
        part = hz.oracle_queries(w, b, idx)
        for k in ("q_lat", "q_r", "o_lat", "o"):
            np.testing.assert_allclose(part[k], full[k][idx], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(part["lse"], full["lse"][idx], rtol=1e-12, atol=1e-12)
