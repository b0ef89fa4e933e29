"""Benchmark one absorbed-MLA decode step on one MI355X.

A step is the whole hot path for one batch: mla_cache_append (the B*Lq new
tokens) -> mla_absorb_q -> mla_decode_attn (split + combine) -> mla_out_up,
with every input already resident in HBM; the timed (captured) step runs the
first two as one launch (mla_append_absorb). The default workload is the
128-head, 16k-context decode (B=32, H=128, L=16384, Lq=1, block tables
randomly permuted over the pool).

Prints one JSON line: throughput (tokens/s) over HIP-graph replays of the
whole step, per-call times from eager steps with HIP events around each call
(median, p10, p90), the attention call's roofline (algorithmic bytes / its
steady-state duration, from replays of a HIP graph of 20 back-to-back calls,
vs 8 TB/s HBM and 2.5 PFLOP/s bf16), the same call against
what this box achieves on a plain stream read and on a loop of bf16 MFMAs,
the call with caches flushed before every step (a 1 GiB read evicts L2 and
the 256 MiB MALL), and the fp64 oracle timed on the host cores on a bounded
sample.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
ROW_BYTES = 576 * 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--cold-steps", type=int, default=20, help="steps timed after a cache flush each")
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="v3_b32_h128_l16384")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cache", choices=("bf16", "fp8", "kvpe"), default="bf16",
                    help="latent cache: the paged pool of bf16 rows, the paged pool of E4M3 codes with one "
                         "fp32 scale per token, or the two-buffer bf16 layout kv_cache [B, max_seq, 512] + "
                         "pe_cache [B, max_seq, 64]")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layer", action="store_true",
                    help="also time the whole layer: the projections around the step (synthetic weights) "
                         "and the residual output projection, eager per call and as one HIP graph")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device read (a sum) and a 1 GiB device write (a fill), "
                         "the calibration of the traffic counters")
    ap.add_argument("--crossover", action="store_true",
                    help="instead of the decode step: time a causal prefill chunk of Lq tokens per sequence "
                         "(B=4, 128 heads, 16,384 cached tokens) in the absorbed form (absorb_q + attention + "
                         "out_up) and in the expanded form (mla_prefill_expanded) for several Lq, one JSON line")
    ap.add_argument("--cross-lq", type=int, nargs="+", default=[32, 64, 128, 256, 512, 1024, 2048],
                    help="chunk sizes (query tokens per sequence) that --crossover times")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="parse two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this bench "
                         "with --copy-calib into profiles/traffic_<cache>_<workload>.json, then exit")
    return ap.parse_args()


COPY_BYTES = 1 << 30
ATTN_GRAPH_CALLS = 20


def traffic_from(fetch_dir: str, write_dir: str, workload: str) -> dict:
    """HBM bytes per mla_decode_attn launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the counter reads for a plain kernel of known
    traffic: a sum over COPY_BYTES (reads them) for FETCH_SIZE, a fill of
    COPY_BYTES (writes them) for WRITE_SIZE."""
    import csv
    import glob

    def per_kernel(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        acc = {}
        last_attn = -1
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            key = ("split" if any(k in name for k in ("attn_own", "attn_rows", "attn_cols")) else
                   "combine" if "attn_combine" in name else
                   "read" if "reduce_kernel" in name else
                   "write" if "FillFunctor" in name else
                   "copy" if "copyBuffer" in name else None)
            if key:
                did = int(row["Dispatch_Id"])
                if key in ("split", "combine"):
                    last_attn = max(last_attn, did)
                acc.setdefault(key, []).append((did, float(row["Counter_Value"]) * 1024.0))
        # calibration kernels run after the last attention call (earlier fills, such as
        # the probe buffer's, have other sizes); the largest of those dispatches, since
        # a reduction may add a small second pass
        return {k: (max(x for d, x in v if d > last_attn) if k in ("read", "write", "copy")
                    else sum(x for _, x in v) / len(v)) for k, v in acc.items()}
    fe, wr = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    # scale from a plain device-to-device copy of COPY_BYTES (reads and writes them);
    # the sum and the fill are kept in raw_kib as a cross-check
    f_scale, w_scale = COPY_BYTES / fe["copy"], COPY_BYTES / wr["copy"]
    fetch = (fe["split"] + fe.get("combine", 0.0)) * f_scale
    write = (wr["split"] + wr.get("combine", 0.0)) * w_scale
    return {"workload": workload, "kernel_source_hash": kernel_hash(),
            "bytes_per_launch": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
            "fetch_scale": f_scale, "write_scale": w_scale,
            "raw_kib": {"fetch": fe, "write": wr}}


def achievable_peaks(torch, dev) -> dict:
    """What this machine reaches with the probes of libmla_probe.so: a plain
    stream read of 2 GiB (16-byte loads, eight in flight per thread, 2048
    workgroups) and a loop of back-to-back bf16 32x32x16 MFMAs on every SIMD;
    median of 10 and of 5 launches, HIP events. The practical ceilings next to
    the datasheet peaks."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(__file__)), "mla_latent_cache_append_amd",
                                   "libmla_probe.so"))
    lib.mla_probe_stream_read.restype = ctypes.c_int
    lib.mla_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.mla_probe_mfma.restype = ctypes.c_int
    lib.mla_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 2 * COPY_BYTES
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    out = torch.empty(2048 * 256 * 4, dtype=torch.float32, device=dev)

    def timed(fn, reps, skip):
        ts = []
        for i in range(reps + skip):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            assert fn() == 0
            e1.record()
            e1.synchronize()
            if i >= skip:
                ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    t_read = timed(lambda: lib.mla_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                                     ctypes.c_void_p(out.data_ptr()), stream), 10, 3)
    waves4, iters = 1024, 2000
    t_mfma = timed(lambda: lib.mla_probe_mfma(waves4, iters, ctypes.c_void_p(out.data_ptr()), stream), 5, 2)
    del buf, out
    return {"hbm_read_GBps": nbytes / t_read / 1e9,
            "hbm_read_probe": "stream read of 2 GiB, 16-byte loads, median of 10",
            "mfma_bf16_TFLOPs": waves4 * 4 * 4 * iters * 32768 / t_mfma / 1e12,
            "mfma_probe": "back-to-back v_mfma_f32_32x32x16_bf16, 4 chains per wave, 16 waves per CU, median of 5"}


def _capture_graph(torch, fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def layer_timing(torch, nat, workloads, w, step, args, to_dev, qpos, slots) -> dict:
    """The step wrapped in its layer: c_kv = Wdkv h, k_pe = Wkr h, qz = Wdq h,
    q_nope = Wuq qz, q_pe = Wqr qz, the decode step, h_out = h + Wo o. Model
    widths: d_model 2048 at 16 heads (V2-Lite), 7168 at 128 heads (V3); query
    latent 1536. Weights N(0, 1/in), hidden states N(0, 1). Per call: HIP
    events around replays of a graph of 20 calls; the whole layer as replays
    of HIP graphs of ten layers (and of one layer)."""
    from mla_latent_cache_append_amd.step import LayerStep
    d_model = 2048 if w.H <= 16 else 7168
    d_cq = 1536
    lw = {k: to_dev(v) for k, v in workloads.layer_weights(args.seed, 0, w.H, d_model, d_cq).items()}
    ls = LayerStep(step, **lw)
    h = to_dev(workloads.hidden_states(args.seed, w.N, d_model))
    N = w.N
    calls = {
        "w_dkv": lambda: nat.mla_linear(h, ls.w_dkv, ls.c_kv, workspace=ls.ws["dkv"]),
        "w_kr": lambda: nat.mla_linear(h, ls.w_kr, ls.k_pe, workspace=ls.ws["kr"]),
        "w_dq": lambda: nat.mla_linear(h, ls.w_dq, ls.qz, workspace=ls.ws["dq"]),
        "w_uq": lambda: nat.mla_linear(ls.qz, ls.w_uq, ls.q_nope.view(N, -1), workspace=ls.ws["uq"]),
        "w_qr": lambda: nat.mla_linear(ls.qz, ls.w_qr, ls.q_pe.view(N, -1), workspace=ls.ws["qr"]),
        "w_o": lambda: nat.mla_linear(step.o.view(N, -1), ls.w_o, ls.out, residual=h, workspace=ls.ws["o"]),
    }
    ls(h, qpos, slots)
    torch.cuda.synchronize()
    # per call: a HIP graph of 20 back-to-back calls, replayed, so that the
    # host's per-call overhead does not enter the GPU time
    per = {}
    for name, fn in calls.items():
        def twenty(fn=fn):
            for _ in range(20):
                fn()
        gc = _capture_graph(torch, twenty)
        for _ in range(2):
            gc.replay()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            gc.replay()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / 20)
        per[name] = float(np.median(ts))
    def layer_graph_us(per_graph):
        g = ls.capture(h, qpos, slots, reps=per_graph)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(args.steps // 4, 10)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * per_graph)

    # ten layers per graph, as a model's stack of layers is captured (the
    # graph launch amortised); one layer per graph beside it
    layer_us = layer_graph_us(10)
    layer_us_one = layer_graph_us(1)
    wbytes = {k: int(v.numel()) * 2 for k, v in lw.items()}
    io = lambda k: N * (lw[k].shape[0] + lw[k].shape[1]) * 2      # activations in and out
    gbps = {k: (wbytes[k] + io(k)) / (per[k] * 1e-6) / 1e9 for k in calls}
    return {"d_model": d_model, "d_cq": d_cq, "call_us_median": per,
            "weight_bytes": wbytes, "GBps": gbps,
            "w_o_frac_of_8TBps": gbps["w_o"] / HBM_PEAK_GBPS,
            "layer_us_graph": layer_us, "layers_per_graph": 10, "layer_us_one_layer_graphs": layer_us_one,
            "layer_tokens_per_s": N / (layer_us * 1e-6)}


def algorithmic(w, fp8: bool = False):
    """Algorithmic bytes and flops of one attention call (and of one step).
    A cache row is 1,152 bytes in bf16, 576 code bytes + a 4-byte scale in FP8."""
    L = w.lens.astype(np.int64)
    rows = w.Lq * w.H
    cache = int(L.sum()) * (576 + 4 if fp8 else ROW_BYTES)
    q_bytes = w.N * w.H * 576 * 2
    olat_bytes = w.N * w.H * 512 * 2 + w.N * w.H * 4
    attn_bytes = cache + q_bytes + olat_bytes
    attn_flops = int((2 * rows * L * (576 + 512)).sum())
    return dict(cache_bytes=cache, attn_bytes=attn_bytes, attn_flops=attn_flops)


def cpu_baseline(w, budget_s: float) -> dict:
    """The fp64 oracle's absorbed path, as it stands, on whole sequences of the
    same workload until about ``budget_s`` seconds of CPU work are done."""
    from oracle import mla as orc
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in info}))
    except Exception:  # threadpoolctl missing: report the affinity set
        threads, blas = len(os.sched_getaffinity(0)), "unknown"
    f = orc.bf16_bits_to_f64
    q_nope, q_pe = w.queries(0)
    wuk, wuv = (f(x) for x in w.weights())
    # whole sequences, cycling over the first few (inputs generated untimed)
    cached = {}
    done_tok, spent, calls = 0, 0.0, 0
    while spent < budget_s:
        b = calls % min(w.B, 4)
        if b not in cached:
            ckv, kpe = w.seq_cache(b)
            sl = slice(b * w.Lq, (b + 1) * w.Lq)
            cached[b] = (f(q_nope[sl]), f(q_pe[sl]), f(ckv), f(kpe), wuk, wuv)
        t0 = time.perf_counter()
        orc.absorbed_decode(*cached[b])
        spent += time.perf_counter() - t0
        done_tok += w.Lq
        calls += 1
    return {"value": done_tok / spent, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{calls} single-sequence decodes (sequences 0..{min(w.B, 4) - 1} of {w.name}, "
                      f"L={int(w.lens[0])}, H={w.H}; fp64 NumPy absorbed path, BLAS {blas}), {spent:.1f} s"}


def crossover(args) -> None:
    """Absorbed against expanded form on one cache: B sequences of HIST
    cached tokens plus a chunk of Lq new ones (already in the cache), every
    query token attending causally. Each form runs as a HIP graph of
    CROSS_CALLS calls when it captures (else eager calls), median of
    CROSS_REPS timed replays; flops are the algorithm's for each form."""
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import workloads
    from mla_latent_cache_append_amd import native as nat
    from mla_latent_cache_append_amd.step import DecodeStep

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    B, H, HIST = 4, 128, 16384
    lqs = tuple(sorted(set(args.cross_lq)))
    if not lqs or lqs[0] < 1 or lqs[-1] > 65536:
        print("--cross-lq takes chunk sizes from 1 to 65536", file=sys.stderr)
        sys.exit(2)
    lmax = HIST + max(lqs)
    dev = torch.device("cuda")
    w = workloads.Workload("crossover_b4_h128", B, H, max(lqs), [lmax] * B, "permuted", args.seed)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    wuk, wuv = (to_dev(x) for x in w.weights())
    pool = torch.empty((w.num_blocks, 64, 576), dtype=torch.bfloat16, device=dev)
    block_table = torch.from_numpy(w.block_table).to(dev)
    dims = nat.mla_dims_default(H)
    for b in range(B):   # every token of the longest chunk in the cache
        ckv, kpe = w.seq_cache(b)
        for s0 in range(0, lmax, 65536):
            p = np.arange(s0, min(lmax, s0 + 65536))
            nat.mla_cache_append(dims, to_dev(ckv[p]), to_dev(kpe[p]), torch.from_numpy(p.astype(np.int32)).to(dev),
                                 torch.from_numpy(w.slots(b, p)).to(dev), pool)
        print(f"[bench] filled sequence {b}/{B}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        mode = "graph"
        try:
            g = _capture_graph(torch, lambda: [fn() for _ in range(CROSS_CALLS)])
            run = g.replay
        except Exception:   # a library call that does not capture: eager calls
            mode = "eager"
            torch.cuda.synchronize()

            def run():
                for _ in range(CROSS_CALLS):
                    fn()
        run()
        us = []
        for _ in range(CROSS_REPS):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            e1.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3 / CROSS_CALLS)
        return float(np.median(us)), mode

    series = []
    for lq in lqs:
        L = HIST + lq
        N = B * lq
        seq_lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        qn = to_dev(workloads.normal_bf16((args.seed, workloads.TAG_QNOPE, lq), (N, H, 128)))
        qp = to_dev(workloads.normal_bf16((args.seed, workloads.TAG_QPE, lq), (N, H, 64)))
        pos = torch.from_numpy(np.tile(np.arange(HIST, L, dtype=np.int32), B)).to(dev)
        q = torch.empty((N, H, 576), dtype=torch.bfloat16, device=dev)
        o_lat = torch.empty((N, H, 512), dtype=torch.bfloat16, device=dev)
        o_a = torch.empty((N, H, 128), dtype=torch.bfloat16, device=dev)
        o_x = torch.empty((N, H, 128), dtype=torch.bfloat16, device=dev)
        ws_a = torch.empty(nat.mla_decode_workspace_size(dims, B, lq), dtype=torch.uint8, device=dev)
        ws_x = torch.empty(nat.mla_prefill_expanded_workspace_size(dims, B, L), dtype=torch.uint8, device=dev)

        def absorbed():
            nat.mla_absorb_q(dims, qn, qp, pos, wuk, q)
            nat.mla_decode_attn(dims, q, pool, block_table, seq_lens, lq, o_lat, workspace=ws_a)
            nat.mla_out_up(dims, o_lat, wuv, o_a)

        def expanded():
            nat.mla_prefill_expanded(dims, qn, qp, pos, pool, block_table, seq_lens, lq, L, wuk, wuv, o_x,
                                     workspace=ws_x)

        a_us, a_mode = timed(absorbed)
        x_us, x_mode = timed(expanded)
        torch.cuda.synchronize()
        # the two forms' outputs on the same inputs agree to bf16 rounding
        diff = (o_a.float() - o_x.float()).abs().mean().item() / max(o_a.float().abs().mean().item(), 1e-30)
        pairs = B * (lq * HIST + lq * (lq + 1) // 2)          # (query, visible key) pairs
        f_a = 2 * H * pairs * (576 + 512) + 2 * 2 * N * H * 128 * 512
        f_x = 2 * B * L * H * 256 * 512 + 2 * H * pairs * (192 + 128)
        series.append(dict(Lq=lq, keys=L, absorbed_us=a_us, expanded_us=x_us, speedup=a_us / x_us,
                           absorbed_tflops=f_a / a_us / 1e6, expanded_tflops=f_x / x_us / 1e6,
                           absorbed_gflop=f_a / 1e9, expanded_gflop=f_x / 1e9, timing=[a_mode, x_mode],
                           mean_rel_diff=diff))
        print(f"[bench] Lq={lq}: absorbed {a_us:.1f} us, expanded {x_us:.1f} us", file=sys.stderr, flush=True)
        del ws_x, ws_a
        torch.cuda.empty_cache()
    cross = None
    for s0, s1 in zip(series, series[1:]):
        if s0["speedup"] < 1.0 <= s1["speedup"]:   # interpolate in log Lq
            t = (1.0 - s0["speedup"]) / (s1["speedup"] - s0["speedup"])
            cross = float(np.exp(np.log(s0["Lq"]) + t * (np.log(s1["Lq"]) - np.log(s0["Lq"]))))
    print(json.dumps({"metric": "prefill chunk time, absorbed vs expanded form", "unit": "us",
                      "config": {"workload": "crossover_b4_h128", "B": B, "H": H, "cached_tokens": HIST,
                                 "Lq": list(lqs)},
                      "series": series, "crossover_Lq": cross, "data": "synthetic"}), flush=True)


CROSS_CALLS = 5
CROSS_REPS = 5


def main():
    args = parse()
    if args.crossover:
        crossover(args)
        return
    if args.traffic_from:
        t = traffic_from(args.traffic_from[0], args.traffic_from[1], args.workload)
        t["cache"] = args.cache
        out = traffic_path(args.cache, args.workload)
        json.dump(t, open(out, "w"), indent=1)
        print(json.dumps(t))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import workloads
    from mla_latent_cache_append_amd import native as nat
    from mla_latent_cache_append_amd.step import DecodeStep

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    nat.lib()
    dev = torch.device("cuda")
    w = workloads.make(args.workload, seed=args.seed)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- setup (untimed): weights, paged pool filled through mla_cache_append
    wuk, wuv = w.weights()
    fp8 = args.cache == "fp8"
    kvpe = args.cache == "kvpe"
    pe_cache = None
    if kvpe:
        # two-buffer layout: room for the longest sequence in every row of the batch
        max_seq = int(w.lens.max())
        pool = torch.empty((w.B, max_seq, 512), dtype=torch.bfloat16, device=dev)
        pe_cache = torch.empty((w.B, max_seq, 64), dtype=torch.bfloat16, device=dev)
    else:
        pool = torch.empty((w.num_blocks, 64, 576), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    pool_scale = torch.empty((w.num_blocks, 64), dtype=torch.float32, device=dev) if fp8 else None
    block_table = torch.from_numpy(w.block_table).to(dev)
    seq_lens = torch.from_numpy(w.lens.astype(np.int32)).to(dev)
    step = DecodeStep(w.H, w.B, w.Lq, pool, block_table, seq_lens, to_dev(wuk), to_dev(wuv), pool_scale=pool_scale,
                      pe_cache=pe_cache)

    def slots_of(b, p):
        """Where positions p of sequence b go: pool slots, or (two-buffer
        layout) the sequence index of each token."""
        p = np.asarray(p)
        return np.full(p.shape, b, np.int32) if kvpe else w.slots(b, p)

    new_ckv = np.zeros((w.N, 512), np.uint16)
    new_kpe = np.zeros((w.N, 64), np.uint16)
    new_slot = np.zeros(w.N, np.int32 if kvpe else np.int64)
    fill_events = 0.0
    t_fill = time.perf_counter()
    for b in range(w.B):
        L = int(w.lens[b])
        ckv, kpe = w.seq_cache(b)
        hist = L - w.Lq
        for s0 in range(0, hist, 65536):
            s1 = min(hist, s0 + 65536)
            p = np.arange(s0, s1)
            c, k = to_dev(ckv[s0:s1]), to_dev(kpe[s0:s1])
            pos = torch.from_numpy(p.astype(np.int32)).to(dev)
            sl = torch.from_numpy(slots_of(b, p)).to(dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step.append(c, k, pos, sl)
            e1.record()
            e1.synchronize()
            fill_events += e0.elapsed_time(e1)
        for i in range(w.Lq):
            p = L - w.Lq + i
            n = b * w.Lq + i
            new_ckv[n], new_kpe[n], new_slot[n] = ckv[p], kpe[p], slots_of(b, [p])[0]
        if b % 8 == 0:
            print(f"[bench] filled sequence {b}/{w.B}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_fill = time.perf_counter() - t_fill
    q_nope, q_pe = w.queries(0)
    args_step = (to_dev(new_ckv), to_dev(new_kpe), to_dev(q_nope), to_dev(q_pe),
                 torch.from_numpy(w.query_positions()).to(dev), torch.from_numpy(new_slot).to(dev))
    ckv_n, kpe_n, qn, qp, qpos, slot_n = args_step

    # ---- timed steps; HIP events around every call on the stream the kernels run on
    names = ("append", "absorb_q", "decode_attn", "out_up")

    def one_step(ev=None):
        if ev is not None:
            ev[0].record()
        step.append(ckv_n, kpe_n, qpos, slot_n)
        if ev is not None:
            ev[1].record()
        nat.mla_absorb_q(step.dims, qn, qp, qpos, step.w_uk, step.q)
        if ev is not None:
            ev[2].record()
        step.decode_attn()
        if ev is not None:
            ev[3].record()
        nat.mla_out_up(step.dims, step.o_lat, step.w_uv, step.o)
        if ev is not None:
            ev[4].record()

    # eager steps: HIP events around every call give the per-call breakdown
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(evs[i])
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t0
    per = {n: [] for n in names}
    for ev in evs:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)   # us
    step_us = [evs[i][0].elapsed_time(evs[i][4]) * 1e3 for i in range(args.steps)]
    med = {n: float(np.median(v)) for n, v in per.items()}
    pct = {n: {"p10": float(np.percentile(v, 10)), "p90": float(np.percentile(v, 90))} for n, v in per.items()}

    # the step's first two calls fused into one launch (what the captured step
    # runs): 20 launches recorded as one HIP graph (so host overhead stays out),
    # replayed five times between two events
    fused_us = None
    if not kvpe:   # the two-buffer step runs append and absorb as two launches
        fused_graph = _capture_graph(torch, lambda: [nat.mla_append_absorb(
            step.dims, ckv_n, kpe_n, slot_n, step.pool, qn, qp, qpos, step.w_uk, step.q,
            pool_scale=step.pool_scale) for _ in range(20)])
        fused = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fused_graph.replay()
            e1.record()
            e1.synchronize()
            fused.append(e0.elapsed_time(e1) * 1e3 / 20)
        fused_us = float(np.median(fused))
        del fused_graph

    # the attention call in steady state: 20 back-to-back calls recorded as
    # one HIP graph, replayed; per call = replay time / 20. No host work sits
    # between the calls, so this is the call's own GPU time (the roofline is
    # taken on it). The eager per-call events above include any wait of the
    # GPU for the host inside the event window.
    attn_graph = _capture_graph(torch, lambda: [step.decode_attn() for _ in range(ATTN_GRAPH_CALLS)])
    for _ in range(3):
        attn_graph.replay()
    attn_graph_us = []
    for _ in range(max(10, args.steps // 10)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        attn_graph.replay()
        e1.record()
        e1.synchronize()
        attn_graph_us.append(e0.elapsed_time(e1) * 1e3 / ATTN_GRAPH_CALLS)
    del attn_graph

    # cold steps: a 1 GiB read between steps evicts L2 and MALL (a read
    # leaves no dirty lines to write back during the step), so every step
    # reads the cache and the weights from HBM; events around each call
    flush = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    cold = {n: [] for n in names}
    for i in range(args.cold_steps):
        flush.sum()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        one_step(ev)
        torch.cuda.synchronize()
        for j, n in enumerate(names):
            cold[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)
    del flush

    # graph steps: S whole steps recorded as one HIP graph and replayed, the
    # way a decode loop captured ahead of time issues them; exactly args.steps
    # steps are timed (S divides it). This is the timed throughput. One step
    # per graph is timed as well, for reference.
    spg = next(k for k in (10, 8, 5, 4, 2, 1) if args.steps % k == 0)

    def time_graph(reps):
        graph = step.capture(*[args_step[i] for i in (0, 1, 2, 3, 4, 5)], reps=reps)
        for _ in range(max(1, args.warmup // reps)):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g0.record()
        for _ in range(args.steps // reps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del graph
        return max(wall * 1e3, g0.elapsed_time(g1)) / args.steps

    ms_per_step_1 = time_graph(1)
    ms_per_step = time_graph(spg)

    layer = layer_timing(torch, nat, workloads, w, step, args, to_dev, qpos, slot_n) if args.layer else None
    ach = achievable_peaks(torch, dev)
    alg = algorithmic(w, fp8)
    attn_us = float(np.median(attn_graph_us))
    attn_s = attn_us * 1e-6
    achieved_gbps = alg["attn_bytes"] / attn_s / 1e9
    tflops = alg["attn_flops"] / attn_s / 1e12
    traffic = None
    tf = traffic_path(args.cache, w.name)
    if os.path.exists(tf):
        try:
            t = json.load(open(tf))
            if (t.get("workload") == w.name and t.get("kernel_source_hash") == kernel_hash()
                    and t.get("cache", "bf16") == args.cache):
                traffic = t.get("bytes_per_launch")
        except Exception:
            traffic = None

    # the bound is whichever floor is higher at the datasheet peaks: the bytes
    # at 8 TB/s or the flops at 2.5 PFLOP/s (many query rows per sequence
    # turn the call into a contraction-bound one)
    if alg["attn_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12) > alg["attn_bytes"] / (HBM_PEAK_GBPS * 1e9):
        roof = {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / MFMA_BF16_PEAK_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": achieved_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved_gbps / HBM_PEAK_GBPS}
    out = {
        "metric": "absorbed-MLA decode tokens/s + latent-cache GB/s & MFMA TFLOP/s (% roofline)",
        "value": w.N / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Lq": w.Lq,
                   "keys_per_seq": int(w.lens.max()) if w.lens.min() == w.lens.max() else "ragged",
                   "total_keys": int(w.lens.sum()), "block_table": w.table_kind, "seed": args.seed,
                   "cache": "fp8-e4m3 (per-token fp32 scale)" if fp8 else
                            "bf16 two-buffer kv_cache + pe_cache" if kvpe else "bf16"},
        "roofline": dict(roof, traffic=traffic,
                         kernel=("mla_decode_attn_fp8" if fp8 else "mla_decode_attn_kvpe" if kvpe else "mla_decode_attn")
                         + " call (split kernel + combine kernel)",
                         algorithmic_bytes_per_launch=alg["attn_bytes"],
                         algorithmic_flops_per_launch=alg["attn_flops"],
                         avg_launch_us=attn_us,
                         timing=f"median per call over replays of a HIP graph of {ATTN_GRAPH_CALLS} "
                                "back-to-back calls (HIP events on the stream the kernels run on)",
                         graph_call_us_p10_p90={"p10": float(np.percentile(attn_graph_us, 10)),
                                                "p90": float(np.percentile(attn_graph_us, 90))},
                         eager_call_us_median=med["decode_attn"],
                         eager_frac=alg["attn_bytes"] / (med["decode_attn"] * 1e-6) / 1e9 / HBM_PEAK_GBPS
                         if roof["bound"] == "hbm" else
                         alg["attn_flops"] / (med["decode_attn"] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS),
        "latent_cache_GBps": alg["cache_bytes"] / attn_s / 1e9,
        "mfma_TFLOPs": tflops,
        "mfma_frac": tflops / MFMA_BF16_PEAK_TFLOPS,
        "call_us_median": dict(med, append_absorb_fused=fused_us),
        "call_us_p10_p90": pct,
        "achievable": dict(ach, frac_hbm=achieved_gbps / ach["hbm_read_GBps"],
                           frac_mfma=tflops / ach["mfma_bf16_TFLOPs"]),
        "cold_cache": {"steps": args.cold_steps,
                       "call_us_median": {n: float(np.median(v)) for n, v in cold.items()},
                       "decode_attn_GBps": alg["attn_bytes"] / (float(np.median(cold["decode_attn"])) * 1e-6) / 1e9},
        "step_mode": f"hip_graph replays of {spg} whole steps per graph, append and absorb "
                     + ("as two launches" if kvpe else "fused in one launch")
                     + " (eager per-call events give call_us_median)",
        "steps_per_graph": spg,
        "ms_per_step_one_step_graphs": ms_per_step_1,
        "eager_ms_per_step": eager_wall * 1e3 / args.steps,
        "eager_step_us_median_events": float(np.median(step_us)),
        "fill": {"tokens": int(w.lens.sum()) - w.N, "append_kernel_s": fill_events * 1e-3,
                 "wall_s_incl_host_generation": t_fill},
    }
    if layer is not None:
        out["layer"] = layer
    if args.copy_calib:
        buf = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(buf)
        for _ in range(3):
            buf.sum()            # reads COPY_BYTES
            buf.fill_(1.0)       # writes COPY_BYTES
            dst.copy_(buf)       # reads and writes COPY_BYTES (device-to-device copy kernel)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def traffic_path(cache: str, workload: str) -> str:
    """Stored HBM traffic of the attention call for one cache format and workload."""
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"traffic_{cache}_{workload}.json")


def kernel_hash() -> str:
    """Hash of the attention kernel source, to tie stored counter data to it."""
    import hashlib
    p = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mla_latent_cache_append_amd", "csrc", "attn.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


if __name__ == "__main__":
    main()
