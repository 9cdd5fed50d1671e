#!/usr/bin/env python3
"""Benchmark of the sparse-MLA-over-NVFP4 hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--warm-s SECONDS] [--workload c3|c2] [--splits S] [--no-cpu-baseline]

One step = one decode step of the whole path for every request of the
workload: quantized write of each request's newest KV row, dedup compaction of
the requests' top-k lists, sparse MLA decode over the compacted lists
(per-split kernel), and the (o, lse) merge.  Inputs (4.6 GB pool, page table,
lists, queries) are resident in HBM before timing; 8 rotating list/query sets
keep the gathered rows from being served out of the 256 MB Infinity Cache.

Prints one JSON line: decode tokens/s (value), the roofline of the dominant
kernel (the per-split decode kernel, timed with HIP events on the stream it
runs on), prefill MFMA utilisation, and the CPU oracle on the host's cores
(the decode step above, then each other config's unit of work, with 1-thread
runs of the tiny decode and the write + compaction).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CPU_BASELINE_SECONDS = 6.0     # oracle decode steps timed; the other configs get shorter budgets
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, published
N_SETS = 8                     # rotating list/query sets
PROFILES = os.path.join(ROOT, "profiles")
WARM_S = 1.0                   # untimed run of the step (and of the prefill) before it is timed
SECTION_WARM_S = [0.3]         # the same before each shorter timed section (scaled by --warm-s)


def warm(fn, dev, seconds=WARM_S):
    """Repeat fn (untimed) for about `seconds`: the GPU raises its clock over
    the first seconds of sustained load (measured: the decode split kernel
    38.8 -> 34 us and the prefill 1.80 -> 1.51 ms over a few seconds), so a
    section is timed at the clock it runs at under steady load."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize(dev)


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3", choices=["c2", "c3"])
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's automatic choice")
    ap.add_argument("--prefill-iters", type=int, default=5)
    ap.add_argument("--warm-s", type=float, default=WARM_S,
                    help="seconds of untimed work before the timed steps and before the prefill timing (the GPU's "
                         "clock rises over the first seconds of load)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-write", action="store_true", help="skip the write + compaction measurement")
    ap.add_argument("--no-rope-free", action="store_true", help="skip the rope-free (288-byte row) decode measurement")
    ap.add_argument("--no-compact", action="store_true", help="skip the global compaction measurements")
    ap.add_argument("--no-c2", action="store_true",
                    help="skip the tiny (batch 1) and batch-8 (one GPU's head share) decode measurements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (a known-size kernel for counter calibration)")
    return ap.parse_args()


# ---------------------------------------------------------------- setup
def build_decode_workload(spec, dev, n_sets=N_SETS):
    """Device pool (all slots quantized by kv4_quant_write from device-drawn
    fp32 rows), page table, rotating lists / queries / new rows."""
    import torch
    import bit_kv_cache_kv4_amd as kv4
    import workloads as W

    pool = torch.empty((spec.n_slots, 352), dtype=torch.uint8, device=dev)
    n_chunks = -(-spec.n_slots // W.KV_CHUNK)
    for c in range(n_chunks):
        x = W.kv_chunk_device(spec, c, dev)
        lo = c * W.KV_CHUNK
        slots = torch.arange(lo, lo + x.shape[0], dtype=torch.int32, device=dev)
        kv4.quant_write(x, slots, pool)
        del x
    pt_h = W.page_table(spec)
    sets = []
    for i in range(n_sets):
        s = W.scaled(spec, seed=spec.seed + 17 * i) if i else spec
        topk_h = W.topk_lists(s)
        q = W.queries(s)
        g = np.random.default_rng([spec.seed, 99, i])
        new_rows = g.standard_normal((spec.n_req, 576), dtype=np.float32)
        sets.append(dict(topk_h=topk_h, topk=torch.from_numpy(topk_h).to(dev), q=q.to(dev),
                         new_rows=torch.from_numpy(new_rows).to(dev)))
    last = spec.ctx - 1
    new_slots = (pt_h[:, last >> 6].astype(np.int64) * 64 + (last & 63)).astype(np.int32)
    torch.cuda.synchronize(dev)
    return dict(pool=pool, pt_h=pt_h, pt=torch.from_numpy(pt_h).to(dev), sets=sets,
                new_slots=torch.from_numpy(new_slots).to(dev), new_slots_h=new_slots)


def gathered_rows_host(spec, pt_h, topk_h, dev):
    """fp32 originals of the rows the lists select, regenerated from the same
    device draws (for the oracle); returns (unique slots, rows [n, 576])."""
    import torch
    import workloads as W
    slots = (pt_h[np.arange(topk_h.shape[0])[:, None], topk_h >> 6].astype(np.int64) * 64 + (topk_h & 63))
    uniq = np.unique(slots)
    rows = np.empty((uniq.size, 576), dtype=np.float32)
    chunk_of = uniq // W.KV_CHUNK
    for c in np.unique(chunk_of):
        sel = np.nonzero(chunk_of == c)[0]
        x = W.kv_chunk_device(spec, int(c), dev)
        idx = torch.from_numpy(uniq[sel] - int(c) * W.KV_CHUNK).to(dev)
        rows[sel] = x.index_select(0, idx).cpu().numpy()
        del x
    return uniq, rows, slots


# ---------------------------------------------------------- measurement
def algorithmic_decode_bytes(n_req, n_heads, k, q_bytes=2, row_bytes=352, dim=576):
    """Per launch: each request's k selected rows (row_bytes: 352, or 288
    rope-free), k list entries and k page-table entries (4 B each), its
    queries (n_heads x dim x q_bytes) and its output (n_heads x 512 fp32 +
    n_heads lse)."""
    per_req = k * row_bytes + k * 4 * 2 + n_heads * dim * q_bytes + n_heads * (512 + 1) * 4
    return per_req * n_req


def prefill_flops(n_rows, n_heads, k):
    """Scores over 576 dims and P.V over 512 dims, 2 flops per multiply-add."""
    return 2.0 * n_rows * n_heads * k * (576 + 512)


ATTN_SOURCES = ("kv4_attn.hip", "kv4_attn.h", "kv4_device.h")   # what the attention kernel is built from


def kernel_source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_kv_cache_kv4_amd", "csrc")
    for name in ATTN_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3
    counter summaries, or None if absent or taken on other kernel sources."""
    path = os.path.join(PROFILES, "sparse_mla_decode_%s_traffic.json" % workload)
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_digest") != kernel_source_digest():
        return None
    return d.get("hbm_bytes_per_launch")


def _time_oracle(fn, budget_s, min_reps=1):
    """Repeat fn until budget_s seconds of it are timed (at least min_reps
    runs); returns (runs, seconds)."""
    reps, dt = 0, 0.0
    while reps < min_reps or dt < budget_s:
        t0 = time.perf_counter()
        fn()
        dt += time.perf_counter() - t0
        reps += 1
    return reps, dt


def _decode_inputs_host(spec, dev):
    """Host inputs of one decode call of a DecodeSpec for the oracle: fp32
    queries, the lists rewritten to index a pool of the rows they select
    (quantized by the oracle from the same fp32 originals as the device pool)."""
    import oracle
    import workloads as W
    pt_h, topk_h = W.page_table(spec), W.topk_lists(spec)
    uniq, rows, slots = gathered_rows_host(spec, pt_h, topk_h, dev)
    pool_h = np.zeros((uniq.size, 352), dtype=np.uint8)
    oracle.quant_write(rows, np.arange(uniq.size, dtype=np.int32), pool_h)
    compact = np.searchsorted(uniq, slots).astype(np.int32)
    q = W.queries(spec).float().numpy()
    return q, pool_h, compact


def run_cpu_baseline(spec, wl, dev):
    """The oracle, as it is, on the host cores: the same decode step (write
    the requests' new rows, dedup their lists, attention) for every request
    of one rotating set, over a host pool of the selected rows that the
    oracle quantized itself (untimed setup); then the other configs' units of
    work (per_config), with 1-thread runs of C1 and C4."""
    import oracle
    import workloads as W
    st = wl["sets"][0]
    uniq, rows, slots = gathered_rows_host(spec, wl["pt_h"], st["topk_h"], dev)
    pool_h = np.zeros((uniq.size + spec.n_req, 352), dtype=np.uint8)
    oracle.quant_write(rows, np.arange(uniq.size, dtype=np.int32), pool_h)
    compact = np.searchsorted(uniq, slots).astype(np.int32)
    q = st["q"].float().cpu().numpy()
    new_rows = st["new_rows"].cpu().numpy()
    new_slots = np.arange(uniq.size, uniq.size + spec.n_req, dtype=np.int32)
    threads = oracle.num_threads()
    affinity = len(os.sched_getaffinity(0))

    def step():
        oracle.quant_write(new_rows, new_slots, pool_h)
        lists, _ = oracle.dedup_compact(compact)
        oracle.sparse_mla(q, pool_h, lists, spec.sm_scale)

    steps, dt = _time_oracle(step, CPU_BASELINE_SECONDS)
    res = {"value": spec.n_req * steps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "affinity_cores": affinity,
           "sample": "%d repetitions of one full decode step of %s: %d requests (write %d new rows, dedup %d lists "
                     "of %d, attention %d heads x %d keys each), host pool of the %d selected rows; %.2f s wall on %d "
                     "threads" % (steps, spec.name, spec.n_req, spec.n_req, spec.n_req, spec.k, spec.n_heads, spec.k,
                                  uniq.size, dt, threads)}
    print("[bench] cpu baseline: other configs", file=sys.stderr, flush=True)
    res["per_config"] = run_cpu_baseline_configs(dev, threads)
    return res


def run_cpu_baseline_configs(dev, threads):
    """Oracle time per unit of each config's GPU measurement: a decode call
    for C1 and C2 (attention of every request), the write of 16,384 tokens and
    the dedup of 4096 lists for C4, and prefill rows for C5 (a stated subset of
    the 4096 rows, extrapolated).  C1 and C4 also on one thread."""
    import oracle
    import workloads as W
    out = {}

    def with_threads(n, fn):
        old = oracle.num_threads()
        oracle.set_num_threads(n)
        try:
            return fn()
        finally:
            oracle.set_num_threads(old)

    for spec, budget in ((W.C1, 1.0), (W.C2, 2.0)):
        q, pool_h, compact = _decode_inputs_host(spec, dev)
        call = lambda: oracle.sparse_mla(q, pool_h, compact, spec.sm_scale)
        n, dt = _time_oracle(call, budget)
        d = {"unit_of_work": "decode call: %d requests x %d heads x %d keys" % (spec.n_req, spec.n_heads, spec.k),
             "ms_per_call": round(dt / n * 1e3, 3), "tokens_per_s": round(spec.n_req * n / dt, 2),
             "threads": threads, "runs": n}
        if spec is W.C1:
            n1, dt1 = with_threads(1, lambda: _time_oracle(call, budget))
            d["one_thread"] = {"ms_per_call": round(dt1 / n1 * 1e3, 3), "tokens_per_s": round(spec.n_req * n1 / dt1, 2),
                               "runs": n1}
        out[spec.name] = d

    spec = W.C4
    rows, wslots = W.write_tokens(spec), W.write_slots(spec)
    pool_h = np.zeros((spec.n_slots, 352), dtype=np.uint8)
    lists = W.dup_lists(spec)
    write = lambda: oracle.quant_write(rows, wslots, pool_h)
    dedup = lambda: oracle.dedup_compact(lists)
    d = {"unit_of_work": "write of %d tokens; dedup of %d lists of %d" % (spec.n_tokens, spec.n_lists, spec.list_len),
         "threads": threads}
    for name, fn, budget in (("write", write, 1.5), ("dedup", dedup, 1.5)):
        n, dt = _time_oracle(fn, budget)
        n1, dt1 = with_threads(1, lambda: _time_oracle(fn, budget))
        d[name] = {"us": round(dt / n * 1e6, 1), "runs": n, "one_thread_us": round(dt1 / n1 * 1e6, 1),
                   "one_thread_runs": n1}
    out[spec.name] = d

    spec = W.C5
    n_rows = 128
    kv = W.kv_rows_host(spec, 0, spec.n_slots)
    pool_h = np.zeros((spec.n_slots, 352), dtype=np.uint8)
    oracle.quant_write(kv, np.arange(spec.n_slots, dtype=np.int32), pool_h)
    del kv
    sel = np.linspace(0, spec.rows - 1, n_rows).astype(np.int64)      # rows spread over all positions
    import torch
    q = W.queries(spec)[torch.from_numpy(sel)].float().numpy()
    topk, pt, rr = W.topk_lists(spec)[sel], W.page_table(spec), W.row_req(spec)[sel]
    n, dt = _time_oracle(lambda: oracle.sparse_mla(q, pool_h, topk, spec.sm_scale, page_table=pt, row_req=rr), 3.0)
    per_row = dt / n / n_rows
    out[spec.name] = {"unit_of_work": "prefill of %d of the %d query rows (evenly spaced) x %d heads x %d keys"
                                      % (n_rows, spec.rows, spec.n_heads, spec.k),
                      "ms_per_row": round(per_row * 1e3, 3), "runs": n, "threads": threads,
                      "full_prefill_s_extrapolated": round(per_row * spec.rows, 2),
                      "query_tokens_per_s": round(1.0 / per_row, 2)}
    return out


def main():
    args = _args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_kv_cache_kv4_amd as kv4
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = W.C3 if args.workload == "c3" else W.C2
    print("[bench] building %s pool: %d slots (%.2f GB)" % (spec.name, spec.n_slots, spec.n_slots * 352 / 1e9),
          file=sys.stderr, flush=True)
    wl = build_decode_workload(spec, dev)
    pool, pt, sets = wl["pool"], wl["pt"], wl["sets"]
    H, R, K = spec.n_heads, spec.n_req, spec.k
    S = args.splits or kv4.sparse_mla_decode_splits(sets[0]["q"], pool, sets[0]["topk"], page_table=pt)
    # the decode workspace, allocated once up front as an engine would at
    # start-up (a workspace allocated after the other buffers made the same
    # steps 0.6-0.9 us slower in one measurement: the placement of the
    # allocation, not the kernels, which are the same)
    ws = torch.empty(max(1, kv4.sparse_mla_decode_workspace(sets[0]["q"], pool, sets[0]["topk"], S, page_table=pt)),
                     dtype=torch.uint8, device=dev)
    part_o = torch.empty((S, R, H, 512), dtype=torch.float16, device=dev)   # as decode's workspace holds them
    part_lse = torch.empty((S, R, H), dtype=torch.float32, device=dev)
    out = torch.empty((R, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    lists = torch.empty((R, K), dtype=torch.int32, device=dev)
    counts = torch.empty((R,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        st = sets[i % len(sets)]
        # the new rows' write and the lists' compaction: one call, one kernel
        kv4.write_and_dedup(st["new_rows"], wl["new_slots"], pool, st["topk"], out_idx=lists, out_count=counts)
        # the decode call: the split kernel (fp16 parts in the workspace) and
        # the merge, which takes each row's parts on the XCD that wrote them
        kv4.sparse_mla_decode(st["q"], pool, lists, spec.sm_scale, page_table=pt, num_splits=S, workspace=ws,
                              out=out, lse=lse)

    # The timed steps run from HIP graphs that hold one step per rotating
    # input set, in order (a step's three calls are launched by the GPU, not
    # by the host), as they would sit inside a model's decode graph; a
    # remainder graph completes K.  For comparison, the same K steps with one
    # graph launch per step, whose host launch gap (~8 us) falls between
    # every two steps.
    step(0)
    torch.cuda.synchronize(dev)
    n_sets = len(sets)

    def capture(first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                step(first + i)
        return g

    per_step = [capture(i, 1) for i in range(n_sets)]
    full = capture(0, n_sets)

    def run_steps(k):
        for _ in range(k // n_sets):
            full.replay()
        if k % n_sets:
            rest.replay()

    rest = capture(0, args.steps % n_sets) if args.steps % n_sets else None
    SECTION_WARM_S[0] = 0.3 * min(1.0, args.warm_s / WARM_S)
    warm(full.replay, dev, args.warm_s)
    for i in range(args.warmup):
        per_step[i % n_sets].replay()
    full.replay()                        # the multi-step graph's first replay, untimed
    torch.cuda.synchronize(dev)
    print("[bench] timing %d steps (splits=%d)" % (args.steps, S), file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    elapsed = t1 - t0
    t2 = time.perf_counter()
    for i in range(args.steps):
        per_step[i % n_sets].replay()
    torch.cuda.synchronize(dev)
    per_step_ms = (time.perf_counter() - t2) / args.steps * 1e3

    # Average launch duration of the split kernel (and of the merge): a graph
    # of LAUNCHES back-to-back launches, launch i on rotating input set i % 8,
    # replayed REPS times between events on the stream they run on.  The
    # workload's lists hold no repeats, so a set's raw lists are its
    # compacted ones.
    LAUNCHES, REPS = 16, 5
    for i in range(n_sets):
        step(i)
        torch.cuda.synchronize(dev)
        if not bool((counts == K).all()):
            raise RuntimeError("input set %d: a list holds repeats, so its raw and compacted lists differ" % i)

    def launch_ms(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(LAUNCHES):
                fn(i % n_sets)
        g.replay()
        torch.cuda.synchronize(dev)
        warm(g.replay, dev, SECTION_WARM_S[0])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(REPS):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / (LAUNCHES * REPS)

    if S > 1:
        split_ms = launch_ms(lambda i: kv4.sparse_mla_decode_partial(sets[i]["q"], pool, sets[i]["topk"], spec.sm_scale,
                                                                     S, page_table=pt, part_o=part_o,
                                                                     part_lse=part_lse))
        merge_ms = launch_ms(lambda i: kv4.merge_states(part_o, part_lse, out=out, lse=lse))
    else:
        split_ms = launch_ms(lambda i: kv4.sparse_mla_decode(sets[i]["q"], pool, sets[i]["topk"], spec.sm_scale,
                                                             page_table=pt, num_splits=1, out=out, lse=lse))
        merge_ms = 0.0

    if args.calib_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        a.fill_(1.0)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize(dev)

    algo = algorithmic_decode_bytes(R, H, K)
    achieved = algo / (split_ms * 1e-3) / 1e9
    decode_flops = prefill_flops(R, H, K)
    result = {
        "metric": "sparse-MLA decode tokens/s + achieved HBM GB/s at top-k 2048; prefill MFMA %",
        "value": round(R * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": spec.name, "requests": R, "context_tokens": spec.ctx, "heads": H, "topk": K,
                   "page_size": 64, "pool_rows": spec.n_slots, "pool_gb": round(spec.n_slots * 352 / 1e9, 3),
                   "q_dtype": spec.q_dtype, "splits": S, "rotating_sets": len(sets)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profiles(args.workload),
                     "kernel": "sparse_mla_bf16_kernel (per-split decode)", "avg_launch_ms": round(split_ms, 5),
                     "algorithmic_bytes": algo,
                     "mfma_tflops": round(decode_flops / (split_ms * 1e-3) / 1e12, 2),
                     "mfma_frac": round(decode_flops / (split_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)},
        "merge_avg_launch_ms": round(merge_ms, 5),
        "ms_per_step_one_graph_per_step": round(per_step_ms, 5),
        "decode_gbs_incl_merge": round(algo / ((split_ms + merge_ms) * 1e-3) / 1e9, 1),
    }

    result["measured_ceilings"] = measure_ceilings(dev)
    result["roofline"]["frac_of_measured_copy"] = round(achieved / result["measured_ceilings"]["copy_gbs"], 4)
    if not args.no_rope_free:
        result["rope_free_decode"] = run_rope_free(spec, wl, dev, S, launch_ms)
    if not args.no_c2 and args.workload == "c3":
        result["c1_decode"] = run_c1_decode(dev)
        result["c2_decode"] = run_c2_decode(dev)
    if not args.no_compact:
        print("[bench] global compaction of the decode lists", file=sys.stderr, flush=True)
        result["global_compact_decode"] = run_global_compact(spec.name + " lists", pool, sets[0]["topk"], pt, None,
                                                             dev)[0]
    if not args.no_prefill:
        del part_o
        result["prefill"] = run_prefill(args, dev)
    if not args.no_write:
        result["write_compaction"] = run_write_compaction(dev)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = run_cpu_baseline(spec, wl, dev)
    print(json.dumps(result), flush=True)


def run_rope_free(spec, wl, dev, S, launch_ms):
    """The same decode over the 288-byte rope-free rows (the latent part of
    the same device-drawn rows, 512-dim queries): the pool is built the same
    way, the lists and page table are the workload's."""
    import torch
    import bit_kv_cache_kv4_amd as kv4
    import workloads as W
    print("[bench] rope-free decode %s" % spec.name, file=sys.stderr, flush=True)
    pool = torch.empty((spec.n_slots, kv4.ROW_BYTES_ROPE_FREE), dtype=torch.uint8, device=dev)
    for c in range(-(-spec.n_slots // W.KV_CHUNK)):
        x = W.kv_chunk_device(spec, c, dev)            # [n, 576]: the write reads the first 512 of each row
        lo = c * W.KV_CHUNK
        kv4.quant_write(x, torch.arange(lo, lo + x.shape[0], dtype=torch.int32, device=dev), pool)
        del x
    sets = wl["sets"]
    qs = [st["q"][:, :, :512].contiguous() for st in sets]
    scale = 1.0 / np.sqrt(512.0)
    R, H, K = spec.n_req, spec.n_heads, spec.k
    ws = torch.empty(max(1, kv4.sparse_mla_decode_workspace(qs[0], pool, sets[0]["topk"], S, page_table=wl["pt"])),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((R, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    ms = launch_ms(lambda i: kv4.sparse_mla_decode(qs[i], pool, sets[i]["topk"], scale, page_table=wl["pt"],
                                                   num_splits=S, workspace=ws, out=out, lse=lse))
    algo = algorithmic_decode_bytes(R, H, K, row_bytes=kv4.ROW_BYTES_ROPE_FREE, dim=512)
    del pool
    torch.cuda.empty_cache()
    gbs = algo / (ms * 1e-3) / 1e9
    return {"workload": spec.name + " with 288-byte rope-free rows", "row_bytes": kv4.ROW_BYTES_ROPE_FREE,
            "splits": S, "decode_ms": round(ms, 5), "tokens_per_s": round(R / (ms * 1e-3), 1),
            "algorithmic_bytes": algo, "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "note": "one decode call (split kernel and merge) per token batch; the step's write and dedup not included"}


def run_c1_decode(dev):
    """Config C1, tiny decode (1 request, 16 heads, fp32 queries, top-256 of a
    4096-token context): latency of one decode call (automatic split count:
    the split kernel and the merge), from a HIP graph of 20 calls replayed 5
    times between events; tokens/s = 1 / t."""
    import torch
    import bit_kv_cache_kv4_amd as kv4
    import workloads as W
    spec = W.C1
    print("[bench] decode %s" % spec.name, file=sys.stderr, flush=True)
    wl = build_decode_workload(spec, dev, n_sets=1)
    st = wl["sets"][0]
    S = kv4.sparse_mla_decode_splits(st["q"], wl["pool"], st["topk"], page_table=wl["pt"])
    ws = torch.empty(max(1, kv4.sparse_mla_decode_workspace(st["q"], wl["pool"], st["topk"], S, page_table=wl["pt"])),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((spec.n_req, spec.n_heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((spec.n_req, spec.n_heads), dtype=torch.float32, device=dev)
    CALLS, REPS = 20, 5

    def call():
        kv4.sparse_mla_decode(st["q"], wl["pool"], st["topk"], spec.sm_scale, page_table=wl["pt"], num_splits=S,
                              workspace=ws, out=out, lse=lse)

    call()
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(CALLS):
            call()
    g.replay()
    torch.cuda.synchronize(dev)
    warm(g.replay, dev, SECTION_WARM_S[0])
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(REPS):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / (CALLS * REPS)
    return {"workload": spec.name, "requests": spec.n_req, "heads": spec.n_heads, "topk": spec.k,
            "context_tokens": spec.ctx, "q_dtype": spec.q_dtype, "splits": S, "decode_us": round(ms * 1e3, 2),
            "tokens_per_s": round(spec.n_req / (ms * 1e-3), 1),
            "note": "launch-latency bound: 0.16 MB and 8.9 MFLOP per call"}


def run_c2_decode(dev, n_pools=6):
    """Config C2, one GPU's 64-head share at batch 8: the decode call
    (automatic split count: the split kernel and the merge) over n_pools
    independent pools with their own page tables, lists and queries (6 x 92 MB,
    so the gathered rows do not sit in the 256 MB MALL); average of a HIP graph
    of 12 calls cycling through them, replayed 5 times between events."""
    import torch
    import bit_kv_cache_kv4_amd as kv4
    import workloads as W
    spec = W.C2
    print("[bench] decode %s" % spec.name, file=sys.stderr, flush=True)
    wls = [build_decode_workload(W.scaled(spec, seed=spec.seed + 101 * i), dev, n_sets=1) for i in range(n_pools)]
    R, H, K = spec.n_req, spec.n_heads, spec.k
    S = kv4.sparse_mla_decode_splits(wls[0]["sets"][0]["q"], wls[0]["pool"], wls[0]["sets"][0]["topk"],
                                     page_table=wls[0]["pt"])
    ws = torch.empty(max(1, kv4.sparse_mla_decode_workspace(wls[0]["sets"][0]["q"], wls[0]["pool"],
                                                            wls[0]["sets"][0]["topk"], S, page_table=wls[0]["pt"])),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((R, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    CALLS, REPS = 12, 5

    def call(i):
        w = wls[i % n_pools]
        kv4.sparse_mla_decode(w["sets"][0]["q"], w["pool"], w["sets"][0]["topk"], spec.sm_scale, page_table=w["pt"],
                              num_splits=S, workspace=ws, out=out, lse=lse)

    call(0)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(CALLS):
            call(i)
    g.replay()
    torch.cuda.synchronize(dev)
    warm(g.replay, dev, SECTION_WARM_S[0])
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(REPS):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / (CALLS * REPS)
    algo = algorithmic_decode_bytes(R, H, K)
    gbs = algo / (ms * 1e-3) / 1e9
    del wls
    torch.cuda.empty_cache()
    return {"workload": spec.name, "requests": R, "heads": H, "topk": K, "context_tokens": spec.ctx, "splits": S,
            "pools": n_pools, "decode_us": round(ms * 1e3, 2), "tokens_per_s": round(R / (ms * 1e-3), 1),
            "algorithmic_bytes": algo, "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "note": "one decode call (split kernel and merge) per token batch of 8"}


def measure_ceilings(dev):
    """What this GPU reaches with library kernels, as context for the roofline
    fractions (which stay against the published peaks): a 1 GiB device copy
    (bytes read + written per second) and a dense fp16 GEMM of 8192^3 through
    torch.matmul, each the best of 5 event-timed runs."""
    import torch
    stream = torch.cuda.current_stream(dev)

    def best_ms(fn, reps=5):
        fn()
        torch.cuda.synchronize(dev)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    copy_ms = best_ms(lambda: b.copy_(a))
    del a, b
    n = 8192
    x = torch.randn((n, n), dtype=torch.float16, device=dev)
    y = torch.randn((n, n), dtype=torch.float16, device=dev)
    z = torch.empty((n, n), dtype=torch.float16, device=dev)
    gemm_ms = best_ms(lambda: torch.matmul(x, y, out=z))
    del x, y, z
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1),
            "gemm_f16_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "note": "1 GiB fp32 device copy (read + write bytes) and an 8192^3 fp16 GEMM via torch.matmul, best of 5"}


def run_global_compact(name, pool, topk, pt, row_req, dev, reps=5):
    """Global dedup across all lists into a compacted pool: average time of a
    HIP graph of `reps` calls (five to seven kernels each); algorithmic bytes = the
    lists read twice (marking, rewriting) and the rewritten lists written, the
    slot bitmap written and read twice, and the distinct rows read and
    written (page-table entries are not counted: they stay in L2)."""
    import torch
    import bit_kv_cache_kv4_amd as kv4
    R, k = topk.shape
    cap = min(pool.shape[0], R * k)
    cpool = torch.empty((max(cap, 1), pool.shape[1]), dtype=torch.uint8, device=dev)
    out_idx = torch.empty((R, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((1,), dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, kv4.global_compact_workspace(pool, topk, page_table=pt, row_req=row_req)),
                     dtype=torch.uint8, device=dev)
    kw = dict(page_table=pt, row_req=row_req, cpool=cpool, out_idx=out_idx, out_count=cnt, workspace=ws)
    kv4.global_compact(pool, topk, **kw)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            kv4.global_compact(pool, topk, **kw)
    g.replay()
    torch.cuda.synchronize(dev)
    warm(g.replay, dev, SECTION_WARM_S[0])
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    us = e0.elapsed_time(e1) / (3 * reps) * 1e3
    n = int(cnt.item())
    bitmap = (pool.shape[0] + 7) // 8
    algo = R * k * 4 * 3 + bitmap * 3 + n * pool.shape[1] * 2
    return {"lists": name, "entries": R * k, "distinct_rows": n, "row_bytes": pool.shape[1], "us": round(us, 2),
            "algorithmic_bytes": algo, "gbs": round(algo / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(algo / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}, cpool[:n], out_idx


def run_write_compaction(dev):
    """Config C4: quantized write of 16,384 fp32 rows into whole free pages of a
    1024-page pool (amax/6 scales, and MSE-searched scales), and dedup of 4096
    lists of 2048 (~25% repeats).  Eight
    independent input sets (about 300 MB of rows and 270 MB of lists) rotate
    through the timed launches so they do not sit in the 256 MB MALL.  Average
    launch time of a HIP graph of 16 launches replayed 5 times between events."""
    import torch
    import bit_kv_cache_kv4_amd as kv4
    import workloads as W
    spec = W.C4
    n_sets, LAUNCHES, REPS = 8, 16, 5
    print("[bench] write + compaction %s" % spec.name, file=sys.stderr, flush=True)
    rows = [torch.from_numpy(W.write_tokens(W.WriteSpec(seed=spec.seed + 11 * i))).to(dev) for i in range(n_sets)]
    slots = torch.from_numpy(W.write_slots(spec)).to(dev)
    pool = torch.empty((spec.n_slots, 352), dtype=torch.uint8, device=dev)
    lists = [torch.from_numpy(W.dup_lists(W.WriteSpec(seed=spec.seed + 11 * i))).to(dev) for i in range(n_sets)]
    out_idx = torch.empty_like(lists[0])
    out_cnt = torch.empty((spec.n_lists,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        fn(0)
        torch.cuda.synchronize(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(LAUNCHES):
                fn(i % n_sets)
        g.replay()
        torch.cuda.synchronize(dev)
        warm(g.replay, dev, SECTION_WARM_S[0])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(REPS):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / (LAUNCHES * REPS)

    w_ms = timed(lambda i: kv4.quant_write(rows[i], slots, pool))
    m_ms = timed(lambda i: kv4.quant_write_mse(rows[i], slots, pool))
    d_ms = timed(lambda i: kv4.dedup_compact(lists[i], out_idx=out_idx, out_count=out_cnt))
    w_bytes = spec.n_tokens * (576 * 4 + 4 + 352)
    d_bytes = spec.n_lists * (2 * spec.list_len * 4 + 4)
    return {"workload": spec.name,
            "write": {"tokens": spec.n_tokens, "us": round(w_ms * 1e3, 2), "algorithmic_bytes": w_bytes,
                      "gbs": round(w_bytes / (w_ms * 1e-3) / 1e9, 1),
                      "hbm_frac": round(w_bytes / (w_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "write_mse": {"tokens": spec.n_tokens, "us": round(m_ms * 1e3, 2), "algorithmic_bytes": w_bytes,
                          "gbs": round(w_bytes / (m_ms * 1e-3) / 1e9, 1),
                          "hbm_frac": round(w_bytes / (m_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "dedup": {"lists": spec.n_lists, "k": spec.list_len, "us": round(d_ms * 1e3, 2), "algorithmic_bytes": d_bytes,
                      "gbs": round(d_bytes / (d_ms * 1e-3) / 1e9, 1),
                      "hbm_frac": round(d_bytes / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}


def run_prefill(args, dev):
    """Sparse MLA prefill over the 65,536-token context (4096 queries x 64 heads
    x top-2048): MFMA utilisation against the dense fp16 peak."""
    import torch
    import bit_kv_cache_kv4_amd as kv4
    import workloads as W
    spec = W.C5
    print("[bench] prefill %s" % spec.name, file=sys.stderr, flush=True)
    kv = torch.from_numpy(W.kv_rows_host(spec, 0, spec.n_slots)).to(dev)
    pool = torch.empty((spec.n_slots, 352), dtype=torch.uint8, device=dev)
    kv4.quant_write(kv, torch.arange(spec.n_slots, dtype=torch.int32, device=dev), pool)
    del kv
    q = W.queries(spec).to(dev)
    topk = torch.from_numpy(W.topk_lists(spec)).to(dev)
    pt = torch.from_numpy(W.page_table(spec)).to(dev)
    rr = torch.from_numpy(W.row_req(spec)).to(dev)
    out = torch.empty((spec.rows, spec.n_heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((spec.rows, spec.n_heads), dtype=torch.float32, device=dev)
    kv4.sparse_mla_prefill(q, pool, topk, spec.sm_scale, page_table=pt, row_req=rr, out=out, lse=lse)
    torch.cuda.synchronize(dev)
    warm(lambda: kv4.sparse_mla_prefill(q, pool, topk, spec.sm_scale, page_table=pt, row_req=rr, out=out, lse=lse), dev,
         args.warm_s)
    stream = torch.cuda.current_stream(dev)
    ms = []
    for _ in range(args.prefill_iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kv4.sparse_mla_prefill(q, pool, topk, spec.sm_scale, page_table=pt, row_req=rr, out=out, lse=lse)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        ms.append(e0.elapsed_time(e1))
    t = float(np.median(ms))
    fl = prefill_flops(spec.rows, spec.n_heads, spec.k)
    tf = fl / (t * 1e-3) / 1e12
    res = {"workload": spec.name, "query_rows": spec.rows, "heads": spec.n_heads, "topk": spec.k,
           "context_tokens": spec.ctx, "ms": round(t, 4), "tflops": round(tf, 2),
           "mfma_peak_tflops": MFMA_F16_PEAK_TFLOPS, "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
           "query_tokens_per_s": round(spec.rows / (t * 1e-3), 1)}
    if not args.no_compact:
        # the prefill lists compacted into one pool, then the prefill over it
        comp, cpool, cidx = run_global_compact(spec.name + " lists", pool, topk, pt, rr, dev)
        kv4.sparse_mla_prefill(q, cpool, cidx, spec.sm_scale, out=out, lse=lse)
        torch.cuda.synchronize(dev)
        warm(lambda: kv4.sparse_mla_prefill(q, cpool, cidx, spec.sm_scale, out=out, lse=lse), dev, args.warm_s)
        cms = []
        for _ in range(args.prefill_iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            kv4.sparse_mla_prefill(q, cpool, cidx, spec.sm_scale, out=out, lse=lse)
            e1.record(stream)
            torch.cuda.synchronize(dev)
            cms.append(e0.elapsed_time(e1))
        comp["prefill_over_compacted_pool_ms"] = round(float(np.median(cms)), 4)
        res["global_compact"] = comp
    return res


if __name__ == "__main__":
    main()
