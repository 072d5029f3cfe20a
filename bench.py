"""Benchmark of the decode-time block indexer on one MI355X.

One step = the whole chain on one batch of the long-context workload
(4 requests x 1,048,576 keys, page_size 256, decode_query_len 8,
plane 32 x 4 x 8192, Top16 over 8 column ranges, the per-range lists merged
by msa_top16_merge):

    msa_score_decode -> msa_top16_select (R=8) -> msa_top16_merge

Two other forms of the same step, with bit-identical rows, are timed beside
it: select and merge in one launch (msa_score_decode ->
msa_top16_select_merge, the range rows kept in LDS;
e2e.one_launch_select_merge), and the plane with the per-range rows in one
launch followed by the merge (msa_score_select -> msa_top16_merge;
e2e.score_select_then_merge). One rank's share of the same workload on a
cache split by rows over 2 or 4 ranks (msa_score_decode_sharded ->
msa_top16_select_mapped, then the owner's msa_top16_merge_dedup) is
reported under e2e.sharded_rank_share.

Inputs are seeded and synthetic (workloads.py) and resident in HBM before
timing. Before every step a read pass over a 1 GiB buffer evicts index-K
from the 256 MB Infinity Cache; it sits outside the step's event pair. (A
read, not a fill: a 1 GiB fill would leave the caches full of dirty lines
whose write-back the next kernel would pay for.) The step time is measured with HIP
events on the stream the kernels run on; a second pass records an event
between the kernels for per-kernel times. The roofline figure takes the
scorer's per-launch duration from K launches back to back between one event
pair, which leaves out the dispatch delay after each event record (that is
what the kernel trace measures). The contract's wall clock brackets all K
steps, fills included, with a synchronize on both sides.

Prints one JSON line. `value` is scored keys/s, i.e. the sum of seq_len over
the mean step time. `roofline` rates the scorer, the dominant kernel, against
HBM. Its algorithmic bytes are 128 B per key, so 536,870,912 B per launch.
`roofline.mfma` is the scorer's MFMA work and busy fraction from rocprofv3
counters (committed under profiles/, valid while the scorer's source hash
matches). `roofline.stream_read_probe` times msa_stream_read_probe, a plain streaming
read with no other work, over as many index-K bytes in the same way: the
streaming ceiling the scorer's rate is read against. `cpu_baseline` times the oracle on the
same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
FLUSH_BYTES = 1 << 30           # read before each step; > 256 MB Infinity Cache
COPY_BYTES = 512 << 20          # calibration copy: reads and writes this many bytes
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic_score_decode_long_b4_s1m.json")
MFMA_FILE = os.path.join(HERE, "profiles", "mfma_score_decode_long_b4_s1m.json")
KERNEL_SOURCES = [os.path.join(HERE, "sparse_attention_block_msa_amd", "csrc", f)
                  for f in ("score_decode.hip", "msa_internal.h")]


def kernel_source_hash() -> str:
    """Hash of the scorer's code: its sources with // and /* */ comments and
    all white space removed, so an edit that only touches comments keeps the
    measured byte counters valid."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", "", text).encode())
    return h.hexdigest()[:16]


def load_traffic(launch_bytes: int):
    """HBM bytes per scorer launch from the committed counter summary, or
    None when it is missing or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return {"fetch_bytes": t["fetch_bytes"], "write_bytes": t["write_bytes"],
            "total_bytes": t["fetch_bytes"] + t["write_bytes"],
            "vs_algorithmic": round((t["fetch_bytes"] + t["write_bytes"]) / launch_bytes, 4),
            "copy_scale": t.get("copy_scale"), "source": os.path.relpath(TRAFFIC_FILE, HERE)}


def load_mfma():
    """The scorer's MFMA counters (flops, busy fraction) from the committed
    summary, or None when it is missing or the kernel source changed."""
    try:
        with open(MFMA_FILE) as f:
            m = json.load(f)
    except (OSError, ValueError):
        return None
    if m.get("kernel_source_hash") != kernel_source_hash():
        return None
    return {"flops_per_launch": m["mfma_flops"], "mfma_busy_frac": m["mfma_util"],
            "source": os.path.relpath(MFMA_FILE, HERE)}


def cpu_host() -> dict:
    """The host the CPU baseline runs on: CPU model, logical CPUs of the
    machine (os.cpu_count) and those this process may run on (nproc)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        nproc = os.cpu_count()
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "nproc": nproc}


CPU_BASELINE_MIN_S = 10.0  # repeat whole passes until this much CPU time is spent
CPU_BASELINE_MAX_PASSES = 30


def cpu_baseline(w):
    """The oracle on the same workload, on this host's cores: whole passes
    (score the full plane, then select and merge) repeated until about ten
    seconds have been spent, so the rate is not one short sample; then one
    more pass on a single thread (`single_thread`)."""
    import oracle

    orc = oracle.default()
    nvp = w.num_valid_pages.numpy()
    q, k, bt, sl = w.index_q.numpy(), w.index_k.numpy(), w.block_table.numpy(), w.seq_lens.numpy()
    score_s = select_s = 0.0
    passes = 0
    while passes < CPU_BASELINE_MAX_PASSES and score_s + select_s < CPU_BASELINE_MIN_S:
        t0 = time.perf_counter()
        plane, _, _ = orc.score_decode(q, k, bt, sl, page_size=w.page_size,
                                       decode_query_len=w.dql, cols=w.cols)
        t1 = time.perf_counter()
        ps, pi, _ = orc.top16_select(plane, nvp, init_blocks=w.init_blocks,
                                     local_blocks=w.local_blocks, num_ranges=w.num_ranges)
        if w.num_ranges > 1:
            orc.top16_merge(ps, pi, nvp, init_blocks=w.init_blocks, local_blocks=w.local_blocks)
        t2 = time.perf_counter()
        score_s += t1 - t0
        select_s += t2 - t1
        passes += 1
    keys = w.total_keys
    total = score_s + select_s
    cores = orc.num_threads()
    # one more whole pass on a single thread
    orc.set_num_threads(1)
    t0 = time.perf_counter()
    plane, _, _ = orc.score_decode(q, k, bt, sl, page_size=w.page_size, decode_query_len=w.dql,
                                   cols=w.cols)
    ps, pi, _ = orc.top16_select(plane, nvp, init_blocks=w.init_blocks,
                                 local_blocks=w.local_blocks, num_ranges=w.num_ranges)
    if w.num_ranges > 1:
        orc.top16_merge(ps, pi, nvp, init_blocks=w.init_blocks, local_blocks=w.local_blocks)
    one = time.perf_counter() - t0
    orc.set_num_threads(cores)
    return {"value": keys * passes / total, "unit": "keys/s", "cores": cores,
            "kind": "oracle", "host": cpu_host(),
            "sample": f"{passes} whole passes over the workload ({keys} keys each): score "
                      f"{score_s / passes:.2f} s, then Top16 select over {w.num_ranges} ranges "
                      f"and merge {select_s / passes:.2f} s, per pass",
            "seconds": round(total, 2),
            "single_thread": {"value": keys / one, "unit": "keys/s", "cores": 1,
                              "sample": "one whole pass over the workload", "seconds": round(one, 2)}}


def mfma_accuracy(tiles: int = 2048, seed: int = 77) -> dict:
    """Accumulation error of the three MFMA forms of msa_contraction_probe
    on 128-dim fp8 dot products (tiles x 16 x 16 of them per distribution),
    against exact float64 sums of torch-decoded codes (every finite e4m3fn
    code is a multiple of 2^-9 below 2^9, so each sum is a multiple of 2^-18
    below 2^43, which float64 holds exactly)."""
    import numpy as np
    import torch

    import sparse_attention_block_msa_amd as msa
    import workloads

    dev = torch.device("cuda:0")
    forms = {"bf16 16x16x32 x4 (the scorer's form)": msa.PROBE_BF16,
             "fp8 16x16x32 x4": msa.PROBE_FP8_16X16X32,
             "f8f6f4 16x16x128 x1": msa.PROBE_F8F6F4_16X16X128}
    g = torch.Generator().manual_seed(seed)
    shape = (tiles, 16, 128)

    def normal(scale):
        return (torch.randn(shape, generator=g) * scale).to(torch.float8_e4m3fn).view(torch.uint8)

    def codes():
        return workloads.FINITE_CODES[torch.randint(0, 254, shape, generator=g)]

    dists = {"q, k ~ N(0,1) -> e4m3fn": (normal(1.0), normal(1.0)),
             "q, k uniform over the 254 finite codes": (codes(), codes()),
             "q ~ N(0,1), k ~ N(0,64) -> e4m3fn": (normal(1.0), normal(8.0))}
    result = {"what": "max |err| / sum|q_i k_i| of 128-dim fp8 dot products, and how many "
                      "exceed 1e-5", "dots_per_distribution": tiles * 256, "seed": seed,
              "results": {}}
    out = torch.empty((tiles, 16, 16), dtype=torch.float32, device=dev)
    for dname, (q, k) in dists.items():
        qd = q.view(torch.float8_e4m3fn).to(torch.float64).numpy()
        kd = k.view(torch.float8_e4m3fn).to(torch.float64).numpy()
        exact = np.einsum("tid,tjd->tij", qd, kd)
        absum = np.einsum("tid,tjd->tij", np.abs(qd), np.abs(kd))
        qg, kg = q.to(dev), k.to(dev)
        row = {}
        for fname, form in forms.items():
            msa.msa_contraction_probe(qg, kg, out, form=form)
            torch.cuda.synchronize()
            rel = np.abs(out.cpu().numpy().astype(np.float64) - exact) / np.maximum(absum, 1e-300)
            row[fname] = {"max_rel_err": float(rel.max()),
                          "over_1e-5": int(np.count_nonzero(rel > 1e-5))}
        result["results"][dname] = row
    return result


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, help="workload number (1..5)")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache-evicting read pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mfma-accuracy", action="store_true",
                    help="only measure the accumulation error of the fp8 and bf16 MFMA forms "
                         "(msa_contraction_probe) and print it as one JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, copy a 512 MiB buffer once (a kernel of known "
                         "traffic for scaling hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the indexer runs on one GPU (got --gpus {args.gpus}); "
              "there is no multi-GPU path to measure", file=sys.stderr)
        sys.exit(2)

    if args.mfma_accuracy:
        print(json.dumps(mfma_accuracy()), flush=True)
        return

    import torch

    import sparse_attention_block_msa_amd as msa
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating workload {args.config}", file=sys.stderr, flush=True)
    w = workloads.config(args.config)
    q, k = w.index_q.to(dev), w.index_k.to(dev)
    bt, sl, nvp = w.block_table.to(dev), w.seq_lens.to(dev), w.num_valid_pages.to(dev)
    T, R = w.num_tokens, w.num_ranges
    plane = torch.empty((T, 4, w.cols), dtype=torch.float32, device=dev)
    part = msa.new_rows(T, 4, R, device=dev)
    final = msa.new_rows(T, 4, device=dev)
    errors = torch.zeros(1, dtype=torch.int32, device=dev)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    msa.msa_warmup()
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        msa.msa_score_decode(q, k, bt, sl, plane, page_size=w.page_size,
                             decode_query_len=w.dql, errors=errors, stream=stream)
        if ev:
            ev[1].record(stream)
        msa.msa_top16_select(plane, nvp, part, init_blocks=w.init_blocks,
                             local_blocks=w.local_blocks, num_ranges=R, errors=errors,
                             stream=stream)
        if ev:
            ev[2].record(stream)
        if R > 1:
            msa.msa_top16_merge(part, nvp, final, init_blocks=w.init_blocks,
                                local_blocks=w.local_blocks, errors=errors, stream=stream)
        if ev:
            ev[3].record(stream)

    def step_fused():
        msa.msa_score_decode(q, k, bt, sl, plane, page_size=w.page_size,
                             decode_query_len=w.dql, errors=errors, stream=stream)
        msa.msa_top16_select_merge(plane, nvp, final, init_blocks=w.init_blocks,
                                   local_blocks=w.local_blocks, num_ranges=R,
                                   errors=errors, stream=stream)

    # select and merge in one launch where that form applies (at most 16
    # ranges of at most 2048 columns)
    fused_applies = 1 < R <= 16 and -(-w.cols // R) <= 2048

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        if not args.no_flush:
            flush.sum()
        step()
        if fused_applies:
            step_fused()
    torch.cuda.synchronize()

    # Timed region 1 (the headline): K steps, an event pair around each step
    # only, so nothing is recorded between the kernels of a step.
    step_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                   for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        if not args.no_flush:
            flush.sum()
        step_events[i][0].record(stream)
        step()
        step_events[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    # Timed region 1b: the same K steps with select and merge in one launch
    # (msa_top16_select_merge), reported beside the headline.
    fused_ms = None
    if fused_applies:
        fused_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                        for _ in range(args.steps)]
        for i in range(args.steps):
            if not args.no_flush:
                flush.sum()
            fused_events[i][0].record(stream)
            step_fused()
            fused_events[i][1].record(stream)
        torch.cuda.synchronize()
        fused_ms = sum(ev[0].elapsed_time(ev[1]) for ev in fused_events) / args.steps

    # Timed region 1c: the same K steps with the plane and the range rows from
    # one launch (msa_score_select), then msa_top16_merge; reported beside the
    # headline.
    ws = msa.score_select_workspace(w.batch, w.dql, w.cols, R, pool=True, device=dev)

    def step_score_select():
        # plane in the workspace's pool (scores unused), range rows and their
        # merge from the same launch
        msa.msa_score_select(q, k, bt, sl, None, nvp, part, ws, page_size=w.page_size,
                             decode_query_len=w.dql, init_blocks=w.init_blocks,
                             local_blocks=w.local_blocks, num_ranges=R, cols=w.cols,
                             merged=final if R <= 64 else None, errors=errors, stream=stream)

    score_select_ms = None
    if -(-w.cols // R) <= 2048:
        for _ in range(args.warmup):
            step_score_select()
        ss_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                     for _ in range(args.steps)]
        for i in range(args.steps):
            if not args.no_flush:
                flush.sum()
            ss_events[i][0].record(stream)
            step_score_select()
            ss_events[i][1].record(stream)
        torch.cuda.synchronize()
        score_select_ms = sum(ev[0].elapsed_time(ev[1]) for ev in ss_events) / args.steps

    # Timed region 1d: one rank's share of the same workload on a cache whose
    # pages are split by rows over world_size ranks (msa_score_decode_sharded
    # -> msa_top16_select_mapped over R ranges), and the owner's merge of all
    # ranks' rows (msa_top16_merge_dedup), for world_size 2 and 4.
    sharded = {}
    if w.page_size % 128 == 0:
        for ws_n in (2, 4):
            rows_per_rank = w.page_size // ws_n
            shard = workloads.shard_rows(w.index_k, 0, ws_n).to(dev)
            scols = max(4, -(-(-(-int(w.seq_lens.max()) // w.page_size)) // 4) * 4)
            splane = torch.empty((T, 4, scols), dtype=torch.float32, device=dev)
            spart = msa.new_rows(T, 4, R, device=dev)
            scale, offset = (1, 0) if w.page_size == 128 else (2, 0)
            # rank 0 holds the positions p with p % page_size < rows_per_rank
            rank_keys = 0
            for sl_b in w.seq_lens.tolist():
                full, rem = divmod(max(0, sl_b), w.page_size)
                rank_keys += full * rows_per_rank + min(rem, rows_per_rank)

            def step_rank():
                msa.msa_score_decode_sharded(q, shard, bt, sl, splane, page_size=w.page_size,
                                             decode_query_len=w.dql, rank=0, world_size=ws_n,
                                             errors=errors, stream=stream)
                msa.msa_top16_select_mapped(splane, nvp, spart, init_blocks=w.init_blocks,
                                            local_blocks=w.local_blocks, num_ranges=R,
                                            index_scale=scale, index_offset=offset,
                                            errors=errors, stream=stream)

            for _ in range(args.warmup):
                step_rank()
            ev_r = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                    for _ in range(args.steps)]
            for i in range(args.steps):
                if not args.no_flush:
                    flush.sum()
                ev_r[i][0].record(stream)
                step_rank()
                ev_r[i][1].record(stream)
            # owner merge of every rank's rows (rank 0's rows stand in for all)
            all_rows = spart.repeat(1, 1, ws_n, 1).contiguous()
            merged = msa.new_rows(T, 4, device=dev)
            for _ in range(args.warmup):
                msa.msa_top16_merge_dedup(all_rows, nvp, merged, init_blocks=w.init_blocks,
                                          local_blocks=w.local_blocks, stream=stream)
            ev_m = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                    for _ in range(args.steps)]
            for i in range(args.steps):
                ev_m[i][0].record(stream)
                msa.msa_top16_merge_dedup(all_rows, nvp, merged, init_blocks=w.init_blocks,
                                          local_blocks=w.local_blocks, stream=stream)
                ev_m[i][1].record(stream)
            torch.cuda.synchronize()
            rank_ms = sum(e[0].elapsed_time(e[1]) for e in ev_r) / args.steps
            merge_ms = sum(e[0].elapsed_time(e[1]) for e in ev_m) / args.steps
            rank_bytes = rank_keys * 128
            sharded[f"world_size_{ws_n}"] = {
                "rank": 0, "rank_keys": rank_keys,
                "rank_step_ms": rank_ms,
                "rank_hbm_gbps": rank_bytes / (rank_ms * 1e-3) / 1e9,
                "rank_frac_of_peak": rank_bytes / (rank_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "owner_merge_ms": merge_ms, "merged_rows_per_head": ws_n * R}
            del shard, splane, spart, all_rows, merged

    # Timed region 2: K steps with an event between every kernel,
    # for per-kernel durations (the events themselves lengthen these steps).
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps per kernel", file=sys.stderr, flush=True)
    for i in range(args.steps):
        if not args.no_flush:
            flush.sum()
        step(events[i])
    torch.cuda.synchronize()
    # Timed region 3: the scorer alone, K launches back to back between one
    # event pair (a cache-evicting read first), for its per-launch duration
    # without the dispatch delay that follows each event record. Launches
    # stream 537 MB each through a 256 MB Infinity Cache with non-temporal
    # loads, so a launch finds little of the previous one's data resident.
    print(f"[bench] timing {args.steps} back-to-back scorer launches", file=sys.stderr,
          flush=True)
    if not args.no_flush:
        flush.sum()
    b2b = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    b2b[0].record(stream)
    for _ in range(args.steps):
        msa.msa_score_decode(q, k, bt, sl, plane, page_size=w.page_size,
                             decode_query_len=w.dql, errors=errors, stream=stream)
    b2b[1].record(stream)
    torch.cuda.synchronize()
    score_b2b_ms = b2b[0].elapsed_time(b2b[1]) / args.steps
    # Timed region 3b: the streaming-read probe (a plain read, no other work)
    # over as many index-K bytes, timed the same way: the streaming ceiling
    # the scorer's rate is read against.
    # as many bytes as the scorer's algorithmic read, in whole 16 KiB blocks
    # from the start of the cache (pages in storage order)
    probe_bytes = max(16384, workloads.index_k_bytes(w) // 16384 * 16384)
    probe_bytes = min(probe_bytes, k.numel() // 16384 * 16384)
    sink = torch.zeros(msa.STREAM_PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
    msa.msa_stream_read_probe(k, sink, nbytes=probe_bytes, stream=stream)
    if not args.no_flush:
        flush.sum()
    b2b_probe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    b2b_probe[0].record(stream)
    for _ in range(args.steps):
        msa.msa_stream_read_probe(k, sink, nbytes=probe_bytes, stream=stream)
    b2b_probe[1].record(stream)
    torch.cuda.synchronize()
    probe_ms = b2b_probe[0].elapsed_time(b2b_probe[1]) / args.steps
    if int(errors.item()) != 0:
        raise RuntimeError(f"device error counter = {int(errors.item())}")
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    step_ms = sorted(ev[0].elapsed_time(ev[1]) for ev in step_events)
    score_ms = [ev[0].elapsed_time(ev[1]) for ev in events]
    select_ms = [ev[1].elapsed_time(ev[2]) for ev in events]
    merge_ms = [ev[2].elapsed_time(ev[3]) for ev in events]
    mean = lambda xs: sum(xs) / len(xs)
    ms_step = mean(step_ms)
    keys = w.total_keys
    launch_bytes = workloads.index_k_bytes(w)
    value = keys / (ms_step * 1e-3)
    e2e_gbps = launch_bytes / (ms_step * 1e-3) / 1e9
    score_mean = mean(score_ms)
    achieved = launch_bytes / (score_b2b_ms * 1e-3) / 1e9
    traffic = load_traffic(launch_bytes)  # HBM bytes per launch, from the committed counters
    probe_gbps = probe_bytes / (probe_ms * 1e-3) / 1e9

    out = {
        "metric": "index-K scored keys/s and achieved HBM GB/s (% of peak), score+Top16, 1 GPU",
        "value": value,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-products-f32-accumulate",
        "data": "synthetic (seeded N(0,1) -> float8_e4m3fn, random page permutation)",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": int(w.seq_lens.max()),
                   "page_size": w.page_size, "decode_query_len": w.dql, "cols": w.cols,
                   "ranges": R, "init_blocks": w.init_blocks, "local_blocks": w.local_blocks,
                   "index_k_bytes": launch_bytes, "parallelism": "single-gpu",
                   "cache_flush_between_steps": not args.no_flush},
        "e2e": {"step": "msa_score_decode -> msa_top16_select" +
                        (" -> msa_top16_merge" if R > 1 else ""),
                "hbm_gbps": e2e_gbps, "frac_of_peak": e2e_gbps / HBM_PEAK_GBPS,
                # each key is scored against its request's 4 * dql query rows
                "dot_products_per_s": value * 4 * w.dql,
                "step_ms_p10": step_ms[len(step_ms) // 10],
                "step_ms_p50": step_ms[len(step_ms) // 2],
                "step_ms_p90": step_ms[(len(step_ms) * 9) // 10],
                "kernels_ms": {"score_decode": score_mean, "top16_select": mean(select_ms),
                               "top16_merge": mean(merge_ms)},
                "score_decode_ms_back_to_back": score_b2b_ms,
                "step_ms_with_kernel_events": mean([ev[0].elapsed_time(ev[3]) for ev in events]),
                "one_launch_select_merge": None if fused_ms is None else {
                    "ms_per_step": fused_ms, "keys_per_s": keys / (fused_ms * 1e-3),
                    "hbm_gbps": launch_bytes / (fused_ms * 1e-3) / 1e9,
                    "frac_of_peak": launch_bytes / (fused_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS},
                "score_select_then_merge": None if score_select_ms is None else {
                    "ms_per_step": score_select_ms,
                    "keys_per_s": keys / (score_select_ms * 1e-3),
                    "hbm_gbps": launch_bytes / (score_select_ms * 1e-3) / 1e9,
                    "frac_of_peak":
                        launch_bytes / (score_select_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS},
                "sharded_rank_share": sharded or None,
                "wall_s_all_steps_incl_flush": wall},
        "roofline": {"kernel": "score_decode", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "algorithmic_bytes_per_launch": launch_bytes,
                     "launch_ms": score_b2b_ms,
                     "launch_ms_source": "K scorer launches back to back between one event pair",
                     "traffic": None if traffic is None else traffic["total_bytes"],
                     "traffic_detail": traffic,
                     "mfma": load_mfma(),
                     "stream_read_probe": {
                         "what": "msa_stream_read_probe over as many index-K bytes, pages "
                                 "in storage order: a plain streaming read with no other work",
                         "launch_ms": probe_ms, "achieved": probe_gbps,
                         "frac_of_peak": probe_gbps / HBM_PEAK_GBPS,
                         "scorer_frac_of_probe": achieved / probe_gbps}},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
