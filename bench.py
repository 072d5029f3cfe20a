"""Benchmark of the decode-time block indexer on one MI355X.

One step = the whole decode path on one batch of the long-context workload
(4 requests x 1,048,576 keys, page_size 256, decode_query_len 8,
plane 32 x 4 x 8192, Top16 over 8 column ranges, the per-range lists merged):

    msa_score_decode -> msa_top16_select_merge (per-range rows written, and
                        their merge, in one launch)

Where that one-launch form does not apply (one range, or more than 16, or
ranges wider than 2048 columns) the step is msa_score_decode ->
msa_top16_select [-> msa_top16_merge]. The other forms of the same step, all
with bit-identical merged rows, are timed beside it under e2e.other_forms:
the three-launch chain (score -> select -> merge), the whole-row select
(select_merge without per-range rows), and msa_score_select (plane in the
workspace pool, range rows and merge in the scoring launch). One rank's
share of the same workload on a cache split by rows over 2 or 4 ranks
(msa_score_decode_sharded -> msa_top16_select_mapped, then the owner's
msa_top16_merge_dedup) is reported under e2e.sharded_rank_share (steps back
to back over rotating shard copies, as the headline, and one per event pair),
and the prefill chain on one 8192-token window under `prefill`.

Inputs are seeded and synthetic (workloads.py) and resident in HBM before
timing. The headline times K steps back to back between one event pair,
with a synchronize on both sides (the contract's wall clock brackets the
same K steps), as a decode loop runs them: step i reads index-K copy
i % n, the copies standing in for successive layers' caches, with at least
768 MiB of other copies read between two uses of one copy so that the
256 MB Infinity Cache holds none of it. 400 untimed back-to-back steps come
first: after an idle spell the first ~175 run slower (about 105 -> 91 us per
step at config 5) while the device settles under sustained load, and the
step then holds steady. Workloads too small for that (more than 4
copies) time an event pair around each step instead. Beside it, every
form of the step is also timed with an event pair around each step after a
read pass over a 1 GiB buffer that evicts index-K (outside the pair; a read,
not a fill, since a fill would leave dirty lines whose write-back the next
kernel would pay for); those per-step times carry the dispatch delay that
back-to-back steps overlap, and give the mean, p10, p50 and p90 with their
fractions of HBM peak. A further pass records an event between the kernels
of the three-launch chain for per-kernel times. The roofline figure takes
the scorer's per-launch duration from K launches back to back between one
event pair, which leaves out the dispatch delay after each event record
(that is what the kernel trace measures); they rotate over the same index-K
copies as the headline, after 400 untimed launches (the scorer alone
settles over ~300 launches from idle).

Prints one JSON line. `value` is scored keys/s, i.e. the sum of seq_len over
the mean step time. `roofline` rates the scorer, the dominant kernel, against
HBM. Its algorithmic bytes are 128 B per key, so 536,870,912 B per launch.
`roofline.mfma` is the scorer's MFMA work and busy fraction from rocprofv3
counters (committed under profiles/, valid while the scorer's source hash
matches). `roofline.stream_read_probe` times msa_stream_read_probe, a plain
streaming read with no other work, over as many index-K bytes (the same
copies, the same warm-up) and over 4 GiB, in the same way and at each of its
shapes: the fastest shape at each size is the streaming ceiling the
scorer's rate is read against. `cpu_baseline` times the oracle on the same
workload.
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
PROBE_BIG_BYTES = 4 << 30       # the long streaming-read probe
PROBE_SHAPES = (0, 2, 4, 8, 16)  # the probe's shapes (0: persistent); the ceiling is the best
ROTATE_MIN_BYTES = 768 << 20    # other index-K bytes read between two uses of one copy
MAX_COPIES = 4                  # index-K copies the headline rotates over, at most
ROTATE_WARMUP_STEPS = 400       # untimed back-to-back steps before the headline's K
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic_score_decode_long_b4_s1m.json")
MFMA_FILE = os.path.join(HERE, "profiles", "mfma_score_decode_long_b4_s1m.json")
KERNEL_SOURCES = [os.path.join(HERE, "sparse_attention_block_msa_amd", "csrc", f)
                  for f in ("score_decode.hip", "score_tile.h", "msa_internal.h")]


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


def timed_steps(fn, steps, stream, flush=None):
    """K calls of fn, each after a cache-evicting read (when given) and inside
    its own event pair; returns the sorted per-step times in ms."""
    import torch

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        if flush is not None:
            flush.sum()
        evs[i][0].record(stream)
        fn()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return sorted(e[0].elapsed_time(e[1]) for e in evs)


def step_stats(ms, launch_bytes, keys):
    """Mean and percentiles of per-step times, as rates against HBM."""
    mean = sum(ms) / len(ms)
    pick = lambda f: ms[min(len(ms) - 1, int(len(ms) * f))]
    frac = lambda t: launch_bytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS
    return {"ms_per_step": mean, "keys_per_s": keys / (mean * 1e-3),
            "hbm_gbps": launch_bytes / (mean * 1e-3) / 1e9, "frac_of_peak": frac(mean),
            "step_ms_p10": pick(0.1), "step_ms_p50": pick(0.5), "step_ms_p90": pick(0.9),
            "frac_of_peak_p50": frac(pick(0.5)), "frac_of_peak_p90": frac(pick(0.9))}


def prefill_figure(dev, stream, runs: int = 10) -> dict:
    """The prefill chain (window plan -> local scoring and select -> merge) on
    one long query window: 8192 query tokens at the end of a 65,536-key
    request, page_size 256. Its contraction is compute-bound (4 * 8192 query
    rows per key), so it is rated in useful MFMA flops: 2 * 128 per (query
    row, visible key), against the bf16 dense peak."""
    import torch

    import sparse_attention_block_msa_amd as msa
    import workloads

    w = workloads.generate(name="prefill_q8192_s64k_p256", batch=1, seq=("fixed", 65536),
                           q_lens=("fixed", 8192), page_size=256, dql=1, init=4, local=4,
                           ranges=1, seed=3105)
    T, R = w.num_tokens, w.num_ranges
    q, k = w.index_q.to(dev), w.index_k.to(dev)
    bt, qo = w.block_table.to(dev), w.qo_indptr.to(dev)
    sl, nvp = w.seq_lens.to(dev), w.num_valid_pages.to(dev)
    plane = torch.empty((T, 4, w.cols), dtype=torch.float32, device=dev)
    plan = msa.new_prefill_plan(T, w.batch, w.cols, device=dev)
    carrier = msa.new_rows(T, 4, R, device=dev)
    merged = msa.new_rows(T, 4, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    sel = dict(init_blocks=w.init_blocks, local_blocks=w.local_blocks)

    def chain():
        msa.msa_prefill_window_plan(qo, sl, plan, num_tokens=T, cols=w.cols, errors=err,
                                    stream=stream)
        msa.msa_prefill_local(q, k, bt, plan, plane, nvp, carrier, page_size=w.page_size,
                              num_ranges=R, errors=err, stream=stream, **sel)
        msa.msa_prefill_merge(carrier, nvp, merged, errors=err, stream=stream, **sel)

    for _ in range(3):
        chain()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record(stream)
    for _ in range(runs):
        chain()
    e[1].record(stream)
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"prefill: device error counter = {int(err.item())}")
    ms = e[0].elapsed_time(e[1]) / runs
    pos = w.positions.to(torch.float64)
    useful = float(2 * 128 * 4 * (pos + 1).sum())
    tflops = useful / (ms * 1e-3) / 1e12
    return {"workload": w.name, "query_tokens": T, "keys": int(w.seq_lens.sum()),
            "step": "msa_prefill_window_plan -> msa_prefill_local -> msa_prefill_merge",
            "ms_per_chain": ms, "chain_timing": f"{runs} chains back to back between one event pair",
            "useful_flop": useful, "achieved_tflops": tflops,
            "peak_tflops": BF16_PEAK_TFLOPS, "frac_of_bf16_peak": tflops / BF16_PEAK_TFLOPS}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, help="workload number (1..5)")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache-evicting read pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill figure")
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
    flush = None if args.no_flush else torch.ones(FLUSH_BYTES // 4, dtype=torch.float32,
                                                 device=dev)
    msa.msa_warmup()
    stream = torch.cuda.current_stream()
    sel = dict(init_blocks=w.init_blocks, local_blocks=w.local_blocks, errors=errors,
               stream=stream)
    keys = w.total_keys
    launch_bytes = workloads.index_k_bytes(w)

    def score(kk=k):
        msa.msa_score_decode(q, kk, bt, sl, plane, page_size=w.page_size,
                             decode_query_len=w.dql, errors=errors, stream=stream)

    # Forms of the step; all leave bit-identical merged rows (the tests check
    # each form against the others and the oracle).
    one_launch = 1 < R <= 16 and -(-w.cols // R) <= 2048

    def step_three(ev=None, kk=k):
        # score -> per-range select -> merge, three launches
        if ev:
            ev[0].record(stream)
        score(kk)
        if ev:
            ev[1].record(stream)
        msa.msa_top16_select(plane, nvp, part, num_ranges=R, **sel)
        if ev:
            ev[2].record(stream)
        if R > 1:
            msa.msa_top16_merge(part, nvp, final, **sel)
        if ev:
            ev[3].record(stream)

    def step_headline(kk=k):
        # score -> per-range select and their merge in one launch (the
        # per-range rows are written as well)
        score(kk)
        msa.msa_top16_select_merge(plane, nvp, final, num_ranges=R, partial=part, **sel)

    def step_row_select():
        # score -> the merged rows straight from the whole row (no per-range rows)
        score()
        msa.msa_top16_select_merge(plane, nvp, final, num_ranges=R, **sel)

    ws = msa.score_select_workspace(w.batch, w.dql, w.cols, R, pool=True, device=dev)

    def step_score_select():
        # range rows and their merge from the scoring launch (plane in the pool)
        msa.msa_score_select(q, k, bt, sl, None, nvp, part, ws, page_size=w.page_size,
                             decode_query_len=w.dql, num_ranges=R, cols=w.cols,
                             merged=final if R <= 64 else None, **sel)

    headline = step_headline if one_launch else step_three
    headline_name = ("msa_score_decode -> msa_top16_select_merge (per-range rows written, "
                     "merged in the same launch)" if one_launch else
                     "msa_score_decode -> msa_top16_select" +
                     (" -> msa_top16_merge" if R > 1 else ""))
    forms = {"three_launch_chain": step_three}
    if one_launch:
        forms["row_select"] = step_row_select
    if -(-w.cols // R) <= 2048:
        forms["fused_score_select"] = step_score_select

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        if flush is not None:
            flush.sum()
        headline()
        for f in forms.values():
            f()
    torch.cuda.synchronize()

    # Timed region 1 (the headline): K steps back to back, bracketed by a
    # synchronize and one event pair, as a decode loop runs them. Step i reads
    # index-K copy i % n: the copies stand in for successive layers' caches,
    # and the (n - 1) copies read between two uses of one copy (at least
    # ROTATE_MIN_BYTES) leave nothing of it in the 256 MB Infinity Cache.
    # Workloads too small for that take an event pair per step after a
    # cache-evicting read instead.
    n_copies = -(-ROTATE_MIN_BYTES // max(1, launch_bytes)) + 1
    rotate = flush is not None and n_copies <= MAX_COPIES
    kcopies = [k] + [k.clone() for _ in range(n_copies - 1)] if rotate else [k]
    if rotate:
        # Untimed back-to-back steps first. Measured on MI355X at config 5
        # (events every 25 steps, two trials after 2 s idle): 105, 101-108,
        # 96-99, 95, 91-93, 90 us per step over the first 150 steps, then
        # 88.6-89.2 us from about step 175 on, for the 1200 steps measured;
        # the device settles under sustained load (about 16 ms here). The
        # timed steps start once it has.
        for i in range(max(args.warmup, ROTATE_WARMUP_STEPS)):
            headline(kk=kcopies[i % n_copies])
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    if rotate:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for i in range(args.steps):
            headline(kk=kcopies[i % n_copies])
        ev[1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_step = ev[0].elapsed_time(ev[1]) / args.steps
        timing = (f"{args.steps} steps back to back between one event pair, step i on "
                  f"index-K copy i % {n_copies} (copies stand in for successive layers' "
                  "caches; the Infinity Cache holds none of a copy when it is reused)")
        step_ms = timed_steps(headline, args.steps, stream, flush)
    else:
        step_ms = timed_steps(headline, args.steps, stream, flush)
        wall = time.perf_counter() - wall0
        ms_step = sum(step_ms) / len(step_ms)
        timing = ("an event pair around each step, after a read of a 1 GiB buffer that "
                  "evicts index-K from the Infinity Cache" if flush is not None else
                  "an event pair around each step (no eviction)")

    # Timed region 1b: the other forms of the step, timed the same way.
    alt = {}
    for name, f in forms.items():
        alt[name] = step_stats(timed_steps(f, args.steps, stream, flush), launch_bytes, keys)
    alt["three_launch_chain"]["step"] = ("msa_score_decode -> msa_top16_select" +
                                         (" -> msa_top16_merge" if R > 1 else ""))
    if "row_select" in alt:
        alt["row_select"]["step"] = ("msa_score_decode -> msa_top16_select_merge without "
                                     "per-range rows (whole-row select)")
    if "fused_score_select" in alt:
        alt["fused_score_select"]["step"] = ("msa_score_select: plane in the workspace pool, "
                                             "range rows and their merge in one launch")

    sink = torch.zeros(msa.STREAM_PROBE_SINK_WORDS, dtype=torch.int32, device=dev)

    def probe_shape_ms(bufs, nbytes, launches, bpw, warm):
        """msa_stream_read_probe over nbytes, bpw blocks per wave: `warm`
        untimed launches, then K launches back to back between one event
        pair, launch i reading bufs[i % len(bufs)] (a cache-evicting read
        first when there is one buffer)."""
        for i in range(warm):
            msa.msa_stream_read_probe(bufs[i % len(bufs)], sink, nbytes=nbytes,
                                      blocks_per_wave=bpw, stream=stream)
        if flush is not None and len(bufs) == 1:
            flush.sum()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for i in range(launches):
            msa.msa_stream_read_probe(bufs[i % len(bufs)], sink, nbytes=nbytes,
                                      blocks_per_wave=bpw, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / launches

    def probe_ms(bufs, nbytes, launches, warm=1):
        """The fastest probe shape's launch time, and every shape's."""
        shapes = {("persistent" if bpw == msa.STREAM_PROBE_PERSISTENT else bpw):
                  probe_shape_ms(bufs, nbytes, launches, bpw, warm) for bpw in PROBE_SHAPES}
        return min(shapes.values()), shapes

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
                msa.msa_top16_select_mapped(splane, nvp, spart, num_ranges=R,
                                            index_scale=scale, index_offset=offset, **sel)

            for _ in range(args.warmup):
                step_rank()
            rank_ms = timed_steps(step_rank, args.steps, stream, flush)
            # the same step back to back over rotating shard copies, as the
            # headline times its steps (a rank of a decode loop runs them so)
            n_shards = -(-ROTATE_MIN_BYTES // shard.numel()) + 1
            rotate_shards = flush is not None and n_shards <= 2 * MAX_COPIES
            shards = ([shard] + [shard.clone() for _ in range(n_shards - 1)]
                      if rotate_shards else [])

            def step_rank_on(kk):
                msa.msa_score_decode_sharded(q, kk, bt, sl, splane, page_size=w.page_size,
                                             decode_query_len=w.dql, rank=0, world_size=ws_n,
                                             errors=errors, stream=stream)
                msa.msa_top16_select_mapped(splane, nvp, spart, num_ranges=R,
                                            index_scale=scale, index_offset=offset, **sel)

            rank_btb_ms = None
            if rotate_shards:
                for i in range(ROTATE_WARMUP_STEPS):
                    step_rank_on(shards[i % n_shards])
                ev_r = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                ev_r[0].record(stream)
                for i in range(args.steps):
                    step_rank_on(shards[i % n_shards])
                ev_r[1].record(stream)
                torch.cuda.synchronize()
                rank_btb_ms = ev_r[0].elapsed_time(ev_r[1]) / args.steps
            # owner merge of every rank's rows (rank 0's rows stand in for all)
            all_rows = spart.repeat(1, 1, ws_n, 1).contiguous()
            merged = msa.new_rows(T, 4, device=dev)

            def owner_merge():
                # rank 0's rows repeated stand in for every rank's: the forced
                # ids other ranks would hold are missing, so no error counter
                msa.msa_top16_merge_dedup(all_rows, nvp, merged, init_blocks=w.init_blocks,
                                          local_blocks=w.local_blocks, stream=stream)

            for _ in range(args.warmup):
                owner_merge()
            merge_ms = timed_steps(owner_merge, args.steps, stream)
            rank_mean = sum(rank_ms) / len(rank_ms)
            rank_bytes = rank_keys * 128
            # the rank's scorer alone, back to back, against a plain read of
            # as many bytes (the ceiling at this size, ramp and tail included),
            # both over the rotating shard copies after the same warm-up when
            # there are copies (one shard alone would sit in the Infinity
            # Cache), else after a cache-evicting read
            rank_bufs = shards if rotate_shards else [shard]

            def rank_score_on(kk):
                msa.msa_score_decode_sharded(q, kk, bt, sl, splane, page_size=w.page_size,
                                             decode_query_len=w.dql, rank=0, world_size=ws_n,
                                             errors=errors, stream=stream)

            if rotate_shards:
                for i in range(ROTATE_WARMUP_STEPS):
                    rank_score_on(rank_bufs[i % len(rank_bufs)])
            elif flush is not None:
                flush.sum()
            ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev_s[0].record(stream)
            for i in range(args.steps):
                rank_score_on(rank_bufs[i % len(rank_bufs)])
            ev_s[1].record(stream)
            torch.cuda.synchronize()
            rank_score_ms = ev_s[0].elapsed_time(ev_s[1]) / args.steps
            rank_probe_bytes = min(rank_bytes, shard.numel()) // 16384 * 16384
            rank_probe_ms, _ = probe_ms(rank_bufs, rank_probe_bytes, args.steps,
                                        ROTATE_WARMUP_STEPS if rotate_shards else 1)
            rank_score_timing = (
                f"{args.steps} launches back to back between one event pair over "
                f"{len(rank_bufs)} rotating shard copies, after {ROTATE_WARMUP_STEPS} untimed"
                if rotate_shards else
                f"{args.steps} launches back to back after a cache-evicting read")
            del shards, rank_bufs
            sharded[f"world_size_{ws_n}"] = {
                "rank": 0, "rank_keys": rank_keys,
                "rank_step_ms_back_to_back": rank_btb_ms,
                "rank_frac_of_peak_back_to_back":
                    rank_bytes / (rank_btb_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS
                    if rank_btb_ms else None,
                "rank_step_timing_back_to_back": (
                    f"{args.steps} steps back to back between one event pair over "
                    f"{n_shards} rotating shard copies, after {ROTATE_WARMUP_STEPS} untimed")
                    if rank_btb_ms else None,
                "rank_step_ms": rank_mean,
                "rank_hbm_gbps": rank_bytes / (rank_mean * 1e-3) / 1e9,
                "rank_frac_of_peak": rank_bytes / (rank_mean * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "rank_scorer_ms_back_to_back": rank_score_ms,
                "rank_scorer_timing": rank_score_timing,
                "rank_scorer_hbm_gbps": rank_bytes / (rank_score_ms * 1e-3) / 1e9,
                "stream_read_probe_same_bytes_ms": rank_probe_ms,
                "rank_scorer_frac_of_probe":
                    (rank_bytes / rank_score_ms) / (rank_probe_bytes / rank_probe_ms),
                "owner_merge_ms": sum(merge_ms) / len(merge_ms),
                "merged_rows_per_head": ws_n * R}
            del shard, splane, spart, all_rows, merged

    # Timed region 2: the three-launch chain with an event between every
    # kernel, for per-kernel durations (the events lengthen these steps).
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps per kernel", file=sys.stderr, flush=True)
    for i in range(args.steps):
        if flush is not None:
            flush.sum()
        step_three(events[i])
    torch.cuda.synchronize()
    # Timed region 3: the scorer alone, K launches back to back between one
    # event pair, for its per-launch duration without the dispatch delay that
    # follows each event record. Where the headline rotates index-K copies,
    # so does this, after ROTATE_WARMUP_STEPS untimed launches: measured at
    # config 5 from idle (events every 25 launches), the scorer alone takes
    # about 300 launches to settle (98 -> 82.4 us per launch). Otherwise the
    # launches follow a cache-evicting read.
    print(f"[bench] timing {args.steps} back-to-back scorer launches", file=sys.stderr,
          flush=True)
    n_rot = len(kcopies)
    if rotate:
        for i in range(ROTATE_WARMUP_STEPS):
            score(kcopies[i % n_rot])
    elif flush is not None:
        flush.sum()
    b2b = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    b2b[0].record(stream)
    for i in range(args.steps):
        score(kcopies[i % n_rot])
    b2b[1].record(stream)
    torch.cuda.synchronize()
    score_b2b_ms = b2b[0].elapsed_time(b2b[1]) / args.steps
    # Timed region 3b: the streaming-read probe (a plain read, no other work)
    # over as many index-K bytes, timed the same way (the same copies, the same
    # warm-up), and over 4 GiB (where the launch's ramp and tail weigh least):
    # the streaming ceilings the scorer's rate is read against.
    probe_bytes = max(16384, launch_bytes // 16384 * 16384)
    probe_bytes = min(probe_bytes, k.numel() // 16384 * 16384)
    probe_launch_ms, probe_shapes = probe_ms(kcopies, probe_bytes, args.steps,
                                             ROTATE_WARMUP_STEPS if rotate else 1)
    del kcopies
    big = torch.empty(PROBE_BIG_BYTES, dtype=torch.uint8, device=dev)
    big_ms, big_shapes = probe_ms([big], PROBE_BIG_BYTES, 10, 2)
    del big
    if int(errors.item()) != 0:
        raise RuntimeError(f"device error counter = {int(errors.item())}")
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    prefill = None
    if not args.no_prefill:
        print("[bench] prefill chain", file=sys.stderr, flush=True)
        prefill = prefill_figure(dev, stream)

    pairs = step_stats(step_ms, launch_bytes, keys)
    score_ms = [ev[0].elapsed_time(ev[1]) for ev in events]
    select_ms = [ev[1].elapsed_time(ev[2]) for ev in events]
    merge_ms = [ev[2].elapsed_time(ev[3]) for ev in events]
    mean = lambda xs: sum(xs) / len(xs)
    value = keys / (ms_step * 1e-3)
    e2e_gbps = launch_bytes / (ms_step * 1e-3) / 1e9
    achieved = launch_bytes / (score_b2b_ms * 1e-3) / 1e9
    traffic = load_traffic(launch_bytes)  # HBM bytes per launch, from the committed counters
    probe_gbps = probe_bytes / (probe_launch_ms * 1e-3) / 1e9
    big_gbps = PROBE_BIG_BYTES / (big_ms * 1e-3) / 1e9

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
                   "cache_flush_between_steps": flush is not None},
        "e2e": {"step": headline_name,
                "timing": timing,
                "hbm_gbps": e2e_gbps, "frac_of_peak": e2e_gbps / HBM_PEAK_GBPS,
                "target_frac_of_peak": 0.70,
                # per-step latency: an event pair around each step after a
                # cache-evicting read (it also holds the dispatch delay that
                # back-to-back steps overlap), with its percentiles
                "per_step_event_pairs": {kk: vv for kk, vv in pairs.items()
                                         if kk != "keys_per_s"},
                # each key is scored against its request's 4 * dql query rows
                "dot_products_per_s": value * 4 * w.dql,
                "kernels_ms_three_launch_chain": {
                    "score_decode": mean(score_ms), "top16_select": mean(select_ms),
                    "top16_merge": mean(merge_ms),
                    "step_with_kernel_events": mean([ev[0].elapsed_time(ev[3])
                                                     for ev in events])},
                "score_decode_ms_back_to_back": score_b2b_ms,
                "other_forms": alt,
                "sharded_rank_share": sharded or None,
                "wall_s_headline_steps": wall},
        "roofline": {"kernel": "score_decode", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "algorithmic_bytes_per_launch": launch_bytes,
                     "launch_ms": score_b2b_ms,
                     "launch_ms_source": (
                         "K scorer launches back to back between one event pair" +
                         (f", launch i on index-K copy i % {n_copies}, after "
                          f"{ROTATE_WARMUP_STEPS} untimed" if rotate else
                          ", after a cache-evicting read")),
                     "traffic": None if traffic is None else traffic["total_bytes"],
                     "traffic_detail": traffic,
                     "mfma": load_mfma(),
                     "stream_read_probe": {
                         "what": "msa_stream_read_probe, a plain streaming read with no other "
                                 "work, launches back to back between one event pair (over "
                                 "as many bytes: the scorer's copies and warm-up); the "
                                 "fastest of its shapes at each size (persistent: one "
                                 "contiguous run per wave, one wave per SIMD; 2-16: that "
                                 "many 16 KiB blocks per wave over a grid covering the buffer)",
                         "same_bytes": {"bytes": probe_bytes, "launch_ms": probe_launch_ms,
                                        "achieved": probe_gbps,
                                        "frac_of_peak": probe_gbps / HBM_PEAK_GBPS,
                                        "launch_ms_by_shape": probe_shapes},
                         "4_gib": {"bytes": PROBE_BIG_BYTES, "launch_ms": big_ms,
                                   "achieved": big_gbps,
                                   "frac_of_peak": big_gbps / HBM_PEAK_GBPS,
                                   "launch_ms_by_shape": big_shapes},
                         "scorer_frac_of_probe_same_bytes": achieved / probe_gbps,
                         "scorer_frac_of_probe_4_gib": achieved / big_gbps}},
        "prefill": prefill,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
