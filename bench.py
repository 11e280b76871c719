"""Paged-attention decode benchmark on one MI355X.

One step = one pass of the whole decode hot path over one batch: the
per-sequence v1/v2 choice, Phase 1 (partition kernel) and Phase 2 (reduce
kernel), one call of the library's C ABI (arguments marshalled once, before
timing).  The headline workload is the largest that fits one GPU: the ragged
MHA ALiBi bf16 batch (256 sequences, 32 query / 32 KV heads, head size 128,
block size 16, lognormal lengths of median 2048 clipped to [16, 32768], about
14 GB of KV; the auto path mixes v1 and v2 there, so both kernels are timed).
The two other long-context workloads (4 x 100000 fp16 tokens; fp8 KV, 32 x
32768) are timed in the same process and reported inside the line
(``also_timed``; ``--also none`` skips them), and the other decode paths
(balanced split, work list, and auto_ws -- the auto call given a counters
buffer, which schedules the batch for balance) on the headline workload's
same inputs (``paths_on_this_workload``; auto_ws on the other two workloads
too; ``--compare none`` skips them).  tmp_out is float32 by default
(``--partials out``: the query dtype).

Inputs are resident in HBM before timing.  By default the step rotates over
``--copies`` independent copies of the KV pool (4 x 14 GB for the headline),
so the 256 MB Infinity Cache cannot serve one step's KV from the previous
step; ``--hot`` times a single copy instead.  W warm-up steps, then exactly K timed steps
between device synchronisations give ms_per_step and value.  The same K
steps are then run again with the library's profiling hook
(pa_set_timing_events): every launch records HIP events at the kernel's own
start and end, giving the average partition-kernel duration used for the
roofline of the dominant kernel (``frac``) and the partition-start to
reduce-end time of the whole step (``step_frac``); the recording adds a few
microseconds per step, so it is not part of the wall-clock region.  The fp64 CPU oracle is timed on a bounded sample of the same
workload for the CPU baseline.  ``--window W`` / ``--softcap C`` turn on the
decode options (sliding window over the last W + 1 keys, logit soft cap);
the KV bytes then count the keys inside the window only.  ``--layout
block_rows`` repacks the same caches into the [num_blocks, num_kv_heads,
block_size, head_size] layout and times the kernels for that layout.

Prints one JSON line (stdout); progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-attn decode µs/step + effective KV HBM GB/s (% of peak), 1 MI355X"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(prefill: bool = False) -> str:
    """Hash of the library sources a measurement depends on (the decode path:
    every source but the prefill kernel's own files and the stream-read
    hook's; prefill: every source but the hook's): counter figures taken on
    other sources are not reported."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_297_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name == "pa_stream.hip" or (not prefill and name.startswith("pa_prefill")):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl, path: str, cu: int, B, window_left: int = -1,
                      partials: str = "f32", kv_layout: str = "decode") -> dict:
    """Bytes each launch must move at minimum (each KV byte inside the window
    once per KV head; partial rows in the partial dtype)."""
    import numpy as np
    lens = wl.lens.astype(np.int64)
    t_lo = np.maximum(0, lens - 1 - window_left) if window_left >= 0 else np.zeros_like(lens)
    eff = lens - t_lo                                 # keys inside the window
    esz_q = wl.query.element_size()
    kv = int(eff.sum()) * wl.num_kv_heads * wl.head_size * 2 * wl.kv_elem_bytes
    q = wl.num_seqs * wl.num_heads * wl.head_size * esz_q
    out = q
    blocks = int(((lens + wl.block_size - 1) // wl.block_size - t_lo // wl.block_size).sum())
    table = blocks * 4 + wl.num_seqs * 4
    # Partitions holding a key of the window.
    parts = np.where(lens > 0, (lens + 511) // 512 - t_lo // 512, 0)
    if path in ("v1", "split", "worklist", "auto_ws"):
        # split / worklist / auto_ws: the pieces' partials are scratch inside one launch,
        # not part of the result; the minimum is that of v1.
        v2 = np.zeros_like(lens, dtype=bool)
    elif path == "v2":
        v2 = np.ones_like(lens, dtype=bool)
    else:
        v2 = np.array([B.should_use_v2(wl.num_seqs, wl.num_kv_heads, int(n), cu) for n in eff])
    h, d = wl.num_heads, wl.head_size
    esz_t = 4 if partials == "f32" else esz_q
    if path == "auto" and B.auto_uses_slots(
            wl.num_seqs, wl.num_heads, wl.num_kv_heads, wl.head_size, wl.block_size,
            wl.max_seq_len, wl.dtype, wl.kv_cache_dtype, window_left, 0.0, kv_layout):
        # The slot form: every sequence of two or more partitions goes through
        # partial rows merged by the reduce -- at least one row per (sequence,
        # head), a statistics pair per partition slot (pieces and padding).
        multi = parts > 1
        rows = int(multi.sum()) * h
        tmp = rows * d * esz_t
        stats = int((parts * multi).sum()) * h * 8
        out_p1 = int((~multi).sum()) * h * d * esz_q
        out_p2 = int(multi.sum()) * h * d * esz_q
        reduce_read = rows * d * esz_t + stats
        return {"kv": kv, "partition": kv + q + table + tmp + stats + out_p1,
                "reduce": reduce_read + out_p2 + wl.num_seqs * 4,
                "step": kv + q + table + tmp + stats + out + reduce_read,
                "any_v2": bool(multi.any())}
    tmp = int((parts * v2).sum()) * h * d * esz_t   # partial outputs
    stats = int((v2 * wl.max_num_partitions).sum()) * h * 8   # values and padding
    multi = v2 & (parts > 1)
    out_p1 = int((~multi).sum()) * h * d * esz_q
    out_p2 = int(multi.sum()) * h * d * esz_q
    reduce_read = int((parts * multi).sum()) * h * (d * esz_t + 8)
    return {"kv": kv, "partition": kv + q + table + tmp + stats + out_p1,
            "reduce": reduce_read + out_p2 + wl.num_seqs * 4,
            "step": kv + q + table + tmp + stats + out + reduce_read,
            "any_v2": bool(v2.any())}


def read_traffic(workload_name: str, src_hash: str, call_path: str, partials: str):
    """HBM bytes per partition launch from the committed counter summary, if
    it was measured on the current kernel sources with the same path and
    partial dtype."""
    path = os.path.join(PROFILES, f"traffic_pa_partition_{workload_name}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        header = f.readline()
        if f"path={call_path}" not in header or f"partials={partials}" not in header:
            return None
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_hash") != src_hash:
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def stream_read_ceiling(B, gib: int, reps: int = 10) -> float:
    """GB/s of the library's plain streaming read (pa_stream_read) over a
    fresh gib-GiB device buffer, one launch per pass: 16-byte loads, one
    workgroup per CU (measured on MI355X: 7.17 TB/s; 2-32 workgroups per CU
    read 6.95-7.04 TB/s), median of ``reps`` passes after two warm-ups.  The
    buffer is far larger than the 256 MB Infinity Cache, so every read comes
    from HBM.  (Reading the workload's own pools instead, a few hundred MB
    per launch, read 6.3-6.9 TB/s: launch ramps weigh more there.)"""
    import numpy as np
    import torch

    n = gib << 30
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(B.device_cu_count(), dtype=torch.int32, device="cuda")
    for _ in range(2):
        B.stream_read(buf, sink)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.stream_read(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del buf
    torch.cuda.empty_cache()
    gbs = n / (float(np.median(ts)) * 1e-3) / 1e9
    log(f"stream read ceiling: {gbs:.1f} GB/s over {gib} GiB")
    return round(gbs, 1)


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or 'unknown'."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s: float, window_left: int = -1, soft_cap: float = 0.0) -> dict:
    """The fp64 oracle as it is, on the host's cores: the first sequences of
    the same batch (up to 4 per thread), one per task on a thread pool as
    wide as the process's CPU affinity (at most 16; one BLAS thread each),
    whole passes over that sample until ``budget_s`` of wall time is spent
    (at least one pass).  Device-to-host copies happen before the clock."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import pa_oracle as O
    from paged_kv_cache_297_amd import workloads as W

    threads = max(1, min(len(os.sched_getaffinity(0)), 16))
    alibi = None if wl.alibi_slopes is None else wl.alibi_slopes.cpu().double().numpy()

    def eff(L: int) -> int:
        return min(L, window_left + 1) if window_left >= 0 else L

    per_token = wl.num_kv_heads * wl.head_size * 2 * wl.kv_elem_bytes
    kv_step = sum(eff(int(L)) for L in wl.lens) * per_token
    sample = list(range(min(wl.num_seqs, 4 * threads)))
    hosts = {s: W.host_subset(wl, [s]) for s in sample}

    def one(s: int) -> int:
        host = hosts[s]
        O.paged_attention(host["query"], host["key_cache"], host["value_cache"],
                          host["block_tables"], host["seq_lens"], wl.scale,
                          q_kind=wl.q_kind, kv_kind=wl.kv_kind, k_scale=wl.k_scale,
                          v_scale=wl.v_scale, alibi_slopes=alibi,
                          max_num_partitions=wl.max_num_partitions, seqs=[s],
                          window_left=window_left, soft_cap=soft_cap)
        return eff(int(wl.lens[s])) * per_token

    passes, kv_done = 0, 0
    with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        while True:
            kv_done += sum(ex.map(one, sample))
            passes += 1
            spent = time.perf_counter() - t0
            if spent >= budget_s or passes >= 50:
                break
    gbs = kv_done / spent / 1e9
    return {"value": round(gbs, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"{passes} passes over the first {len(sample)} of the batch's "
                       f"{wl.num_seqs} sequences ({kv_done / 1e6:.1f} MB of KV), v1 + v2 "
                       f"partials + merge in fp64, {threads} threads (one sequence per task, one "
                       f"BLAS thread each), {spent:.1f} s wall; device-to-host copies excluded"),
            "us_per_step_extrapolated": round(spent / kv_done * kv_step * 1e6, 1)}


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 matrix peak


def prefill_flops(qlens, klens, num_heads: int, head_size: int) -> int:
    """Useful flops of a causal prefill batch: 2 * D multiply-adds for QK^T and
    2 * D for PV per visible (query, key) pair and head.  Query i of a
    sequence sits at position nk - nq + i and sees keys 0 .. that position."""
    pairs = 0
    for nq, nk in zip(qlens, klens):
        nq, nk = int(nq), int(nk)
        lo = nk - nq  # keys visible to query 0, minus one
        for_all = sum(max(0, min(nk, lo + i + 1)) for i in range(nq))
        pairs += for_all
    return 4 * head_size * num_heads * pairs


def bench_prefill(args) -> int:
    """Times paged_prefill on a prefill workload; prints the JSON line."""
    import numpy as np
    import torch

    from paged_kv_cache_297_amd import binding as B
    from paged_kv_cache_297_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    B.load_library()
    wl = W.make_prefill_workload(args.prefill, device="cuda")
    stream = torch.cuda.current_stream()
    out = torch.empty_like(wl.query)
    call = B.PreparedPrefill(out, wl.query, wl.key_cache, wl.value_cache, wl.num_kv_heads,
                             wl.scale, wl.block_tables, wl.cu_seq_q, wl.cu_seq_k, wl.max_seq_q,
                             wl.max_seq_k, causal=True, stream=stream)
    lib = B.load_library()
    # At least 50 warm-up launches: the compute-bound kernel's launch time
    # falls over its first ~40 launches as the GPU clock ramps up under load
    # (kernel traces: 390 -> 330 us on the fresh-prompt batch).
    warmup = max(args.warmup, 50)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for ev in events:
        for e in ev:
            e.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for ev in events:
        lib.pa_set_timing_events(ev[0].cuda_event, ev[1].cuda_event, None, None)
        call()
    torch.cuda.synchronize()
    B.set_timing_events()
    kern_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    flops = prefill_flops(wl.qlens, wl.klens, wl.num_heads, wl.head_size)
    ms = wall * 1e3 / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    kavg = float(kern_ms.mean())
    achieved = flops / (kavg * 1e-3) / 1e12
    result = {
        "metric": "paged prefill attention TFLOP/s (causal), 1 MI355X",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {torch.float16: "f16", torch.bfloat16: "bf16"}[wl.dtype], "data": "synthetic",
        "config": {"workload": (f"{wl.name}: paged prefill, num_seqs={wl.num_seqs}, "
                                f"query tokens {int(wl.qlens.min())}..{int(wl.qlens.max())}, "
                                f"keys {int(wl.klens.min())}..{int(wl.klens.max())}, "
                                f"num_heads={wl.num_heads}, num_kv_heads={wl.num_kv_heads}, "
                                f"head_size={wl.head_size}, block_size={wl.block_size}, causal"),
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "kernel": "pa_prefill_kernel", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops_per_launch": flops, "avg_launch_ms": round(kavg, 5),
                     "kernel_source_hash": kernel_source_hash(prefill=True)},
    }
    print(json.dumps(result), flush=True)
    return 0


def prepare(number: int, args, B, W, paths):
    """Builds workload ``number`` with ``--copies`` rotating copies (same bytes at
    other addresses) and the marshalled calls of each path in ``paths``;
    returns (base, {path: calls}, hold)."""
    import torch

    copies = 1 if args.hot else max(1, args.copies)
    log(f"building workload {number} x{copies}")
    base = W.make_workload(number, device="cuda", seed=1000 + number)
    if args.layout == "block_rows":
        base.key_cache, base.value_cache = W.to_block_rows(base.key_cache, base.value_cache)
        torch.cuda.empty_cache()
    wls = [base]
    for _ in range(1, copies):
        # Same bytes at other addresses: identical work, no cache reuse across steps.
        w2 = W.Workload(**{**base.__dict__})
        w2.key_cache = base.key_cache.clone()
        w2.value_cache = base.value_cache.clone()
        w2.query = base.query.clone()
        w2.block_tables = base.block_tables.clone()
        wls.append(w2)
    stream = torch.cuda.current_stream()
    calls, keep = {path: [] for path in paths}, []
    for wl in wls:
        out, es, ml, to = wl.alloc_outputs(args.partials)
        keep.append((out, es, ml, to))
        common = (out, es, ml, to, wl.query, wl.key_cache, wl.value_cache, wl.num_kv_heads,
                  wl.scale, wl.block_tables, wl.seq_lens, wl.block_size, wl.max_seq_len)
        kw = dict(alibi_slopes=wl.alibi_slopes, kv_cache_dtype=wl.kv_cache_dtype,
                  k_scale=wl.k_scale, v_scale=wl.v_scale, stream=stream,
                  window_left=args.window, logits_soft_cap=args.softcap,
                  kv_layout=args.layout)
        # Arguments are checked and marshalled once per input copy; a timed step
        # is one C call (v1 = partition kernel only; v2 / auto = partition +
        # reduce; split, worklist = one launch).
        for path in paths:
            if path == "v1":
                calls[path].append(lambda out=out, wl=wl, kw=kw: B.paged_attention_v1(
                    out, wl.query, wl.key_cache, wl.value_cache, wl.num_kv_heads, wl.scale,
                    wl.block_tables, wl.seq_lens, wl.block_size, wl.max_seq_len, **kw))
            elif path in ("split", "worklist", "auto_ws"):
                calls[path].append(B.PreparedCall(
                    path, *common, **kw, counters=B.split_counters(wl.num_seqs, wl.num_heads)))
            else:
                calls[path].append(B.PreparedCall(path, *common, **kw))
    return base, calls, (wls, keep)


def time_steps(calls, steps: int, warmup: int, B):
    """W warm-up steps, K timed steps between device synchronisations (wall
    clock), then the same K steps again with the library's profiling hook
    recording each kernel's own start / end.  Returns (wall_s, partition_ms,
    reduce_ms, step_ms) with the event arrays per step."""
    import numpy as np
    import torch

    lib = B.load_library()
    stream = torch.cuda.current_stream()
    n = len(calls)

    def launch(i: int, ev=None):
        if ev is not None:
            # The library records these at each kernel's own start and end.
            lib.pa_set_timing_events(*ev)
        calls[i % n]()

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    # partition start/stop, reduce start/stop of every timed step; each event
    # is recorded once here so that its handle exists.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for ev in events:
        for e in ev:
            e.record(stream)
    handles = [tuple(e.cuda_event for e in ev) for ev in events]
    log(f"timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        launch(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The same K steps again with the kernels recording their own start / end
    # (the recording adds a few microseconds per step, so it is kept out of
    # the wall-clock region above).
    log(f"timing {steps} steps per kernel")
    for i in range(steps):
        launch(i, handles[i])
    torch.cuda.synchronize()
    B.set_timing_events()
    part = np.array([e[0].elapsed_time(e[1]) for e in events])
    red = np.array([e[2].elapsed_time(e[3]) for e in events])
    step = np.array([e[0].elapsed_time(e[3]) for e in events])
    return wall, part, red, step


def measure(number: int, args, B, W, cu: int, keep_base: bool = False,
            other_paths=()) -> dict:
    """Times workload ``number`` on the chosen path; the figures of one bench
    line (the step, the dominant kernel's roofline, the whole step's).  With
    ``keep_base`` the first copy of the inputs is returned too (for the CPU
    baseline); the others are freed.  ``other_paths`` are timed afterwards on
    the same inputs (wall clock of the same K steps) for comparison."""
    import numpy as np
    import torch

    paths = [args.path] + [q for q in other_paths if q != args.path]
    base, calls, hold = prepare(number, args, B, W, paths)
    ab = algorithmic_bytes(base, args.path, cu, B, args.window, args.partials, args.layout)
    wall, part_ms, red_ms, step_ms = time_steps(calls[args.path], args.steps, args.warmup, B)
    if args.path in ("v1", "split", "worklist", "auto_ws") or not ab["any_v2"]:
        # No reduce kernel runs (an all-v1 auto call records its reduce events
        # back to back; their gap is event overhead, not work).
        red_ms = np.zeros(len(part_ms))
        step_ms = part_ms
    ms = wall * 1e3 / args.steps
    others = {}
    for q in paths[1:]:
        log(f"timing {args.steps} steps of path {q}")
        w2, pm2, _, _ = time_steps(calls[q], args.steps, args.warmup, B)
        others[q] = {"us_per_step": round(w2 * 1e6 / args.steps, 2),
                     "kv_gbs": round(ab["kv"] / (w2 / args.steps) / 1e9, 1),
                     "kernel_avg_ms": round(float(pm2.mean()), 5)}
    part_avg = float(part_ms.mean())
    step_avg = float(step_ms.mean())
    achieved = ab["partition"] / (part_avg * 1e-3) / 1e9
    step_achieved = ab["step"] / (step_avg * 1e-3) / 1e9
    options = args.window != -1 or args.softcap != 0.0
    lens = base.lens
    dtype = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[base.dtype]
    if base.kv_cache_dtype == "fp8_e4m3":
        dtype = f"{dtype} (fp8 e4m3 KV)"
    copies = len(calls[args.path])
    res = {
        "name": base.name,
        "dtype": dtype,
        "workload": (f"{base.name}: paged-attention decode, num_seqs={base.num_seqs}, "
                     f"num_heads={base.num_heads}, num_kv_heads={base.num_kv_heads}, "
                     f"head_size={base.head_size}, block_size={base.block_size}, "
                     f"seq_lens {int(lens.min())}..{int(lens.max())} "
                     f"(sum {int(lens.sum())}), path={args.path}, partials={args.partials}"
                     + (f", kv_layout={args.layout}" if args.layout != "decode" else "")
                     + (f", window_left={args.window}, soft_cap={args.softcap:g}"
                        if options else "")),
        "ms_per_step": ms,
        "kv_gbs": ab["kv"] / (ms * 1e-3) / 1e9,
        "ab": ab,
        "part_avg": part_avg,
        "red_avg": float(red_ms.mean()),
        "step_avg": step_avg,
        "step_p": [float(np.percentile(step_ms, q)) * 1e3 for q in (10, 50, 90)],
        "achieved": achieved,
        "step_achieved": step_achieved,
        "copies": copies,
        "options": options,
        "other_paths": others,
        "base": base if keep_base else None,
    }
    del calls, hold, base
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5],
                    help="the headline workload (default 4: ragged MHA ALiBi bf16, the "
                         "largest that fits one GPU)")
    ap.add_argument("--compare", default="split,worklist,auto_ws",
                    help="other decode paths timed on the headline workload, reported inside the "
                         "line (comma list, or 'none')")
    ap.add_argument("--also", default="3,5",
                    help="other workloads timed in the same process, reported inside the line "
                         "(comma list, or 'none')")
    ap.add_argument("--path", default="auto",
                    choices=["auto", "v2", "v1", "split", "worklist", "auto_ws"])
    ap.add_argument("--partials", default="f32", choices=["f32", "out"],
                    help="dtype of tmp_out: float32 (the default contract) or the query dtype")
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--hot", action="store_true", help="one copy of the inputs (cache-hot)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--window", type=int, default=-1, metavar="W",
                    help="sliding window: attend to the last W + 1 keys (-1: off)")
    ap.add_argument("--softcap", type=float, default=0.0, metavar="C",
                    help="logit soft cap C * tanh(s / C) (0: off)")
    ap.add_argument("--layout", default="decode", choices=["decode", "block_rows"],
                    help="KV cache layout of the decode call (16-bit caches for block_rows)")
    ap.add_argument("--stream-gib", type=int, default=4, metavar="GIB",
                    help="also time the library's streaming read of GIB GiB: the practical HBM "
                         "read ceiling (0: skip)")
    ap.add_argument("--prefill", default=None, choices=["prefill_bf16", "chunked_bf16"],
                    help="time paged prefill on this workload instead of decode")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode path "
              "has no multi-GPU part in this library.", file=sys.stderr)
        return 2

    if args.prefill:
        return bench_prefill(args)

    import torch

    from paged_kv_cache_297_amd import binding as B
    from paged_kv_cache_297_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    B.load_library()
    torch.cuda.set_device(0)
    cu = B.device_cu_count()
    also = [] if args.also.strip().lower() in ("", "none") else [
        int(x) for x in args.also.split(",") if int(x) != args.workload]

    compare = [] if args.compare.strip().lower() in ("", "none") else [
        q.strip() for q in args.compare.split(",")]
    for q in compare:
        if q not in ("auto", "v2", "v1", "split", "worklist", "auto_ws"):
            print(f"unknown path {q!r} in --compare", file=sys.stderr)
            return 2
    head = measure(args.workload, args, B, W, cu, keep_base=not args.no_cpu_baseline,
                   other_paths=compare)
    others = [measure(n, args, B, W, cu, other_paths=[q for q in compare if q == "auto_ws"])
              for n in also]

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy: {n} bytes x3")

    # The stream-read ceiling, after the timed steps (allocating its buffer
    # before them slowed the steps by 6%).
    stream_gbs = stream_read_ceiling(B, args.stream_gib) if args.stream_gib > 0 else None

    src_hash = kernel_source_hash()
    ab = head["ab"]
    traffic = (read_traffic(head["name"], src_hash, args.path, args.partials)
               if head["copies"] > 1 and not head["options"] and args.layout == "decode"
               else None)
    ms = head["ms_per_step"]
    result = {
        "metric": METRIC,
        "value": round(head["kv_gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "pct_of_peak": round(100.0 * head["kv_gbs"] / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": {
            "workload": head["workload"],
            "path": args.path,
            "partials": args.partials,
            "window_left": args.window,
            "logits_soft_cap": args.softcap,
            "kv_layout": args.layout,
            "kv_bytes_per_step": ab["kv"],
            "inputs": ("cache-hot single copy" if head["copies"] == 1 else
                       f"{head['copies']} rotating copies of the KV pool (L2/MALL-cold)"),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("pa_partition (Phase 1)" if args.layout == "decode"
                       else "pa_partition_nhd (Phase 1, block-rows layout)"),
            "achieved": round(head["achieved"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["achieved"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": ab["partition"],
            "avg_launch_ms": round(head["part_avg"], 5),
            "reduce_avg_launch_ms": round(head["red_avg"], 5),
            "step_algorithmic_bytes": ab["step"],
            "step_avg_ms": round(head["step_avg"], 5),
            "step_achieved": round(head["step_achieved"], 1),
            "step_frac": round(head["step_achieved"] / HBM_PEAK_GBS, 4),
            "event_step_us_p10_p50_p90": [round(x, 2) for x in head["step_p"]],
            "kernel_source_hash": src_hash,
            "stream_read_gbs": stream_gbs,
            "frac_of_stream_read": (round(head["achieved"] / stream_gbs, 4)
                                    if stream_gbs else None),
        },
        "paths_on_this_workload": head["other_paths"],
        "also_timed": [{
            "workload": o["workload"], "dtype": o["dtype"],
            "us_per_step": round(o["ms_per_step"] * 1e3, 2),
            "kv_gbs": round(o["kv_gbs"], 1),
            "pct_of_peak": round(100.0 * o["kv_gbs"] / HBM_PEAK_GBS, 2),
            "kernel_avg_ms": round(o["part_avg"], 5),
            "kernel_frac": round(o["achieved"] / HBM_PEAK_GBS, 4),
            "reduce_avg_ms": round(o["red_avg"], 5),
            "step_frac": round(o["step_achieved"] / HBM_PEAK_GBS, 4),
            "event_step_us_p10_p50_p90": [round(x, 2) for x in o["step_p"]],
            "paths_on_this_workload": o["other_paths"],
        } for o in others],
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(head["base"], args.cpu_budget, args.window,
                                              args.softcap)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
