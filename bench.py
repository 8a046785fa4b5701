#!/usr/bin/env python3
"""Throughput of the generation-logprob reduction on one MI355X.

One step = one flare_logprobs_run over one frame of the speculative-verify
workload: 128 slots x T=8 verify rows x V=248,320 bf16 logits, emitted counts
uniform in 1..8 (rows past each slot's prefix hold NaN/+inf garbage and are
never read), K=20 natural alternatives.  Inputs are seeded synthetic logits
(Gumbel plus a +10 peak), resident in HBM before timing; `--copies` rotated
copies of the logits keep the 256 MB Infinity Cache from serving repeats.

Prints one JSON line: rows/s over the whole timed region (each call made
through a prepared binding, Plan.bind, so that one call is one C call), the
roofline of the reduction launch (algorithmic bytes / its mean duration, from a
second region of the same number of reduction launches back to back, HIP events
only at its ends, on the launch stream), and the CPU oracle timed on a bounded
sample of the same rows.  The HBM traffic of the reduction launch and its
rocprofv3 trace average come from the summary under profiles/, and only while
the kernel source is the one that summary was taken on.

`--prompt P1` (or P2) measures prompt scoring instead: one step scores one
prefill chunk (P1: 128 rows x V=248,320 bf16, each row's target logprob, rank
and twenty alternatives), reported the same way in its own JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
# Calls captured in the timed HIP graph.  Each replay costs a fixed few
# microseconds of launch (about 6 us for a one-call graph of C1 or C3), so
# the graph holds a serving loop's worth of calls, cycling the logits copies.
GRAPH_CALLS = 32
# Calls in each diagnostic region (the reduction launches alone, the merge
# launches alone, the graph replay): at least this many, so that their
# averages describe a warm GPU whatever --steps is.
DIAG_CALLS = 200
# Whole calls the GPU has run before the diagnostic regions start: when the
# warm-up and the timed steps were fewer, untimed calls make up the rest.
# The first few hundred calls after an idle GPU run slower while it ramps up,
# and the diagnostic regions describe the kernels on a warm GPU.
DIAG_WARM_CALLS = 800
KERNEL_SOURCES = ("full_vocab_logprob_amd/csrc/flp_kernels.hip",
                  "full_vocab_logprob_amd/csrc/flp_internal.h")
# The rocprofv3 summary of each workload (kernel trace average and HBM bytes
# per reduction launch), keyed by the workload's tag (see workload_tag).
TRAFFIC_SUMMARIES = {
    "C1": "profiles/reduce_kernel_plain_decode_fp32_K20.txt",
    "C2": "profiles/reduce_kernel_decode_batch_fp32_K20.txt",
    "C3": "profiles/reduce_kernel_speculative_verify_bf16_K20.txt",
    "C3-K0": "profiles/reduce_kernel_speculative_verify_bf16_K0.txt",
    "C4": "profiles/reduce_kernel_tie_stress_bf16_selected40.txt",
    "C5": "profiles/reduce_kernel_large_batch_fp32_K20.txt",
    "C5-K0": "profiles/reduce_kernel_large_batch_fp32_K0.txt",
    "C5-sel": "profiles/reduce_kernel_large_batch_fp32_selected128.txt",
    "P1": "profiles/reduce_kernel_prompt_scoring_bf16.txt",
    "P2": "profiles/reduce_kernel_prompt_scoring_fp32.txt",
}


def workload_tag(config: str, K=None, selected=None) -> str:
    """The summary key of a generation workload: the configuration, with the
    K or selected-ID override of a sweep."""
    if selected == "all":
        return f"{config}-sel"
    if K is not None:
        return f"{config}-K{K}"
    return config


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profile_field(config: str, name: str):
    """A number from the committed rocprofv3 summary of this workload (HBM
    bytes per reduction launch, the trace's average launch duration), or None
    when the summary is missing, covers another workload, or was taken on a
    different kernel source."""
    if config not in TRAFFIC_SUMMARIES:
        return None
    path = os.path.join(ROOT, TRAFFIC_SUMMARIES[config])
    if not os.path.exists(path):
        return None
    text = open(path).read()
    fields = dict(re.findall(r"^([a-z_0-9]+):\s*(\S+)\s*$", text, flags=re.M))
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    if fields.get("workload") != config:
        return None
    try:
        return float(fields[name])
    except (KeyError, ValueError):
        return None


def host_cpu() -> str:
    """The host CPU model and its logical core count (lscpu's model name)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical cores"


def timed_regions(step, K: int, warmup: int, stream, graph=None):
    """The timed part of a bench, after `warmup` untimed whole calls:
    region 1, K whole calls back to back (the throughput); then, once the GPU
    has run DIAG_WARM_CALLS whole calls in all, region 2, the same calls'
    reduction launches alone, back to back, max(K, DIAG_CALLS) of them (the
    reduction's mean duration: the roofline); region 3, as many merge
    launches alone; then `graph()`, if given, for the graph-replay rate.
    Every region is
    bracketed by a synchronization and HIP events at its two ends only, on
    the launch stream, so no event sits between two launches."""
    import torch

    for i in range(warmup):
        step(i)

    def region(phase, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record(stream)
        for i in range(n):
            step(warmup + i, phase)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, time.perf_counter() - w0

    ms_per_step, wall = region("all", K)
    for i in range(max(0, DIAG_WARM_CALLS - warmup - K)):
        step(i)
    reduce_ms, _ = region("reduce", max(K, DIAG_CALLS))
    merge_ms, _ = region("merge", max(K, DIAG_CALLS))
    g = graph() if graph is not None else None
    if reduce_ms > ms_per_step:
        print(f"[bench] warning: reduction launches took {reduce_ms * 1e3:.1f} us each, more "
              f"than a whole call ({ms_per_step * 1e3:.1f} us): clock drift between regions",
              file=sys.stderr, flush=True)
    return ms_per_step, wall, reduce_ms, merge_ms, g


def roofline(config: str, kernel: str, algo_bytes: float, reduce_ms: float, packed=False):
    achieved = algo_bytes / (reduce_ms / 1e3) / 1e9
    trace_ns = None if packed else profile_field(config, "reduce_trace_average_ns")
    return {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
            "traffic": None if packed else profile_field(config, "traffic_bytes_per_launch"),
            "profile_trace_average_us": None if trace_ns is None else trace_ns / 1e3,
            "profile_frac": None if trace_ns is None
            else algo_bytes / (trace_ns / 1e9) / 1e9 / PEAK_HBM_GBPS}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=600,
                    help="untimed calls right before the timed region (about 45 ms of load: "
                         "the first few hundred calls after an idle GPU run slower)")
    ap.add_argument("--config", default="C3")
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--K", type=int, default=None,
                    help="override the configuration's K (throughput sweeps, e.g. K=0)")
    ap.add_argument("--selected", default=None, choices=("all",),
                    help="every slot lists 128 caller-selected IDs (the 128-ID sweep)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the CPU oracle baseline (0 disables it)")
    ap.add_argument("--check-rows", type=int, default=4,
                    help="oracle rows compared with the GPU output before timing")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run a plain elementwise FP32 copy of this many MiB "
                         "three times (scales HBM byte counters; 0 disables it)")
    ap.add_argument("--graph", type=int, default=1,
                    help="also time the calls replayed from one captured HIP graph (0: skip)")
    ap.add_argument("--prompt", default=None,
                    help="measure prompt scoring on this chunk (P1 or P2) instead")
    ap.add_argument("--records", type=int, default=0,
                    help="1: emitted counts and tokens read from int64 completion records")
    ap.add_argument("--packed", type=int, default=0,
                    help="1: the frame's committed rows packed into P physical rows "
                         "(shuffled slot order) and read through row offsets")
    ap.add_argument("--shards", type=int, default=0,
                    help="N > 0: the vocabulary split into N shards on this GPU (N shard "
                         "passes, then the cross-shard merge)")
    return ap.parse_args()


def copy_kernel(dev, mib):
    """A kernel of known traffic (reads and writes `mib` MiB each) so that
    profiler byte counters can be converted into bytes."""
    import torch
    src = torch.ones(mib * (1 << 18), dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def bench_prompt(args):
    """Prompt scoring: the same three timed regions as the generation bench."""
    import numpy as np
    import torch

    import __graft_entry__
    __graft_entry__._ensure_built()
    import full_vocab_logprob_amd as flp
    import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    spec = synth.PROMPT_CONFIGS[args.prompt]
    bf16 = spec.dtype == synth.BF16
    print(f"[bench] generating {spec.name}: {spec.description}", file=sys.stderr, flush=True)
    w = synth.make_prompt(spec)
    valid = w.valid_rows()
    algo_bytes = w.algorithmic_bytes()
    lg = torch.from_numpy(w.logits.view(np.int16) if bf16 else w.logits).to(dev)
    lg = (lg.view(torch.bfloat16) if bf16 else lg).reshape(-1)
    copies = [lg] + [lg.clone() for _ in range(1, args.copies)]
    targets = torch.from_numpy(np.ascontiguousarray(w.targets, np.int32)).to(dev)
    plan = flp.PromptPlan(w.rows, spec.V, spec.V_pad,
                          dtype=torch.bfloat16 if bf16 else torch.float32, device=0)
    ws = plan.workspace()
    out = plan.new_out(int(synth.POISON))
    stream = torch.cuda.current_stream()

    sh = stream.cuda_stream
    bound = {(c, ph): plan.bind(copies[c], targets, out, ws, phase=ph)
             for c in range(len(copies)) for ph in ("all", "reduce", "merge")}

    def step(i, phase="all"):
        bound[(i % len(copies), phase)](sh)

    def graph():
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        gr = torch.cuda.CUDAGraph()
        n = GRAPH_CALLS
        with torch.cuda.stream(side):
            with torch.cuda.graph(gr, stream=side):
                for c in range(n):
                    plan.run(copies[c % len(copies)], targets, out, ws)
        torch.cuda.synchronize()
        reps = max(1, max(args.steps, DIAG_CALLS) // n)
        for _ in range(2):
            gr.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(reps):
            gr.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        per_call = g0.elapsed_time(g1) / (reps * n)
        del gr
        return {"ms_per_call": per_call, "rows_per_s": w.rows / (per_call / 1e3),
                "calls": reps * n, "calls_per_graph": n}

    # Warm-up straight into the timed regions; the oracle check of the
    # output comes after them, so the GPU does not idle before timing.
    K = args.steps
    ms_per_step, wall, mean_reduce_ms, mean_merge_ms, graph_res = timed_regions(
        step, K, args.warmup, stream, graph if args.graph else None)
    step(0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    checked = 0
    vrows = np.nonzero((w.targets >= 0) & (w.targets < spec.V))[0]
    if args.check_rows > 0:
        import oracle
        o = oracle.get()
        for r in vrows[:: max(1, len(vrows) // args.check_rows)][: args.check_rows]:
            words, _ = o.prompt_row(w.logits[r], int(w.targets[r]), V=spec.V)
            g_ = got[r]
            assert g_[0] == words[0] and g_[2] == words[2], f"bench check: row {r}"
            assert np.array_equal(g_[3::2], words[3::2]), f"bench check: ids differ on row {r}"
            gv = np.concatenate([g_[1:2], g_[4::2]]).view(np.float32).astype(np.float64)
            rv = np.concatenate([words[1:2], words[4::2]]).view(np.float32).astype(np.float64)
            assert np.all(np.abs(gv - rv) <= 2e-5), f"values differ on row {r}"
            checked += 1

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        o = oracle.get()
        n = 0
        c0 = time.perf_counter()
        while n < w.rows and time.perf_counter() - c0 < args.cpu_seconds:
            o.prompt_row(w.logits[n], int(w.targets[n]), V=spec.V)
            n += 1
        dt = time.perf_counter() - c0
        cpu = {"value": n / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"first {n} rows of {spec.name} (of {w.rows}, {valid} valid), "
                         f"single-threaded oracle, {dt:.1f} s", "cpu": host_cpu()}
    if args.copy_mib > 0:
        copy_kernel(dev, args.copy_mib)

    res = {
        "metric": f"scored prompt rows/s and achieved HBM GB/s (% of peak) at V={spec.V}, "
                  f"{w.rows}-row chunk",
        "value": w.rows / (ms_per_step / 1e3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "fp32",
        "data": "synthetic (seeded logits + peak; targets: half the peak lane, half uniform, "
                "an image span and the prompt end invalid)",
        "config": {"workload": f"{spec.name}: {w.rows} rows x V={spec.V} "
                               f"{'bf16' if bf16 else 'fp32'}, prompt scoring",
                   "rows": w.rows, "valid_rows": valid, "V": spec.V, "copies": len(copies),
                   "oracle_rows_checked": checked},
        "roofline": roofline(spec.name, "reduce_kernel (scoring)", algo_bytes, mean_reduce_ms),
        "reduce_ms": mean_reduce_ms,
        "diagnostic_calls": max(K, DIAG_CALLS),
        "diagnostic_after_calls": max(DIAG_WARM_CALLS, args.warmup + K),
        "merge_ms": mean_merge_ms,
        "graph_replay": graph_res,
        "algorithmic_bytes_per_launch": algo_bytes,
        "wall_s": wall,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the reduction is sharded by rows with no "
              "exchange, so N GPUs run N independent copies; multi-GPU runs are not "
              "part of this build (use --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.prompt:
        bench_prompt(args)
        return

    import numpy as np
    import torch

    import __graft_entry__
    __graft_entry__._ensure_built()
    import full_vocab_logprob_amd as flp
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    spec = synth.CONFIGS[args.config]
    if args.K is not None:
        spec = spec.with_(K=args.K)
    if args.selected:
        spec = spec.with_(selected=args.selected)
    bf16 = spec.dtype == synth.BF16
    print(f"[bench] generating {spec.name}: {spec.description}", file=sys.stderr, flush=True)
    w = synth.make(spec)
    rows = spec.capacity * spec.T
    active = w.active_rows()
    algo_bytes = w.algorithmic_bytes()

    def upload(a):
        t = torch.from_numpy(a.view(np.int16) if bf16 else a).to(dev)
        return t.view(torch.bfloat16).reshape(-1) if bf16 else t.reshape(-1)

    g = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)  # noqa
    packed_rows, offsets = None, None
    if args.packed:
        # Slot order shuffled, each slot's committed rows directly after another's.
        e = np.where(w.requested != 0, np.clip(w.emitted, 0, spec.T), 0)
        off = np.zeros(spec.capacity, dtype=np.int32)
        P = 0
        for sl in np.random.default_rng(spec.seed).permutation(spec.capacity):
            off[sl] = P
            P += int(e[sl])
        packed = np.empty((P, spec.V_pad), dtype=w.logits.dtype)
        for sl in range(spec.capacity):
            packed[off[sl]:off[sl] + e[sl]] = w.logits[sl * spec.T:sl * spec.T + e[sl]]
        copies = [upload(packed)]
        packed_rows, offsets = P, g(off)
    else:
        copies = [upload(w.logits)]
    for _ in range(1, args.copies):
        copies.append(copies[0].clone())
    tokens, emitted, requested = g(w.tokens), g(w.emitted), g(w.requested)
    id_counts, ids = g(w.id_counts), g(w.ids)
    plan = flp.Plan(spec.capacity, spec.T, spec.V, spec.V_pad,
                    dtype=torch.bfloat16 if bf16 else torch.float32, K=spec.K, device=0,
                    packed_rows=packed_rows, shards=args.shards or None)
    ws = plan.workspace()
    out = plan.new_out(int(synth.POISON))
    stream = torch.cuda.current_stream()

    # Each call validated and marshalled once (Plan.bind): a timed step is one
    # C call per launch, so the host keeps ahead of the GPU.
    sh = stream.cuda_stream
    if args.shards:
        # "reduce" is every shard pass (what the ranks run side by side), "merge"
        # the cross-shard merge.
        def bind(c, ph):
            if ph == "reduce":
                return [plan.bind(copies[c], tokens, emitted, requested, id_counts, ids, out, ws,
                                  phase=f"shard:{r}") for r in range(args.shards)]
            return plan.bind(copies[c], tokens, emitted, requested, id_counts, ids, out, ws,
                             phase=ph)
        bound = {(c, ph): bind(c, ph) for c in range(len(copies))
                 for ph in ("all", "reduce", "merge")}
    else:
        bound = {(c, ph): plan.bind(copies[c], tokens, emitted, requested, id_counts, ids, out,
                                    ws, phase=ph, row_offsets=offsets)
                 for c in range(len(copies)) for ph in ("all", "reduce", "merge")}
    if args.records:
        # Timed calls read the counts and tokens from completion records
        # (emitted count in field 3); the split launches keep the int32 inputs.
        rec = np.zeros((spec.capacity, 16 + spec.T), dtype=np.int64)
        rec[:, 3] = w.emitted
        rec[:, 16:] = w.tokens.reshape(spec.capacity, spec.T)
        rec_t = torch.from_numpy(rec).to(dev)
        for c in range(len(copies)):
            bound[(c, "all")] = plan.bind_records(copies[c], rec_t, requested, out, ws, 3,
                                                  id_counts=id_counts, ids=ids)

    def step(i, phase="all"):
        b = bound[(i % len(copies), phase)]
        for call in (b if isinstance(b, list) else [b]):
            call(sh)

    def graph():
        # The same calls replayed from one HIP graph (GRAPH_CALLS calls over the
        # logits copies captured, replayed until about K calls have run).
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        gr = torch.cuda.CUDAGraph()
        n = GRAPH_CALLS
        with torch.cuda.stream(side):
            with torch.cuda.graph(gr, stream=side):
                for c in range(n):
                    plan.run(copies[c % len(copies)], tokens, emitted, requested, id_counts, ids,
                             out, ws, row_offsets=offsets)
        torch.cuda.synchronize()
        reps = max(1, max(args.steps, DIAG_CALLS) // n)
        for _ in range(2):
            gr.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(reps):
            gr.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        per_call = g0.elapsed_time(g1) / (reps * n)
        del gr
        return {"ms_per_call": per_call, "rows_per_s": active / (per_call / 1e3),
                "calls": reps * n, "calls_per_graph": n}

    # Warm-up straight into the timed regions; the oracle check of the
    # output comes after them, so the GPU does not idle before timing.
    K = args.steps
    ms_per_step, wall, mean_reduce_ms, mean_merge_ms, graph_res = timed_regions(
        step, K, args.warmup, stream, graph if args.graph else None)
    rows_per_s = active / (ms_per_step / 1e3)

    step(0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    act_rows = np.nonzero(w.active_mask().reshape(-1))[0]
    checked = 0
    if args.check_rows > 0:
        import oracle
        o = oracle.get()
        for r in act_rows[:: max(1, len(act_rows) // args.check_rows)][: args.check_rows]:
            sl, t = divmod(int(r), spec.T)
            n_sel = int(np.clip(w.id_counts[sl], 0, 128))
            sel = w.ids[sl * 128: sl * 128 + n_sel] if n_sel > 0 else None
            words, _ = o.row(w.logits[r], token=int(w.tokens[r]), K=spec.K, sel=sel, V=spec.V)
            g_ = got[sl, t, :len(words)]
            assert np.array_equal(g_[0::2], words[0::2]), f"bench check: ids differ on row {r}"
            d = np.abs(g_[1::2].view(np.float32).astype(np.float64)
                       - words[1::2].view(np.float32).astype(np.float64))
            assert np.all((d <= 2e-5) | (g_[1::2] == words[1::2])), f"values differ on row {r}"
            checked += 1

    cpu = cpu_threads = None
    if args.cpu_seconds > 0:
        import oracle
        o = oracle.get()
        n = 0
        c0 = time.perf_counter()
        while n < len(act_rows) and time.perf_counter() - c0 < args.cpu_seconds:
            r = int(act_rows[n])
            n_sel = int(np.clip(w.id_counts[r // spec.T], 0, 128))
            o.row(w.logits[r], token=int(w.tokens[r]), K=spec.K, V=spec.V,
                  sel=w.ids[(r // spec.T) * 128:(r // spec.T) * 128 + n_sel] if n_sel else None)
            n += 1
        dt = time.perf_counter() - c0
        cpu = {"value": n / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"first {n} active rows of {spec.name} (of {active}), "
                         f"single-threaded oracle, {dt:.1f} s", "cpu": host_cpu()}
        # The same per-row oracle over every active row, rows split across
        # host threads (ctypes releases the GIL during each row).
        from concurrent.futures import ThreadPoolExecutor
        threads = max(1, min(16, os.cpu_count() or 1))

        def one(r):
            r = int(r)
            n_sel = int(np.clip(w.id_counts[r // spec.T], 0, 128))
            o.row(w.logits[r], token=int(w.tokens[r]), K=spec.K, V=spec.V,
                  sel=w.ids[(r // spec.T) * 128:(r // spec.T) * 128 + n_sel] if n_sel else None)

        c0 = time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, act_rows))
        dt = time.perf_counter() - c0
        cpu_threads = {"value": len(act_rows) / dt, "unit": "rows/s", "cores": threads,
                       "kind": "oracle", "sample": f"all {len(act_rows)} active rows of "
                       f"{spec.name}, one row per task over {threads} threads, {dt:.1f} s"}

    if args.copy_mib > 0:
        copy_kernel(dev, args.copy_mib)

    res = {
        "metric": f"logprob rows/s and achieved HBM GB/s (% of peak) at V={spec.V:,}, T={spec.T}, "
                  f"{spec.capacity} slots",
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "fp32",
        "data": f"synthetic, seeded ({spec.description.split(': ', 1)[1]}; rows past each "
                f"slot's prefix hold NaN/+inf garbage)",
        "config": {"workload": f"{spec.name}: {spec.capacity} slots x T={spec.T} x V={spec.V} "
                               f"{'bf16' if bf16 else 'fp32'}, emitted 1..{spec.T}, K={spec.K}"
                               + (f", packed into {packed_rows} rows" if packed_rows else "")
                               + (", counts and tokens from completion records"
                                  if args.records else "")
                               + (f", vocabulary in {args.shards} shards" if args.shards else "")
                               + (", 128 selected IDs per slot" if args.selected else ""),
                   "active_rows": active, "capacity": spec.capacity, "T": spec.T, "V": spec.V,
                   "K": spec.K, "copies": len(copies), "oracle_rows_checked": checked},
        "roofline": roofline(workload_tag(spec.name, args.K, args.selected)
                             if not args.records and not args.shards
                             else "", "reduce_kernel" if not args.shards
                             else f"reduce_kernel + shard_finalize_kernel, {args.shards} shard passes",
                             algo_bytes, mean_reduce_ms, packed=bool(packed_rows or args.shards)),
        "reduce_ms": mean_reduce_ms,
        "diagnostic_calls": max(K, DIAG_CALLS),
        "diagnostic_after_calls": max(DIAG_WARM_CALLS, args.warmup + K),
        "merge_ms": mean_merge_ms,
        "graph_replay": graph_res,
        "algorithmic_bytes_per_launch": algo_bytes,
        "wall_s": wall,
        "cpu_baseline": cpu,
        "cpu_baseline_threads": cpu_threads,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
