#!/usr/bin/env python
"""Benchmark of the paged-KV hot path on one MI355X.

A step is one pass of the whole path over one batch: the KV block write of
the step's new tokens, then paged attention (device-side plan, split-context
decode, partition merge, prefill).

Default run (``--workload all``): the headline is the 70B-shaped long-context
decode batch (64 requests, 64 query / 8 KV heads, head_dim 128, one new token
each over a cached context uniform in [32768, 131072], blocks scattered at
random in a pool of about 0.92 of free HBM); ``value`` is the KV bytes
attention must read (L * 2 * Hkv * D * 2 per request) per second of
whole-step time.  The other four workloads follow as line items under
``items`` (the 8B-shaped decode batch, the prefill batch, the
continuous-batching step and the tiny mixed step), each with the same fields.

Per workload:
* ``ms_per_step``: exactly ``--steps`` steps between two events (the tiny
  mixed step: 50 times as many), and ``step_us_median`` / ``step_us_min``
  from events around each step in a second pass;
* ``roofline`` for the dominant kernel (decode: HBM GB/s of algorithmic KV
  bytes; prefill: TFLOP/s of unmasked (query, key) pairs against the bf16
  dense MFMA peak): algorithmic work per launch / the kernel's mean launch
  duration, timed with two HIP events on the launch stream around that
  kernel only; the continuous-batching step has both (``roofline`` for its
  decode part, ``roofline_chunk`` for its chunk) and its lower bounds;
* ``traffic``: HBM bytes per launch from committed counter summaries;
* ``cpu_baseline``: the fp64 CPU oracle on a bounded sample of the same
  workload (gather + attention timed; data generation not).

Inputs are synthetic: lengths and block placement from the seeded workload
generators, values N(0,1) drawn on the GPU with a seeded generator.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode KV-read GB/s (% HBM peak) + prefill attn TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6

DESCRIPTIONS = {
    "tiny_mixed": "TinyLlama-shaped mixed step: 6-token prefill + 1-token decode over 37 cached "
                  "tokens; 32 q / 4 kv heads, head_dim 64, 64-block pool",
    "decode_8b": "Llama-3-8B-shaped decode batch: 256 requests x 1 new token, cached context "
                 "U[512,4096]; 32 q / 8 kv heads, head_dim 128; pool sized to the total",
    "prefill_8b": "Llama-3-8B-shaped prefill batch: 16 prompts U[256,2048] packed end to end, "
                  "causal, no history; 32 q / 8 kv heads, head_dim 128",
    "cb_step_8b": "continuous-batching step (8192-token budget): 192 decodes over U[1024,8192] "
                  "(64 share a 1024-token prefix) + one 2048-token chunk over 16384 cached tokens",
    "long_decode_70b": "70B-shaped layer share: 64 requests x 1 new token over U[32768,131072]; "
                       "64 q / 8 kv heads, head_dim 128; pool ~0.92 of free HBM",
    "spec_verify_8b": "8B-shaped speculative-decoding check: 128 requests x 4 new tokens (3 drafted) "
                      "over cached context U[2048,16384]; 32 q / 8 kv heads, head_dim 128",
    "spec_verify_70b": "70B-shaped speculative-decoding check: 64 requests x 4 new tokens (3 drafted) "
                       "over cached context U[4096,16384]; 64 q / 8 kv heads, head_dim 128",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Setup:
    """A workload resident on the GPU, values drawn on the device."""

    def __init__(self, wl, pool_blocks=None):
        import torch
        import paged_kv_cache_469_amd as pkv

        self.wl = wl
        dev = torch.device("cuda:0")
        gen = torch.Generator(device=dev)
        gen.manual_seed(469)
        hkv, d = wl.num_kv_heads, wl.head_dim
        nb = wl.num_blocks if pool_blocks is None else pool_blocks
        self.pool = torch.empty((nb, 2, 16, hkv, d), dtype=torch.bfloat16, device=dev)
        used = np.unique(wl.block_tables[wl.block_tables >= 0]).astype(np.int64)
        ids = torch.from_numpy(used).to(dev)
        chunk = 1 << 14
        for i in range(0, ids.numel(), chunk):
            sel = ids[i:i + chunk]
            vals = torch.randn((sel.numel(), 2, 16, hkv, d), generator=gen, device=dev)
            self.pool.index_copy_(0, sel, vals.to(torch.bfloat16))
            del vals
        t = wl.num_tokens
        self.q = torch.randn((t, wl.num_q_heads, d), generator=gen, device=dev).to(torch.bfloat16)
        self.k = torch.randn((t, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
        self.v = torch.randn((t, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
        self.out = torch.empty_like(self.q)
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.slots = up(wl.slot_mapping)
        self.bt = up(wl.block_tables)
        self.cu = up(wl.cu_seqlens_q)
        self.lens = up(wl.seq_lens)
        self.ws = torch.empty(pkv.paged_attention_workspace_size(
            wl.num_seqs, t, wl.num_q_heads, hkv, d, wl.max_blocks_per_seq),
            dtype=torch.uint8, device=dev)
        self.pkv = pkv

    def step(self):
        self.pkv.paged_kv_write(self.k, self.v, self.slots, self.pool)
        self.pkv.paged_attention(self.q, self.pool, self.bt, self.cu, self.lens, self.wl.scale,
                                 out=self.out, workspace=self.ws)


STAGES = ["plan", "decode", "decode_merge", "prefill"]

# Passes over the steps of one workload, in this order, each of the same
# number of steps (``trace_summary`` splits a kernel trace of a bench run by
# the same plan):
#   timed      nothing but the calls between two events: the step time;
#   per-step   two events around every step: median and min of a step;
#   kernel <k> two events around kernel k only, once for each roofline kernel
#              of the workload: its mean, median and min launch duration;
#   stages     events around every kernel: the per-kernel breakdown (each
#              record leaves a gap of a few microseconds between kernels, so
#              these times are not used for the rooflines).
# One warm-up pass of `warmup` steps comes first.
def passes_of(dominant):
    return ["timed", "per_step"] + [f"kernel:{k}" for k in dominant] + ["stages"]


def run_steps(setup, steps, warmup, dominant):
    """Runs the passes above; returns a dict of their results."""
    import torch

    pkv = setup.pkv
    mk = lambda: torch.cuda.Event(enable_timing=True)

    def made(evs):                     # create the HIP events outside the timed regions
        for e in evs:
            e.record()
        return evs

    stage_sets = [made([mk() for _ in range(5)]) for _ in range(steps)]
    write_sets = [made([mk(), mk()]) for _ in range(steps)]
    step_sets = [made([mk(), mk()]) for _ in range(steps)]
    dom_sets = {k: [made([mk(), mk()]) for _ in range(steps)] for k in dominant}
    start, end = made([mk(), mk()])
    for _ in range(warmup):
        setup.step()
    torch.cuda.synchronize()
    # timed: exactly `steps` steps between two events
    start.record()
    for _ in range(steps):
        setup.step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # per step
    for a, b in step_sets:
        a.record()
        setup.step()
        b.record()
    torch.cuda.synchronize()
    step_us = [1e3 * a.elapsed_time(b) for a, b in step_sets]
    # each roofline kernel alone: events around it only
    dom = {}
    for k in dominant:
        i = STAGES.index(k)
        for evs2 in dom_sets[k]:
            evs = [None] * 5
            evs[i], evs[i + 1] = evs2
            pkv.paged_attention_set_stage_events(evs)
            setup.step()
        torch.cuda.synchronize()
        pkv.paged_attention_set_stage_events(None)
        d = [1e3 * a.elapsed_time(b) for a, b in dom_sets[k]]
        dom[k] = {"mean": float(np.mean(d)), "median": float(np.median(d)), "min": float(np.min(d))}
    # every kernel
    for i in range(steps):
        pkv.paged_attention_set_stage_events(stage_sets[i])
        write_sets[i][0].record()
        pkv.paged_kv_write(setup.k, setup.v, setup.slots, setup.pool)
        write_sets[i][1].record()
        pkv.paged_attention(setup.q, setup.pool, setup.bt, setup.cu, setup.lens, setup.wl.scale,
                            out=setup.out, workspace=setup.ws)
    torch.cuda.synchronize()
    pkv.paged_attention_set_stage_events(None)
    us = {n: 1e3 * float(np.mean([s[i].elapsed_time(s[i + 1]) for s in stage_sets]))
          for i, n in enumerate(STAGES)}
    us["kv_write"] = 1e3 * float(np.mean([a.elapsed_time(b) for a, b in write_sets]))
    status = pkv.paged_attention_device_status(setup.ws)
    if status:
        raise RuntimeError(f"device status {status}: metadata rejected")
    return {"ms": ms, "step_us": {"median": float(np.median(step_us)), "min": float(np.min(step_us))},
            "kernels_us": us, "dominant": dom}


# ------------------------------------------------------------------ oracle beside it

def _oracle_pool(wl, sel):
    """A host pool holding the K/V of segments `sel` (their blocks renumbered
    contiguously) and their tables: untimed set-up of a CPU baseline."""
    from oracle import paged

    hkv, d = wl.num_kv_heads, wl.head_dim
    nblk = [(int(wl.seq_lens[s]) + 15) // 16 for s in sel]
    pool = np.empty((sum(nblk), 2, 16, hkv, d), dtype=np.uint16)
    tables = np.full((len(sel), max(nblk)), -1, dtype=np.int32)
    c = 0
    for i, s in enumerate(sel):
        tables[i, :nblk[i]] = np.arange(c, c + nblk[i])
        length = int(wl.seq_lens[s])
        k, v = wl.request_kv(s)
        pos = np.arange(length)
        paged.kv_write(k, v, (tables[i][pos // 16].astype(np.int64) * 16 + pos % 16), pool)
        c += nblk[i]
    return pool, tables


def cpu_baseline_decode(wl, sample):
    """The fp64 oracle on `sample` decode requests of a batch: gather from a
    host pool + attention, timed; generation and pool filling untimed."""
    from threadpoolctl import threadpool_limits

    from oracle import paged

    cores = len(os.sched_getaffinity(0))
    dec = [s for s in range(wl.num_seqs) if 1 <= wl.new_tokens[s] <= 8]
    sel = dec[:sample]
    hkv, d = wl.num_kv_heads, wl.head_dim
    pool, tables = _oracle_pool(wl, sel)
    q = wl.q()
    cu = wl.cu_seqlens_q
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in sel])
    cu_sub = np.zeros(len(sel) + 1, dtype=np.int32)
    cu_sub[1:] = np.cumsum([int(wl.new_tokens[s]) for s in sel])
    lens = wl.seq_lens[sel]
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        paged.attend(q[rows], pool, tables, cu_sub, lens, wl.scale)
        dt = time.perf_counter() - t0
    kv = int(lens.astype(np.int64).sum()) * 2 * hkv * d * 2
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(sel)} of {len(dec)} decode requests of the same batch "
                      f"({kv / 1e9:.3f} GB of KV), gather + fp64 attention timed: {dt:.2f} s"}


def cpu_baseline_prefill(wl, seg, rows=None):
    """The fp64 oracle on segment `seg` of a batch (all its rows, or the
    `rows` last ones), gather from a host pool + attention timed."""
    from threadpoolctl import threadpool_limits

    from oracle import bf16, paged

    cores = len(os.sched_getaffinity(0))
    n = int(wl.new_tokens[seg])
    length = int(wl.seq_lens[seg])
    h = length - n
    r = n if rows is None else min(rows, n)
    pool, tables = _oracle_pool(wl, [seg])
    q = wl.q()[wl.cu_seqlens_q[seg] + n - r:wl.cu_seqlens_q[seg + 1]]
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        k, v = paged.gather(pool, tables[0], length)
        paged.attend_dense(bf16.to_f64(q), bf16.to_f64(k), bf16.to_f64(v), wl.scale, h + n - r)
        dt = time.perf_counter() - t0
    pairs = r * (h + n - r) + r * (r + 1) // 2
    flops = 4 * wl.head_dim * wl.num_q_heads * pairs
    what = f"all {n} rows" if r == n else f"the last {r} of its {n} rows"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"segment {seg} ({what}, {h + n - r} keys before the first) of the same "
                      f"batch: {flops / 1e9:.1f} GFLOP, gather + fp64 attention timed: {dt:.2f} s"}


def cpu_baseline_step(wl, reps):
    """The fp64 oracle on the whole step, `reps` times: time per step."""
    from threadpoolctl import threadpool_limits

    from oracle import paged

    cores = len(os.sched_getaffinity(0))
    sel = list(range(wl.num_seqs))
    pool, tables = _oracle_pool(wl, sel)
    q = wl.q()
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for _ in range(reps):
            paged.attend(q, pool, tables, wl.cu_seqlens_q, wl.seq_lens, wl.scale)
        dt = time.perf_counter() - t0
    return {"value": 1e6 * dt / reps, "unit": "us/step", "cores": cores, "kind": "oracle",
            "sample": f"the whole step, {reps} times (gather + fp64 attention): {dt:.2f} s"}


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of ``nbytes``: it reads and writes
    exactly ``nbytes`` each, so the counters it reads give the scale between
    counter units and HBM bytes."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


# HBM traffic of a kernel, from two rocprofv3 counter runs (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for
# the plain 1 GiB copy of --copy-calibration.  The summary (a text file under
# profiles/) records a hash of the kernel's sources; bench reports the
# traffic only while the sources still hash the same.
KERNEL_SOURCES = {
    # the plan decides the order of the work items, which sets how much of
    # the K/V a kernel fetches from beyond L2
    "decode_kernel": ["decode.hip", "plan.hip", "common.hpp", "kernels.hpp"],
    "prefill_kernel": ["prefill.hip", "matrix_phase.inc", "plan.hip", "common.hpp", "kernels.hpp"],
}


def _code_only(text):
    """Source text without // comments and blank space, so that editing a
    comment does not count as changing the kernel."""
    out = []
    for line in text.splitlines():
        code = line.split("//", 1)[0].strip()
        if code:
            out.append(" ".join(code.split()))
    return "\n".join(out)


def kernel_source_hash(kernel, read=None):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        path = os.path.join("paged_kv_cache_469_amd", "csrc", f)
        if read is None:
            with open(os.path.join(ROOT, path)) as fh:
                text = fh.read()
        else:
            text = read(path)
        h.update(_code_only(text).encode())
    return h.hexdigest()[:16]


def traffic_file(kernel, workload):
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")


def stored_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel's sources changed since it was taken."""
    path = traffic_file(kernel, workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    return float(fields["hbm_bytes_per_launch"])


def _counter_means(path_glob, name_filter):
    vals = {}
    for f in glob.glob(path_glob):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if name_filter(r["Kernel_Name"]):
                    vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def pmc_summary(args):
    """Turns the four counter runs into the summary text bench reads back."""
    copy_kib = (1 << 30) / 1024.0
    cf, _ = _counter_means(os.path.join(args.calib_fetch, "*counter_collection.csv"), lambda n: "copyBuffer" in n)
    cw, _ = _counter_means(os.path.join(args.calib_write, "*counter_collection.csv"), lambda n: "copyBuffer" in n)
    kf, nf = _counter_means(os.path.join(args.fetch, "*counter_collection.csv"), lambda n: args.kernel in n)
    kw, nw = _counter_means(os.path.join(args.write, "*counter_collection.csv"), lambda n: args.kernel in n)
    f_scale = copy_kib / cf["FETCH_SIZE"]
    w_scale = copy_kib / cw["WRITE_SIZE"]
    fetch = kf["FETCH_SIZE"] * f_scale * 1024.0
    write = kw["WRITE_SIZE"] * w_scale * 1024.0
    lines = [
        f"# HBM traffic of {args.kernel}<128>, workload {args.workload}",
        "#",
        "# Commands (from the repository root, on one MI355X):",
        f"#   rocprofv3 --pmc FETCH_SIZE --kernel-include-regex {args.kernel} -f csv -d <F> -o k -- "
        f"python bench.py --workload {args.workload} --steps 3 --warmup 1 --no-cpu-baseline",
        f"#   rocprofv3 --pmc WRITE_SIZE --kernel-include-regex {args.kernel} -f csv -d <W> -o k -- "
        f"python bench.py --workload {args.workload} --steps 3 --warmup 1 --no-cpu-baseline",
        "#   rocprofv3 --pmc FETCH_SIZE -f csv -d <CF> -o copy -- python bench.py --copy-calibration",
        "#   rocprofv3 --pmc WRITE_SIZE -f csv -d <CW> -o copy -- python bench.py --copy-calibration",
        f"#   python bench.py --pmc-summary --kernel {args.kernel} --workload {args.workload} "
        "--fetch <F> --write <W> --calib-fetch <CF> --calib-write <CW>",
        "#",
        "# The copy moves 1 GiB each way; the counters' KiB for it give the scales.",
        f"copy_fetch_kib_per_dispatch: {cf['FETCH_SIZE']:.1f}",
        f"copy_write_kib_per_dispatch: {cw['WRITE_SIZE']:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"kernel_dispatches: fetch {nf.get('FETCH_SIZE', 0)} write {nw.get('WRITE_SIZE', 0)}",
        f"kernel_fetch_kib_per_dispatch: {kf['FETCH_SIZE']:.1f}",
        f"kernel_write_kib_per_dispatch: {kw['WRITE_SIZE']:.1f}",
        f"hbm_fetch_bytes_per_launch: {fetch:.0f}",
        f"hbm_write_bytes_per_launch: {write:.0f}",
        f"hbm_bytes_per_launch: {fetch + write:.0f}",
        f"source_sha256_16: {kernel_source_hash(args.kernel)}",
    ]
    print("\n".join(lines))


MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_BUSY_CYCLES",
                 "GRBM_GUI_ACTIVE"]


def mfma_summary(args):
    """Matrix-core busy time and the shader clock of one kernel, from one
    rocprofv3 run with --pmc of MFMA_COUNTERS and --kernel-trace (durations of
    the same dispatches).  GRBM_GUI_ACTIVE comes summed over the XCDs (one
    instance each), so cycles = GRBM_GUI_ACTIVE / XCDs:
      busy  = SQ_VALU_MFMA_BUSY_CYCLES / (cycles * CUs * 4 SIMDs)
      clock = cycles / dispatch duration (cycles per ns = GHz)
      executed flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 (every MFMA the
      kernel issues, masked products included), against the algorithmic
      flops of the workload's segments on that kernel."""
    import workloads

    trace = glob.glob(os.path.join(args.trace, "*kernel_trace.csv"))[0]
    dur = {}
    with open(trace) as fh:
        for r in csv.DictReader(fh):
            if args.kernel in r["Kernel_Name"]:
                dur[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    per = {}
    for f in glob.glob(os.path.join(args.counters, "*counter_collection.csv")):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if args.kernel in r["Kernel_Name"]:
                    per.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
    ids = sorted((i for i in per if i in dur and len(per[i]) == len(MFMA_COUNTERS)), key=int)
    cus = args.cus
    wl = workloads.make(args.workload) if args.workload != "long_decode_70b" else None
    alg = None
    if wl is not None:
        _, pre, _ = _decode_split(wl)
        alg = wl.attention_flops(segments=pre) if pre.size else 0
    rows = []
    for i in ids:
        c, ns = per[i], dur[i]
        cyc = c["GRBM_GUI_ACTIVE"] / args.xcds          # the dispatch's cycles on one XCD
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * cus * 4)
        ghz = cyc / ns
        exe = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        rows.append((i, ns / 1e3, busy, ghz, exe, c["SQ_BUSY_CYCLES"]))
    lines = [
        f"# Matrix-core busy time and shader clock of {args.kernel}<128>, workload {args.workload}",
        "#",
        "# Commands (from the repository root, on one MI355X):",
        f"#   rocprofv3 --kernel-trace --pmc {' '.join(MFMA_COUNTERS)} --kernel-include-regex "
        f"{args.kernel} -f csv -d <C> -o m -- python bench.py --workload {args.workload} "
        "--steps 3 --warmup 1 --no-cpu-baseline",
        f"#   python bench.py --mfma-summary --kernel {args.kernel} --workload {args.workload} "
        "--counters <C> --trace <C>",
        "#",
        "# cycles = GRBM_GUI_ACTIVE / 8: rocprofv3 sums the counter over its 8 instances (one per",
        "#   XCD; each counts the dispatch's cycles at the shader clock);",
        "# busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles * 256 CUs * 4 SIMDs): the share of the",
        "#   dispatch's cycles in which an average SIMD's matrix core was busy;",
        "# clock = cycles / duration, in GHz; the 2516.6 TFLOP/s peak assumes 2.4 GHz.  Check:",
        "#   busy * clock * 1024 flop per SIMD-cycle * 1024 SIMDs = executed flops per second;",
        "# executed = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512: the flops of every MFMA issued, masked",
        "#   or idle products included; algorithmic = 4 * D * Hq per unmasked (query, key) pair.",
        "#   Counter collection serialises dispatches, so durations here may differ a little",
        "#   from the bench's own events.",
        f"cus: {cus}",
        f"algorithmic_flops_per_launch: {alg}",
        "",
        "| dispatch | us | MFMA busy | clock GHz | busy x clock x 1 PFLOP/GHz | executed TFLOP | "
        "executed TFLOP/s | algorithmic TFLOP/s | algorithmic / executed |",
        "|---|---|---|---|---|---|---|---|---|",
    ]
    for i, us, busy, ghz, exe, _ in rows:
        a = f"{alg / (us * 1e-6) / 1e12:.0f}" if alg else "-"
        r = f"{alg / exe:.3f}" if alg else "-"
        lines.append(f"| {i} | {us:.1f} | {100 * busy:.1f} % | {ghz:.3f} | "
                     f"{busy * ghz * 1024 * 1024 / 1e3:.0f} | {exe / 1e12:.4f} | "
                     f"{exe / (us * 1e-6) / 1e12:.0f} | {a} | {r} |")
    if rows:
        m = lambda k: float(np.mean([x[k] for x in rows]))
        lines += ["", f"mean_us: {m(1):.1f}", f"mean_mfma_busy: {m(2):.4f}",
                  f"mean_clock_ghz: {m(3):.3f}",
                  f"mean_executed_tflops_per_s: {np.mean([x[4] / (x[1] * 1e-6) / 1e12 for x in rows]):.1f}"]
        if alg:
            lines.append(f"mean_algorithmic_tflops_per_s: {np.mean([alg / (x[1] * 1e-6) / 1e12 for x in rows]):.1f}")
    print("\n".join(lines))


# The default run: the long-context decode batch as the headline, then the
# other four workloads as line items, in this order.  Per workload: the
# kernels whose rooflines are reported, and the step count (the tiny mixed
# step is timed over 50 times as many steps: it takes tens of microseconds).
DEFAULT_RUN = ["long_decode_70b", "decode_8b", "prefill_8b", "cb_step_8b", "tiny_mixed"]
DOMINANT = {"prefill_8b": ["prefill"], "cb_step_8b": ["decode", "prefill"], "tiny_mixed": []}
STEP_FACTOR = {"tiny_mixed": 50}


def dominant_of(name):
    return DOMINANT.get(name, ["decode"])


def run_plan(workload, steps, warmup):
    """[(workload, steps, warmup, passes)] of a bench run, in order."""
    names = DEFAULT_RUN if workload == "all" else [workload]
    plan = []
    for n in names:
        f = STEP_FACTOR.get(n, 1) if workload == "all" else 1
        plan.append((n, steps * f, warmup * f, passes_of(dominant_of(n))))
    return plan


def trace_summary(args):
    """Per-kernel durations from a rocprofv3 --kernel-trace CSV of a bench
    command, split into the bench's phases (workloads and passes) by counting
    the KV-write dispatch that opens every step, in the order of run_plan."""
    path = glob.glob(os.path.join(args.trace, "*kernel_trace.csv"))[0]
    with open(path) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))
    rows = [r for r in rows if "pkv::" in r["Kernel_Name"]]
    plan = run_plan(args.workload, args.steps, args.warmup)
    # phase boundaries in KV-write dispatches
    bounds = []
    for name, steps, warmup, passes in plan:
        bounds.append((name, "warm-up", warmup))
        for ps in passes:
            bounds.append((name, ps, steps))
    phases, bi, seen = [], -1, 0
    for r in rows:
        if "kv_write" in r["Kernel_Name"]:
            if bi < 0 or seen == bounds[bi][2]:
                bi += 1
                seen = 0
                phases.append((bounds[bi][0], bounds[bi][1], []))
            seen += 1
        phases[-1][2].append(r)
    flag = "" if args.workload == "all" else f" --workload {args.workload}"
    title = ("default bench (long_decode_70b headline; decode_8b, prefill_8b, cb_step_8b, "
             "tiny_mixed line items)" if args.workload == "all"
             else f"{args.workload}: {DESCRIPTIONS[args.workload]}")
    out = [f"# Kernel trace: {title}", "",
           "Command (from the repository root, on one MI355X):", "",
           f"    rocprofv3 --kernel-trace --stats -f csv -d <T> -o kt -- python bench.py{flag} "
           f"--steps {args.steps} --warmup {args.warmup} --no-cpu-baseline",
           f"    python bench.py --trace-summary --trace <T>{flag} --steps {args.steps} "
           f"--warmup {args.warmup}",
           "",
           "Durations in microseconds (end - start of each dispatch).  Per workload the bench "
           "runs a warm-up, then passes of the same number of steps: timed (the step time), "
           "per-step (events around each step), one pass per roofline kernel (events around "
           "that kernel only: the pass whose times the bench line reports for it) and stages "
           "(events around every kernel).", ""]

    def table(rs):
        by = {}
        for r in rs:
            name = (r["Kernel_Name"].replace("void ", "").replace("(anonymous namespace)::", "")
                    .split("(")[0])
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            by.setdefault(name, {"d": [], "r": r})["d"].append(d)
        t = ["| kernel | calls | avg us | median us | min us | max us | grid (threads) | wg | "
             "vgpr | lds B |", "|---|---|---|---|---|---|---|---|---|---|"]
        for name, v in sorted(by.items(), key=lambda kv: -sum(kv[1]["d"])):
            d, r = v["d"], v["r"]
            t.append(f"| {name} | {len(d)} | {np.mean(d):.1f} | {np.median(d):.1f} | {min(d):.1f} | "
                     f"{max(d):.1f} | {r['Grid_Size_X']} | {r['Workgroup_Size_X']} | "
                     f"{r['VGPR_Count']} | {r['LDS_Block_Size']} |")
        return t

    for name, _, _, _ in plan:
        mine = [ph for ph in phases if ph[0] == name]
        allrows = [r for ph in mine for r in ph[2]]
        out += [f"## {name}", "", "All passes but the warm-up:", ""]
        out += table([r for ph in mine if ph[1] != "warm-up" for r in ph[2]])
        for ph in mine:
            if ph[1].startswith("kernel:"):
                k = ph[1].split(":", 1)[1]
                out += ["", f"Pass `{ph[1]}` (the {k} kernel's roofline time in the bench line "
                        f"comes from this pass's events):", ""]
                out += table(ph[2])
        out.append("")
        del allrows
    print("\n".join(out))


def make_workload(name):
    import torch
    import workloads

    if name == "long_decode_70b":
        free, _ = torch.cuda.mem_get_info()
        wl0 = workloads.make(name, num_blocks=1 << 20)
        reserve = (wl0.num_tokens * wl0.num_q_heads * wl0.head_dim * 2 * 2
                   + (2 << 30))                       # q, out, workspace and slack first
        nb = int(0.92 * (free - reserve) // 65536)
        return workloads.make(name, num_blocks=nb), nb
    return workloads.make(name), None


def _decode_split(wl):
    """(decode segments, prefill segments, algorithmic KV bytes of the decode
    kernel: unique bytes, each shared prefix block counted once)."""
    # segments on the split-context decode path: n * G <= 32 and n <= 8
    max_dec = min(8, 32 // (wl.num_q_heads // wl.num_kv_heads))
    dec = np.nonzero((wl.new_tokens >= 1) & (wl.new_tokens <= max_dec))[0]
    pre = np.nonzero(wl.new_tokens > max_dec)[0]
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * 2
    dec_bytes = int(wl.seq_lens[dec].astype(np.int64).sum()) * per_tok
    if wl.shared_prefix:
        dec_bytes = wl.kv_bytes_unique() - int(wl.seq_lens[pre].astype(np.int64).sum()) * per_tok
    return dec, pre, dec_bytes


def _roofline(kind, work, kernel_times, traffic_key):
    """Roofline entry of one kernel: `work` algorithmic bytes or flops per
    launch over its mean launch duration."""
    us = kernel_times["mean"]
    if kind == "decode":
        ach = work / (us * 1e-6) / 1e9
        return {"kernel": "decode_kernel<128>", "bound": "hbm", "achieved": ach,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "kernel_us": us,
                "kernel_us_median": kernel_times["median"], "kernel_us_min": kernel_times["min"],
                "algorithmic_bytes": work, "traffic": stored_traffic("decode_kernel", traffic_key)}
    ach = work / (us * 1e-6) / 1e12
    return {"kernel": "prefill_kernel<128>", "bound": "mfma", "achieved": ach,
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFLOPS,
            "kernel_us": us, "kernel_us_median": kernel_times["median"],
            "kernel_us_min": kernel_times["min"], "algorithmic_flops": work,
            "traffic": stored_traffic("prefill_kernel", traffic_key)}


def bench_workload(name, steps, warmup, with_cpu, cpu_sample=None):
    """Times one workload (set-up untimed) and returns its entry of the line."""
    import torch

    wl, nb = make_workload(name)
    log(f"[bench] {name}: S={wl.num_seqs} T={wl.num_tokens} NB={wl.num_blocks}, {steps} steps")
    st = Setup(wl, pool_blocks=nb)
    res = run_steps(st, steps, warmup, dominant_of(name))
    del st
    torch.cuda.empty_cache()
    ms = res["ms"]
    dec, pre, dec_bytes = _decode_split(wl)
    flops = wl.attention_flops()
    pre_flops = wl.attention_flops(segments=pre) if pre.size else 0
    kv_bytes = wl.kv_bytes_unique()
    e = {"workload": f"{name}: {DESCRIPTIONS[name]}", "steps": steps, "warmup": warmup,
         "ms_per_step": ms, "step_us_median": res["step_us"]["median"],
         "step_us_min": res["step_us"]["min"],
         "config": {"num_seqs": wl.num_seqs, "num_tokens": wl.num_tokens,
                    "heads": [wl.num_q_heads, wl.num_kv_heads], "head_dim": wl.head_dim,
                    "block_size": 16, "pool_blocks": wl.num_blocks, "kv_bytes": kv_bytes,
                    "attention_flops": flops}}
    dom = res["dominant"]
    if name == "prefill_8b":
        e.update(value=flops / (ms * 1e-3) / 1e12, unit="TFLOP/s")
        e["roofline"] = _roofline("prefill", pre_flops, dom["prefill"], name)
    elif name == "tiny_mixed":
        e.update(value=1e3 * ms, unit="us/step")
        e["roofline"] = None
        e["roofline_note"] = "latency-bound step (a few kernels of a few microseconds each)"
    else:
        e.update(value=kv_bytes / (ms * 1e-3) / 1e9, unit="GB/s")
        e["roofline"] = _roofline("decode", dec_bytes, dom["decode"], name)
    if name == "cb_step_8b":
        e["config"]["kv_bytes_logical"] = wl.kv_bytes_logical()
        chunk = _roofline("prefill", pre_flops, dom["prefill"], name)
        e["roofline_chunk"] = chunk
        # lower bounds of the step at the peaks: decode and chunk overlapped, or serialised
        t_dec = dec_bytes / (HBM_PEAK_GBS * 1e9) * 1e6
        t_chk = pre_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6
        e["step_bound_us"] = {"overlapped": max(t_dec, t_chk), "serialised": t_dec + t_chk}
    if name == "long_decode_70b":
        e["config"]["pool_holds_tokens"] = wl.num_blocks * 16
    e["kernels_us"] = res["kernels_us"]
    if with_cpu:
        log(f"[bench] {name}: CPU oracle")
        if name == "prefill_8b":
            seg = int(np.argsort(wl.new_tokens)[wl.num_seqs // 2])   # a median-length prompt
            e["cpu_baseline"] = cpu_baseline_prefill(wl, seg)
        elif name == "tiny_mixed":
            e["cpu_baseline"] = cpu_baseline_step(wl, 200)
        else:
            e["cpu_baseline"] = cpu_baseline_decode(wl, cpu_sample or 4)
            if name == "cb_step_8b":
                e["cpu_baseline_chunk"] = cpu_baseline_prefill(wl, int(pre[0]), rows=256)
    return e


CPU_SAMPLE = {"long_decode_70b": 3, "decode_8b": 64, "cb_step_8b": 16, "spec_verify_8b": 8,
              "spec_verify_70b": 8}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(DESCRIPTIONS),
                    help="all (default): the long-context decode batch as the headline and the "
                         "other four workloads as line items; or one workload alone")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--group-members", type=int, default=0,
                    help="most members of a shared-prefix group (0: automatic, 1: no groups)")
    ap.add_argument("--pmc-summary", action="store_true",
                    help="summarise four rocprofv3 counter runs (see --fetch .. --calib-write)")
    ap.add_argument("--trace-summary", action="store_true",
                    help="summarise a rocprofv3 kernel-trace CSV of a bench run (--trace DIR)")
    ap.add_argument("--trace")
    ap.add_argument("--mfma-summary", action="store_true",
                    help="summarise a rocprofv3 run with MFMA counters and a kernel trace "
                         "(--counters DIR --trace DIR)")
    ap.add_argument("--counters")
    ap.add_argument("--cus", type=int, default=256)
    ap.add_argument("--xcds", type=int, default=8)
    ap.add_argument("--kernel", default="decode_kernel")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--calib-fetch")
    ap.add_argument("--calib-write")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (5 times), the reference kernel "
                         "that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.trace_summary:
        trace_summary(args)
        return
    if args.mfma_summary:
        mfma_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_469_amd as pkv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    pkv.lib()
    if args.partition_tokens:
        pkv.paged_attention_set_partition_tokens(args.partition_tokens)
    if args.group_members:
        pkv.paged_attention_set_group_members(args.group_members)
    props = torch.cuda.get_device_properties(0)
    log(f"[bench] device {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs")

    plan = run_plan(args.workload, args.steps, args.warmup)
    entries = {}
    for name, steps, warmup, _ in plan:
        entries[name] = bench_workload(name, steps, warmup, not args.no_cpu_baseline,
                                       CPU_SAMPLE.get(name))
    head_name = plan[0][0]
    head = entries[head_name]
    out = {"metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
           "higher_is_better": head["unit"] != "us/step", "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic"}
    cfg = dict(head["config"])
    cfg = {"workload": head["workload"], **cfg}
    out["config"] = cfg
    for k in ("roofline", "roofline_chunk", "roofline_note", "step_bound_us", "cpu_baseline",
              "cpu_baseline_chunk", "step_us_median", "step_us_min", "kernels_us"):
        if k in head:
            out[k] = head[k]
    if len(plan) > 1:
        out["items"] = {n: entries[n] for n, _, _, _ in plan[1:]}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
