#!/usr/bin/env python
"""Benchmark of the paged-KV hot path on one MI355X.

A step is one pass of the whole path over one batch: the KV block write of
the step's new tokens, then paged attention (device-side plan, split-context
decode, partition merge, prefill).  Default workload: the Llama-3-8B-shaped
decode batch (256 requests, 32 query / 8 KV heads, head_dim 128, one new
token each over a cached context uniform in [512, 4096], blocks scattered at
random in a pool sized to the total).  ``value`` is KV bytes attention must
read (per request, L * 2 * Hkv * D * 2) per second of whole-step time.

Also reported on the same line:
* ``roofline`` for the dominant kernel (decode): algorithmic KV bytes per
  launch / the kernel's mean duration, timed with two HIP events recorded on
  the launch stream around that kernel only, over as many steps again as the
  timed ones (``kernels_us`` breaks a step down with events around every
  kernel, in a third pass);
* ``prefill``: the prefill batch (16 prompts of 256..2048 tokens), attention
  TFLOP/s of the prefill kernel against the bf16 dense MFMA peak;
* ``cpu_baseline``: the fp64 CPU oracle on a bounded sample of the same
  decode batch (gather + attention timed; data generation not).

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


def run_steps(setup, steps, warmup, dominant):
    """Time `steps` steps; returns (ms_per_step, per-kernel mean us, mean us
    of the `dominant` kernel).

    The whole-step time comes from the timed steps alone (nothing but the
    calls between the two events).  The dominant kernel's time (the one the
    roofline is reported for) comes from the same number of steps run again
    with only the two HIP events around that kernel; the per-kernel breakdown
    from a third such pass with events around every kernel (each record adds
    a few microseconds between kernels, and the idle gaps slow the prefill
    kernel that follows them by several per cent, so the roofline does not
    use that pass)."""
    import torch

    pkv = setup.pkv
    mk = lambda: torch.cuda.Event(enable_timing=True)
    stage_sets = [[mk() for _ in range(5)] for _ in range(steps)]
    write_sets = [(mk(), mk()) for _ in range(steps)]
    for evs in stage_sets + write_sets:        # create the HIP events outside the timed region
        for e in evs:
            e.record()
    for _ in range(warmup):
        setup.step()
    torch.cuda.synchronize()
    start, end = mk(), mk()
    start.record()
    for _ in range(steps):
        setup.step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps

    # the dominant kernel alone: events around it only
    names = ["plan", "decode", "decode_merge", "prefill"]
    k = names.index(dominant)
    dom_sets = [[mk(), mk()] for _ in range(steps)]
    for evs in dom_sets:
        for e in evs:
            e.record()
    torch.cuda.synchronize()
    for i in range(steps):
        evs = [None] * 5
        evs[k], evs[k + 1] = dom_sets[i]
        pkv.paged_attention_set_stage_events(evs)
        pkv.paged_kv_write(setup.k, setup.v, setup.slots, setup.pool)
        pkv.paged_attention(setup.q, setup.pool, setup.bt, setup.cu, setup.lens, setup.wl.scale,
                            out=setup.out, workspace=setup.ws)
    torch.cuda.synchronize()
    pkv.paged_attention_set_stage_events(None)
    dom_us = 1e3 * float(np.mean([a.elapsed_time(b) for a, b in dom_sets]))

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
          for i, n in enumerate(names)}
    us["kv_write"] = 1e3 * float(np.mean([a.elapsed_time(b) for a, b in write_sets]))
    status = pkv.paged_attention_device_status(setup.ws)
    if status:
        raise RuntimeError(f"device status {status}: metadata rejected")
    return ms, us, dom_us


def cpu_baseline_decode(wl, sample):
    """The fp64 oracle on `sample` requests of a decode batch: gather from a
    host pool + attention, timed; generation and pool filling untimed."""
    from threadpoolctl import threadpool_limits

    from oracle import paged

    cores = len(os.sched_getaffinity(0))
    sel = list(range(min(sample, wl.num_seqs)))
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
            "sample": f"{len(sel)} of {wl.num_seqs} requests of the same batch "
                      f"({kv / 1e9:.3f} GB of KV), gather + fp64 attention timed: {dt:.2f} s"}


def prefill_cpu_baseline(wl):
    from threadpoolctl import threadpool_limits

    from oracle import bf16, paged

    cores = len(os.sched_getaffinity(0))
    s = int(np.argmin(wl.new_tokens))
    n = int(wl.new_tokens[s])
    k, v = wl.request_kv(s)
    q = wl.q()[wl.cu_seqlens_q[s]:wl.cu_seqlens_q[s + 1]]
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        paged.attend_dense(bf16.to_f64(q), bf16.to_f64(k), bf16.to_f64(v), wl.scale, 0)
        dt = time.perf_counter() - t0
    flops = 4 * wl.head_dim * wl.num_q_heads * n * (n + 1) // 2
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"segment {s} ({n} tokens) of the prefill batch: {dt:.2f} s"}


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
    "decode_kernel": ["decode.hip", "common.hpp", "kernels.hpp"],
    "prefill_kernel": ["prefill.hip", "common.hpp", "kernels.hpp"],
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
        f"python bench.py --workload {args.workload} --steps 3 --warmup 1 --no-prefill --no-cpu-baseline",
        f"#   rocprofv3 --pmc WRITE_SIZE --kernel-include-regex {args.kernel} -f csv -d <W> -o k -- "
        f"python bench.py --workload {args.workload} --steps 3 --warmup 1 --no-prefill --no-cpu-baseline",
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


def trace_summary(args):
    """Per-kernel durations from a rocprofv3 --kernel-trace CSV of a bench
    command.  For the default command (decode_8b) the trace is split into its
    two phases (decode_8b, then prefill_8b) by counting the KV-write
    dispatches that open every step; for another --workload it is one phase."""
    path = glob.glob(os.path.join(args.trace, "*kernel_trace.csv"))[0]
    with open(path) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))
    rows = [r for r in rows if "pkv::" in r["Kernel_Name"]]
    default = args.workload == "decode_8b"
    wl_flag = "" if default else f" --workload {args.workload}"
    if default:
        n_dec = args.warmup + 3 * args.steps             # decode_8b steps (timed + two event passes)
        phases, seen = {"decode_8b": [], "prefill_8b": []}, 0
        for r in rows:
            if "kv_write" in r["Kernel_Name"]:
                seen += 1
            phases["decode_8b" if seen <= n_dec else "prefill_8b"].append(r)
        title = "default bench (decode_8b headline, prefill_8b line item)"
    else:
        phases = {args.workload: rows}
        title = f"{args.workload}: {DESCRIPTIONS[args.workload]}"
    out = [f"# Kernel trace: {title}", "",
           "Command (from the repository root, on one MI355X):", "",
           f"    rocprofv3 --kernel-trace --stats -f csv -d <T> -o kt -- python bench.py{wl_flag} "
           f"--steps {args.steps} --warmup {args.warmup} --no-cpu-baseline",
           f"    python bench.py --trace-summary --trace <T>{wl_flag} --steps {args.steps} --warmup {args.warmup}",
           "", "Durations in microseconds (end - start of each dispatch): per step one warm-up, then "
           "three passes of the steps (timed; events around the roofline kernel; events around "
           "every kernel).", ""]
    for ph, rs in phases.items():
        by = {}
        for r in rs:
            name = r["Kernel_Name"].replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            by.setdefault(name, {"d": [], "r": r})["d"].append(d)
        out += [f"### phase: {ph}", "", "| kernel | calls | avg us | min us | max us | grid (threads) | wg | vgpr | lds B |",
                "|---|---|---|---|---|---|---|---|---|"]
        for name, v in sorted(by.items(), key=lambda kv: -sum(kv[1]["d"])):
            d, r = v["d"], v["r"]
            out.append(f"| {name} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | {max(d):.1f} | "
                       f"{r['Grid_Size_X']} | {r['Workgroup_Size_X']} | {r['VGPR_Count']} | {r['LDS_Block_Size']} |")
        out.append("")
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


def measure(name, steps, warmup):
    import torch

    wl, nb = make_workload(name)
    log(f"[bench] {name}: S={wl.num_seqs} T={wl.num_tokens} NB={wl.num_blocks}")
    st = Setup(wl, pool_blocks=nb)
    dominant = "prefill" if name == "prefill_8b" else "decode"
    ms, us, dom_us = run_steps(st, steps, warmup, dominant)
    res = {"wl": wl, "ms": ms, "us": us, "dom_us": dom_us, "pool_tokens": wl.num_blocks * 16}
    del st
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode_8b", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-batch line item")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=160, help="decode requests the oracle runs")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--group-members", type=int, default=0,
                    help="most members of a shared-prefix group (0: automatic, 1: no groups)")
    ap.add_argument("--pmc-summary", action="store_true",
                    help="summarise four rocprofv3 counter runs (see --fetch .. --calib-write)")
    ap.add_argument("--trace-summary", action="store_true",
                    help="summarise a rocprofv3 kernel-trace CSV of the default bench (--trace DIR)")
    ap.add_argument("--trace")
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

    main_res = measure(args.workload, args.steps, args.warmup)
    wl = main_res["wl"]
    ms = main_res["ms"]
    us = main_res["us"]
    dom_us = main_res["dom_us"]
    kv_bytes = wl.kv_bytes_unique()
    flops = wl.attention_flops()
    # segments on the split-context decode path: n * G <= 32 and n <= 8
    max_dec = min(8, 32 // (wl.num_q_heads // wl.num_kv_heads))
    decode_segs = np.nonzero((wl.new_tokens >= 1) & (wl.new_tokens <= max_dec))[0]
    prefill_segs = np.nonzero(wl.new_tokens > max_dec)[0]
    dec_bytes = int(wl.seq_lens[decode_segs].astype(np.int64).sum()) * 2 * wl.num_kv_heads * wl.head_dim * 2
    if wl.shared_prefix:
        dec_bytes = kv_bytes - int(wl.seq_lens[prefill_segs].astype(np.int64).sum()) * 2 * wl.num_kv_heads * wl.head_dim * 2
    pre_flops = wl.attention_flops(segments=prefill_segs) if prefill_segs.size else 0

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic"}
    cfg = {"workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}",
           "num_seqs": wl.num_seqs, "num_tokens": wl.num_tokens,
           "heads": [wl.num_q_heads, wl.num_kv_heads], "head_dim": wl.head_dim,
           "block_size": 16, "pool_blocks": wl.num_blocks,
           "kv_bytes": kv_bytes, "attention_flops": flops}
    if args.workload == "prefill_8b":
        out.update(value=flops / (ms * 1e-3) / 1e12, unit="TFLOP/s")
        ach = pre_flops / (dom_us * 1e-6) / 1e12
        out["roofline"] = {"kernel": "prefill_kernel<128>", "bound": "mfma", "achieved": ach,
                           "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / MFMA_BF16_PEAK_TFLOPS, "kernel_us": dom_us,
                           "traffic": stored_traffic("prefill_kernel", args.workload)}
    elif args.workload == "tiny_mixed":
        out.update(value=kv_bytes / (ms * 1e-3) / 1e9, unit="GB/s")
        out["roofline"] = None
    else:
        out.update(value=kv_bytes / (ms * 1e-3) / 1e9, unit="GB/s")
        ach = dec_bytes / (dom_us * 1e-6) / 1e9
        out["roofline"] = {"kernel": "decode_kernel<128>", "bound": "hbm", "achieved": ach,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                           "kernel_us": dom_us,
                           "traffic": stored_traffic("decode_kernel", args.workload),
                           "algorithmic_bytes": dec_bytes}
    out["config"] = cfg
    out["kernels_us"] = us
    if args.workload == "long_decode_70b":
        cfg["pool_holds_tokens"] = main_res["pool_tokens"]
    if args.workload == "cb_step_8b":
        cfg["kv_bytes_logical"] = wl.kv_bytes_logical()
        out["chunk_prefill_tflops"] = pre_flops / (us["prefill"] * 1e-6) / 1e12

    if args.workload == "decode_8b" and not args.no_prefill:
        pr = measure("prefill_8b", max(5, args.steps // 2), args.warmup)
        pwl = pr["wl"]
        pflops = pwl.attention_flops()
        ach = pflops / (pr["dom_us"] * 1e-6) / 1e12
        out["prefill"] = {"workload": f"prefill_8b: {DESCRIPTIONS['prefill_8b']}",
                          "ms_per_step": pr["ms"], "attention_flops": pflops,
                          "tflops_step": pflops / (pr["ms"] * 1e-3) / 1e12,
                          "roofline": {"kernel": "prefill_kernel<128>", "bound": "mfma",
                                       "achieved": ach, "peak": MFMA_BF16_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFLOPS,
                                       "kernel_us": pr["dom_us"],
                                       "traffic": stored_traffic("prefill_kernel", "prefill_8b")},
                          "kernels_us": pr["us"]}

    if not args.no_cpu_baseline:
        if args.workload in ("decode_8b", "long_decode_70b", "cb_step_8b", "spec_verify_8b",
                             "spec_verify_70b"):
            import workloads
            base_wl = workloads.make("decode_8b") if args.workload == "decode_8b" else wl
            if args.workload == "decode_8b":
                out["cpu_baseline"] = cpu_baseline_decode(base_wl, args.cpu_sample)
            else:
                out["cpu_baseline"] = cpu_baseline_decode(base_wl, 4)
        elif args.workload == "prefill_8b":
            out["cpu_baseline"] = prefill_cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
