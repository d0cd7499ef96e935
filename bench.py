"""Benchmark: one flash-decoding step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fp8_32k] [--num-partitions 0]
                    [--block-size B] [--seq-len T] [--layout contiguous|ordered|fragmented] [--batch N]

The last four override the named workload (page-size / length / layout sweeps); the default run
uses none of them.

Prints ONE JSON line. After W warmup steps, untimed steps continue for --settle-ms (200 ms) so
that the GPU clocks have ramped (reported as `settle`). A step is one fd_decode_attention call
(split-KV partition kernel + combine kernel) over one batch of synthetic, seeded inputs already
resident in HBM. Each step reads a different copy of the KV cache (the copies are rotated) so no
step is served from the 256 MB Infinity Cache left warm by the previous one.

value           = KV-read bytes (K + V payload + scales) per step / mean step time, in GB/s;
                  value_chunks = the same rate over consecutive chunks of the K timed steps
                  (events between chunks), min / median / max; step_us_p10_p50_p90 = the
                  spread of single steps timed with events each.
roofline        = the partition kernel: the same algorithmic bytes / its mean duration from
                  HIP events recorded around it on its stream, against 8 TB/s HBM peak; traffic =
                  HBM bytes per launch from committed rocprofv3 counter runs of the same sources.
read_probe      = streaming reads of 4 GiB, best over three load designs (plain grid-stride 128-bit
                  loads; nontemporal loads with 4 or 8 per lane in flight over 1 KB chunks) and
                  four grid sizes: the practical read ceiling.
warm            = the same steps on one KV copy (possibly Infinity-Cache-served; context only).
graph           = the same step captured once per KV copy in a HIP graph and replayed (launch
                  overhead removed; `value` stays the eager call).
cpu_baseline    = the fp64 oracle on the host threads this process may use (its CPU affinity, capped
                  by OMP_NUM_THREADS where the machine sets one), the whole step, same inputs;
                  one_core = the oracle on one thread over a bounded sample of whole sequences.
context         = the one profiling observation the decode-attention pages give for their own
                  hardware (H100), quoted as context only.
gpu_state       = GPU clock levels and power (amdgpu sysfs) right after the timed steps.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved KV-read HBM GB/s (% of peak) and µs per decode step"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
KERNEL_SRCS = [os.path.join(ROOT, "decode_attention_06_amd", "csrc", f)
               for f in ("fd_kernels.hip", "fd_wide.hip", "fd_direct.hip", "fd_device.h", "fd_internal.h")]


def strip_comments(src: str) -> str:
    """C/C++ source without comments and with runs of whitespace collapsed (string literals
    kept; a '//' inside one does not start a comment)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c == '"':
            j = i + 1
            while j < n and src[j] != '"':
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_hash() -> str:
    """Hash of the device code (comments and layout ignored): committed counter runs count only
    while it is unchanged."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(strip_comments(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def partition_kernel_name(case) -> str:
    """Which partition kernel the library's plan runs for this case: E4M3 or INT8 KV, head_dim 128
    and a multiple of 64 query heads per kv head take the wide-group kernel (f16 / bf16 KV: a
    multiple of 128 heads; any query window); otherwise E4M3 KV, head_dim 128 and a multiple of 32
    MFMA columns per kv head (query heads x query tokens) the 32-column kernel; everything else
    the 16-head kernel."""
    if case.d == 128 and (
            (case.kv_dtype in ("fp8_e4m3", "int8") and case.group % 64 == 0)
            or (case.kv_dtype in ("f16", "bf16") and case.group % 128 == 0)):
        return "wide_partition_kernel"
    if case.kv_dtype == "fp8_e4m3" and case.d == 128 and (case.group * case.nq) % 32 == 0:
        return "direct_partition_kernel"
    return "partition_kernel"


def compute_note(case) -> str:
    """The arithmetic the partition kernel runs for this case's dtypes."""
    kern = partition_kernel_name(case)
    wide_fp8 = kern in ("wide_partition_kernel", "direct_partition_kernel")
    qk = {"fp8_e4m3": ("E4M3 K on FP8 MFMAs with q as exact E4M3 terms, f16 MFMA p.v" if wide_fp8
                       else f"E4M3 K -> {case.q_dtype} MFMA q.k, f16 MFMA p.v"),
          "int8": ("INT8 K and V staged as exact f16 (once per workgroup), f16 MFMA q.k (q scaled "
                   "exactly into f16) and p.v" if kern == "wide_partition_kernel"
                   else "INT8 K/V -> f16 (exact) MFMA q.k (q scaled into f16) and p.v"),
          "f16": ("f16 MFMA q.k and p.v, K/V tiles shared through LDS" if kern == "wide_partition_kernel"
                  else "f16 MFMA q.k and p.v"),
          "bf16": ("bf16 MFMA q.k, bf16 MFMA p.v (p split into two bf16 terms), K/V tiles shared through LDS"
                   if kern == "wide_partition_kernel"
                   else "bf16 MFMA q.k, bf16 MFMA p.v (p split into two bf16 terms)")}[case.kv_dtype]
    return qk + ", f32 softmax and accumulate"


def measured_traffic(workload: str, partitions: int, overridden: bool = False):
    """HBM traffic per partition launch from committed rocprofv3 counter runs, if they were
    taken on the current device code, with the same partition count, on the workload as
    defined; else None."""
    if overridden:
        return None
    path = os.path.join(ROOT, "profiles", f"traffic_partition_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_src_sha256_16") != kernel_hash() or rec.get("partitions") != partitions:
        return None
    return rec.get("traffic_bytes_per_launch")


def kv_append_timing(fd, torch, case, target, stream, reps=50):
    """fd_kv_append of one new token per sequence (bf16 rows, quantised into the cache): mean
    launch duration over `reps` back-to-back calls.  Each call rewrites the last existing row of
    every sequence (pos = seq_len - 1), always a valid row of the cache."""
    dev = target.k_cache.device
    g = torch.Generator(device=dev).manual_seed(1)
    k_new = torch.randn((case.batch, case.hkv, case.d), generator=g, device=dev).to(torch.bfloat16)
    v_new = torch.randn((case.batch, case.hkv, case.d), generator=g, device=dev).to(torch.bfloat16)
    pos = (target.seq_len.to(torch.int64) - 1).clamp(min=-1).to(torch.int32)

    def call():
        fd.kv_append(k_new, v_new, target.k_cache, target.v_cache, pos, kv_dtype=case.kv_dtype,
                     block_table=target.block_table, kv_start=target.kv_start,
                     block_size=case.block_size, scale_mode=case.scale_mode, k_scale=target.k_scale,
                     v_scale=target.v_scale, stream=stream.cuda_stream)

    for _ in range(3):
        call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    rows = int((target.seq_len > 0).sum()) * case.hkv * 2
    eb = {"fp8_e4m3": 1, "int8": 1, "f16": 2, "bf16": 2}[case.kv_dtype]
    moved = rows * case.d * (2 + eb) + (rows * 4 if case.scale_mode == "token_head" else 0)
    us = a.elapsed_time(b) * 1e3 / reps
    return {"us_per_call": round(us, 2), "rows": rows, "bytes_moved": moved,
            "what": "fd_kv_append: one bf16 K and V row per (sequence, kv head) into the cache"}


def one_core_oracle(oracle, prob, case, np, min_tokens=20000):
    """The oracle on one host thread over a bounded sample: whole sequences in index order until
    they hold at least `min_tokens` tokens; the rate is that sample's KV bytes over its time."""
    seqs, tok = [], 0
    for b, n in enumerate(case.seq_lens):
        if n > 0:
            seqs.append(b)
            tok += n
        if tok >= min_tokens:
            break
    if not seqs:
        return None
    per_token = case.kv_read_bytes() / max(sum(case.seq_lens), 1)
    t0 = time.perf_counter()
    oracle.decode_attention(prob, seqs=seqs, nthreads=1)
    dt = time.perf_counter() - t0
    return {"value": round(per_token * tok / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "sample": f"sequences {seqs[0]}..{seqs[-1]} ({len(seqs)} sequences, {tok} tokens, all heads), "
                      f"one run: {dt:.2f} s wall"}


def gpu_state():
    """Clock levels and power of the GPU right after the timed steps (boost clocks change kernel
    times from run to run), read from the amdgpu driver's sysfs files -- no program is started.
    None where the files are not visible."""
    import glob
    for dev in sorted(glob.glob("/sys/class/drm/card[0-9]*/device")):
        try:
            if open(os.path.join(dev, "vendor")).read().strip() != "0x1002":
                continue
        except OSError:
            continue
        state = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            try:
                levels = open(os.path.join(dev, name)).read().splitlines()
            except OSError:
                continue
            cur = [ln.split(":", 1)[-1].strip(" *") for ln in levels if ln.rstrip().endswith("*")]
            state[name[7:] + "_current"] = cur[0] if cur else None
        for hw in glob.glob(os.path.join(dev, "hwmon", "hwmon*")):
            for f in ("power1_average", "power1_input"):
                try:
                    state[f + "_W"] = int(open(os.path.join(hw, f)).read()) / 1e6
                except (OSError, ValueError):
                    pass
        if state:
            return {"source": dev, **state}
    return None


def graph_step_timing(torch, step, ncopy, steps, stream):
    """The same step captured once per KV copy in a HIP graph (the library is capture-safe: no
    allocation, memset or host sync) and replayed `steps` times, rotating the copies as the eager
    loop does.  Returns microseconds per step."""
    graphs = []
    for i in range(ncopy):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i, torch.cuda.current_stream().cuda_stream)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(3 * ncopy):
        graphs[i % ncopy].replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(steps):
        graphs[i % ncopy].replay()
    b.record()
    torch.cuda.synchronize()
    return round(a.elapsed_time(b) * 1e3 / steps, 2)


PROBE_KINDS = {0: "plain 128-bit loads, grid-stride, 4 per lane in flight",
               1: "nontemporal 128-bit loads over 1 KB chunks, 4 per lane in flight",
               2: "nontemporal 128-bit loads over 1 KB chunks, 8 per lane in flight"}


def read_probe(fd, torch, dev, stream, nbytes=4 << 30, reps=5):
    """The practical HBM read ceiling: streaming reads of a 4 GiB buffer (fd_hbm_read_probe), best
    over three load designs and four grid sizes, mean of `reps` back-to-back reads each; every
    design's best is reported too."""
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    best, per_kind = (0.0, 0, 0), {}
    for kind in PROBE_KINDS:
        for blocks in (512, 768, 1024, 2048):
            out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
            fd.hbm_read_probe(buf, out, blocks, kind=kind, stream=stream.cuda_stream)  # warm
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fd.hbm_read_probe(buf, out, blocks, kind=kind, stream=stream.cuda_stream)
            b.record(stream)
            torch.cuda.synchronize()
            gbs = nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
            best = max(best, (gbs, blocks, kind))
            per_kind[kind] = max(per_kind.get(kind, 0.0), gbs)
    del buf
    return {"gbs": round(best[0], 1), "bytes": nbytes, "blocks_of_256": best[1], "kind": PROBE_KINDS[best[2]],
            "best_per_design": {PROBE_KINDS[k]: round(v, 1) for k, v in per_kind.items()}}


class Roctx:
    """roctx ranges around phases of the run, visible in a rocprofv3 marker trace (the AMD
    counterpart of NVTX ranges); no-ops when the library is not there."""

    def __init__(self):
        import ctypes
        self.lib = None
        for name in ("libroctx64.so", "/opt/rocm/lib/libroctx64.so"):
            try:
                self.lib = ctypes.CDLL(name)
                self.lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
                break
            except OSError:
                continue

    def push(self, name: str):
        if self.lib:
            self.lib.roctxRangePushA(name.encode())

    def pop(self):
        if self.lib:
            self.lib.roctxRangePop()


# The decode-attention pages' own profiling observation (one H100-SXM5 trace of a long-context
# FP8-KV decode), reported next to the result as context, never as a target.
CONTEXT = {"source": "从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash-Decode, section 1",
           "hardware": "H100-SXM5 (sm_90)",
           "observation": "about 73 % of SM cycles stalled waiting on L2 refills during the flash-decode kernel",
           "workload": "long-context MQA decode with FP8 KV and FP16 compute"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed steps after the warmup until the GPU has been busy this long")
    ap.add_argument("--workload", default="fp8_32k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--num-partitions", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="KV copies rotated across steps (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--no-read-probe", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing")
    ap.add_argument("--block-size", type=int, default=None, help="page size override (16, 32, 64)")
    ap.add_argument("--seq-len", type=int, default=None, help="every sequence this many tokens")
    ap.add_argument("--layout", choices=("contiguous", "ordered", "fragmented"), default=None,
                    help="contiguous rows, or pages in table order / shuffled")
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--nq", type=int, default=None, help="query tokens per sequence (a verify window)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this decode path is single-GPU by design.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import decode_attention_06_amd as fd
    import workloads

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    overrides, seq_lens = {}, None
    if args.batch is not None:
        overrides["batch"] = args.batch
    if args.nq is not None:
        overrides["nq"] = args.nq
    if args.block_size is not None:
        overrides["block_size"] = args.block_size
    if args.layout is not None:
        overrides["paged"] = args.layout != "contiguous"
        overrides["shuffle"] = args.layout == "fragmented"
    if args.seq_len is not None:
        nb = args.batch if args.batch is not None else workloads.WORKLOADS[args.workload]["batch"]
        seq_lens = [args.seq_len] * nb
        overrides["max_seq_len"] = args.seq_len
    case = workloads.make_case(args.workload, seed=args.seed, device=dev, seq_lens=seq_lens, **overrides)
    kv_bytes = case.kv_read_bytes()
    ncopy = args.copies or max(2, math.ceil(2 * MALL_BYTES / max(kv_bytes, 1)) + 1)
    copies = [case]
    for _ in range(ncopy - 1):
        c = workloads.Case(**{k: getattr(case, k) for k in case.__dataclass_fields__})
        c.k_cache = case.k_cache.clone()
        c.v_cache = case.v_cache.clone()
        if case.k_scale is not None:
            c.k_scale = case.k_scale.clone()
            c.v_scale = case.v_scale.clone()
        copies.append(c)
    # [batch][hq][d] -- or [batch][nq][hq][d] for a window of nq query tokens: the kernels write
    # one row per query row, so the buffers take q's shape
    out = torch.empty(tuple(case.q.shape), dtype=torch.float32, device=dev)
    lse = torch.empty(tuple(case.q.shape[:-1]), dtype=torch.float32, device=dev)
    wsb = fd.workspace_bytes(case.batch, case.hq, case.hkv, case.d, case.max_seq_len, case.block_size,
                             case.kv_dtype, args.num_partitions, num_query=case.nq)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    nparts = fd.plan_partitions(case.batch, case.hq, case.hkv, case.d, case.max_seq_len,
                                case.block_size, case.kv_dtype, args.num_partitions, num_query=case.nq)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        fd.decode_case(copies[i % ncopy], out=out, lse=lse, workspace=ws,
                       num_partitions=args.num_partitions, stream=stream.cuda_stream)

    for i in range(args.warmup):
        step(i)
    # clock settle: after idle the GPU's clocks take ~10 ms of load to ramp (steps run up to 10 %
    # slower meanwhile), so untimed steps continue until the GPU has been busy for settle_ms;
    # the timed steps then see steady-state decode, as a serving loop does
    torch.cuda.synchronize()
    settle_steps, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        for _ in range(8):
            step(args.warmup + settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t0) * 1e3

    # ---- timed region: exactly K steps, back to back (events between chunks of them give the
    # spread of the same measurement)
    roctx = Roctx()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    nchunk = max(1, min(8, args.steps // 10))
    bounds = [round(j * args.steps / nchunk) for j in range(nchunk + 1)]
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(nchunk + 1)]
    torch.cuda.synchronize()
    roctx.push(f"timed steps ({args.steps})")
    t_start.record(stream)
    cev[0].record(stream)
    for j in range(nchunk):
        for i in range(bounds[j], bounds[j + 1]):
            step(i)
        cev[j + 1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    roctx.pop()
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps
    chunk_gbs = sorted(kv_bytes * (bounds[j + 1] - bounds[j]) / (cev[j].elapsed_time(cev[j + 1]) * 1e-3) / 1e9
                       for j in range(nchunk) if bounds[j + 1] > bounds[j])
    state = gpu_state()

    # ---- the same K steps on one KV copy: warm, served from the 256 MB Infinity Cache when the
    # step's KV fits in it (context only; `value` is the rotated, cold measurement above)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(0)
    t_end.record(stream)
    torch.cuda.synchronize()
    warm_ms = t_start.elapsed_time(t_end) / args.steps

    # ---- partition-kernel durations from HIP events recorded around it, on its stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:  # create the underlying HIP events (torch creates them on first record)
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        fd.set_profile_events(*evs[i])
        step(i)
    fd.set_profile_events(None, None)
    torch.cuda.synchronize()
    kdur_ms = [a.elapsed_time(b) for a, b in evs]
    kmean_ms = float(np.mean(kdur_ms))

    # ---- each step on its own: events around every whole step (partition + combine); the events
    # leave gaps between steps, so this gives the spread, not `value`
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    sdur_us = [a.elapsed_time(b) * 1e3 for a, b in evs]
    k_achieved = kv_bytes / (kmean_ms * 1e-3) / 1e9

    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"steps": settle_steps, "ms": round(settle_ms, 1),
                   "what": "untimed steps after the warmup until the clocks reach steady state"},
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "value_chunks": {"n": len(chunk_gbs), "min": round(chunk_gbs[0], 1),
                         "median": round(float(np.median(chunk_gbs)), 1), "max": round(chunk_gbs[-1], 1),
                         "what": "GB/s over consecutive chunks of the timed steps"},
        "step_us_p10_p50_p90": [round(float(np.percentile(sdur_us, q)), 2) for q in (10, 50, 90)],
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"int8": "f16", "f16": "f16"}.get(case.kv_dtype, case.q_dtype),
        "data": "synthetic",
        "config": {
            "workload": args.workload, "batch": case.batch, "num_q_heads": case.hq,
            "num_kv_heads": case.hkv, "head_dim": case.d, "kv_dtype": case.kv_dtype,
            "q_dtype": case.q_dtype, "scale_mode": case.scale_mode, "block_size": case.block_size,
            "tokens": int(sum(case.seq_lens)), "max_seq_len": case.max_seq_len,
            "kv_read_bytes": kv_bytes, "partitions": nparts,
            "kv_copies_rotated": ncopy, "seed": args.seed,
            "overrides": {"block_size": args.block_size, "seq_len": args.seq_len, "layout": args.layout,
                          "batch": args.batch, "nq": args.nq} if (overrides or seq_lens) else None,
            "compute": compute_note(case),
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": partition_kernel_name(case),
            "bound": "hbm",
            "achieved": round(k_achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(k_achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.workload, nparts, bool(overrides or seq_lens)),
            "kernel_us_mean": round(kmean_ms * 1e3, 2),
            "kernel_us_p10_p90": [round(float(np.percentile(kdur_ms, 10)) * 1e3, 2),
                                  round(float(np.percentile(kdur_ms, 90)) * 1e3, 2)],
            "algorithmic_bytes_per_launch": kv_bytes,
        },
        "cpu_baseline": None,
    }

    result["warm"] = {"us_per_step": round(warm_ms * 1e3, 2),
                      "gbs": round(kv_bytes / (warm_ms * 1e-3) / 1e9, 2),
                      "what": "the same KV copy every step, back to back: possibly served from the "
                              "256 MB Infinity Cache (context, not the value)"}
    result["kv_append"] = kv_append_timing(fd, torch, case, copies[0], stream)

    if not args.no_graph:
        def graph_step(i, s):
            fd.decode_case(copies[i % ncopy], out=out, lse=lse, workspace=ws,
                           num_partitions=args.num_partitions, stream=s)
        result["graph"] = {"us_per_step": graph_step_timing(torch, graph_step, ncopy, args.steps, stream),
                           "what": "the same step captured once per KV copy in a HIP graph, replayed"}

    if not args.no_read_probe:
        result["read_probe"] = read_probe(fd, torch, dev, stream)
        result["roofline"]["frac_of_read_probe"] = round(k_achieved / result["read_probe"]["gbs"], 4)

    if not args.no_cpu_baseline:
        import oracle
        threads = args.cpu_threads or oracle.host_threads()
        prob = oracle.Problem.from_case(case)
        # the whole step on the host cores (the oracle's cost is linear in tokens x heads);
        # median of 3 wall-clock runs (a single run for steps over 2M tokens)
        runs = 1 if sum(case.seq_lens) > 2_000_000 else 3
        times = []
        for _ in range(runs):
            t0 = time.perf_counter()
            oracle.decode_attention(prob, nthreads=threads)
            times.append(time.perf_counter() - t0)
        dt = float(np.median(times))
        result["cpu_baseline"] = {
            "value": round(kv_bytes / dt / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "host_cpus": {"os_cpu_count": os.cpu_count(),
                          "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
                          "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")},
            "kind": "oracle",
            "sample": f"the whole step ({case.batch} sequences, {sum(case.seq_lens)} tokens, all heads), "
                      f"median of {runs} run(s): {dt:.2f} s wall",
            "us_per_step": round(dt * 1e6, 1),
            "one_core": one_core_oracle(oracle, prob, case, np),
        }
    result["gpu_state"] = state
    result["context"] = CONTEXT
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
