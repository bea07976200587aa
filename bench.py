#!/usr/bin/env python3
"""Benchmark of the MoE token-reordering hot path on one MI355X.

One step = one pass of the whole path over the four large synthetic workloads, each a
single library call on the current stream:
  batching BF16   A=16 BS=32 K+1=9  H=7168, 256 experts (Zipf 1.1), 5% masked
  batching INT8   A=64 BS=64 K+1=9  H=7168 + FP32 scale, 16 layers x 64 experts, 20% masked
  unpermute non-padded  T=16384 topK=8 E=128 H=4096 BF16, FP32 probs, 10% empty slots
  unpermute padded      E=64 C=512 T=8192 H=5120 FP16, FP16 probs (top-4)
The printed value is effective HBM bandwidth: the step's algorithmic bytes (every input
byte the operations need, read once, plus every output byte, written once) divided by
the measured step time.  Inputs are resident in HBM before timing; the step's working
set (~2 GB) is far above the 256 MB Infinity Cache, so steps do not hit in it.

Also reported, per workload: the median, p10 and p90 call time with L2 and the
Infinity Cache flushed (a 1 GiB write) before every iteration, the warm back-to-back
time, and a plain device copy moving the same number of bytes (what a streaming kernel
reaches); the roofline of the dominant kernel (the non-padded gather-reduce, timed with
HIP events bound to its launch, so the span is that kernel alone); and the CPU oracle
timed on the host (median of 3 runs per workload).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# row bytes of each workload (the unit its row mover copies)
ROW_BYTES = {"batching_bf16": 7168 * 2, "batching_int8": 7168, "unpermute_nonpadded": 4096 * 2,
             "unpermute_padded": 5120 * 2}
METRIC = "effective HBM GB/s (and % of peak) for batching and unpermute; rows/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "unpermute_reduce_nonpadded_bf16_T16384_topk8_H4096.traffic.txt")
REDUCE_SOURCES = ["unpermute_ffnwb_batching_amd/csrc/reduce_kernels.hpp",
                  "unpermute_ffnwb_batching_amd/csrc/device_common.hpp"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--detail-iters", type=int, default=100, help="per-workload timed iterations (0 = skip)")
    ap.add_argument("--no-next-rows", action="store_true", help="skip the measurements outside the step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma list of workloads to keep (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


# ----------------------------------------------------------------------------- timing helpers

_FLUSH = []


def flushed_times(run, stream, iters):
    """Call times (ms) of run(stream), L2 and the 256 MB Infinity Cache flushed by a 1 GiB
    write before each call (outside the timed bracket)."""
    import torch
    if not _FLUSH:
        _FLUSH.append(torch.empty(1 << 30, dtype=torch.uint8, device="cuda"))
    flush = _FLUSH[0]
    ts = []
    for _ in range(iters):
        flush.fill_(1)
        b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record(stream)
        run(stream)
        e.record(stream)
        e.synchronize()
        ts.append(b.elapsed_time(e))
    return np.array(ts)


def warm_ms(run, stream, iters):
    """Mean time (ms) of back-to-back calls."""
    import torch
    b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.record(stream)
    for _ in range(iters):
        run(stream)
    e.record(stream)
    torch.cuda.synchronize()
    return b.elapsed_time(e) / iters


PROBE_LIB = os.path.join(ROOT, "unpermute_ffnwb_batching_amd", "_lib", "libffnwb_probe.so")
_PROBE = []


def probe_copy_gbps(nbytes, row_bytes, stream, iters, shuffled=False):
    """The library's row-mover access pattern as a plain copy (one wavefront per row,
    16-byte non-temporal loads and stores; rows in a random order when shuffled) moving
    nbytes (reads plus writes) in rows of row_bytes, flushed like the calls: the
    achievable rate for that byte count and pattern on this GPU."""
    import ctypes
    import torch
    if not _PROBE:
        lib = ctypes.CDLL(PROBE_LIB)
        lib.ffnwb_probe_copy_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_void_p, ctypes.c_void_p]
        lib.ffnwb_probe_copy_rows.restype = ctypes.c_int
        _PROBE.append(lib)
    lib = _PROBE[0]
    nrows = max(int(nbytes) // (2 * row_bytes), 1)
    src = torch.empty(nrows * row_bytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    order = torch.randperm(nrows, dtype=torch.int32, device="cuda") if shuffled else None
    optr = ctypes.c_void_p(order.data_ptr()) if order is not None else None

    def run(st):
        if lib.ffnwb_probe_copy_rows(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), row_bytes,
                                     nrows, optr, ctypes.c_void_p(st.cuda_stream)) != 0:
            raise RuntimeError("probe copy rejected")
    ts = flushed_times(run, stream, iters)
    del src, dst, order
    return round(2 * nrows * row_bytes / float(np.median(ts)) / 1e6, 1)


def copy_gbps(nbytes, stream, iters):
    """A plain device copy whose reads plus writes equal nbytes, flushed like the calls."""
    import torch
    n = max(int(nbytes) // 2, 1)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ts = flushed_times(lambda st: dst.copy_(src), stream, iters)
    del src, dst
    return round(2 * n / float(np.median(ts)) / 1e6, 1)


# ----------------------------------------------------------------------------- algorithmic bytes

def batching_bytes(c, actual):
    Y = c["A"] * c["BS"] * c["K1"]
    row = c["H"] * (1 if c["token_dtype"] == 2 else 2)
    b = 4 * Y + (Y if c["mask"] is not None else 0) + (4 * c["A"] if c["layer_ids"] is not None else 0)
    b += actual * (2 * row + 16 + (8 if c["token_dtype"] == 2 else 0))
    b += 16 * c["expert_num"] + 8
    return b


def nonpadded_bytes(c):
    T, H = c["restore_shape"]
    sI = c["sorted_indices"]
    N = sI.size
    elt = 4 if c["dtype"] == 3 else 2
    pelt = 4 if c["probs_dtype"] == 3 else 2
    valid = int(((sI >= 0) & (sI < N)).sum())
    nnz = int((c["routing_map"] != 0).sum())
    E = c["routing_map"].shape[1]
    return T * E + nnz * pelt + 4 * N + valid * H * elt + T * H * elt + N * pelt + 8 * N


def nonpadded_reduce_bytes(c):
    """Bytes the gather-reduce kernel alone must move: indices, valid rows and their
    weights, and the output rows."""
    T, H = c["restore_shape"]
    sI = c["sorted_indices"]
    N = sI.size
    elt = 4 if c["dtype"] == 3 else 2
    pelt = 4 if c["probs_dtype"] == 3 else 2
    valid = int(((sI >= 0) & (sI < N)).sum())
    return 4 * N + valid * (H * elt + pelt) + T * H * elt


def padded_bytes(c):
    T, H = c["restore_shape"]
    sI = c["sorted_indices"]
    N = sI.size
    elt = 4 if c["dtype"] == 3 else 2
    pelt = 4 if c["probs_dtype"] == 3 else 2
    nval = int(((sI >= 0) & (sI < T)).sum())
    return 4 * N + nval * pelt + nval * H * elt + T * H * elt + N * pelt + 8 * N


def permute_bytes(c, ref_nnz):
    """Forward permute: the map, each token row once, every output row, the indices
    (non-padded: N rows and slots; padded: the E*C capacity rows and entries)."""
    elt = {0: 2, 1: 2, 2: 1, 3: 4}[c["dtype"]]
    n_out = c["E"] * c["C"] if c.get("padded") else c["N"]
    return c["T"] * c["E"] + c["T"] * c["H"] * elt + n_out * c["H"] * elt + 4 * n_out


def padded_skip_bytes(c):
    """Padded unpermute with the zero-weight skip: as padded_bytes, but only the rows whose
    weight is non-zero are read (every valid entry's weight still is)."""
    T, H = c["restore_shape"]
    sI = c["sorted_indices"]
    N = sI.size
    E = c["probs"].shape[1]
    elt = 4 if c["dtype"] == 3 else 2
    pelt = 4 if c["probs_dtype"] == 3 else 2
    ok = (sI >= 0) & (sI < T)
    i = np.nonzero(ok)[0]
    p = c["probs"]
    if c["probs_dtype"] == 1:      # BF16 bits: widen to FP32
        p = (p.astype(np.uint32) << np.uint32(16)).view(np.float32)
    w = p.astype(np.float32)[sI[i], i // (N // E)]
    nval, nread = int(ok.sum()), int((w != 0).sum())
    return 4 * N + nval * pelt + nread * H * elt + T * H * elt + N * pelt + 8 * N, nread


def measure_skip(args, stream, c):
    """The padded workload with the opt-in zero-weight skip: the rows whose weight is zero
    are not read.  Flushed-cache median and steady-state time; parity with the oracle
    run with the same option."""
    import torch
    from _gpu import prepare_unpermute, fetch_unpermute
    call = prepare_unpermute(c, skip_zero_weight=True)
    for _ in range(3):
        call.run(stream)
    torch.cuda.synchronize()
    alg, nread = padded_skip_bytes(c)
    K = max(args.steps, 5)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(K):
        call.run(stream)
    s1.record(stream)
    torch.cuda.synchronize()
    call_ms = s0.elapsed_time(s1) / K
    nval = int(((c["sorted_indices"] >= 0) & (c["sorted_indices"] < c["restore_shape"][0])).sum())
    res = {"shape": "padded E=64 C=512 T=8192 H=5120 fp16, skip_zero_weight=1",
           "rows_valid": nval, "rows_read": nread, "alg_bytes": alg,
           "us_per_call": round(call_ms * 1e3, 2), "GBps": round(alg / call_ms / 1e6, 1)}
    if args.detail_iters > 0:
        ts = flushed_times(call.run, stream, args.detail_iters)
        res["us_median_flushed"] = round(float(np.median(ts)) * 1e3, 2)
    if not args.no_cpu_baseline:
        from _gpu import oracle_unpermute, check_unpermute
        t1 = time.perf_counter()
        ref = oracle_unpermute(c, skip_zero_weight=True)
        res["cpu_oracle_s"] = round(time.perf_counter() - t1, 3)
        try:
            check_unpermute(c, fetch_unpermute(call, c), ref)
            res["parity"] = True
        except AssertionError as ex:
            res["parity"] = False
            print(f"# parity FAILED for the skip: {ex}", file=sys.stderr, flush=True)
    return res


def ctx_bytes(area, actual):
    """Batching from a ScheduleContext: the context words read, the chosen chunks'
    descriptors, the moved rows (read and written), the per-row ids and group_list."""
    A, n, E = area["A"], area["BS"] * area["K1"], area["expert_num"]
    row = area["row"] - (4 if area["token_dtype"] == 2 else 0)
    return 424 + A * (8 + 4 * n) + actual * (2 * row + 16 + (8 if area["token_dtype"] == 2 else 0)) + 16 * E + 8


def measure_ctx(args, stream):
    """Batching fed by a ScheduleContext at the BF16 batching workload's shape: A=16
    sessions x 4 micro-batches of BS=32, K+1=9 slots, H=7168 BF16 rows, 256 experts;
    the call batches micro-batch 3 with needSchedule=1 (every flag read, all ready)."""
    import torch
    import synth
    from _gpu import prepare_ctx, fetch_batching
    area = synth.schedule_area(13, 16, 4, 32, 9, 7168, 256, 1, synth.BF16)
    call = prepare_ctx(area, 3, 1)
    for _ in range(3):
        call.run(stream)
    torch.cuda.synchronize()
    actual = int(call.out["actual_token_num"].item())
    alg = ctx_bytes(area, actual)
    K = max(args.steps, 5)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(K):
        call.run(stream)
    s1.record(stream)
    torch.cuda.synchronize()
    call_ms = s0.elapsed_time(s1) / K
    res = {"shape": "A=16 M=4 BS=32 K+1=9 H=7168 bf16, 256 experts, micro-batch 3, needSchedule=1",
           "rows": actual, "alg_bytes": alg, "us_per_call": round(call_ms * 1e3, 2),
           "GBps": round(alg / call_ms / 1e6, 1)}
    if args.detail_iters > 0:
        ts = flushed_times(call.run, stream, args.detail_iters)
        res["us_median_flushed"] = round(float(np.median(ts)) * 1e3, 2)
    if not args.no_cpu_baseline:
        from _gpu import oracle_ctx, check_ctx
        t1 = time.perf_counter()
        ref = oracle_ctx(area, call)
        res["cpu_oracle_s"] = round(time.perf_counter() - t1, 3)
        try:
            check_ctx(area, call, fetch_batching(call), ref)
            res["parity"] = True
        except AssertionError as ex:
            res["parity"] = False
            print(f"# parity FAILED for the context batching: {ex}", file=sys.stderr, flush=True)
    return res


def measure_update_expert(args, stream):
    """MoeUpdateExpert at its largest token count: BS=512 tokens x topK=8 over 256
    logical experts placed as 320 instances on 64 ranks (F=9), BF16 scales with a
    per-slot threshold, 400 active tokens, balance by rank.  One launch of 4096 slots:
    its time is latency (three dependent load rounds), not bandwidth."""
    import torch
    import synth
    from _gpu import prepare_update_expert, check_update_expert
    c = synth.update_expert_case(15, 512, 8, 256, 64, 5, F=9, local_rank_id=37, scale_dtype=synth.BF16,
                                 n_active=400)
    call = prepare_update_expert(c)
    for _ in range(3):
        call.run(stream)
    torch.cuda.synchronize()
    K = max(args.steps, 5) * 10
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(K):
        call.run(stream)
    s1.record(stream)
    torch.cuda.synchronize()
    us = s0.elapsed_time(s1) / K * 1e3
    n = 512 * 8
    res = {"shape": "BS=512 topK=8, 256 experts on 64 ranks x 5 instances, F=9, bf16 scales, by rank",
           "us_per_call": round(us, 2), "slots_per_s": round(n / us * 1e6, 1)}
    if not args.no_cpu_baseline:
        t1 = time.perf_counter()
        try:
            check_update_expert(c, call)
            res["parity"] = True
        except AssertionError as ex:
            res["parity"] = False
            print(f"# parity FAILED for the expert update: {ex}", file=sys.stderr, flush=True)
        res["cpu_oracle_s"] = round(time.perf_counter() - t1, 3)
    return res


def measure_permute(args, stream, padded=False):
    """The forward permute (a widening of the path) at the non-padded (or padded)
    unpermute workload's shape: flushed-cache medians, the row-copy kernel's steady-state
    time from fence-free HIP events, and (with the CPU leg) parity with the oracle."""
    import torch
    import synth
    from _gpu import prepare_permute, fetch_permute
    from unpermute_ffnwb_batching_amd.hip_events import HipEvent
    c = synth.permute_padded_config() if padded else synth.permute_config()
    call = prepare_permute(c)
    for _ in range(3):
        call.run(stream)
    torch.cuda.synchronize()
    alg = permute_bytes(c, None)
    K = max(args.steps, 5)
    ev = [(HipEvent(), HipEvent()) for _ in range(K)]
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for i in range(K):
        call.set_copy_events(*ev[i])
        call.run(stream)
    s1.record(stream)
    torch.cuda.synchronize()
    call_ms = s0.elapsed_time(s1) / K
    copy_ms = float(np.mean([b.elapsed_ms(e) for b, e in ev]))
    call.set_copy_events(None, None)
    shape = ("E=64 C=512 T=8192 H=5120 fp16, 4 uniform experts per token" if padded
             else "T=16384 topK=8 E=128 H=4096 bf16, 8 uniform experts per token")
    res = {"shape": shape,
           "alg_bytes": alg, "us_per_call": round(call_ms * 1e3, 2), "GBps": round(alg / call_ms / 1e6, 1),
           "copy_kernel_us": round(copy_ms * 1e3, 2),
           "copy_kernel_GBps": round((alg - c["T"] * c["E"]) / copy_ms / 1e6, 1)}
    if args.detail_iters > 0:
        ts = flushed_times(call.run, stream, args.detail_iters)
        res["us_median_flushed"] = round(float(np.median(ts)) * 1e3, 2)
    if not args.no_cpu_baseline:
        from _gpu import oracle_permute, check_permute
        t1 = time.perf_counter()
        ref = oracle_permute(c)
        res["cpu_oracle_s"] = round(time.perf_counter() - t1, 3)
        res["cpu_oracle_GBps"] = round(alg / res["cpu_oracle_s"] / 1e9, 4)
        try:
            check_permute(c, fetch_permute(call), ref)
            res["parity"] = True
        except AssertionError as ex:
            res["parity"] = False
            print(f"# parity FAILED for the permute: {ex}", file=sys.stderr, flush=True)
    return res


def kernel_source_hash():
    h = hashlib.sha256()
    for p in REDUCE_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(per_launch_alg):
    """HBM traffic of the dominant kernel from the committed rocprofv3 counter summary,
    or None when the summary is missing or was taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build targets one GPU; --gpus {args.gpus} is not supported "
              "(every workload is one GPU's share; see the sharding notes in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import unpermute_ffnwb_batching_amd as F
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from _gpu import (prepare_batching, prepare_unpermute, fetch_batching, fetch_unpermute,
                      check_batching, check_unpermute)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    t0 = time.time()
    names = ["batching_bf16", "batching_int8", "unpermute_nonpadded", "unpermute_padded"]
    if args.only:
        names = [n for n in names if n in args.only.split(",")]
    cases = {}
    for n in names:
        cases[n] = {"batching_bf16": lambda: synth.batching_config(2),
                    "batching_int8": lambda: synth.batching_config(3),
                    "unpermute_nonpadded": lambda: synth.unpermute_config(4),
                    "unpermute_padded": lambda: synth.unpermute_config(5)}[n]()
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    calls = {}
    # the non-padded call's out_index / permute_token_id sort runs on an auxiliary stream
    # the caller owns (default priority), forked and joined inside the call
    aux_stream = torch.cuda.Stream()
    for n, c in cases.items():
        if n.startswith("batching"):
            calls[n] = prepare_batching(c)
        else:
            calls[n] = prepare_unpermute(c, aux_stream=aux_stream if n == "unpermute_nonpadded" else None)
    torch.cuda.synchronize()

    # algorithmic bytes and rows per workload (actual_token_num from the first run)
    for call in calls.values():
        call.run()
    torch.cuda.synchronize()
    alg, rows = {}, {}
    for n, c in cases.items():
        if n.startswith("batching"):
            act = int(calls[n].out["actual_token_num"].item())
            alg[n], rows[n] = batching_bytes(c, act), act
        elif n == "unpermute_nonpadded":
            alg[n] = nonpadded_bytes(c)
            sI = c["sorted_indices"]
            rows[n] = int(((sI >= 0) & (sI < sI.size)).sum())
        else:
            alg[n] = padded_bytes(c)
            rows[n] = int(((c["sorted_indices"] >= 0) & (c["sorted_indices"] < c["restore_shape"][0])).sum())
    step_bytes = sum(alg.values())

    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup
    have_np = "unpermute_nonpadded" in calls
    from unpermute_ffnwb_batching_amd.hip_events import HipEvent
    # fence-free HIP events, bound by the library to the gather-reduce kernel's launch
    hot = [(HipEvent(), HipEvent()) for _ in range(K)]

    def step(i=None):
        for n, call in calls.items():
            if n == "unpermute_nonpadded":
                if i is None:
                    call.set_reduce_events(None, None)
                else:
                    call.set_reduce_events(*hot[i])
            call.run(stream)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    if args.calibrate_copy:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give the scale
        # that converts the counters of the library's kernels into bytes
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(K):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    hot_ms = float(np.mean([b.elapsed_ms(e) for b, e in hot])) if have_np else None
    print(f"# {K} steps, {ms:.4f} ms/step", file=sys.stderr, flush=True)
    # the same steps without the timing hooks, for reference
    s2, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s2.record(stream)
    for _ in range(K):
        step()
    e2.record(stream)
    torch.cuda.synchronize()
    ms_nohook = s2.elapsed_time(e2) / K

    # context: the same four calls issued on four streams (the library keeps no shared
    # state, so independent calls overlap: one call's ordering kernels run beside another's
    # row traffic); each stream waits for the step start and the step ends when all are done
    concurrent = None
    if len(calls) > 1:
        cstreams = {n: torch.cuda.Stream() for n in calls}
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def cstep():
            ev = torch.cuda.Event()
            ev.record(stream)
            for n, call in calls.items():
                cstreams[n].wait_event(ev)
                call.run(cstreams[n])
            for n in calls:
                stream.wait_stream(cstreams[n])
        for _ in range(W):
            cstep()
        torch.cuda.synchronize()
        c0.record(stream)
        for _ in range(K):
            cstep()
        c1.record(stream)
        torch.cuda.synchronize()
        cms = c0.elapsed_time(c1) / K
        concurrent = {"ms_per_step": round(cms, 4), "GBps": round(step_bytes / (cms * 1e-3) / 1e9, 1),
                      "note": "the four calls of a step on four streams (context; value is the one-stream step)"}

    # per workload: flushed-cache times (10 warm-ups first), the warm back-to-back time,
    # and a plain copy of the same byte count for context
    detail = {}
    if args.detail_iters > 0:
        for n, call in calls.items():
            for _ in range(10):
                call.run(stream)
            ts = flushed_times(call.run, stream, args.detail_iters)
            med = float(np.median(ts))
            warm = warm_ms(call.run, stream, 20)
            detail[n] = {"us_median": round(med * 1e3, 2), "us_p10": round(float(np.percentile(ts, 10)) * 1e3, 2),
                         "us_p90": round(float(np.percentile(ts, 90)) * 1e3, 2), "iters": args.detail_iters,
                         "alg_bytes": alg[n], "GBps": round(alg[n] / med / 1e6, 1),
                         "pct_hbm_peak": round(100 * alg[n] / med / 1e6 / HBM_PEAK_GBS, 1),
                         "rows_per_s": round(rows[n] / med * 1e3, 1),
                         "us_warm": round(warm * 1e3, 2), "GBps_warm": round(alg[n] / warm / 1e6, 1),
                         "copy_same_bytes_GBps": copy_gbps(alg[n], stream, 20),
                         "achievable_copy_GBps": probe_copy_gbps(alg[n], ROW_BYTES[n], stream, 20),
                         "achievable_copy_shuffled_rows_GBps": probe_copy_gbps(alg[n], ROW_BYTES[n], stream, 20,
                                                                               shuffled=True)}

    # parity of the timed outputs and the CPU oracle baseline, on the host
    parity = None
    cpu = None
    if not args.no_cpu_baseline and cases:
        from _gpu import oracle_batching, oracle_unpermute
        t_or = {}
        refs = {}
        for n, c in cases.items():
            runs = []
            for _ in range(3):
                t1 = time.perf_counter()
                refs[n] = oracle_batching(c) if n.startswith("batching") else oracle_unpermute(c)
                runs.append(time.perf_counter() - t1)
            t_or[n] = float(np.median(runs))
        secs = sum(t_or.values())
        cpu = {"value": round(step_bytes / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": "one full step (all four workloads) through the NumPy oracle, single-threaded, median "
                         f"of 3 runs per workload; {secs:.1f} s on {os.cpu_count()} visible host cores",
               "per_workload": {n: {"s": round(v, 3), "GBps": round(alg[n] / v / 1e9, 4),
                                    "rows_per_s": round(rows[n] / v, 1)} for n, v in t_or.items()}}
        parity = True
        for n, c in cases.items():
            try:
                if n.startswith("batching"):
                    check_batching(c, fetch_batching(calls[n]), refs[n])
                else:
                    check_unpermute(c, fetch_unpermute(calls[n], c), refs[n])
            except AssertionError as ex:
                parity = False
                print(f"# parity FAILED for {n}: {ex}", file=sys.stderr, flush=True)

    # workload 1 (tiny, latency-bound): call time in microseconds, flushed and warm
    latency = None
    if args.detail_iters > 0 and not args.only:
        c1 = synth.batching_config(1)
        call1 = prepare_batching(c1)
        for _ in range(10):
            call1.run(stream)
        torch.cuda.synchronize()
        act1 = int(call1.out["actual_token_num"].item())
        ts = flushed_times(call1.run, stream, args.detail_iters)
        warm = warm_ms(call1.run, stream, 100)
        # device time per call without host submission: 100 calls captured in one graph
        gstream = torch.cuda.Stream()
        gstream.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gstream):
            with torch.cuda.graph(g, stream=gstream):
                for _ in range(100):
                    call1.run(gstream)
        stream.wait_stream(gstream)
        g.replay()
        torch.cuda.synchronize()
        gb, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gb.record(stream)
        for _ in range(5):
            g.replay()
        ge.record(stream)
        torch.cuda.synchronize()
        graph_us = gb.elapsed_time(ge) / 500 * 1e3
        latency = {"batching_tiny": {
            "shape": "A=2 BS=8 K+1=3 (Y=48) H=128 fp16, 16 experts, 5 slots masked",
            "us_median": round(float(np.median(ts)) * 1e3, 2), "us_p10": round(float(np.percentile(ts, 10)) * 1e3, 2),
            "us_p90": round(float(np.percentile(ts, 90)) * 1e3, 2), "iters": args.detail_iters,
            "us_warm": round(warm * 1e3, 2), "us_per_call_in_graph": round(graph_us, 2), "rows": act1,
            "rows_per_s": round(act1 / float(np.median(ts)) * 1e3, 1)}}
        if not args.no_cpu_baseline:
            from _gpu import oracle_batching
            ref1 = oracle_batching(c1)
            try:
                check_batching(c1, fetch_batching(call1), ref1)
                latency["batching_tiny"]["parity"] = True
            except AssertionError as ex:
                latency["batching_tiny"]["parity"] = False
                print(f"# parity FAILED for the tiny batching: {ex}", file=sys.stderr, flush=True)
        # the non-padded call with its auxiliary sort on the caller's stream (no aux stream)
        if have_np:
            c4 = cases["unpermute_nonpadded"]
            call4 = prepare_unpermute(c4)
            for _ in range(10):
                call4.run(stream)
            ts4 = flushed_times(call4.run, stream, args.detail_iters)
            detail["unpermute_nonpadded"]["us_median_aux_on_caller_stream"] = round(float(np.median(ts4)) * 1e3, 2)
            del call4

    roof = None
    if have_np:
        red_bytes = nonpadded_reduce_bytes(cases["unpermute_nonpadded"])
        achieved = red_bytes / (hot_ms * 1e-3) / 1e9
        traffic = read_traffic(red_bytes)
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "unpermute_reduce_kernel (non-padded, BF16 rows, FP32 weights)",
                "alg_bytes_per_launch": red_bytes, "avg_launch_us": round(hot_ms * 1e3, 2)}

    next_rows = {}
    if args.no_next_rows:
        pass
    elif not args.only or "permute" in args.only.split(","):
        next_rows["moe_permute_nonpadded"] = measure_permute(args, stream)
        next_rows["moe_permute_padded"] = measure_permute(args, stream, padded=True)
    if not args.no_next_rows and (not args.only or "context" in args.only.split(",")):
        next_rows["batching_from_context"] = measure_ctx(args, stream)
    if not args.no_next_rows and (not args.only or "update_expert" in args.only.split(",")):
        next_rows["moe_update_expert"] = measure_update_expert(args, stream)
    if not args.no_next_rows and "unpermute_padded" in cases:
        next_rows["unpermute_padded_skip_zero_weight"] = measure_skip(args, stream, cases["unpermute_padded"])
    next_rows = next_rows or None

    value = step_bytes / (ms * 1e-3) / 1e9 if step_bytes else 0.0
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 4), "ms_per_step_without_timing_hooks": round(ms_nohook, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "moe_reorder_suite: " + "+".join(names),
                   "step_alg_bytes": step_bytes, "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
                   "element_types": "bf16/int8 rows moved; fp32 accumulation in unpermute"},
        "roofline": roof, "cpu_baseline": cpu, "configs": detail, "latency": latency,
        "step_on_four_streams": concurrent, "parity": parity,
        "next_rows": next_rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
