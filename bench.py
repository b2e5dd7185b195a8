#!/usr/bin/env python3
"""Throughput of the paged-KV hot path on one MI355X.

A step is one call of the path on one batch of synthetic input that is
already resident in HBM. The headline line is batch prefill over a paged
cache (bf16, batch 16, ragged q lengths U[256, 2048] on cached prefixes
U[0, 2048], 32 qo / 8 kv heads, head dim 128, HND pages of 16 tokens in a
65536-page pool, bottom-right causal, fp32 LSE), reported as TFLOP/s of the
unmasked (query, key) pairs. The same JSON line also carries decode (KV-read
GB/s: batch 256, seq U[512, 8192], bf16) and append-then-speculative-decode
(fp8 KV, window 4095, sinks, 4 drafts) and bulk append (262144 fp8 rows)
measurements, each against the MI355X roofline, and the float64 oracle timed
on the host for comparison.

Rates come from warm back-to-back calls; each leg also reports the median of
calls made after a 1 GiB read has evicted the caches ("flushed"). The
speculative step and the append page's Example (append then causal fp16
prefill, launch-bound) are also timed as captured HIP graphs, of one step
and of 8 steps back to back (per-step figures). The measured
ceilings (a pure MFMA loop, a streaming read, copies) put the rates beside
what this GPU reaches at all. The float64 oracle is timed on a bounded
sample of every workload (cpu_baseline; its "configs" holds each one). An
append scaling sweep (2^12 to 2^20 rows of the append Example's shape) closes
the line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-sweep]
       python bench.py --only {prefill,fp8prefill,decode,spec,append,copy,ceilings,append_sweep,
                               example}
"""

import argparse
import collections
import ctypes
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

METRIC = "prefill TFLOP/s and decode KV-read GB/s, paged KV, as fraction of MI355X peak"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "attention_paged_kv_cache_amd", "csrc")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--settle-ms", type=float, default=250.0,
                   help="untimed back-to-back calls of each workload for at least this long "
                        "before its warm-up steps (0: none; profiling runs pass 0)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the append scaling sweep")
    p.add_argument("--no-flush", action="store_true",
                   help="skip the cold-cache timings and the measured ceilings (kernel traces)")
    p.add_argument("--only", choices=["prefill", "decode", "spec", "fp8prefill", "append", "copy",
                                      "ceilings", "append_sweep", "example"],
                   default=None, help="time one workload (profiling runs); 'copy' times a "
                                      "plain 1 GiB device copy used to calibrate HBM counters; "
                                      "'append_sweep' times the append at 2^12..2^20 rows of "
                                      "the append example's shape")
    return p.parse_args()


# ---- algorithmic work (what the method must do) ------------------------------

def prefill_flops(lq, lkv, h_qo, d_qk, d_vo):
    """2 (d_qk + d_vo) H_qo per allowed (query, key) pair, bottom-right causal."""
    pairs = 0
    for q, k in zip(lq, lkv):
        q, k = int(q), int(k)
        if k >= q:
            pairs += q * (k - q) + q * (q + 1) // 2
        else:  # rows t < q - k see nothing
            n = k
            pairs += n * (n + 1) // 2
    return 2 * (d_qk + d_vo) * h_qo * pairs


def decode_bytes(seq, q_len, window, h_qo, h_kv, d, kv_elem, q_elem, out_elem, page_size):
    """K/V bytes of every key some query may see, plus Q, O and page ids."""
    keys = 0
    pages = 0
    for s in seq:
        s = int(s)
        n = min(s, window + q_len) if window >= 0 else s
        keys += n
        pages += (n + page_size - 1) // page_size
    kv = keys * h_kv * 2 * d * kv_elem
    qo = len(seq) * q_len * h_qo * d * (q_elem + out_elem)
    return kv + qo + pages * 4 + len(seq) * 4


def append_bytes(nnz, h_kv, d, elem):
    return 4 * nnz * h_kv * d * elem + 8 * nnz


# ---- timing -------------------------------------------------------------------

Timing = collections.namedtuple("Timing", "region_ms launch_ms min_ms median_ms")


def _stats(per, region_ms):
    per = sorted(per)
    return Timing(region_ms, sum(per) / len(per), per[0], statistics.median(per))


# Untimed back-to-back calls before each workload's warm-up steps, in ms (set
# from --settle-ms). The host builds each workload for seconds while the GPU
# idles; after such a gap the GPU's clocks go through a transient of 20 to
# 40 ms (measured: speculative decode ran one fast 20-call window, then
# 5.0 TB/s, recovering to its steady 5.8 over about 160 calls; the first
# prefill round read 851 to 857 TFLOP/s against about 935 after), longer
# than 10 warm-up calls of the short workloads. Settling first makes every
# leg a steady-state measurement.
SETTLE_MS = 250.0

# Steps captured in one HIP graph for the multi-step graph timings of the
# launch-bound steps.
GRAPH_STEPS = 8


def settle(fn):
    """Call `fn` back to back, untimed, for at least SETTLE_MS of wall time."""
    import torch
    if SETTLE_MS <= 0:
        return
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < SETTLE_MS:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def time_steps(fn, steps, warmup):
    """Warm caches: settle (see SETTLE_MS), `warmup` untimed calls, then two
    timed passes of `steps` calls back to back.
    region_ms: the first pass, with events only at its two ends, per step.
    launch/min/median_ms: the second pass, from events around each call.
    Each event pair on the GPU's timeline adds about 5 us to the call it
    brackets (the kernel trace's durations are that much shorter), so the
    rates come from region_ms and the per-call figures give the spread.
    Events sit on the current stream, which is the stream the library
    enqueues on."""
    import torch
    settle(fn)
    for _ in range(warmup):
        fn()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    region = start.elapsed_time(end) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return _stats([a.elapsed_time(b) for a, b in ev], region)


def new_flush_buffer(torch):
    """1 GiB of float32 that time_flushed reads to evict the caches."""
    return torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")


def time_flushed(fn, steps, flush):
    """Cold caches: before each timed call, read the whole of `flush` (1 GiB),
    which evicts the L2s and the 256 MB last-level cache. A read, not a
    write: a written buffer would leave up to 256 MB of dirty lines whose
    write-back then runs during the timed call (that costs a 0.17 ms decode
    a third of its rate). The read also drains any dirty lines left by
    earlier calls before the timed one starts. Only the call itself sits
    between its events. None when `flush` is None."""
    import torch
    if flush is None:
        return None
    sink = torch.empty(1, dtype=flush.dtype, device=flush.device)
    fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        torch.sum(flush, dim=(0,), keepdim=True, out=sink)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return _stats([a.elapsed_time(b) for a, b in ev], None)


# Sources each kernel is compiled from: a counter summary taken on other
# sources is not reported (an edit elsewhere leaves it valid).
PREFILL_SRC = ("prefill.hip", "pkv_common.h", "launch_prefill.h")
DECODE_SRC = ("decode.hip", "pkv_common.h", "launch_decode.h")
APPEND_SRC = ("append.hip", "pkv_common.h", "launch_append.h")


def kernel_hash(*files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic(name, src_files, per_launch_units=1):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{name}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_sha") != kernel_hash(*src_files):
        return None
    return c.get("hbm_bytes_per_launch")


def roofline(bound, achieved, peak, unit, traffic_bytes):
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic_bytes}


# ---- workloads -----------------------------------------------------------------

def bench_prefill(pkv, torch, workloads, fp8=False):
    """(workload, algorithmic FLOP, step)."""
    dev = "cuda:0"
    w = workloads.fp8_prefill(dev) if fp8 else workloads.batch_prefill(dev)
    lq, lkv = w["seq_lens_q"], w["seq_lens_kv"]
    ws = torch.zeros(pkv.prefill_workspace_size(lq.shape[0]), dtype=torch.uint8, device=dev)
    lq_d, lkv_d, bt_d = lq.to(dev), lkv.to(dev), w["block_tables"].to(dev)
    out = torch.empty(w["q"].shape[0], w["num_qo_heads"], w["d_vo"],
                      dtype=torch.bfloat16, device=dev)
    lse = torch.empty(w["q"].shape[0], w["num_qo_heads"], dtype=torch.float32, device=dev)
    sc = {k: (None if w[k] is None else w[k].to(dev)) for k in ("q_scale", "k_scale", "v_scale")}
    mq, mk = int(lq.max()), int(lkv.max())

    def step():
        pkv.batch_prefill_with_kv_cache(
            w["q"], w["k_cache"], w["v_cache"], w["scale"], ws, max_token_per_sequence=mq,
            max_sequence_kv=mk, actual_seq_lens_q=lq_d, actual_seq_lens_kv=lkv_d,
            block_tables=bt_d, causal=True, out=out, lse=lse, kv_layout=w["layout"], **sc)

    flops = prefill_flops(lq.tolist(), lkv.tolist(), w["num_qo_heads"], w["d_qk"], w["d_vo"])
    return w, flops, step


def bench_decode(pkv, torch, workloads):
    """(workload, algorithmic bytes, step)."""
    dev = "cuda:0"
    w = workloads.batch_decode(dev)
    ws = torch.zeros(max(pkv.decode_workspace_size(
        256, 1, 32, 8, 128, w["max_seq_len"], -1), 16), dtype=torch.uint8, device=dev)
    bt, seq = w["block_tables"].to(dev), w["seq_lens"].to(dev)
    out = torch.empty_like(w["query"])

    def step():
        pkv.batch_decode_with_kv_cache(w["query"], w["kv_cache"], ws, bt, seq, w["max_seq_len"],
                                       bmm1_scale=w["bmm1_scale"], bmm2_scale=1.0, out=out,
                                       kv_layout="HND")

    nbytes = decode_bytes(w["seq_lens"].tolist(), 1, -1, 32, 8, 128, 2, 2, 2, 16)
    return w, nbytes, step


def bench_spec(pkv, torch, workloads):
    """Append 4 drafts per request, then decode them (one step = both).
    (workload, decode bytes, append bytes, append, decode)."""
    dev = "cuda:0"
    w = workloads.spec_decode(dev)
    B, ql = 64, 4
    ws = torch.zeros(max(pkv.decode_workspace_size(
        B, ql, 64, 8, 128, w["max_seq_len"], w["window_left"]), 16), dtype=torch.uint8, device=dev)
    bt, seq = w["block_tables"].to(dev), w["seq_lens"].to(dev)
    seq32 = w["seq_lens"].to(torch.int32).to(dev)
    ai = w["append_indptr"].to(dev)
    idx, indptr, last = (w["kv_indices"].to(dev), w["kv_indptr"].to(dev),
                         w["kv_last_page_len"].to(dev))
    sinks = w["sinks"].to(dev)
    out = torch.empty_like(w["query"])
    nnz = w["k_append"].shape[0]
    bi, pos = pkv.get_batch_indices_positions(ai, seq32, nnz)

    def append():
        pkv.append_paged_kv_cache(w["k_append"], w["v_append"], bi, pos, w["kv_cache"], idx,
                                  indptr, last, kv_layout="HND")

    def decode():
        pkv.batch_decode_with_kv_cache(w["query"], w["kv_cache"], ws, bt, seq, w["max_seq_len"],
                                       bmm1_scale=w["bmm1_scale"], bmm2_scale=w["bmm2_scale"],
                                       window_left=w["window_left"], out=out, sinks=sinks,
                                       kv_layout="HND", q_len_per_req=ql)

    nbytes = decode_bytes(w["seq_lens"].tolist(), ql, w["window_left"], 64, 8, 128, 1, 2, 2, 32)
    abytes = append_bytes(nnz, 8, 128, 1)
    return w, nbytes, abytes, append, decode


def bench_append(pkv, torch, w):
    """(algorithmic bytes, step) for an append workload dict."""
    dev = "cuda:0"
    nnz = w["k_append"].shape[0]
    seq = w["seq_lens"].to(dev)
    bi, pos = pkv.get_batch_indices_positions(w["append_indptr"].to(dev), seq, nnz)
    idx, indptr, last = (w["kv_indices"].to(dev), w["kv_indptr"].to(dev),
                         w["kv_last_page_len"].to(dev))

    def step():
        pkv.append_paged_kv_cache(w["k_append"], w["v_append"], bi, pos, w["kv_cache"], idx,
                                  indptr, last, kv_layout=w["layout"])

    elem = w["k_append"].element_size()
    return append_bytes(nnz, w["num_kv_heads"], w["head_dim"], elem), step


# nnz of the append scaling sweep: the append Example's shape family (fp16, 32
# kv heads, d 128, NHD page 16) from 2^12 to 2^20 rows, an extra measurement
# (not one of the workloads) that shows whether the scatter itself is bound
# by HBM bandwidth, which the workloads' small appends cannot show.
SWEEP_NNZ = [1 << k for k in range(12, 21)]


def bench_append_sweep(pkv, torch, workloads, steps, warmup, flush, nnzs=SWEEP_NNZ):
    """Warm (region) and flushed (per-call median) rates of the append at each
    nnz of `nnzs`; one dict per size."""
    G = 1e9
    points = []
    for nnz in nnzs:
        w = workloads.append_sweep("cuda:0", nnz=nnz)
        nb, step = bench_append(pkv, torch, w)
        t = time_steps(step, steps, warmup)
        f = time_flushed(step, steps, flush)
        pt = {"nnz": nnz, "bytes": nb, "GB/s": round(rate(nb, t.region_ms, G), 1),
              "ms_per_step": round(t.region_ms, 4)}
        if f is not None:
            pt["flushed_GB/s"] = round(rate(nb, f.median_ms, G), 1)
            pt["flushed_ms_median"] = round(f.median_ms, 4)
        points.append(pt)
        del w, step
        torch.cuda.empty_cache()
    return points


def bench_example(pkv, torch, workloads):
    """The append page's Example (fp16, NHD 5D cache, 4 requests of 45/8/25/22
    tokens, 100 rows), then a causal prefill of the appended tokens. One step
    is the whole chain: get_seq_lens, get_batch_indices_positions, append,
    csr_to_block_tables, prefill. Returns (workload, prefill FLOP, append
    bytes, step, append part, prefill part)."""
    dev = "cuda:0"
    w = workloads.append_example(dev)
    cache = w["paged_kv_cache"]
    indptr, last, idx, ai = (w[k].to(dev) for k in ("kv_indptr", "kv_last_page_len",
                                                     "kv_indices", "append_indptr"))
    lens = w["append_lengths"].to(dev)
    ws = torch.zeros(pkv.prefill_workspace_size(4), dtype=torch.uint8, device=dev)
    out = torch.empty(100, 32, 128, dtype=torch.float16, device=dev)
    lse = torch.empty(100, 32, dtype=torch.float32, device=dev)

    def append():
        seq = pkv.get_seq_lens(indptr, last, 16)
        bi, pos = pkv.get_batch_indices_positions(ai, seq, 100)
        pkv.append_paged_kv_cache(w["k_append"], w["v_append"], bi, pos, cache, idx, indptr,
                                  last, kv_layout="NHD")

    def prefill():
        bt = pkv.csr_to_block_tables(indptr, idx, 3)
        pkv.batch_prefill_with_kv_cache(
            w["q"], cache[:, 0], cache[:, 1], w["scale"], ws, max_token_per_sequence=45,
            max_sequence_kv=45, actual_seq_lens_q=lens, actual_seq_lens_kv=lens,
            block_tables=bt, causal=True, out=out, lse=lse, kv_layout="NHD")

    def step():
        append()
        prefill()

    L = w["append_lengths"].tolist()
    flops = prefill_flops(L, L, 32, 128, 128)
    # rows read and written, their indices, and the index arrays the chain reads
    abytes = append_bytes(100, 32, 128, 2) + 4 * (5 + 4 + 8 + 5)
    return w, flops, abytes, step, append, prefill


def time_graph(torch, fn, steps, warmup, per_graph=1):
    """The same timing as time_steps for `per_graph` calls of `fn` captured
    once in a HIP graph and replayed: what the step costs on the GPU without
    the host's per-call argument handling and launch gaps. With per_graph > 1
    one replay runs that many steps back to back (a serving loop's steps in
    one graph), and every figure is divided by per_graph: the per-replay
    launch cost is then shared by those steps."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    torch.cuda.synchronize()
    t = time_steps(g.replay, steps, warmup)
    del g
    return Timing(*(x / per_graph for x in t))


# ---- measured ceilings -------------------------------------------------------------

def measured_ceilings(torch, steps=10):
    """Rates of a pure bf16 MFMA loop, a streaming 4 GiB read, a 1 GiB
    device copy and a hand-written 512 MiB copy on this GPU
    (libpkv_ceiling.so), each over `steps` back-to-back calls after warm-up,
    timed as the workloads are (region_ms)."""
    path = os.path.join(ROOT, "attention_paged_kv_cache_amd", "libpkv_ceiling.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build first "
                           "(python -m attention_paged_kv_cache_amd.build)")
    lib = ctypes.CDLL(path)
    lib.pkv_ceiling_mfma_bf16.restype = ctypes.c_int
    lib.pkv_ceiling_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p]
    lib.pkv_ceiling_mfma_bf16_flop.restype = ctypes.c_double
    lib.pkv_ceiling_mfma_bf16_flop.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.pkv_ceiling_read.restype = ctypes.c_int
    lib.pkv_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_void_p]
    dev = "cuda:0"
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} launch failed with hipError {rc}")

    blocks, iters = 2048, 2000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    t = time_steps(lambda: ok(lib.pkv_ceiling_mfma_bf16(blocks, iters, out.data_ptr(), stream),
                              "mfma loop"), steps, 3)
    mfma = lib.pkv_ceiling_mfma_bf16_flop(blocks, iters) / (t.region_ms * 1e-3) / 1e12
    del out

    nbytes, rblocks = 4 << 30, 2048
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    words = torch.empty(rblocks * 256, dtype=torch.int32, device=dev)
    t = time_steps(lambda: ok(lib.pkv_ceiling_read(buf.data_ptr(), nbytes, rblocks,
                                                   words.data_ptr(), stream), "read stream"),
                   steps, 3)
    read = nbytes / (t.region_ms * 1e-3) / 1e9
    del buf, words

    x = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    t = time_steps(lambda: y.copy_(x), steps, 3)
    copy = 2 * x.numel() * 4 / (t.region_ms * 1e-3) / 1e9
    del x, y

    # hand-written streaming copy of 512 MiB (the bulk append's read and
    # write sizes): plain and non-temporal loads and stores, 4 or 8 loads in
    # flight per thread, 2048 or 8192 workgroups; the fastest is the ceiling
    lib.pkv_ceiling_copy.restype = ctypes.c_int
    lib.pkv_ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p]
    cbytes = 512 << 20
    src = torch.empty(cbytes, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty_like(src)
    kcopy = {}
    for nt in (0, 1):
        for unroll in (4, 8):
            for cblocks in (2048, 8192):
                t = time_steps(lambda: ok(lib.pkv_ceiling_copy(src.data_ptr(), dst.data_ptr(),
                                                               cbytes, cblocks, nt, unroll,
                                                               stream), "copy stream"),
                               steps, 3)
                kcopy[(nt, unroll, cblocks)] = 2 * cbytes / (t.region_ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    best = max(kcopy, key=kcopy.get)
    return {"mfma_bf16_loop_TFLOPs": round(mfma, 1), "hbm_read_4GiB_GBs": round(read, 1),
            "hbm_copy_1GiB_GBs": round(copy, 1),
            "hbm_copy_kernel_512MiB_GBs": round(kcopy[best], 1),
            "hbm_copy_kernel_best": {"nontemporal": bool(best[0]), "loads_per_thread": best[1],
                                     "workgroups": best[2]},
            "hbm_copy_kernel_plain_GBs": round(max(v for k, v in kcopy.items() if not k[0]), 1),
            "hbm_copy_kernel_nontemporal_GBs": round(max(v for k, v in kcopy.items() if k[0]), 1),
            "what": "pure v_mfma_f32_32x32x16_bf16 loop (8 chains per wave, 8192 waves); "
                    "non-temporal 16-byte loads over 4 GiB (2048 workgroups, one contiguous "
                    "span each); torch copy_ of 1 GiB (read + write counted); a hand-written "
                    "copy of 512 MiB (one contiguous span per workgroup, 4 or 8 loads of 16 "
                    "bytes in flight per thread before their stores, 2048 or 8192 workgroups, "
                    "plain or non-temporal: the fastest of the eight reported, its shape in "
                    "hbm_copy_kernel_best; read + write counted); each over 10 "
                    "back-to-back calls"}


def _cpu_cores(torch):
    cores = torch.get_num_threads()
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 0) for i in info] + [cores])
    except Exception:
        pass
    return cores


def _baseline(torch, value, unit, sample):
    return {"value": value, "unit": unit, "cores": _cpu_cores(torch), "kind": "oracle",
            "sample": f"{sample}; float64 numpy on {cpu_model()} "
                      f"({os.cpu_count()} logical CPUs visible)"}


def cpu_baseline(w, budget_s=6.0):
    """The float64 oracle on a bounded sample of the batch-prefill workload:
    whole requests, in order, until about budget_s seconds of CPU work."""
    import numpy as np
    import torch
    import oracle
    from tests.helpers import bits, fmt
    from workloads import compact_pages
    lq, lkv = w["seq_lens_q"], w["seq_lens_kv"]
    ps = w["page_size"]
    q_all = bits(w["q"])
    cq = np.concatenate([[0], np.cumsum(lq.numpy())])
    flops = 0
    n_req = 0
    spent = 0.0
    for b in range(lq.shape[0]):
        n = (int(lkv[b]) + ps - 1) // ps
        bt = w["block_tables"][b:b + 1]
        kc, bt1 = compact_pages(w["k_cache"], bt, [n])
        vc, _ = compact_pages(w["v_cache"], bt, [n])
        kb, vb = bits(kc), bits(vc)
        q = q_all[cq[b]:cq[b + 1]]
        t0 = time.perf_counter()
        oracle.batch_prefill(q, fmt(w["q"]), kb, vb, fmt(w["k_cache"]), bt1.numpy(),
                             lq[b:b + 1].numpy(), lkv[b:b + 1].numpy(), w["scale"], True,
                             w["layout"])
        spent += time.perf_counter() - t0
        flops += prefill_flops([int(lq[b])], [int(lkv[b])], w["num_qo_heads"], w["d_qk"],
                               w["d_vo"])
        n_req += 1
        if spent > budget_s:
            break
    return _baseline(torch, round(flops / spent / 1e12, 6), "TFLOP/s",
                     f"first {n_req} of {lq.shape[0]} requests of the batch-prefill workload "
                     f"({flops / 1e9:.1f} GFLOP algorithmic) in {spent:.1f} s")


def cpu_example(w, reps=3):
    """The oracle on the whole append Example plus its causal prefill (the
    same chain as the GPU step: seq lens, row coordinates, append, block
    tables, prefill), the fastest of `reps` runs. Only the 8 pages the
    Example uses are handed over (the append touches nothing else)."""
    import numpy as np
    import torch
    import oracle
    from tests.helpers import bits, fmt
    cache = bits(w["paged_kv_cache"][:8])
    kb, vb, qb = bits(w["k_append"]), bits(w["v_append"]), bits(w["q"])
    indptr, last = w["kv_indptr"].numpy(), w["kv_last_page_len"].numpy()
    idx, ai = w["kv_indices"].numpy(), w["append_indptr"].numpy()
    L = w["append_lengths"].numpy()
    f = fmt(w["q"])
    best = float("inf")
    for _ in range(reps):
        t0 = time.perf_counter()
        seq = oracle.get_seq_lens(indptr, last, 16)
        bi, pos = oracle.get_batch_indices_positions(ai, seq, 100)
        kc, vc = cache[:, 0].copy(), cache[:, 1].copy()
        oracle.append_paged_kv_cache(kb, vb, bi, pos, kc, vc, idx, indptr, last, "NHD")
        bt = oracle.csr_to_block_tables(indptr, idx, 3)
        oracle.batch_prefill(qb, f, kc, vc, f, bt, L, L, w["scale"], True, "NHD")
        best = min(best, time.perf_counter() - t0)
    flops = prefill_flops(L.tolist(), L.tolist(), 32, 128, 128)
    return _baseline(torch, round(best * 1e6, 1), "us per step",
                     f"the whole append Example (100 rows) and its causal prefill "
                     f"({flops / 1e6:.1f} MFLOP, {flops / best / 1e9:.3f} GFLOP/s), fastest of "
                     f"{reps} runs")


def cpu_fp8_prefill(w, n_req=4, rows_per_req=64, seed=0):
    """The oracle on sampled query rows of the fp8 prefill workload (all
    heads of each row; the request's pages are gathered and decoded as part
    of the timed call)."""
    import numpy as np
    import torch
    import oracle
    from tests.helpers import bits, fmt
    from workloads import compact_pages
    rng = np.random.default_rng(seed)
    lq = w["seq_lens_q"].numpy()
    rows = [(b, int(t)) for b in range(n_req) for t in rng.integers(0, lq[b], rows_per_req)]
    ps = w["page_size"]
    used = [(int(w["seq_lens_kv"][b]) + ps - 1) // ps if b < n_req else 0
            for b in range(len(lq))]
    kc, bt = compact_pages(w["k_cache"], w["block_tables"], used)
    vc, _ = compact_pages(w["v_cache"], w["block_tables"], used)
    kb, vb, qb = bits(kc), bits(vc), bits(w["q"])
    sc = lambda x: float(x.reshape(-1)[0])
    t0 = time.perf_counter()
    oracle.batch_prefill(qb, fmt(w["q"]), kb, vb, fmt(w["k_cache"]), bt.numpy(), lq,
                         w["seq_lens_kv"].numpy(), w["scale"], True, w["layout"],
                         q_scale=sc(w["q_scale"]), k_scale=sc(w["k_scale"]),
                         v_scale=sc(w["v_scale"]), rows=rows)
    dt = time.perf_counter() - t0
    shift = int(w["seq_lens_kv"][0]) - int(lq[0])
    pairs = sum(t + 1 + shift for _, t in rows)
    flops = 2 * (w["d_qk"] + w["d_vo"]) * w["num_qo_heads"] * pairs
    return _baseline(torch, round(flops / dt / 1e12, 6), "TFLOP/s",
                     f"{len(rows)} random query rows (all {w['num_qo_heads']} heads) of the first {n_req} "
                     f"requests of the fp8 prefill workload ({flops / 1e9:.2f} GFLOP "
                     f"algorithmic) in {dt:.1f} s")


def cpu_decode(w, reqs, append=False):
    """The oracle on a sample of whole requests of a decode workload (with
    `append`: the speculative step, the 4 draft rows of each sampled request
    appended by the oracle first). Returns (time, decode bytes of the
    sample)."""
    import numpy as np
    import torch
    import oracle
    from tests.helpers import bits, fmt
    from workloads import compact_pages
    ps = w["page_size"]
    seq = w["seq_lens"].to(torch.int64)
    used = [0] * seq.shape[0]
    for b in reqs:
        used[b] = (int(seq[b]) + ps - 1) // ps
    sub, bt = compact_pages(w["kv_cache"], w["block_tables"], used)
    kb, vb = bits(sub[:, 0]), bits(sub[:, 1])
    qb = bits(w["query"])
    sinks = None if w["sinks"] is None else w["sinks"].double().numpy()
    ql = w["q_len_per_req"]
    if append:
        ka, va = bits(w["k_append"]), bits(w["v_append"])
        # the sampled requests' CSR page lists, renumbered into the compacted pool
        n_pages = [used[b] for b in reqs]
        indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
        idx = np.concatenate([bt[b, :used[b]].numpy() for b in reqs]).astype(np.int32)
        last = np.array([(int(seq[b]) - 1) % ps + 1 for b in reqs], dtype=np.int32)
        ai = np.arange(len(reqs) + 1, dtype=np.int32) * ql
        rows = np.concatenate([np.arange(b * ql, (b + 1) * ql) for b in reqs])
        ka_s, va_s = ka[rows], va[rows]
    t0 = time.perf_counter()
    if append:
        s_seq = oracle.get_seq_lens(indptr, last, ps)
        bi, pos = oracle.get_batch_indices_positions(ai, s_seq, len(rows))
        oracle.append_paged_kv_cache(ka_s, va_s, bi, pos, kb, vb, idx, indptr, last, w["layout"])
    oracle.batch_decode(qb, fmt(w["query"]), kb, vb, fmt(w["kv_cache"]), bt.numpy(),
                        seq.numpy(), w["bmm1_scale"], w["bmm2_scale"], w["window_left"], sinks,
                        w["layout"], ql, requests=reqs)
    dt = time.perf_counter() - t0
    elem = w["kv_cache"].element_size()
    nbytes = decode_bytes([int(seq[b]) for b in reqs], ql, w["window_left"],
                          w["num_qo_heads"], w["num_kv_heads"], w["head_dim"], elem, 2, 2, ps)
    return dt, nbytes


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown CPU"


def rate(work, ms, scale):
    return work / (ms * 1e-3) / scale


def mixed_fp8_peak(d_qk, d_vo):
    """Dense peak of a prefill whose QK^T runs on fp8 MFMA and whose PV runs
    on bf16 MFMA (P is rounded to bf16): each part at its own peak, in
    proportion to its share of the FLOP."""
    share_qk = d_qk / (d_qk + d_vo)
    return 1.0 / (share_qk / PEAK_FP8_TFLOPS + (1.0 - share_qk) / PEAK_BF16_TFLOPS)


def main():
    global SETTLE_MS
    args = parse()
    SETTLE_MS = args.settle_ms
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import attention_paged_kv_cache_amd as pkv
    import workloads

    if args.only:
        only(args, torch, pkv, workloads)
        return

    flush = None if args.no_flush else new_flush_buffer(torch)
    T, G = 1e12, 1e9
    cpu = not args.no_cpu_baseline
    base = {}

    print("bench: prefill (bf16, batch 16)", file=sys.stderr, flush=True)
    w, flops, step = bench_prefill(pkv, torch, workloads)
    t1 = time_steps(step, args.steps, args.warmup)
    f1 = time_flushed(step, args.steps, flush)
    tokens, kv_tokens = int(w["seq_lens_q"].sum()), int(w["seq_lens_kv"].sum())
    if cpu:
        print("bench: float64 oracle, batch prefill sample", file=sys.stderr, flush=True)
        base["batch_prefill"] = cpu_baseline(w)
    del w, step
    torch.cuda.empty_cache()

    print("bench: fp8 prefill (d_qk 192)", file=sys.stderr, flush=True)
    w, flops3, step = bench_prefill(pkv, torch, workloads, fp8=True)
    t3 = time_steps(step, args.steps, args.warmup)
    f3 = time_flushed(step, args.steps, flush)
    if cpu:
        print("bench: float64 oracle, fp8 prefill sample", file=sys.stderr, flush=True)
        base["fp8_prefill"] = cpu_fp8_prefill(w)
    del w, step
    torch.cuda.empty_cache()

    print("bench: decode (bf16, batch 256)", file=sys.stderr, flush=True)
    w, bytes4, step = bench_decode(pkv, torch, workloads)
    t4 = time_steps(step, args.steps, args.warmup)
    f4 = time_flushed(step, args.steps, flush)
    if cpu:
        print("bench: float64 oracle, decode sample", file=sys.stderr, flush=True)
        reqs = list(range(96))
        dt, nb = cpu_decode(w, reqs)
        base["decode"] = _baseline(torch, round(nb / dt / 1e9, 4), "GB/s",
                                   f"the first {len(reqs)} of 256 requests of the decode "
                                   f"workload ({nb / 1e6:.1f} MB algorithmic) in {dt:.1f} s")
    del w, step
    torch.cuda.empty_cache()

    print("bench: append + speculative decode (fp8 KV)", file=sys.stderr, flush=True)
    w, bytes5, abytes5, append5, decode5 = bench_spec(pkv, torch, workloads)

    def step5():
        append5()
        decode5()

    t5 = time_steps(step5, args.steps, args.warmup)
    t5d = time_steps(decode5, args.steps, args.warmup)
    t5a = time_steps(append5, args.steps, args.warmup)
    f5d = time_flushed(decode5, args.steps, flush)
    t5g = time_graph(torch, step5, args.steps, args.warmup)
    t5ag = time_graph(torch, append5, args.steps, args.warmup)
    t5g8 = time_graph(torch, step5, args.steps, args.warmup, GRAPH_STEPS)
    t5ag8 = time_graph(torch, append5, args.steps, args.warmup, GRAPH_STEPS)
    if cpu:
        print("bench: float64 oracle, speculative step sample", file=sys.stderr, flush=True)
        reqs = list(range(16))
        dt, nb = cpu_decode(w, reqs, append=True)
        base["spec_decode"] = _baseline(
            torch, round(nb / dt / 1e9, 4), "GB/s",
            f"requests 0-{len(reqs) - 1} of 64 of the speculative step, their "
            f"{4 * len(reqs)} draft rows appended and their {4 * len(reqs)} queries decoded "
            f"({nb / 1e6:.1f} MB of decode reads) in {dt:.1f} s")
    del w, append5, decode5
    torch.cuda.empty_cache()

    print("bench: bulk append (fp8 KV, 262144 rows)", file=sys.stderr, flush=True)
    w = workloads.bulk_append("cuda:0")
    bytes6, step = bench_append(pkv, torch, w)
    t6 = time_steps(step, args.steps, args.warmup)
    f6 = time_flushed(step, args.steps, flush)
    del w, step
    torch.cuda.empty_cache()

    print("bench: append example + causal prefill (fp16, NHD)", file=sys.stderr, flush=True)
    w, flops0, abytes0, step0, append0, prefill0 = bench_example(pkv, torch, workloads)
    t0s = time_steps(step0, args.steps, args.warmup)
    t0a = time_steps(append0, args.steps, args.warmup)
    t0p = time_steps(prefill0, args.steps, args.warmup)
    t0g = time_graph(torch, step0, args.steps, args.warmup)
    t0g8 = time_graph(torch, step0, args.steps, args.warmup, GRAPH_STEPS)
    if cpu:
        print("bench: float64 oracle, append example", file=sys.stderr, flush=True)
        base["append_example"] = cpu_example(w)
    del w, step0, append0, prefill0
    torch.cuda.empty_cache()

    sweep = None
    if not args.no_sweep:
        print("bench: append scaling sweep (fp16, NHD, 2^12 to 2^20 rows)", file=sys.stderr,
              flush=True)
        sweep = bench_append_sweep(pkv, torch, workloads, args.steps, args.warmup, flush)
    flush = None
    torch.cuda.empty_cache()

    ceil = None
    if not args.no_flush:
        print("bench: measured ceilings (MFMA loop, HBM read, copies)", file=sys.stderr,
              flush=True)
        ceil = measured_ceilings(torch)

    def timing(t, f, work, scale):
        d = {"ms_median": round(t.median_ms, 4), "ms_min": round(t.min_ms, 4)}
        if f is not None:
            d["flushed"] = {"ms_median": round(f.median_ms, 4),
                            "value": round(rate(work, f.median_ms, scale), 1)}
        return d

    p_l = rate(flops, t1.region_ms, T)
    p3_l = rate(flops3, t3.region_ms, T)
    d4_l = rate(bytes4, t4.region_ms, G)
    d5_l = rate(bytes5, t5d.region_ms, G)
    a6_l = rate(bytes6, t6.region_ms, G)
    mixed = mixed_fp8_peak(192, 128)
    line = {
        "metric": METRIC,
        "value": round(rate(flops, t1.region_ms, T), 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(t1.region_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "batch prefill over a paged KV cache: bf16, batch 16, q_len U[256,2048], "
                        "kv_len = q_len + U[0,2048], 32 qo / 8 kv heads, d_qk = d_vo = 128, HND, "
                        "page 16, 65536-page pool in random order, bottom-right causal, fp32 LSE",
            "seed": 2,
            "tokens": tokens,
            "kv_tokens": kv_tokens,
            "flop_per_step": flops,
        },
        "roofline": roofline("mfma", p_l, PEAK_BF16_TFLOPS, "TFLOP/s",
                             traffic("prefill_bf16", PREFILL_SRC)),
        "timing": timing(t1, f1, flops, T),
        "fp8_prefill": {
            "workload": "e4m3 prefill, d_qk 192 / d_vo 128, batch 8, q_len = kv_len = 4096, "
                        "16/16 heads, page 64, per-tensor scales, causal, bf16 out",
            "value": round(rate(flops3, t3.region_ms, T), 2), "unit": "TFLOP/s",
            "ms_per_step": round(t3.region_ms, 4),
            "roofline": roofline("mfma", p3_l, PEAK_FP8_TFLOPS, "TFLOP/s",
                                 traffic("prefill_e4m3_d192", PREFILL_SRC)),
            "frac_of_bf16_peak": round(p3_l / PEAK_BF16_TFLOPS, 4),
            "mixed_peak_TFLOPs": round(mixed, 1),
            "frac_of_mixed_peak": round(p3_l / mixed, 4),
            **timing(t3, f3, flops3, T),
        },
        "decode": {
            "workload": "decode over block_tables: bf16, batch 256, seq U[512,8192], 32/8 heads, "
                        "d 128, HND page 16, random pages, 1 query per request",
            "value": round(rate(bytes4, t4.region_ms, G), 1), "unit": "GB/s",
            "ms_per_step": round(t4.region_ms, 4), "bytes_per_step": bytes4,
            "roofline": roofline("hbm", d4_l, PEAK_HBM_GBS, "GB/s",
                                 traffic("decode_bf16", DECODE_SRC)),
            **timing(t4, f4, bytes4, G),
        },
        "spec_decode": {
            "workload": "append 4 drafts/request then decode: fp8 e4m3 KV, batch 64, "
                        "seq U[4096,32768], 64/8 heads, d 128, HND page 32, window_left 4095, "
                        "sinks, q_len_per_req 4",
            "ms_per_step": round(t5.region_ms, 4),
            "graph_ms_per_step": round(t5g.region_ms, 4),
            f"graph{GRAPH_STEPS}_ms_per_step": round(t5g8.region_ms, 4),
            "decode_value": round(d5_l, 1), "unit": "GB/s",
            "decode_bytes": bytes5,
            "roofline": roofline("hbm", d5_l, PEAK_HBM_GBS, "GB/s",
                                 traffic("spec_decode_e4m3", DECODE_SRC)),
            "decode": timing(t5d, f5d, bytes5, G),
            "append_ms": round(t5a.region_ms, 4),
            "append_graph_ms": round(t5ag.region_ms, 4),
            f"append_graph{GRAPH_STEPS}_ms": round(t5ag8.region_ms, 4),
            "append_GBs": round(rate(abytes5, t5a.region_ms, G), 1),
            "append_roofline": roofline("hbm", rate(abytes5, t5ag8.region_ms, G), PEAK_HBM_GBS,
                                        "GB/s", traffic("append_spec_e4m3", APPEND_SRC)),
        },
        "bulk_append": {
            "workload": "append 1024 rows into each of 256 requests: e4m3 KV, 8 kv heads, d 128, "
                        "HND page 32, seq U[4096,8192] after the append, pages in random order",
            "value": round(rate(bytes6, t6.region_ms, G), 1), "unit": "GB/s",
            "ms_per_step": round(t6.region_ms, 4), "bytes_per_step": bytes6,
            "roofline": roofline("hbm", a6_l, PEAK_HBM_GBS, "GB/s",
                                 traffic("append_bulk_e4m3", APPEND_SRC)),
            **timing(t6, f6, bytes6, G),
        },
        "append_example": {
            "workload": "the append page's Example (fp16, NHD 5D cache of 1000 pages x 16 "
                        "tokens x 32 heads x 128, 100 rows into 4 requests of 45/8/25/22 "
                        "tokens) then a causal fp16 prefill of those tokens (32/32 heads, "
                        "scale 1/sqrt(128), fp32 LSE): get_seq_lens, "
                        "get_batch_indices_positions, append, csr_to_block_tables, prefill",
            "us_per_step": round(t0s.region_ms * 1e3, 2),
            "graph_us_per_step": round(t0g.region_ms * 1e3, 2),
            f"graph{GRAPH_STEPS}_us_per_step": round(t0g8.region_ms * 1e3, 2),
            "us_median": round(t0s.median_ms * 1e3, 2), "us_min": round(t0s.min_ms * 1e3, 2),
            "append_us": round(t0a.region_ms * 1e3, 2),
            "prefill_us": round(t0p.region_ms * 1e3, 2),
            "append_GBs": round(rate(abytes0, t0a.region_ms, G), 1),
            "prefill_TFLOPs": round(rate(flops0, t0p.region_ms, T), 3),
            "bound": "launch latency (3.3 MB moved, 27 MFLOP)",
        },
    }
    if sweep is not None:
        line["append_sweep"] = {
            "what": "extra measurement, not a workload: the append Example's shape family "
                    "(fp16, 32 kv heads, d 128, NHD page 16), each request appending its "
                    "whole sequence into its own pages in random order, nnz from 2^12 to "
                    "2^20 rows; bytes = rows read + rows written + indices; GB/s over the "
                    "timed region (back to back), flushed_GB/s the median of calls after a "
                    "1 GiB read",
            "points": sweep,
        }
    if ceil is not None:
        line["measured_ceilings"] = {
            **ceil,
            "prefill_frac_of_mfma_loop": round(p_l / ceil["mfma_bf16_loop_TFLOPs"], 4),
            "decode_frac_of_read": round(d4_l / ceil["hbm_read_4GiB_GBs"], 4),
            "spec_decode_frac_of_read": round(d5_l / ceil["hbm_read_4GiB_GBs"], 4),
            "bulk_append_frac_of_copy": round(a6_l / ceil["hbm_copy_1GiB_GBs"], 4),
            "bulk_append_frac_of_copy_kernel": round(
                a6_l / ceil["hbm_copy_kernel_512MiB_GBs"], 4),
        }
    if cpu:
        head = dict(base["batch_prefill"])
        head["configs"] = base
        line["cpu_baseline"] = head
    print(json.dumps(line), flush=True)


def only(args, torch, pkv, workloads):
    """One workload alone (profiling runs), or the append sweep, or the
    ceilings; prints one JSON line per measurement."""
    T, G = 1e12, 1e9
    if args.only == "copy":
        x = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        y = torch.empty_like(x)
        t = time_steps(lambda: y.copy_(x), args.steps, args.warmup)
        r = {"GB/s": rate(2 * x.numel() * 4, t.region_ms, G), "bytes_read": x.numel() * 4,
             "bytes_written": x.numel() * 4, "ms_per_step": t.region_ms,
             "ms_launch": t.launch_ms}
    elif args.only in ("prefill", "fp8prefill"):
        w, flops, step = bench_prefill(pkv, torch, workloads, fp8=args.only == "fp8prefill")
        t = time_steps(step, args.steps, args.warmup)
        r = {"TFLOP/s": rate(flops, t.region_ms, T), "ms_per_step": t.region_ms,
             "ms_launch": t.launch_ms,
             "ms_min": t.min_ms}
    elif args.only == "append":
        bytes6, step = bench_append(pkv, torch, workloads.bulk_append("cuda:0"))
        t = time_steps(step, args.steps, args.warmup)
        r = {"GB/s": rate(bytes6, t.region_ms, G), "ms_per_step": t.region_ms,
             "ms_launch": t.launch_ms, "ms_min": t.min_ms}
    elif args.only == "decode":
        w, nb, step = bench_decode(pkv, torch, workloads)
        t = time_steps(step, args.steps, args.warmup)
        r = {"GB/s": rate(nb, t.region_ms, G), "ms_per_step": t.region_ms,
             "ms_launch": t.launch_ms, "ms_min": t.min_ms}
    elif args.only == "spec":
        w, nb, ab, append, decode = bench_spec(pkv, torch, workloads)
        td = time_steps(decode, args.steps, args.warmup)
        ta = time_steps(append, args.steps, args.warmup)
        def step():
            append()
            decode()

        tg = time_graph(torch, step, args.steps, args.warmup)
        tg8 = time_graph(torch, step, args.steps, args.warmup, GRAPH_STEPS)
        r = {"decode GB/s": rate(nb, td.region_ms, G), "ms_decode": td.region_ms,
             "ms_decode_launch": td.launch_ms, "ms_append": ta.region_ms,
             "graph_ms_per_step": tg.region_ms,
             f"graph{GRAPH_STEPS}_ms_per_step": tg8.region_ms}
    elif args.only == "ceilings":
        r = measured_ceilings(torch)
    elif args.only == "example":
        w, flops0, abytes0, step0, _, _ = bench_example(pkv, torch, workloads)
        t = time_steps(step0, args.steps, args.warmup)
        tg = time_graph(torch, step0, args.steps, args.warmup)
        tg8 = time_graph(torch, step0, args.steps, args.warmup, GRAPH_STEPS)
        r = {"us_per_step": t.region_ms * 1e3, "us_median": t.median_ms * 1e3,
             "graph_us_per_step": tg.region_ms * 1e3,
             f"graph{GRAPH_STEPS}_us_per_step": tg8.region_ms * 1e3}
    else:  # append_sweep
        flush = new_flush_buffer(torch)
        for pt in bench_append_sweep(pkv, torch, workloads, args.steps, args.warmup, flush):
            print(json.dumps({"only": "append_sweep", **pt}), flush=True)
        return
    print(json.dumps({"only": args.only,
                      **{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}}),
          flush=True)


if __name__ == "__main__":
    main()
