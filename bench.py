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

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import hashlib
import json
import math
import os
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
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", choices=["prefill", "decode", "spec", "fp8prefill", "append", "copy"],
                   default=None, help="time one workload (profiling runs); 'copy' times a "
                                      "plain 1 GiB device copy used to calibrate HBM counters")
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

def time_steps(fn, steps, warmup):
    """(average ms per step over the whole region, average ms per launch from
    events around each call). Events sit on the current stream, which is the
    stream the library enqueues on."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    end.record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    return start.elapsed_time(end) / steps, sum(per) / len(per), min(per)


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

def bench_prefill(pkv, torch, workloads, steps, warmup, fp8=False):
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

    ms, ms_launch, ms_min = time_steps(step, steps, warmup)
    flops = prefill_flops(lq.tolist(), lkv.tolist(), w["num_qo_heads"], w["d_qk"], w["d_vo"])
    return w, flops, ms, ms_launch, ms_min


def bench_decode(pkv, torch, workloads, steps, warmup):
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

    ms, ms_launch, ms_min = time_steps(step, steps, warmup)
    nbytes = decode_bytes(w["seq_lens"].tolist(), 1, -1, 32, 8, 128, 2, 2, 2, 16)
    return w, nbytes, ms, ms_launch, ms_min


def bench_spec(pkv, torch, workloads, steps, warmup):
    """Append 4 drafts per request, then decode them (one step = both)."""
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

    def step():
        append()
        decode()

    ms, _, _ = time_steps(step, steps, warmup)
    _, ms_dec, ms_dec_min = time_steps(decode, steps, warmup)
    _, ms_app, _ = time_steps(append, steps, warmup)
    nbytes = decode_bytes(w["seq_lens"].tolist(), ql, w["window_left"], 64, 8, 128, 1, 2, 2, 32)
    abytes = append_bytes(nnz, 8, 128, 1)
    return w, nbytes, abytes, ms, ms_dec, ms_dec_min, ms_app


def bench_bulk_append(pkv, torch, workloads, steps, warmup):
    """Append 1024 rows into each of 256 requests (e4m3, 8 heads, d 128, HND
    page 32): 512 MiB of K/V read and written per step."""
    dev = "cuda:0"
    w = workloads.bulk_append(dev)
    nnz = w["k_append"].shape[0]
    seq = w["seq_lens"].to(dev)
    bi, pos = pkv.get_batch_indices_positions(w["append_indptr"].to(dev), seq, nnz)
    idx, indptr, last = (w["kv_indices"].to(dev), w["kv_indptr"].to(dev),
                         w["kv_last_page_len"].to(dev))

    def step():
        pkv.append_paged_kv_cache(w["k_append"], w["v_append"], bi, pos, w["kv_cache"], idx,
                                  indptr, last, kv_layout=w["layout"])

    ms, ms_launch, ms_min = time_steps(step, steps, warmup)
    return w, append_bytes(nnz, w["num_kv_heads"], w["head_dim"], 1), ms, ms_launch, ms_min


def cpu_baseline(w, budget_s=12.0):
    """The float64 oracle on a bounded sample of the prefill workload: whole
    requests, in order, until about budget_s seconds of CPU work."""
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
    t0 = time.perf_counter()
    for b in range(lq.shape[0]):
        n = (int(lkv[b]) + ps - 1) // ps
        bt = w["block_tables"][b:b + 1]
        kc, bt1 = compact_pages(w["k_cache"], bt, [n])
        vc, _ = compact_pages(w["v_cache"], bt, [n])
        q = q_all[cq[b]:cq[b + 1]]
        oracle.batch_prefill(q, fmt(w["q"]), bits(kc), bits(vc), fmt(w["k_cache"]), bt1.numpy(),
                             lq[b:b + 1].numpy(), lkv[b:b + 1].numpy(), w["scale"], True,
                             w["layout"])
        flops += prefill_flops([int(lq[b])], [int(lkv[b])], w["num_qo_heads"], w["d_qk"],
                               w["d_vo"])
        n_req += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    cores = torch.get_num_threads()
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 0) for i in info] + [cores])
    except Exception:
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {n_req} of 16 requests of the prefill workload "
                      f"({flops / 1e9:.1f} GFLOP algorithmic) in {dt:.1f} s, float64 numpy"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import attention_paged_kv_cache_amd as pkv
    import workloads

    if args.only:
        if args.only == "copy":
            x = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
            y = torch.empty_like(x)
            ms, ms_l, ms_min = time_steps(lambda: y.copy_(x), args.steps, args.warmup)
            r = {"GB/s": 2 * x.numel() * 4 / (ms_l * 1e-3) / 1e9, "bytes_read": x.numel() * 4,
                 "bytes_written": x.numel() * 4, "ms_launch": ms_l}
        elif args.only in ("prefill", "fp8prefill"):
            w, flops, ms, ms_l, ms_min = bench_prefill(pkv, torch, workloads, args.steps,
                                                       args.warmup, fp8=args.only == "fp8prefill")
            r = {"TFLOP/s": flops / (ms_l * 1e-3) / 1e12, "ms_launch": ms_l, "ms_min": ms_min}
        elif args.only == "append":
            w, nb, ms, ms_l, ms_min = bench_bulk_append(pkv, torch, workloads, args.steps,
                                                        args.warmup)
            r = {"GB/s": nb / (ms_l * 1e-3) / 1e9, "ms_launch": ms_l, "ms_min": ms_min}
        elif args.only == "decode":
            w, nb, ms, ms_l, ms_min = bench_decode(pkv, torch, workloads, args.steps, args.warmup)
            r = {"GB/s": nb / (ms_l * 1e-3) / 1e9, "ms_launch": ms_l, "ms_min": ms_min}
        else:
            w, nb, ab, ms, ms_d, ms_dmin, ms_a = bench_spec(pkv, torch, workloads, args.steps,
                                                            args.warmup)
            r = {"decode GB/s": nb / (ms_d * 1e-3) / 1e9, "ms_decode": ms_d,
                 "ms_append": ms_a, "ms_step": ms}
        print(json.dumps({"only": args.only, **{k: round(v, 4) for k, v in r.items()}}),
              flush=True)
        return

    print("bench: prefill (bf16, batch 16)", file=sys.stderr, flush=True)
    w, flops, ms, ms_launch, ms_min = bench_prefill(pkv, torch, workloads, args.steps,
                                                    args.warmup)
    tflops = flops / (ms * 1e-3) / 1e12
    tflops_launch = flops / (ms_launch * 1e-3) / 1e12
    prefill_src = ("prefill.hip", "pkv_common.h", "launch.h")
    decode_src = ("decode.hip", "pkv_common.h", "launch.h")
    append_src = ("append.hip", "pkv_common.h", "launch.h")

    print("bench: fp8 prefill (d_qk 192)", file=sys.stderr, flush=True)
    w3, flops3, ms3, ms3_launch, _ = bench_prefill(pkv, torch, workloads, args.steps,
                                                   args.warmup, fp8=True)
    del w3
    torch.cuda.empty_cache()

    print("bench: decode (bf16, batch 256)", file=sys.stderr, flush=True)
    w4, bytes4, ms4, ms4_launch, ms4_min = bench_decode(pkv, torch, workloads, args.steps,
                                                        args.warmup)
    del w4
    torch.cuda.empty_cache()

    print("bench: append + speculative decode (fp8 KV)", file=sys.stderr, flush=True)
    w5, bytes5, abytes5, ms5, ms5_dec, ms5_dec_min, ms5_app = bench_spec(
        pkv, torch, workloads, args.steps, args.warmup)
    del w5
    torch.cuda.empty_cache()

    print("bench: bulk append (fp8 KV, 262144 rows)", file=sys.stderr, flush=True)
    w6, bytes6, ms6, ms6_launch, _ = bench_bulk_append(pkv, torch, workloads, args.steps,
                                                       args.warmup)
    del w6
    torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
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
            "tokens": int(w["seq_lens_q"].sum()),
            "kv_tokens": int(w["seq_lens_kv"].sum()),
            "flop_per_step": flops,
        },
        "roofline": roofline("mfma", tflops_launch, PEAK_BF16_TFLOPS, "TFLOP/s",
                             traffic("prefill_bf16", prefill_src)),
        "fp8_prefill": {
            "workload": "e4m3 prefill, d_qk 192 / d_vo 128, batch 8, q_len = kv_len = 4096, "
                        "16/16 heads, page 64, per-tensor scales, causal, bf16 out",
            "value": round(flops3 / (ms3 * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(ms3, 4),
            "roofline": roofline("mfma", flops3 / (ms3_launch * 1e-3) / 1e12, PEAK_FP8_TFLOPS,
                                 "TFLOP/s", traffic("prefill_e4m3_d192", prefill_src)),
            "frac_of_bf16_peak": round(flops3 / (ms3_launch * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        },
        "decode": {
            "workload": "decode over block_tables: bf16, batch 256, seq U[512,8192], 32/8 heads, "
                        "d 128, HND page 16, random pages, 1 query per request",
            "value": round(bytes4 / (ms4 * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(ms4, 4), "bytes_per_step": bytes4,
            "roofline": roofline("hbm", bytes4 / (ms4_launch * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s",
                                 traffic("decode_bf16", decode_src)),
        },
        "spec_decode": {
            "workload": "append 4 drafts/request then decode: fp8 e4m3 KV, batch 64, "
                        "seq U[4096,32768], 64/8 heads, d 128, HND page 32, window_left 4095, "
                        "sinks, q_len_per_req 4",
            "ms_per_step": round(ms5, 4),
            "decode_value": round(bytes5 / (ms5_dec * 1e-3) / 1e9, 1), "unit": "GB/s",
            "decode_bytes": bytes5,
            "roofline": roofline("hbm", bytes5 / (ms5_dec * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s",
                                 traffic("spec_decode_e4m3", decode_src)),
            "append_ms": round(ms5_app, 4),
            "append_GBs": round(abytes5 / (ms5_app * 1e-3) / 1e9, 1),
        },
        "bulk_append": {
            "workload": "append 1024 rows into each of 256 requests: e4m3 KV, 8 kv heads, d 128, "
                        "HND page 32, seq U[4096,8192] after the append, pages in random order",
            "value": round(bytes6 / (ms6 * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(ms6, 4), "bytes_per_step": bytes6,
            "roofline": roofline("hbm", bytes6 / (ms6_launch * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s",
                                 traffic("append_bulk_e4m3", append_src)),
        },
    }
    if not args.no_cpu_baseline:
        print("bench: float64 oracle on the host (bounded sample)", file=sys.stderr, flush=True)
        w, *_ = bench_prefill(pkv, torch, workloads, 1, 0)
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
