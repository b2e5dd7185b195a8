"""Seeded random sweeps of small shapes against the float64 oracle.

Each case draws its shape from one generator seed: batch 1-8, lengths
1-300, page size 16/32/64, NHD or HND, GQA group 1/2/4/8, d_qk 128/192 (for
prefill), fp16/bf16/e4m3, window -1/0/7/100, sinks on or off and 1-4 queries
per request (for decode). Two more sweeps cross the decode extensions
(ragged query counts, random or tree draft masks, e4m3 output, device-tensor
scales) and unpaged prefill with every batch offset in a random order with
gaps. A last sweep crosses the element types: prefill inputs fp16/bf16/e4m3
with fp16 or bf16 output, decode queries fp16 or bf16 over K/V of the
query's type or e4m3 with fp16/bf16/e4m3 output. The per-dimension tests pin
each feature alone; the sweeps cross them at random.
"""

import numpy as np
import pytest
import torch

import workloads
from tests.helpers import assert_lse_close, assert_out_close, oracle_decode, oracle_prefill
from tests.test_gpu_decode import run_decode
from tests.test_gpu_prefill import run_prefill

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def pkv():
    import attention_paged_kv_cache_amd as m
    return m


def _pick(rng, xs):
    return xs[int(rng.integers(len(xs)))]


@pytest.mark.parametrize("case", range(16))
def test_prefill_sweep(pkv, case):
    rng = np.random.default_rng(1000 + case)
    B = int(rng.integers(1, 9))
    hkv = _pick(rng, [1, 2, 4])
    G = _pick(rng, [1, 2, 4, 8])
    dtype = _pick(rng, [torch.float16, torch.bfloat16, torch.float8_e4m3fn])
    d_qk = _pick(rng, [128, 192])
    ps = _pick(rng, [16, 32, 64])
    layout = _pick(rng, ["NHD", "HND"])
    q_hi = int(rng.integers(1, 301))
    kw = dict(batch=B, q_len=(1, q_hi), prefix=(0, int(rng.integers(0, 301))),
              num_qo_heads=hkv * G, num_kv_heads=hkv, d_qk=d_qk, page_size=ps, layout=layout,
              pool_pages=B * (600 // ps + 2) + 5)
    if dtype == torch.float8_e4m3fn:
        w = workloads.batch_prefill(DEV, seed=1000 + case, dtype=torch.bfloat16, **kw)
        sc = torch.rand(3, generator=torch.Generator().manual_seed(case)) * 1.5 + 0.5
        for key in ("q", "k_cache", "v_cache"):
            w[key] = w[key].to(torch.float8_e4m3fn)
        w["q_scale"], w["k_scale"], w["v_scale"] = (sc[i].reshape(1, 1, 1, 1) for i in range(3))
    else:
        w = workloads.batch_prefill(DEV, seed=1000 + case, dtype=dtype, **kw)
    w["causal"] = bool(rng.integers(0, 2))
    print(f"case {case}: B {B} G {G} hkv {hkv} {dtype} d_qk {d_qk} ps {ps} {layout} "
          f"causal {w['causal']} lq {w['seq_lens_q'].tolist()} lkv {w['seq_lens_kv'].tolist()}",
          flush=True)
    out, lse = run_prefill(pkv, w)
    ref_o, ref_l = oracle_prefill(w)
    assert_out_close(out, ref_o, out.dtype)
    assert_lse_close(lse, ref_l)


@pytest.mark.parametrize("case", range(16))
def test_decode_sweep(pkv, case):
    rng = np.random.default_rng(2000 + case)
    B = int(rng.integers(1, 9))
    hkv = _pick(rng, [1, 2, 4])
    G = _pick(rng, [1, 2, 4, 8])
    ql = int(rng.integers(1, 5))
    kv_dtype = _pick(rng, [torch.bfloat16, torch.float8_e4m3fn])
    w = workloads.batch_decode(DEV, seed=2000 + case, batch=B, seq=(1, int(rng.integers(1, 301))),
                               num_qo_heads=hkv * G, num_kv_heads=hkv, q_len_per_req=ql,
                               page_size=_pick(rng, [16, 32, 64]),
                               layout=_pick(rng, ["NHD", "HND"]), kv_dtype=kv_dtype,
                               window_left=_pick(rng, [-1, 0, 7, 100]),
                               sinks=bool(rng.integers(0, 2)))
    w["bmm2_scale"] = float(rng.uniform(0.5, 2.0))
    print(f"case {case}: B {B} G {G} hkv {hkv} ql {ql} {kv_dtype} ps {w['page_size']} "
          f"{w['layout']} window {w['window_left']} sinks {w['sinks'] is not None} "
          f"seq {w['seq_lens'].tolist()}", flush=True)
    out = run_decode(pkv, w)
    assert_out_close(out, oracle_decode(w), out.dtype)


@pytest.mark.parametrize("case", range(16))
def test_decode_feature_sweep(pkv, case):
    # decode features crossed at random: ragged query counts, a draft mask
    # (random or tree), e4m3 output with o_scale, device-tensor bmm scales
    from tests.test_gpu_decode import _tree_mask, check_fp8_out, oracle_decode_ragged
    from tests.helpers import assert_out_close as close
    rng = np.random.default_rng(3000 + case)
    B = int(rng.integers(1, 9))
    hkv = _pick(rng, [1, 2, 4])
    q_max = int(rng.integers(1, 5))
    G = _pick(rng, [g for g in (1, 2, 4, 8, 16) if g * q_max <= 64])
    kv_dtype = _pick(rng, [torch.bfloat16, torch.float8_e4m3fn])
    window = _pick(rng, [-1, 0, 5, 300])
    w = workloads.batch_decode(DEV, seed=3000 + case, batch=B, seq=(1, int(rng.integers(1, 3001))),
                               num_qo_heads=hkv * G, num_kv_heads=hkv, q_len_per_req=q_max,
                               page_size=_pick(rng, [16, 32, 64]),
                               layout=_pick(rng, ["NHD", "HND"]), kv_dtype=kv_dtype,
                               window_left=window, sinks=bool(rng.integers(0, 2)))
    w["bmm1_scale"] = float(rng.uniform(0.03, 0.2))
    w["bmm2_scale"] = float(rng.uniform(0.5, 2.0))
    ragged = bool(rng.integers(0, 2))
    counts = rng.integers(0, q_max + 1, size=B) if ragged else np.full(B, q_max)
    cum = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    kind = _pick(rng, ["none", "random", "tree"]) if q_max > 1 else "none"
    mask = None
    if kind == "random":
        mask = torch.from_numpy(rng.random((B, q_max, q_max)) < 0.5).to(DEV)
    elif kind == "tree":
        mask = torch.from_numpy(_tree_mask(B, q_max, rng)).to(DEV)
    fp8_out = bool(rng.integers(0, 2))
    o_scale = float(rng.uniform(0.2, 2.0)) if fp8_out else 1.0
    dev_scales = bool(rng.integers(0, 2))
    b1, b2 = w["bmm1_scale"], w["bmm2_scale"]
    if dev_scales:
        b1 = torch.tensor([b1], dtype=torch.float32, device=DEV)
        b2 = torch.tensor([b2], dtype=torch.float32, device=DEV)
    print(f"case {case}: B {B} G {G} hkv {hkv} q_max {q_max} counts {counts.tolist()} "
          f"{kv_dtype} ps {w['page_size']} {w['layout']} window {window} "
          f"sinks {w['sinks'] is not None} mask {kind} fp8 out {fp8_out} "
          f"device scales {dev_scales} seq {w['seq_lens'].tolist()}", flush=True)
    ws = torch.zeros(max(pkv.decode_workspace_size(
        B, q_max, hkv * G, hkv, 128, w["max_seq_len"], window), 16), dtype=torch.uint8,
        device=DEV)
    got = pkv.batch_decode_with_kv_cache(
        w["query"], w["kv_cache"], ws, w["block_tables"].to(DEV), w["seq_lens"].to(DEV),
        w["max_seq_len"], bmm1_scale=b1, bmm2_scale=b2, window_left=window,
        sinks=None if w["sinks"] is None else w["sinks"].to(DEV), kv_layout=w["layout"],
        mask=mask, max_q_len=q_max if ragged else None,
        cum_seq_lens_q=torch.from_numpy(cum).to(DEV) if ragged else None,
        q_len_per_req=1 if ragged else q_max,
        out_dtype=torch.float8_e4m3fn if fp8_out else None, o_scale=o_scale)
    torch.cuda.synchronize()
    n = int(cum[-1])
    ref = oracle_decode_ragged(w, cum, mask)
    if fp8_out:
        check_fp8_out(got[:n], ref, o_scale)
    else:
        close(got[:n], ref, got.dtype)


@pytest.mark.parametrize("case", range(10))
def test_prefill_unpaged_offsets_sweep(pkv, case):
    # unpaged prefill (block_tables=None) with every batch offset set: each
    # tensor's requests in their own random order with random gaps; empty
    # requests and L_kv < L_q included; rows no request owns stay untouched
    import oracle
    from tests.helpers import assert_lse_close as close_lse, assert_out_close as close, bits, fmt
    rng = np.random.default_rng(4000 + case)
    B = int(rng.integers(1, 7))
    hkv = _pick(rng, [1, 2, 4])
    G = _pick(rng, [1, 2, 4, 8])
    dtype = _pick(rng, [torch.float16, torch.bfloat16, torch.float8_e4m3fn])
    d_qk = _pick(rng, [128, 192])
    causal = bool(rng.integers(0, 2))
    lq = rng.integers(0, 301, size=B)
    lkv = lq + rng.integers(0, 301, size=B)
    short = rng.random(B) < 0.25
    lkv[short] = rng.integers(0, lq[short] + 1)

    def place(lens):
        order = rng.permutation(B)
        offs = np.zeros(B, dtype=np.int64)
        cur = 0
        for b in order:
            offs[b] = cur
            cur += int(lens[b]) + int(rng.integers(0, 6))
        return offs, max(cur, 1)

    (oq, nq), (oo, no), (os_, ns) = place(lq), place(lq), place(lq)
    (ok_, nk), (ov, nv) = place(lkv), place(lkv)
    gen = torch.Generator(device=DEV).manual_seed(4000 + case)
    H = hkv * G
    rnd = lambda *shape: torch.randn(*shape, generator=gen, device=DEV).to(dtype)
    q, k, v = rnd(nq, H, d_qk), rnd(nk, hkv, d_qk), rnd(nv, hkv, 128)
    if dtype == torch.float8_e4m3fn:
        sc = [float(x) for x in rng.uniform(0.5, 2.0, 3)]
    else:
        sc = [1.0, 1.0, 1.0]
    n_out = max(no, ns)
    o_dtype = torch.float16 if dtype == torch.float16 else torch.bfloat16
    out = torch.full((n_out, H, 128), float("nan"), dtype=o_dtype, device=DEV)
    lse = torch.full((n_out, H), float("nan"), dtype=torch.float32, device=DEV)
    scale = 1.0 / np.sqrt(d_qk)
    print(f"case {case}: B {B} G {G} hkv {hkv} {dtype} d_qk {d_qk} causal {causal} "
          f"lq {lq.tolist()} lkv {lkv.tolist()}", flush=True)
    ws = torch.zeros(pkv.prefill_workspace_size(B), dtype=torch.uint8, device=DEV)
    t = lambda x: torch.tensor(x, dtype=torch.int32, device=DEV)
    st = lambda x: torch.tensor([x], dtype=torch.float32, device=DEV)
    fp8 = dtype == torch.float8_e4m3fn
    pkv.batch_prefill_with_kv_cache(
        q, k, v, scale, ws, max_token_per_sequence=int(lq.max()),
        max_sequence_kv=int(lkv.max()), actual_seq_lens_q=t(lq), actual_seq_lens_kv=t(lkv),
        block_tables=None, causal=causal, q_scale=st(sc[0]) if fp8 else None,
        k_scale=st(sc[1]) if fp8 else None, v_scale=st(sc[2]) if fp8 else None,
        out=out, lse=lse, batch_offsets_q=t(oq), batch_offsets_o=t(oo), batch_offsets_k=t(ok_),
        batch_offsets_v=t(ov), batch_offsets_stats=t(os_))
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.batch_prefill_ragged(
        bits(q), fmt(q), bits(k), bits(v), fmt(k), lq, lkv, scale, causal, q_scale=sc[0],
        k_scale=sc[1], v_scale=sc[2], offsets_q=oq, offsets_o=oo, offsets_k=ok_,
        offsets_v=ov, offsets_stats=os_, out_rows=n_out)
    wo = ~np.isnan(ref_o[:, 0, 0])
    wl = ~np.isnan(ref_l[:, 0])
    if wo.any():
        close(out[torch.from_numpy(wo).to(DEV)], ref_o[wo], o_dtype)
    if wl.any():
        close_lse(lse[torch.from_numpy(wl).to(DEV)], ref_l[wl])
    assert torch.isnan(out[torch.from_numpy(~wo).to(DEV)].float()).all()
    assert torch.isnan(lse[torch.from_numpy(~wl).to(DEV)]).all()


@pytest.mark.parametrize("case", range(12))
def test_dtype_sweep(pkv, case):
    # input and output element types crossed at random, each case drawing a
    # prefill and a decode: prefill q/k/v fp16, bf16 or e4m3 with fp16 or
    # bf16 output; decode query fp16 or bf16, K/V the query's type or e4m3,
    # output fp16, bf16 or e4m3; lengths long enough for split-KV merges
    from tests.test_gpu_decode import check_fp8_out
    rng = np.random.default_rng(5000 + case)
    dtype = _pick(rng, [torch.float16, torch.bfloat16, torch.float8_e4m3fn])
    o_dtype = _pick(rng, [torch.float16, torch.bfloat16])
    hkv = _pick(rng, [1, 2])
    G = _pick(rng, [1, 4, 8])
    d_qk = _pick(rng, [128, 192])
    B = int(rng.integers(1, 5))
    kw = dict(batch=B, q_len=(1, int(rng.integers(1, 260))), prefix=(0, 200),
              num_qo_heads=hkv * G, num_kv_heads=hkv, d_qk=d_qk,
              page_size=_pick(rng, [16, 32, 64]), layout=_pick(rng, ["NHD", "HND"]),
              pool_pages=B * (500 // 16 + 2) + 5)
    if dtype == torch.float8_e4m3fn:
        w = workloads.batch_prefill(DEV, seed=5000 + case, dtype=torch.bfloat16, **kw)
        for key in ("q", "k_cache", "v_cache"):
            w[key] = w[key].to(torch.float8_e4m3fn)
        sc = rng.uniform(0.5, 2.0, 3)
        w["q_scale"], w["k_scale"], w["v_scale"] = (
            torch.tensor([float(x)], dtype=torch.float32) for x in sc)
    else:
        w = workloads.batch_prefill(DEV, seed=5000 + case, dtype=dtype, **kw)
    print(f"case {case} prefill: {dtype} -> {o_dtype} B {B} G {G} hkv {hkv} d_qk {d_qk} "
          f"lq {w['seq_lens_q'].tolist()} lkv {w['seq_lens_kv'].tolist()}", flush=True)
    out, lse = run_prefill(pkv, w, o_dtype)
    assert out.dtype == o_dtype
    ref_o, ref_l = oracle_prefill(w)
    assert_out_close(out, ref_o, o_dtype)
    assert_lse_close(lse, ref_l)

    q_dtype = _pick(rng, [torch.float16, torch.bfloat16])
    kv_dtype = _pick(rng, [q_dtype, torch.float8_e4m3fn])
    d_out = _pick(rng, [torch.float16, torch.bfloat16, torch.float8_e4m3fn])
    ql = int(rng.integers(1, 5))
    Gd = _pick(rng, [g for g in (1, 2, 4, 8, 16) if g * ql <= 64])
    window = _pick(rng, [-1, 7, 1500])
    w = workloads.batch_decode(DEV, seed=6000 + case, batch=int(rng.integers(1, 7)),
                               seq=(1, int(rng.integers(1, 6001))), num_qo_heads=hkv * Gd,
                               num_kv_heads=hkv, q_len_per_req=ql,
                               page_size=_pick(rng, [16, 32, 64]),
                               layout=_pick(rng, ["NHD", "HND"]), kv_dtype=kv_dtype,
                               q_dtype=q_dtype, window_left=window,
                               sinks=bool(rng.integers(0, 2)))
    w["bmm2_scale"] = float(rng.uniform(0.5, 2.0))
    print(f"case {case} decode: q {q_dtype} kv {kv_dtype} out {d_out} G {Gd} hkv {hkv} ql {ql} "
          f"ps {w['page_size']} {w['layout']} window {window} seq {w['seq_lens'].tolist()}",
          flush=True)
    got = run_decode(pkv, w, out_dtype=d_out)
    assert got.dtype == d_out
    ref = oracle_decode(w)
    if d_out == torch.float8_e4m3fn:
        check_fp8_out(got, ref, 1.0)
    else:
        assert_out_close(got, ref, d_out)
