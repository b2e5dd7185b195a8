"""A seeded random sweep of small shapes against the float64 oracle.

Each case draws its shape from one generator seed: batch 1-8, lengths
1-300, page size 16/32/64, NHD or HND, GQA group 1/2/4/8, d_qk 128/192 (for
prefill), fp16/bf16/e4m3, window -1/0/7/100, sinks on or off and 1-4 queries
per request (for decode). The per-dimension tests pin each feature alone;
the sweep crosses them at random.
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
