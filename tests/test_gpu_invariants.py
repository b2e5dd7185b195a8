"""Invariants of the method checked on the GPU path itself, with no oracle:

* layout: the same K/V stored NHD and HND give bit-identical outputs (only
  addresses differ);
* GQA: H_kv heads shared by G qo heads equal K/V repeated to H_qo heads
  (prefill bit for bit; decode within tolerance);
* decode equals prefill: decode of q_len_per_req queries with bmm1 / bmm2
  equals a causal prefill of those queries over the request's keys with
  scale = bmm1 and v_scale = bmm2 (the prefill and decode pages define the
  same masked softmax).
"""

import pytest
import torch

import workloads
from tests.helpers import assert_out_close
from tests.test_gpu_decode import run_decode
from tests.test_gpu_prefill import run_prefill

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def pkv():
    import attention_paged_kv_cache_amd as m
    return m


def _same_bits(a, b):
    ia = a.view(torch.int16) if a.element_size() == 2 else a.view(torch.int32)
    ib = b.view(torch.int16) if b.element_size() == 2 else b.view(torch.int32)
    return torch.equal(ia, ib)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float8_e4m3fn])
def test_prefill_nhd_equals_hnd_bitwise(pkv, dtype):
    if dtype == torch.float8_e4m3fn:
        w = workloads.fp8_prefill(DEV, seed=80, batch=3, seq_len=200, num_heads=4, d_qk=128,
                                  page_size=32)
    else:
        w = workloads.batch_prefill(DEV, seed=81, batch=3, q_len=(1, 300), prefix=(0, 250),
                                    num_qo_heads=16, num_kv_heads=4, dtype=dtype, pool_pages=150)
    assert w["layout"] == "HND"
    o_h, l_h = run_prefill(pkv, w)
    nhd = dict(w, layout="NHD", k_cache=w["k_cache"].transpose(1, 2).contiguous(),
               v_cache=w["v_cache"].transpose(1, 2).contiguous())
    o_n, l_n = run_prefill(pkv, nhd)
    assert _same_bits(o_h, o_n) and _same_bits(l_h, l_n)


@pytest.mark.parametrize("kv_dtype", [torch.bfloat16, torch.float8_e4m3fn])
def test_decode_nhd_equals_hnd_bitwise(pkv, kv_dtype):
    w = workloads.batch_decode(DEV, seed=82, batch=5, seq=(1, 3000), num_qo_heads=16,
                               num_kv_heads=4, q_len_per_req=3, kv_dtype=kv_dtype,
                               window_left=500, sinks=True)
    o_h = run_decode(pkv, w)
    kv_nhd = w["kv_cache"].transpose(2, 3).contiguous()  # [P, 2, ps, H, d]
    o_n = run_decode(pkv, dict(w, layout="NHD"), kv_cache=kv_nhd)
    assert _same_bits(o_h, o_n)


def test_prefill_gqa_equals_replicated_heads(pkv):
    G = 4
    w = workloads.batch_prefill(DEV, seed=83, batch=3, q_len=(1, 300), prefix=(0, 250),
                                num_qo_heads=8, num_kv_heads=2, pool_pages=150)
    o_g, l_g = run_prefill(pkv, w)
    rep = dict(w, num_kv_heads=8,
               k_cache=w["k_cache"].repeat_interleave(G, dim=1).contiguous(),
               v_cache=w["v_cache"].repeat_interleave(G, dim=1).contiguous())
    o_r, l_r = run_prefill(pkv, rep)
    # every row sees the same 64-key tiles in the same order either way (rows
    # beyond a row's keys add exact zeros), so the results are bit-identical
    assert _same_bits(o_g, o_r) and _same_bits(l_g, l_r)


def test_decode_gqa_equals_replicated_heads(pkv):
    G = 8
    w = workloads.batch_decode(DEV, seed=84, batch=4, seq=(1, 2000), num_qo_heads=16,
                               num_kv_heads=2, q_len_per_req=2, sinks=True)
    o_g = run_decode(pkv, w)
    kv = w["kv_cache"].repeat_interleave(G, dim=2).contiguous()  # HND: [P, 2, H, ps, d]
    o_r = run_decode(pkv, dict(w, num_kv_heads=16), kv_cache=kv)
    # 8x the (request, kv head) units changes the split-KV chunk length, so
    # the two runs merge different partial sums: equal within tolerance
    assert_out_close(o_r, o_g.double().cpu().numpy(), o_g.dtype)


@pytest.mark.parametrize("ql", [1, 4])
def test_decode_equals_causal_prefill_of_the_last_positions(pkv, ql):
    w = workloads.batch_decode(DEV, seed=85, batch=6, seq=(ql, 2500), num_qo_heads=16,
                               num_kv_heads=4, q_len_per_req=ql)
    w["bmm1_scale"], w["bmm2_scale"] = 0.07, 1.6
    o_dec = run_decode(pkv, w)
    B = w["seq_lens"].shape[0]
    ws = torch.zeros(pkv.prefill_workspace_size(B), dtype=torch.uint8, device=DEV)
    lens_q = torch.full((B,), ql, dtype=torch.int32, device=DEV)
    lens_kv = w["seq_lens"].to(torch.int32).to(DEV)
    kv = w["kv_cache"]
    o_pre, _ = pkv.batch_prefill_with_kv_cache(
        w["query"], kv[:, 0], kv[:, 1], w["bmm1_scale"], ws, max_token_per_sequence=ql,
        max_sequence_kv=w["max_seq_len"], actual_seq_lens_q=lens_q, actual_seq_lens_kv=lens_kv,
        block_tables=w["block_tables"].to(DEV), causal=True,
        v_scale=torch.tensor([w["bmm2_scale"]], dtype=torch.float32, device=DEV),
        kv_layout="HND")
    torch.cuda.synchronize()
    assert_out_close(o_dec, o_pre.double().cpu().numpy(), o_dec.dtype)
