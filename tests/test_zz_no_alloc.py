"""The allocation-free decode entry point against the workspace one.

pkv_batch_decode_with_kv_cache_no_alloc keeps its split partials in the
library's static scratch array. Called through the C ABI (via the binding)
twice in a row, the second time with a smaller input, it must give the same
output as pkv_batch_decode_with_kv_cache with a caller's workspace: the
same split plan and kernels, so bit for bit, and within the oracle bound.
The second call reuses scratch that still holds the first call's partials.
"""

import numpy as np
import pytest
import torch

import workloads
from tests.helpers import assert_out_close, oracle_decode

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def pkv():
    import attention_paged_kv_cache_amd as m
    return m


def _with_workspace(pkv, w):
    ws = torch.zeros(max(pkv.decode_workspace_size(
        w["seq_lens"].shape[0], w["q_len_per_req"], w["num_qo_heads"], w["num_kv_heads"],
        128, w["max_seq_len"], w["window_left"]), 16), dtype=torch.uint8, device=DEV)
    out = pkv.batch_decode_with_kv_cache(
        w["query"], w["kv_cache"], ws, w["block_tables"].to(DEV), w["seq_lens"].to(DEV),
        w["max_seq_len"], bmm1_scale=w["bmm1_scale"], bmm2_scale=w["bmm2_scale"],
        window_left=w["window_left"],
        sinks=None if w["sinks"] is None else w["sinks"].to(DEV), kv_layout=w["layout"],
        q_len_per_req=w["q_len_per_req"])
    torch.cuda.synchronize()
    return out


def _no_alloc(pkv, w, out):
    pkv.batch_decode_with_kv_cache_no_alloc(
        w["query"], w["kv_cache"], w["block_tables"].to(DEV), w["seq_lens"].to(DEV),
        w["max_seq_len"], out=out, bmm1_scale=w["bmm1_scale"], bmm2_scale=w["bmm2_scale"],
        window_left=w["window_left"],
        sinks=None if w["sinks"] is None else w["sinks"].to(DEV), kv_layout=w["layout"],
        q_len_per_req=w["q_len_per_req"])
    torch.cuda.synchronize()
    return out


def _needs_scratch(pkv, w):
    return pkv.decode_workspace_size(w["seq_lens"].shape[0], w["q_len_per_req"],
                                     w["num_qo_heads"], w["num_kv_heads"], 128,
                                     w["max_seq_len"], w["window_left"]) > 0


@pytest.mark.parametrize("kv_dtype", [torch.bfloat16, torch.float8_e4m3fn])
def test_no_alloc_equals_workspace_decode_twice(pkv, kv_dtype):
    big = workloads.batch_decode(DEV, seed=150, batch=6, seq=(3000, 12000), num_qo_heads=16,
                                 num_kv_heads=2, q_len_per_req=2, window_left=-1, sinks=True,
                                 kv_dtype=kv_dtype)
    small = workloads.batch_decode(DEV, seed=151, batch=3, seq=(2500, 7000), num_qo_heads=16,
                                   num_kv_heads=2, q_len_per_req=2, window_left=4000,
                                   sinks=True, kv_dtype=kv_dtype)
    # both calls go through split partials, so the second reads scratch the
    # first one also wrote
    assert _needs_scratch(pkv, big) and _needs_scratch(pkv, small)
    for w in (big, small):
        ref = _with_workspace(pkv, w)
        out = torch.full_like(w["query"], float("nan"))
        got = _no_alloc(pkv, w, out)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        err = assert_out_close(got, oracle_decode(w), got.dtype)
        print(f"batch {w['seq_lens'].shape[0]}: bitwise equal to the workspace call, "
              f"max |out err| {err:.3g}", flush=True)


def test_no_alloc_single_split_and_full_size(pkv):
    # a plan with one split needs no scratch at all; the batch-decode
    # workload (256 requests up to 8192 tokens) fits the scratch array
    w = workloads.batch_decode(DEV, seed=152, batch=4, seq=(1, 600), num_qo_heads=8,
                               num_kv_heads=2, q_len_per_req=3, sinks=True)
    assert not _needs_scratch(pkv, w)
    ref = _with_workspace(pkv, w)
    got = _no_alloc(pkv, w, torch.empty_like(w["query"]))
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    w = workloads.batch_decode(DEV)
    assert _needs_scratch(pkv, w)
    ref = _with_workspace(pkv, w)
    got = _no_alloc(pkv, w, torch.empty_like(w["query"]))
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    reqs = [0, 100, int(torch.argmax(w["seq_lens"].to(torch.int64)))]
    assert_out_close(got.index_select(0, torch.tensor(reqs, device=DEV)),
                     oracle_decode(w, reqs), got.dtype)


def test_no_alloc_rejects_plans_beyond_the_scratch(pkv):
    # a split plan larger than the static array is refused on the host,
    # before anything is enqueued
    w = workloads.batch_decode(DEV, seed=153, batch=2, seq=(100, 200), num_qo_heads=64,
                               num_kv_heads=8, q_len_per_req=4)
    big_len = 1 << 20
    assert pkv.decode_workspace_size(64, 4, 64, 8, 128, big_len, -1) > 64 << 20
    q = torch.zeros(64 * 4, 64, 128, dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros(64, big_len // 16, dtype=torch.int32, device=DEV)
    seq = torch.ones(64, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(ValueError, match="static scratch"):
        pkv.batch_decode_with_kv_cache_no_alloc(q, w["kv_cache"], bt, seq, big_len, out=out,
                                                q_len_per_req=4)
