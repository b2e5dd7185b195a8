"""Batch prefill without paging (block_tables=None) and with batch offsets.

Without paging, k_cache / v_cache are [total_kv_rows, H_kv, d] and each
request's rows start at batch_offsets_k / batch_offsets_v (packed in request
order when absent); batch_offsets_q / _o / _stats place each request's rows
in q, out and lse. Checked against the float64 oracle, and bitwise against
the paged kernel on the same data (the tile loop is the same code).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import assert_lse_close, assert_out_close, bits, fmt
from tests.test_gpu_prefill import run_prefill

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def pkv():
    import attention_paged_kv_cache_amd as m
    return m


def contiguous_rows(cache, bt, lens, layout):
    """[sum L_kv, H, d] rows of each request, in request order, from a paged
    cache (a plain gather on the device)."""
    ps = cache.shape[2] if layout == "HND" else cache.shape[1]
    parts = []
    for b in range(bt.shape[0]):
        L = int(lens[b])
        n = (L + ps - 1) // ps
        pages = cache.index_select(0, bt[b, :n].to(torch.long).to(cache.device))
        if layout == "HND":
            pages = pages.permute(0, 2, 1, 3)
        parts.append(pages.reshape(n * ps, pages.shape[2], pages.shape[3])[:L])
    return torch.cat(parts).contiguous()


def unpaged_call(pkv, w, k, v, offs=None, out=None, lse=None, rows_q=None):
    lq, lkv = w["seq_lens_q"], w["seq_lens_kv"]
    ws = torch.zeros(pkv.prefill_workspace_size(lq.shape[0]), dtype=torch.uint8, device=DEV)
    dev = lambda x: None if x is None else x.to(DEV)
    offs = offs or {}
    q = w["q"] if rows_q is None else rows_q
    o, l = pkv.batch_prefill_with_kv_cache(
        q, k, v, w["scale"], ws, max_token_per_sequence=int(lq.max()),
        max_sequence_kv=int(lkv.max()), actual_seq_lens_q=lq.to(DEV),
        actual_seq_lens_kv=lkv.to(DEV), block_tables=None, causal=w["causal"],
        q_scale=dev(w["q_scale"]), k_scale=dev(w["k_scale"]), v_scale=dev(w["v_scale"]),
        out=out, lse=lse, **{f"batch_offsets_{n}": dev(t) for n, t in offs.items()})
    torch.cuda.synchronize()
    return o, l


@pytest.mark.parametrize("seed,kw", [
    (110, dict(batch=4, q_len=(1, 300), prefix=(0, 200))),
    (111, dict(batch=3, q_len=(100, 400), prefix=(0, 700), num_qo_heads=8, num_kv_heads=1)),
    (112, dict(batch=3, q_len=(50, 260), prefix=(0, 90), d_qk=192, dtype=torch.float16,
               layout="NHD", page_size=32)),
])
def test_unpaged_equals_paged_bitwise(pkv, seed, kw):
    w = workloads.batch_prefill(DEV, seed=seed, pool_pages=400, **kw)
    out_p, lse_p = run_prefill(pkv, w)
    bt = w["block_tables"]
    k = contiguous_rows(w["k_cache"], bt, w["seq_lens_kv"], w["layout"])
    v = contiguous_rows(w["v_cache"], bt, w["seq_lens_kv"], w["layout"])
    out_u, lse_u = unpaged_call(pkv, w, k, v)
    assert torch.equal(out_p.view(torch.int16), out_u.view(torch.int16))
    assert torch.equal(lse_p.view(torch.int32), lse_u.view(torch.int32))


def test_unpaged_packed_offsets_past_the_inline_limit(pkv):
    """80 requests: the packed q and key/value row offsets come from the
    prefix-sum launches, not from the in-kernel sum; the unpaged run still
    equals the paged one bitwise."""
    w = workloads.batch_prefill(DEV, seed=116, batch=80, q_len=(0, 40), prefix=(0, 60),
                                pool_pages=720)
    out_p, lse_p = run_prefill(pkv, w)
    bt = w["block_tables"]
    k = contiguous_rows(w["k_cache"], bt, w["seq_lens_kv"], w["layout"])
    v = contiguous_rows(w["v_cache"], bt, w["seq_lens_kv"], w["layout"])
    out_u, lse_u = unpaged_call(pkv, w, k, v)
    assert torch.equal(out_p.view(torch.int16), out_u.view(torch.int16))
    assert torch.equal(lse_p.view(torch.int32), lse_u.view(torch.int32))


def _place(lens, order, gap):
    offs = np.zeros(len(lens), dtype=np.int64)
    cur = 0
    for b in order:
        offs[b] = cur
        cur += int(lens[b]) + gap
    return offs, cur


@pytest.mark.parametrize("fp8", [False, True])
def test_offsets_reorder_with_gaps_against_oracle(pkv, fp8):
    if fp8:
        w = workloads.fp8_prefill(DEV, seed=113, batch=4, seq_len=300)
        lq = torch.tensor([300, 0, 170, 33], dtype=torch.int32)
        lkv = torch.tensor([300, 40, 170, 20], dtype=torch.int32)  # L_kv < L_q in one
    else:
        w = workloads.batch_prefill(DEV, seed=114, batch=4, q_len=(1, 280), prefix=(0, 300),
                                    pool_pages=400)
        lq, lkv = w["seq_lens_q"].clone(), w["seq_lens_kv"].clone()
        lq[1], lkv[2] = 0, 0  # an empty request and one with no keys
    full_q, full_kv = w["seq_lens_q"], w["seq_lens_kv"]
    bt = w["block_tables"]
    k_all = contiguous_rows(w["k_cache"], bt, full_kv, w["layout"])
    v_all = contiguous_rows(w["v_cache"], bt, full_kv, w["layout"])
    cq = np.concatenate([[0], np.cumsum(full_q.numpy())])
    ck = np.concatenate([[0], np.cumsum(full_kv.numpy())])
    order = [2, 0, 3, 1]
    oq, nq = _place(lq.numpy(), order, 3)
    oo, no = _place(lq.numpy(), [1, 3, 0, 2], 2)
    os_, ns = _place(lq.numpy(), order, 5)
    ok_, nk = _place(lkv.numpy(), [3, 2, 1, 0], 7)
    ov, nv = _place(lkv.numpy(), order, 1)
    H_qo, d_qk = w["q"].shape[1], w["q"].shape[2]
    H_kv = k_all.shape[1]
    q2 = torch.zeros(nq, H_qo, d_qk, dtype=w["q"].dtype, device=DEV)
    k2 = torch.zeros(nk, H_kv, d_qk, dtype=k_all.dtype, device=DEV)
    v2 = torch.zeros(nv, H_kv, v_all.shape[2], dtype=v_all.dtype, device=DEV)
    for b in range(4):
        q2[oq[b]:oq[b] + int(lq[b])] = w["q"][cq[b]:cq[b] + int(lq[b])]
        k2[ok_[b]:ok_[b] + int(lkv[b])] = k_all[ck[b]:ck[b] + int(lkv[b])]
        v2[ov[b]:ov[b] + int(lkv[b])] = v_all[ck[b]:ck[b] + int(lkv[b])]
    n_out = max(no, ns)
    out = torch.full((n_out, H_qo, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((n_out, H_qo), float("nan"), dtype=torch.float32, device=DEV)
    w2 = dict(w, seq_lens_q=lq, seq_lens_kv=lkv)
    t = lambda x: torch.tensor(x, dtype=torch.int32)
    unpaged_call(pkv, w2, k2, v2, offs=dict(q=t(oq), o=t(oo), k=t(ok_), v=t(ov), stats=t(os_)),
                 out=out, lse=lse, rows_q=q2)
    sc = lambda x: 1.0 if x is None else float(x.reshape(-1)[0])
    ref_o, ref_l = oracle.batch_prefill_ragged(
        bits(q2), fmt(q2), bits(k2), bits(v2), fmt(k2), lq.numpy(), lkv.numpy(), w["scale"],
        w["causal"], q_scale=sc(w["q_scale"]), k_scale=sc(w["k_scale"]),
        v_scale=sc(w["v_scale"]), offsets_q=oq, offsets_o=oo, offsets_k=ok_, offsets_v=ov,
        offsets_stats=os_, out_rows=n_out)
    written_o = ~np.isnan(ref_o[:, 0, 0])
    written_l = ~np.isnan(ref_l[:, 0])
    assert_out_close(out[torch.from_numpy(written_o).to(DEV)], ref_o[written_o], out.dtype)
    assert_lse_close(lse[torch.from_numpy(written_l).to(DEV)], ref_l[written_l])
    # rows no request owns are never written
    assert torch.isnan(out[torch.from_numpy(~written_o).to(DEV)].float()).all()
    assert torch.isnan(lse[torch.from_numpy(~written_l).to(DEV)]).all()


def test_full_size_unpaged_equals_paged_bitwise(pkv):
    # the benchmark's prefill workload (batch 16, 65536-page pool), gathered
    # into packed rows
    w = workloads.batch_prefill(DEV)
    out_p, lse_p = run_prefill(pkv, w)
    bt = w["block_tables"]
    k = contiguous_rows(w["k_cache"], bt, w["seq_lens_kv"], w["layout"])
    v = contiguous_rows(w["v_cache"], bt, w["seq_lens_kv"], w["layout"])
    out_u, lse_u = unpaged_call(pkv, w, k, v)
    assert torch.equal(out_p.view(torch.int16), out_u.view(torch.int16))
    assert torch.equal(lse_p.view(torch.int32), lse_u.view(torch.int32))
