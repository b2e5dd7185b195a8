"""GPU parity of batch prefill against the float64 oracle.

Bar: |out - ref| <= 2e-2 + half an output ulp of ref, elementwise;
|lse - ref| <= 1e-3. Inputs come from workloads/ with the same seeds on both
sides. Scaled cases span several 128-row query tiles and 64-key kv tiles with
ragged tails; full-size cases are checked on sampled rows.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from tests.helpers import assert_lse_close, assert_out_close, oracle_prefill

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def pkv():
    import attention_paged_kv_cache_amd as m
    return m


def run_prefill(pkv, w, o_dtype=None):
    lq, lkv = w["seq_lens_q"], w["seq_lens_kv"]
    ws = torch.zeros(pkv.prefill_workspace_size(lq.shape[0]), dtype=torch.uint8, device=DEV)
    dev = lambda x: None if x is None else x.to(DEV)
    out, lse = pkv.batch_prefill_with_kv_cache(
        w["q"], w["k_cache"], w["v_cache"], w["scale"], ws,
        max_token_per_sequence=int(lq.max()), max_sequence_kv=int(lkv.max()),
        actual_seq_lens_q=lq.to(DEV), actual_seq_lens_kv=lkv.to(DEV),
        block_tables=w["block_tables"].to(DEV), causal=w["causal"],
        q_scale=dev(w["q_scale"]), k_scale=dev(w["k_scale"]), v_scale=dev(w["v_scale"]),
        o_data_type=o_dtype, kv_layout=w["layout"])
    torch.cuda.synchronize()
    return out, lse


def small_prefill(**kw):
    args = dict(device=DEV, seed=20, batch=3, q_len=(1, 300), prefix=(0, 200),
                pool_pages=120)
    args.update(kw)
    return workloads.batch_prefill(**args)


def check(pkv, w, o_dtype=None):
    out, lse = run_prefill(pkv, w, o_dtype)
    ref_o, ref_l = oracle_prefill(w)
    e1 = assert_out_close(out, ref_o, out.dtype)
    e2 = assert_lse_close(lse, ref_l)
    print(f"max |out err| {e1:.3g}  max |lse err| {e2:.3g}", flush=True)
    return out, lse


@pytest.mark.parametrize("batch", [64, 65, 80])
def test_packed_offsets_on_both_sides_of_the_inline_limit(pkv, batch):
    """Without batch offsets the requests' rows are packed. Up to 64
    requests the kernel sums the lengths before its request itself; beyond
    that a prefix-sum launch writes the offsets to the workspace. Both match
    the oracle, zero-length requests included."""
    w = small_prefill(seed=40 + batch, batch=batch, q_len=(0, 40), prefix=(0, 60),
                      pool_pages=batch * 8 + 8)
    assert int((w["seq_lens_q"] == 0).sum()) > 0
    check(pkv, w)


def test_append_example_then_prefill_fp16_nhd(pkv):
    w = workloads.append_example(DEV)
    cache = w["paged_kv_cache"]
    seq = pkv.get_seq_lens(w["kv_indptr"].to(DEV), w["kv_last_page_len"].to(DEV), 16)
    bi, pos = pkv.get_batch_indices_positions(w["append_indptr"].to(DEV), seq, 100)
    pkv.append_paged_kv_cache(w["k_append"], w["v_append"], bi, pos, cache,
                              w["kv_indices"].to(DEV), w["kv_indptr"].to(DEV),
                              w["kv_last_page_len"].to(DEV), kv_layout="NHD")
    bt = pkv.csr_to_block_tables(w["kv_indptr"].to(DEV), w["kv_indices"].to(DEV), 3)
    lens = w["append_lengths"]
    pw = dict(q=w["q"], k_cache=cache[:, 0], v_cache=cache[:, 1], block_tables=bt.cpu(),
              seq_lens_q=lens, seq_lens_kv=lens, page_size=16, scale=w["scale"],
              layout="NHD", causal=True, q_scale=None, k_scale=None, v_scale=None)
    check(pkv, pw)


@pytest.mark.parametrize("hqo,hkv", [(32, 8), (8, 8), (16, 2), (6, 3)])
def test_bf16_gqa_hnd(pkv, hqo, hkv):
    check(pkv, small_prefill(num_qo_heads=hqo, num_kv_heads=hkv, seed=hqo + hkv))


@pytest.mark.parametrize("ps", [16, 32, 64])
def test_page_sizes_and_nhd(pkv, ps):
    check(pkv, small_prefill(page_size=ps, layout="NHD", seed=ps, num_qo_heads=8,
                             num_kv_heads=2, dtype=torch.float16, pool_pages=200))


@pytest.mark.parametrize("hqo,hkv,dtype,d_qk", [
    (9, 3, torch.bfloat16, 128),        # group 3: 42 tokens x 3 heads per 128-row tile
    (10, 2, torch.bfloat16, 128),       # group 5: 25 tokens, rows 125-127 unused
    (12, 2, torch.float8_e4m3fn, 192),  # group 6: 21 tokens, 192-byte rows
    (24, 2, torch.float8_e4m3fn, 128),  # group 12: 10 tokens, 128-byte rows
    (12, 1, torch.float16, 192),        # group 12, 384-byte rows
    (130, 1, torch.bfloat16, 128),      # group 130: two head chunks (128 + 2), 1 token
])
def test_row_groups(pkv, hqo, hkv, dtype, d_qk):
    """Query tiles whose 128 rows pack a number of tokens that is not a power
    of two (or heads spread over two workgroups): the row -> (token, head)
    mapping of the Q operands and of the output rows, unused rows included,
    against the oracle over several ragged query tiles."""
    small = hqo > 64
    w = small_prefill(seed=60 + hqo, num_qo_heads=hqo, num_kv_heads=hkv, dtype=dtype,
                      d_qk=d_qk, batch=2 if small else 3, q_len=(1, 40 if small else 130),
                      prefix=(0, 30 if small else 100))
    check(pkv, w)


def test_d192_bf16(pkv):
    check(pkv, small_prefill(d_qk=192, num_qo_heads=8, num_kv_heads=4, seed=7))


def test_non_causal(pkv):
    w = small_prefill(seed=8, num_qo_heads=4, num_kv_heads=4)
    w["causal"] = False
    check(pkv, w)


def test_fp8_d192_scales(pkv):
    w = workloads.fp8_prefill(DEV, seed=9, batch=2, seq_len=333, num_heads=4)
    check(pkv, w)


def test_fp8_d128_fp16_out(pkv):
    w = workloads.fp8_prefill(DEV, seed=10, batch=2, seq_len=200, num_heads=2, d_qk=128,
                              page_size=16)
    check(pkv, w, o_dtype=torch.float16)


@pytest.mark.parametrize("dtype,o_dtype", [(torch.float16, torch.bfloat16),
                                            (torch.bfloat16, torch.float16)])
@pytest.mark.parametrize("d_qk", [128, 192])
def test_output_dtype_other_than_input(pkv, dtype, o_dtype, d_qk):
    # o_data_type picks the output's 16-bit type independently of q/k/v
    w = small_prefill(seed=15 + d_qk, dtype=dtype, d_qk=d_qk, num_qo_heads=8, num_kv_heads=2)
    out, _ = check(pkv, w, o_dtype)
    assert out.dtype == o_dtype


def test_fp8_d192_fp16_out(pkv):
    w = workloads.fp8_prefill(DEV, seed=16, batch=2, seq_len=290, num_heads=4)
    out, _ = check(pkv, w, o_dtype=torch.float16)
    assert out.dtype == torch.float16


def test_edge_lengths(pkv):
    # L_q = 1, L_kv < L_q (leading rows see no key), and an empty request
    w = small_prefill(seed=11, batch=4, q_len=(300, 300), prefix=(0, 0),
                      num_qo_heads=4, num_kv_heads=2)
    w["seq_lens_q"] = torch.tensor([1, 70, 0, 130], dtype=torch.int32)
    w["seq_lens_kv"] = torch.tensor([1, 40, 5, 300], dtype=torch.int32)
    w["q"] = w["q"][:201].contiguous()
    out, lse = check(pkv, w)
    # rows 1..30 (request 1, tokens 0..29) have no allowed key: out 0, lse -inf
    assert torch.all(out[1:31] == 0)
    assert torch.all(torch.isneginf(lse[1:31]))


def test_negative_scale(pkv):
    w = small_prefill(seed=12, num_qo_heads=4, num_kv_heads=1)
    w["scale"] = -0.05
    check(pkv, w)


def test_poisoned_unused_memory_is_never_read(pkv):
    # NaN in every byte the method must not read: pool pages no request uses,
    # tail slots past each sequence in its last page, and block-table padding
    # pointing at a NaN page. The output must be bit-identical.
    w = small_prefill(seed=13, num_qo_heads=8, num_kv_heads=2, pool_pages=150)
    out0, lse0 = run_prefill(pkv, w)
    ps = w["page_size"]
    used = set()
    for b in range(w["block_tables"].shape[0]):
        n = (int(w["seq_lens_kv"][b]) + ps - 1) // ps
        used.update(int(x) for x in w["block_tables"][b, :n])
    unused = [p for p in range(w["k_cache"].shape[0]) if p not in used]
    kc, vc = w["k_cache"].clone(), w["v_cache"].clone()
    nan = float("nan")
    kc[unused] = nan
    vc[unused] = nan
    for b in range(w["block_tables"].shape[0]):
        L = int(w["seq_lens_kv"][b])
        if L % ps:
            p = int(w["block_tables"][b, L // ps])
            kc[p, :, L % ps:] = nan
            vc[p, :, L % ps:] = nan
    bt = w["block_tables"].clone()
    bt[bt < 0] = unused[0]
    w2 = dict(w, k_cache=kc, v_cache=vc, block_tables=bt)
    out1, lse1 = run_prefill(pkv, w2)
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0.view(torch.int32), lse1.view(torch.int32))


def test_deterministic_and_paged_equals_contiguous(pkv):
    w = small_prefill(seed=14, num_qo_heads=8, num_kv_heads=2)
    o1, l1 = run_prefill(pkv, w)
    o2, l2 = run_prefill(pkv, w)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    # the same sequences laid out in pages 0, 1, 2, ... in order
    ps = w["page_size"]
    bt = w["block_tables"]
    n = [(int(L) + ps - 1) // ps for L in w["seq_lens_kv"]]
    order = torch.cat([bt[b, :n[b]] for b in range(bt.shape[0])]).long().to(DEV)
    kc = w["k_cache"].index_select(0, order)
    vc = w["v_cache"].index_select(0, order)
    bt2 = torch.full_like(bt, -1)
    off = 0
    for b in range(bt.shape[0]):
        bt2[b, :n[b]] = torch.arange(off, off + n[b], dtype=torch.int32)
        off += n[b]
    o3, l3 = run_prefill(pkv, dict(w, k_cache=kc, v_cache=vc, block_tables=bt2))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(l1, l3)


def _sample_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    lq = w["seq_lens_q"].numpy()
    rows = []
    for _ in range(n):
        b = int(rng.integers(0, len(lq)))
        rows.append((b, int(rng.integers(0, lq[b]))))
    # always include the first and last row of one request
    rows += [(0, 0), (0, int(lq[0]) - 1)]
    return rows


def _rows_of(t, w, rows):
    cq = np.concatenate([[0], np.cumsum(w["seq_lens_q"].numpy())])
    idx = torch.tensor([int(cq[b] + r) for b, r in rows], device=t.device)
    return t.index_select(0, idx)


def test_full_size_bf16_gqa_sampled(pkv):
    w = workloads.batch_prefill(DEV)
    out, lse = run_prefill(pkv, w)
    rows = _sample_rows(w, 24, 0)
    ref_o, ref_l = oracle_prefill(w, rows=rows)
    assert_out_close(_rows_of(out, w, rows), ref_o, out.dtype)
    assert_lse_close(_rows_of(lse, w, rows), ref_l)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_full_size_fp8_d192_sampled(pkv):
    w = workloads.fp8_prefill(DEV)
    out, lse = run_prefill(pkv, w)
    rows = _sample_rows(w, 16, 1)
    ref_o, ref_l = oracle_prefill(w, rows=rows)
    assert_out_close(_rows_of(out, w, rows), ref_o, out.dtype)
    assert_lse_close(_rows_of(lse, w, rows), ref_l)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
