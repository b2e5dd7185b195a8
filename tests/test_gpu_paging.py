"""GPU parity of the index math and the append scatter (bit-exact).

The oracle and the HIP path receive the same seeded inputs; index arrays and
the whole post-append cache (every byte, touched or not) must be identical.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.conftest import GOLDEN
from tests.helpers import bits

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def pkv():
    import attention_paged_kv_cache_amd as m
    return m


def _golden():
    with open(os.path.join(GOLDEN, "append_example.json")) as f:
        return json.load(f)


def test_index_math_matches_printed_example(pkv):
    g = _golden()
    indptr = torch.tensor([0, 3, 4, 6, 8], dtype=torch.int32, device=DEV)
    last = torch.tensor(g["kv_last_page_len"], dtype=torch.int32, device=DEV)
    seq = pkv.get_seq_lens(indptr, last, g["page_size"])
    assert seq.cpu().tolist() == g["seq_lens_from_comments"]
    ai = torch.tensor(g["kv_append_indptr"], dtype=torch.int32, device=DEV)
    bi, pos = pkv.get_batch_indices_positions(ai, seq, g["nnz_kv"])
    torch.cuda.synchronize()
    assert bi.cpu().tolist() == g["batch_indices"]
    assert pos.cpu().tolist() == g["positions"]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_index_math_random_equals_oracle(pkv, seed):
    rng = np.random.default_rng(seed)
    B, ps = int(rng.integers(1, 40)), int(rng.choice([16, 32, 64]))
    pages = rng.integers(0, 9, size=B)
    indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    last = np.where(pages > 0, rng.integers(1, ps + 1, size=B), 0).astype(np.int32)
    seq_ref = oracle.get_seq_lens(indptr, last, ps)
    seq = pkv.get_seq_lens(torch.tensor(indptr, device=DEV), torch.tensor(last, device=DEV), ps)
    assert seq.cpu().numpy().tolist() == seq_ref.tolist()
    n_app = np.minimum(rng.integers(0, 6, size=B), seq_ref)
    ai = np.concatenate([[0], np.cumsum(n_app)]).astype(np.int32)
    nnz = int(ai[-1])
    bi_ref, pos_ref = oracle.get_batch_indices_positions(ai, seq_ref, nnz)
    bi, pos = pkv.get_batch_indices_positions(torch.tensor(ai, device=DEV), seq, nnz)
    assert bi.cpu().numpy().tolist() == bi_ref.tolist()
    assert pos.cpu().numpy().tolist() == pos_ref.tolist()
    indices = rng.permutation(int(indptr[-1]) + 3)[: int(indptr[-1])].astype(np.int32)
    width = int(max(pages.max(), 1))
    bt = pkv.csr_to_block_tables(torch.tensor(indptr, device=DEV), torch.tensor(indices, device=DEV), width)
    assert np.array_equal(bt.cpu().numpy(), oracle.csr_to_block_tables(indptr, indices, width))


def test_append_example_bit_exact(pkv):
    w = workloads.append_example(DEV)
    cache = w["paged_kv_cache"]
    before = bits(cache)
    seq = pkv.get_seq_lens(w["kv_indptr"].to(DEV), w["kv_last_page_len"].to(DEV), w["page_size"])
    bi, pos = pkv.get_batch_indices_positions(w["append_indptr"].to(DEV), seq, 100)
    pkv.append_paged_kv_cache(w["k_append"], w["v_append"], bi, pos, cache,
                              w["kv_indices"].to(DEV), w["kv_indptr"].to(DEV),
                              w["kv_last_page_len"].to(DEV), kv_layout="NHD")
    torch.cuda.synchronize()
    ref = before.copy()
    oracle.append_paged_kv_cache(bits(w["k_append"]), bits(w["v_append"]), bi.cpu().numpy(),
                                 pos.cpu().numpy(), ref[:, 0], ref[:, 1],
                                 w["kv_indices"].numpy(), w["kv_indptr"].numpy(),
                                 w["kv_last_page_len"].numpy(), "NHD")
    got = bits(cache)
    assert np.array_equal(got, ref)
    assert not np.array_equal(got, before)


def test_streaming_append_bitwise(pkv):
    # an append whose rows reach the 256 MiB from which the kernel uses
    # non-temporal loads and stores (131072 e4m3 rows of 8 heads x 128 for
    # K and V, into 64 requests' random pages): the whole cache, touched and
    # untouched bytes, equals the oracle's bit for bit
    w = workloads.bulk_append(DEV, seed=61, batch=64, seq=(4096, 8192), rows=2048)
    nnz = w["k_append"].shape[0]
    assert 2 * w["k_append"].numel() * w["k_append"].element_size() >= 256 << 20
    kv = w["kv_cache"]
    before = bits(kv)
    bi, pos = pkv.get_batch_indices_positions(w["append_indptr"].to(DEV),
                                              w["seq_lens"].to(DEV), nnz)
    pkv.append_paged_kv_cache(w["k_append"], w["v_append"], bi, pos, kv,
                              w["kv_indices"].to(DEV), w["kv_indptr"].to(DEV),
                              w["kv_last_page_len"].to(DEV), kv_layout="HND")
    torch.cuda.synchronize()
    ref = before.copy()
    oracle.append_paged_kv_cache(bits(w["k_append"]), bits(w["v_append"]), bi.cpu().numpy(),
                                 pos.cpu().numpy(), ref[:, 0], ref[:, 1],
                                 w["kv_indices"].numpy(), w["kv_indptr"].numpy(),
                                 w["kv_last_page_len"].numpy(), "HND")
    got = bits(kv)
    assert np.array_equal(got, ref)
    assert not np.array_equal(got, before)


@pytest.mark.parametrize("layout,dtype,ps,tuple_form,B,H,D,seq_lo,seq_hi,app_hi", [
    ("HND", torch.bfloat16, 16, False, 5, 3, 128, 1, 200, 40),
    ("NHD", torch.float16, 32, True, 5, 3, 128, 1, 200, 40),
    ("HND", torch.float8_e4m3fn, 32, False, 5, 3, 128, 1, 200, 40),
    ("NHD", torch.float8_e4m3fn, 64, True, 5, 3, 128, 1, 200, 40),
    # more than 8192 rows: several rows per wave, a ragged last wave
    ("HND", torch.bfloat16, 16, False, 64, 2, 128, 200, 2000, 1000),
    # 24-chunk heads (head_dim 192 e4m3), 36 chunks a row
    ("HND", torch.float8_e4m3fn, 64, False, 40, 3, 192, 500, 1500, 1500),
    # ~900k rows of 128 bytes: 64 rows per wave, several unrolled passes
    ("NHD", torch.float16, 16, True, 400, 1, 64, 1500, 3000, 10 ** 6),
])
def test_append_random_equals_oracle(pkv, layout, dtype, ps, tuple_form, B, H, D, seq_lo,
                                     seq_hi, app_hi):
    rng = np.random.default_rng(ps + B)
    seq = rng.integers(seq_lo, seq_hi, size=B)
    npg = (seq + ps - 1) // ps
    pool = int(npg.sum()) + 7
    perm = rng.permutation(pool).astype(np.int32)
    indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    indices = perm[: indptr[-1]]
    last = ((seq - 1) % ps + 1).astype(np.int32)
    n_app = np.minimum(rng.integers(0, app_hi, size=B), seq)
    ai = np.concatenate([[0], np.cumsum(n_app)]).astype(np.int32)
    nnz = int(ai[-1])
    print(f"nnz {nnz}", flush=True)
    bi, pos = oracle.get_batch_indices_positions(ai, seq, nnz)
    page_shape = (ps, H, D) if layout == "NHD" else (H, ps, D)
    gen = torch.Generator(device=DEV).manual_seed(ps + B)
    mk = lambda *s: torch.randn(*s, generator=gen, device=DEV).to(dtype)
    if tuple_form:
        cache = (mk(pool, *page_shape), mk(pool, *page_shape))
        before_k, before_v = bits(cache[0]), bits(cache[1])
    else:
        cache = mk(pool, 2, *page_shape)
        b5 = bits(cache)
        before_k, before_v = b5[:, 0].copy(), b5[:, 1].copy()
    ka, va = mk(nnz, H, D), mk(nnz, H, D)
    t = lambda x: torch.tensor(x, device=DEV)
    pkv.append_paged_kv_cache(ka, va, t(bi), t(pos), cache, t(indices), t(indptr), t(last),
                              kv_layout=layout)
    torch.cuda.synchronize()
    oracle.append_paged_kv_cache(bits(ka), bits(va), bi, pos, before_k, before_v, indices,
                                 indptr, last, layout)
    if tuple_form:
        got_k, got_v = bits(cache[0]), bits(cache[1])
    else:
        b5 = bits(cache)
        got_k, got_v = b5[:, 0], b5[:, 1]
    assert np.array_equal(got_k, before_k)
    assert np.array_equal(got_v, before_v)


def test_append_empty_is_noop(pkv):
    cache = torch.zeros(4, 2, 16, 2, 128, dtype=torch.bfloat16, device=DEV)
    z = torch.zeros(0, 2, 128, dtype=torch.bfloat16, device=DEV)
    e = torch.zeros(0, dtype=torch.int32, device=DEV)
    pkv.append_paged_kv_cache(z, z, e, e, cache, torch.zeros(1, dtype=torch.int32, device=DEV),
                              torch.tensor([0, 1], dtype=torch.int32, device=DEV),
                              torch.tensor([1], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert int(cache.float().abs().sum()) == 0


def test_bulk_append_full_size_sampled(pkv):
    # the benchmark's bulk append (262144 e4m3 rows, HND page 32): every page
    # of a sample of requests, touched slots and untouched ones, bit-exact
    w = workloads.bulk_append(DEV)
    kv = w["kv_cache"]
    reqs = [0, 1, 77, 128, 255]
    bt = w["block_tables"][reqs]
    seq = w["seq_lens"][reqs]
    ps = w["page_size"]
    rows = int(w["append_indptr"][1])
    n_pages = [(int(s) + ps - 1) // ps for s in seq]
    before, bt_c = workloads.compact_pages(kv, bt, n_pages)
    before = bits(before)
    seq_d = w["seq_lens"].to(DEV)
    nnz = w["k_append"].shape[0]
    bi, pos = pkv.get_batch_indices_positions(w["append_indptr"].to(DEV), seq_d, nnz)
    pkv.append_paged_kv_cache(w["k_append"], w["v_append"], bi, pos, kv,
                              w["kv_indices"].to(DEV), w["kv_indptr"].to(DEV),
                              w["kv_last_page_len"].to(DEV), kv_layout="HND")
    torch.cuda.synchronize()
    got, _ = workloads.compact_pages(kv, bt, n_pages)
    got = bits(got)
    indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
    indices = np.concatenate([bt_c[i, :n_pages[i]].numpy() for i in range(len(reqs))])
    last = ((seq.numpy() - 1) % ps + 1).astype(np.int32)
    ai = np.arange(len(reqs) + 1, dtype=np.int32) * rows
    bi_r, pos_r = oracle.get_batch_indices_positions(ai, seq.numpy(), rows * len(reqs))
    src = np.concatenate([np.arange(b * rows, (b + 1) * rows) for b in reqs])
    idx = torch.tensor(src, device=DEV)
    ref = before.copy()
    oracle.append_paged_kv_cache(bits(w["k_append"].index_select(0, idx)),
                                 bits(w["v_append"].index_select(0, idx)), bi_r, pos_r,
                                 ref[:, 0], ref[:, 1], indices, indptr, last, "HND")
    assert np.array_equal(got, ref)
    assert not np.array_equal(got, before)
    # the device's batch indices and positions are the oracle's for the sample
    bi_all, pos_all = bi.cpu().numpy(), pos.cpu().numpy()
    assert np.array_equal(pos_all[src], pos_r)
    assert np.array_equal(bi_all[src], np.repeat(reqs, rows))
