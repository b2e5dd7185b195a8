"""Pins for the oracle's index math, append and gather (CPU only).

Sources: flashinfer.page.append_paged_kv_cache -- Example (printed
batch_indices / positions, and the comments 45 = (3-1)*16+13 etc.), Parameters
and Note; the block_tables parameter of the prefill and decode pages.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle.paging import NHD, HND
from tests.conftest import GOLDEN


def _golden():
    with open(os.path.join(GOLDEN, "append_example.json")) as f:
        return json.load(f)


def test_seq_lens_match_page_comments():
    g = _golden()
    indptr = np.concatenate([[0], np.cumsum(g["num_pages_per_req"])])
    seq = oracle.get_seq_lens(indptr, g["kv_last_page_len"], g["page_size"])
    assert seq.tolist() == g["seq_lens_from_comments"]
    assert indptr.tolist() == [0, 3, 4, 6, 8]


def test_batch_indices_positions_match_printed_example():
    g = _golden()
    indptr = np.concatenate([[0], np.cumsum(g["num_pages_per_req"])])
    seq = oracle.get_seq_lens(indptr, g["kv_last_page_len"], g["page_size"])
    bi, pos = oracle.get_batch_indices_positions(g["kv_append_indptr"], seq, g["nnz_kv"])
    assert bi.tolist() == g["batch_indices"]
    assert pos.tolist() == g["positions"]


def test_positions_are_the_last_positions_of_the_sequence():
    # Note of the append page: the page table already includes the appended
    # rows, so 4 rows appended to a 100-token sequence are positions 96..99.
    bi, pos = oracle.get_batch_indices_positions([0, 4, 5], [100, 1], 5)
    assert bi.tolist() == [0, 0, 0, 0, 1]
    assert pos.tolist() == [96, 97, 98, 99, 0]


def test_csr_to_block_tables_hand_example():
    bt = oracle.csr_to_block_tables([0, 3, 4, 6], [7, 2, 9, 5, 1, 0], 4)
    assert bt.tolist() == [[7, 2, 9, -1], [5, -1, -1, -1], [1, 0, -1, -1]]


def _example_cache(layout, rng, pages=1000):
    g = _golden()
    H, D, ps = g["num_kv_heads"], g["head_dim"], g["page_size"]
    shape = (pages, ps, H, D) if layout == NHD else (pages, H, ps, D)
    return rng.integers(0, 2 ** 16, size=(pages, 2) + shape[1:], dtype=np.uint16)


@pytest.mark.parametrize("layout", [NHD, HND])
def test_append_example_writes_rows_and_nothing_else(layout):
    g = _golden()
    rng = np.random.default_rng(0)
    H, D, ps = g["num_kv_heads"], g["head_dim"], g["page_size"]
    cache = _example_cache(layout, rng, pages=64)
    before = cache.copy()
    k_app = rng.integers(0, 2 ** 16, size=(100, H, D), dtype=np.uint16)
    v_app = rng.integers(0, 2 ** 16, size=(100, H, D), dtype=np.uint16)
    indptr = np.concatenate([[0], np.cumsum(g["num_pages_per_req"])])
    oracle.append_paged_kv_cache(k_app, v_app, g["batch_indices"], g["positions"],
                                 cache[:, 0], cache[:, 1], g["kv_page_indices"],
                                 indptr, g["kv_last_page_len"], layout)
    seq = g["seq_lens_from_comments"]
    ai = g["kv_append_indptr"]
    bt = oracle.csr_to_block_tables(indptr, g["kv_page_indices"], 3)
    touched = np.zeros(cache.shape, dtype=bool)
    for b in range(4):
        # seq_len == append length here, so the gathered request is its rows
        kb = oracle.gather_pages(cache[:, 0], bt[b], seq[b], layout)
        vb = oracle.gather_pages(cache[:, 1], bt[b], seq[b], layout)
        assert np.array_equal(kb, k_app[ai[b]:ai[b + 1]])
        assert np.array_equal(vb, v_app[ai[b]:ai[b + 1]])
        for p in range(seq[b]):
            page = bt[b][p // ps]
            if layout == NHD:
                touched[page, :, p % ps] = True
            else:
                touched[page, :, :, p % ps] = True
    assert np.array_equal(cache[~touched], before[~touched])
    # the last page of request 0 keeps its slots 13..15
    assert np.array_equal(cache[2, :, 13:] if layout == NHD else cache[2, :, :, 13:],
                          before[2, :, 13:] if layout == NHD else before[2, :, :, 13:])


def test_append_onto_existing_prefix_keeps_prefix():
    rng = np.random.default_rng(1)
    ps, H, D = 32, 2, 16
    cache = rng.integers(0, 256, size=(20, 2, H, ps, D), dtype=np.uint8)
    before = cache.copy()
    seq = np.array([70, 33])          # final lengths, 4 new rows each
    pages = [[5, 11, 2], [19, 0]]
    indptr = [0, 3, 5]
    indices = pages[0] + pages[1]
    last = [(s - 1) % ps + 1 for s in seq]
    assert oracle.get_seq_lens(indptr, last, ps).tolist() == seq.tolist()
    bi, pos = oracle.get_batch_indices_positions([0, 4, 8], seq, 8)
    k_app = rng.integers(0, 256, size=(8, H, D), dtype=np.uint8)
    v_app = rng.integers(0, 256, size=(8, H, D), dtype=np.uint8)
    oracle.append_paged_kv_cache(k_app, v_app, bi, pos, cache[:, 0], cache[:, 1],
                                 indices, indptr, last, HND)
    for b in range(2):
        kb = oracle.gather_pages(cache[:, 0], pages[b], seq[b], HND)
        kb0 = oracle.gather_pages(before[:, 0], pages[b], seq[b], HND)
        assert np.array_equal(kb[-4:], k_app[4 * b:4 * b + 4])
        assert np.array_equal(kb[:-4], kb0[:-4])
        vb = oracle.gather_pages(cache[:, 1], pages[b], seq[b], HND)
        assert np.array_equal(vb[-4:], v_app[4 * b:4 * b + 4])


def test_append_rejects_position_outside_allocation():
    cache = np.zeros((4, 2, 16, 1, 8), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.append_paged_kv_cache(np.zeros((1, 1, 8), np.uint16), np.zeros((1, 1, 8), np.uint16),
                                     [0], [5], cache[:, 0], cache[:, 1], [0], [0, 1], [5], NHD)


@pytest.mark.parametrize("layout", [NHD, HND])
@pytest.mark.parametrize("ps", [1, 3, 16])
def test_gather_of_random_pages_equals_contiguous(layout, ps):
    rng = np.random.default_rng(ps)
    H, D, L = 3, 8, 37
    seq = rng.integers(0, 2 ** 16, size=(L, H, D), dtype=np.uint16)
    n_pages = -(-L // ps)
    pool = 2 * n_pages + 3
    perm = rng.permutation(pool)[:n_pages]
    cache = rng.integers(0, 2 ** 16, size=(pool, ps, H, D) if layout == NHD else (pool, H, ps, D),
                         dtype=np.uint16)
    # place token j by hand at page perm[j // ps], slot j % ps
    for j in range(L):
        if layout == NHD:
            cache[perm[j // ps], j % ps] = seq[j]
        else:
            cache[perm[j // ps], :, j % ps] = seq[j]
    assert np.array_equal(oracle.gather_pages(cache, perm, L, layout), seq)
