"""Page-table index math, append and page gather, on raw bits.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: ``flashinfer.page.append_paged_kv_cache`` (Parameters, Example, Note),
and the ``block_tables`` parameter of the prefill and decode pages.

Cache conventions (append page, Parameters, ``paged_kv_cache``):
  NHD  k_cache/v_cache  [max_num_pages, page_size, num_kv_heads, head_dim]
  HND  k_cache/v_cache  [max_num_pages, num_kv_heads, page_size, head_dim]
The single 5D form ``[max_num_pages, 2, ...]`` is the pair
``(cache[:, 0], cache[:, 1])``; callers pass those two views.

All cache and row arrays here are numpy integer arrays holding raw element
bits, so that append and gather are exact copies.
"""

import numpy as np

NHD, HND = "NHD", "HND"


def get_seq_lens(kv_indptr, kv_last_page_len, page_size):
    """Tokens held by each request's pages.

    Append page, Example: the comments there give each length as
    (pages - 1) * page_size + entries in the last page, e.g. 45 = (3-1)*16+13.
    """
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    batch = len(last)
    out = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        pages = kv_indptr[b + 1] - kv_indptr[b]
        out[b] = (pages - 1) * page_size + last[b] if pages > 0 else 0
    return out


def get_batch_indices_positions(append_indptr, seq_lens, nnz):
    """Request index and absolute position of every appended row.

    Append page, Example and Note: the rows of request b are
    ``append_indptr[b] .. append_indptr[b+1]-1`` and the page table already
    covers them, so they are the last n_b positions of a sequence of
    ``seq_lens[b]`` tokens: row k of request b sits at seq_len - n_b + k.
    """
    ai = np.asarray(append_indptr, dtype=np.int64)
    seq = np.asarray(seq_lens, dtype=np.int64)
    batch_indices = np.full(nnz, -1, dtype=np.int32)
    positions = np.full(nnz, -1, dtype=np.int32)
    for b in range(len(seq)):
        n_b = ai[b + 1] - ai[b]
        for k in range(n_b):
            i = ai[b] + k
            if i < nnz:
                batch_indices[i] = b
                positions[i] = seq[b] - n_b + k
    return batch_indices, positions


def csr_to_block_tables(kv_indptr, kv_indices, max_pages_per_seq):
    """CSR page list -> dense ``block_tables[b, k]`` (padding = -1).

    The append page stores pages as kv_indptr/kv_indices; the prefill and
    decode pages take a ``block_tables`` [batch, pages_per_seq]. Entry k of
    request b is the same page in both forms. Unused entries are -1.
    """
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    batch = len(kv_indptr) - 1
    bt = np.full((batch, max_pages_per_seq), -1, dtype=np.int32)
    for b in range(batch):
        for k in range(kv_indptr[b + 1] - kv_indptr[b]):
            if k < max_pages_per_seq:
                bt[b, k] = kv_indices[kv_indptr[b] + k]
    return bt


def _slot_view(cache, page, slot, layout):
    """Index expression selecting all heads of one token in a page."""
    if layout == NHD:
        return (page, slot)                      # -> [H, D]
    if layout == HND:
        return (page, slice(None), slot)         # -> [H, D]
    raise ValueError(f"unknown layout {layout!r}")


def append_paged_kv_cache(append_key, append_value, batch_indices, positions,
                          k_cache, v_cache, kv_indices, kv_indptr,
                          kv_last_page_len, kv_layout=NHD):
    """Scatter appended K/V rows into their pages, in place.

    Append page, Parameters and Note: row i of ``append_key``/``append_value``
    ([nnz, num_kv_heads, head_dim]) belongs to request ``batch_indices[i]`` at
    position ``positions[i]``. Position p lives in the request's page number
    p // page_size (looked up through kv_indptr/kv_indices) at slot
    p % page_size. Nothing else in the cache is touched.
    """
    page_size = k_cache.shape[1] if kv_layout == NHD else k_cache.shape[2]
    seq = get_seq_lens(kv_indptr, kv_last_page_len, page_size)
    for i in range(len(batch_indices)):
        b = int(batch_indices[i])
        p = int(positions[i])
        if not (0 <= p < seq[b]):
            raise ValueError(f"row {i}: position {p} outside request {b}'s "
                             f"{seq[b]} allocated tokens")
        page = int(kv_indices[int(kv_indptr[b]) + p // page_size])
        where = _slot_view(k_cache, page, p % page_size, kv_layout)
        k_cache[where] = append_key[i]
        v_cache[where] = append_value[i]


def gather_pages(cache, block_table_row, seq_len, kv_layout):
    """Contiguous [seq_len, num_kv_heads, head_dim] copy of one request.

    Token j of the request is slot j % page_size of page
    ``block_table_row[j // page_size]`` (the ``block_tables`` parameter of the
    prefill and decode pages; the cache shapes of the decode page). Copied one
    page at a time; slots past ``seq_len`` in the last page are not read.
    """
    if kv_layout == NHD:
        page_size, heads, dim = cache.shape[1], cache.shape[2], cache.shape[3]
    elif kv_layout == HND:
        page_size, heads, dim = cache.shape[2], cache.shape[1], cache.shape[3]
    else:
        raise ValueError(f"unknown layout {kv_layout!r}")
    out = np.empty((seq_len, heads, dim), dtype=cache.dtype)
    for k in range((seq_len + page_size - 1) // page_size):
        page = int(block_table_row[k])
        n = min(page_size, seq_len - k * page_size)
        if kv_layout == NHD:
            out[k * page_size:k * page_size + n] = cache[page, :n]
        else:
            out[k * page_size:k * page_size + n] = cache[page, :, :n].transpose(1, 0, 2)
    return out
