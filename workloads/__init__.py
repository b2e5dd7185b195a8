"""Seeded synthetic inputs for the paged-KV path.

Shared by the tests, the benchmark and the smoke check; it is the only code
that both the HIP path and the oracle see, and it holds none of the method's
arithmetic: it draws lengths, page permutations and values, and lays pages
out. The five workloads follow the shapes of FlashInfer's API pages (the
append page's Example, and prefill / decode shapes with the pages' parameter
names); ``scaled`` variants keep the structure at sizes a float64 oracle
finishes in seconds.

Lengths and page permutations come from a CPU ``torch.Generator`` seeded
with the workload's seed, so they are identical on every machine. Tensor
values come from a generator on the target device, seeded with the same
seed: the same device type gives the same bytes, and tests hand the oracle
the bytes that were actually used.
"""

import math

import torch

HND, NHD = "HND", "NHD"


def _gens(seed, device):
    host = torch.Generator(device="cpu").manual_seed(seed)
    dev = torch.Generator(device=device).manual_seed(seed)
    return host, dev


def _randn(shape, dev_gen, device, dtype):
    x = torch.randn(shape, generator=dev_gen, device=device, dtype=torch.float32)
    return x.to(dtype)


def _uniform_int(host, lo, hi, n):
    """n integers uniform on [lo, hi] inclusive."""
    return torch.randint(lo, hi + 1, (n,), generator=host)


def _page_tables(seq_lens, page_size, pool_pages, host):
    """Block tables over a randomly permuted pool: request b takes the next
    ceil(seq/page_size) ids of one permutation. Padding entries are -1."""
    n_pages = [math.ceil(int(s) / page_size) for s in seq_lens]
    total = sum(n_pages)
    if pool_pages is None:
        pool_pages = total
    if total > pool_pages:
        raise ValueError("pool too small")
    perm = torch.randperm(pool_pages, generator=host).to(torch.int32)
    width = max(max(n_pages), 1)
    bt = torch.full((len(n_pages), width), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(n_pages):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, pool_pages


def append_example(device="cpu", seed=1):
    """The append page's Example, then a causal fp16 prefill of the same 100
    tokens (NHD 5D cache [1000, 2, 16, 32, 128], lengths 45/8/25/22 in pages
    3/1/2/2 with indices 0..7 and last-page lengths 13/8/9/6). The query is a
    fresh randn draw after the rows and the pool."""
    _, dev = _gens(seed, device)
    nnz, hkv, d, ps, pages = 100, 32, 128, 16, 1000
    k_append = _randn((nnz, hkv, d), dev, device, torch.float16)
    v_append = _randn((nnz, hkv, d), dev, device, torch.float16)
    cache = _randn((pages, 2, ps, hkv, d), dev, device, torch.float16)
    q = _randn((nnz, 32, d), dev, device, torch.float16)
    lengths = torch.tensor([45, 8, 25, 22], dtype=torch.int32)
    pages_per_req = torch.tensor([3, 1, 2, 2], dtype=torch.int32)
    return dict(
        k_append=k_append, v_append=v_append, paged_kv_cache=cache, q=q,
        append_lengths=lengths,
        append_indptr=torch.cat([torch.zeros(1, dtype=torch.int32), lengths.cumsum(0)]).int(),
        kv_indptr=torch.cat([torch.zeros(1, dtype=torch.int32), pages_per_req.cumsum(0)]).int(),
        kv_indices=torch.arange(8, dtype=torch.int32),
        kv_last_page_len=torch.tensor([13, 8, 9, 6], dtype=torch.int32),
        page_size=ps, num_kv_heads=hkv, num_qo_heads=32, head_dim=d,
        scale=1.0 / math.sqrt(d), layout=NHD,
    )


def batch_prefill(device="cpu", seed=2, batch=16, q_len=(256, 2048), prefix=(0, 2048),
                  num_qo_heads=32, num_kv_heads=8, d_qk=128, d_vo=128, page_size=16,
                  pool_pages=65536, dtype=torch.bfloat16, layout=HND):
    """Ragged batch prefill over a paged cache (bf16, GQA 4:1, HND, page 16,
    pool of 65536 pages by default). L_q ~ U{q_len}, L_kv = L_q + U{prefix}."""
    host, dev = _gens(seed, device)
    lq = _uniform_int(host, q_len[0], q_len[1], batch).to(torch.int32)
    pre = _uniform_int(host, prefix[0], prefix[1], batch).to(torch.int32)
    lkv = (lq + pre).to(torch.int32)
    bt, pool = _page_tables(lkv.tolist(), page_size, pool_pages, host)
    q = _randn((int(lq.sum()), num_qo_heads, d_qk), dev, device, dtype)
    kshape = (pool, num_kv_heads, page_size, d_qk) if layout == HND else (pool, page_size, num_kv_heads, d_qk)
    vshape = kshape[:-1] + (d_vo,)
    k_cache = _randn(kshape, dev, device, dtype)
    v_cache = _randn(vshape, dev, device, dtype)
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=bt,
                seq_lens_q=lq, seq_lens_kv=lkv, page_size=page_size,
                num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                d_qk=d_qk, d_vo=d_vo, scale=1.0 / math.sqrt(d_qk), layout=layout,
                q_scale=None, k_scale=None, v_scale=None, causal=True)


def fp8_prefill(device="cpu", seed=3, batch=8, seq_len=4096, num_heads=16, d_qk=192,
                d_vo=128, page_size=64):
    """fp8 e4m3 prefill with d_qk 192 / d_vo 128: L_q = L_kv = seq_len, H 16/16,
    page 64, per-tensor fp32 scales ~ U[0.5, 2], values N(0,1) -> e4m3."""
    host, dev = _gens(seed, device)
    lq = torch.full((batch,), seq_len, dtype=torch.int32)
    bt, pool = _page_tables(lq.tolist(), page_size, None, host)
    scales = (torch.rand(3, generator=host) * 1.5 + 0.5).to(torch.float32)
    e4 = torch.float8_e4m3fn
    q = _randn((batch * seq_len, num_heads, d_qk), dev, device, e4)
    k_cache = _randn((pool, num_heads, page_size, d_qk), dev, device, e4)
    v_cache = _randn((pool, num_heads, page_size, d_vo), dev, device, e4)
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=bt,
                seq_lens_q=lq, seq_lens_kv=lq.clone(), page_size=page_size,
                num_qo_heads=num_heads, num_kv_heads=num_heads, d_qk=d_qk, d_vo=d_vo,
                scale=1.0 / math.sqrt(d_qk), layout=HND,
                q_scale=scales[0:1], k_scale=scales[1:2], v_scale=scales[2:3], causal=True)


def batch_decode(device="cpu", seed=4, batch=256, seq=(512, 8192), num_qo_heads=32,
                 num_kv_heads=8, head_dim=128, page_size=16, q_len_per_req=1,
                 kv_dtype=torch.bfloat16, layout=HND, window_left=-1, sinks=False,
                 q_dtype=torch.bfloat16):
    """Batch decode over block_tables: seq_lens uint32 ~ U{seq}, HND page 16,
    random page order, bf16 K/V and query ~ N(0,1), bmm1 = 1/sqrt(128),
    bmm2 = 1, window -1, one query per request. ``q_dtype`` (bf16 or fp16)
    is the query's type; a 16-bit ``kv_dtype`` must match it."""
    host, dev = _gens(seed, device)
    sl = _uniform_int(host, seq[0], seq[1], batch).to(torch.int64)
    bt, pool = _page_tables(sl.tolist(), page_size, None, host)
    shape = (pool, 2, num_kv_heads, page_size, head_dim) if layout == HND \
        else (pool, 2, page_size, num_kv_heads, head_dim)
    kv = _randn(shape, dev, device, kv_dtype)
    q = _randn((batch * q_len_per_req, num_qo_heads, head_dim), dev, device, q_dtype)
    sk = None
    if sinks:
        sk = torch.randn(num_qo_heads, generator=host).to(torch.float32)
    return dict(query=q, kv_cache=kv, block_tables=bt, seq_lens=sl.to(torch.uint32),
                max_seq_len=int(sl.max()), page_size=page_size, num_qo_heads=num_qo_heads,
                num_kv_heads=num_kv_heads, head_dim=head_dim, q_len_per_req=q_len_per_req,
                bmm1_scale=1.0 / math.sqrt(head_dim), bmm2_scale=1.0,
                window_left=window_left, sinks=sk, layout=layout)


def spec_decode(device="cpu", seed=5, batch=64, seq=(4096, 32768), num_qo_heads=64,
                num_kv_heads=8, head_dim=128, page_size=32, q_len_per_req=4,
                window_left=4095):
    """Append 4 draft K/V rows per request into an fp8 e4m3 HND cache (page
    32), then decode 4 queries per request causally with window_left 4095,
    per-head fp32 sinks ~ N(0,1) and per-tensor k/v scales ~ U[0.5, 2] folded
    into bmm1 / bmm2. seq_lens ~ U{seq} are the lengths after the append."""
    host, dev = _gens(seed, device)
    sl = _uniform_int(host, seq[0], seq[1], batch).to(torch.int64)
    bt, pool = _page_tables(sl.tolist(), page_size, None, host)
    n_pages = [(int(s) + page_size - 1) // page_size for s in sl]
    kv_indptr = torch.zeros(batch + 1, dtype=torch.int32)
    kv_indptr[1:] = torch.tensor(n_pages, dtype=torch.int32).cumsum(0)
    kv_indices = torch.cat([bt[b, :n_pages[b]] for b in range(batch)])
    last = ((sl - 1) % page_size + 1).to(torch.int32)
    scales = (torch.rand(2, generator=host) * 1.5 + 0.5).to(torch.float32)
    sinks = torch.randn(num_qo_heads, generator=host).to(torch.float32)
    e4 = torch.float8_e4m3fn
    kv = _randn((pool, 2, num_kv_heads, page_size, head_dim), dev, device, e4)
    nnz = batch * q_len_per_req
    k_append = _randn((nnz, num_kv_heads, head_dim), dev, device, e4)
    v_append = _randn((nnz, num_kv_heads, head_dim), dev, device, e4)
    q = _randn((nnz, num_qo_heads, head_dim), dev, device, torch.bfloat16)
    ks, vs = float(scales[0]), float(scales[1])
    return dict(query=q, kv_cache=kv, block_tables=bt, seq_lens=sl.to(torch.uint32),
                max_seq_len=int(sl.max()), page_size=page_size, num_qo_heads=num_qo_heads,
                num_kv_heads=num_kv_heads, head_dim=head_dim, q_len_per_req=q_len_per_req,
                k_append=k_append, v_append=v_append,
                append_indptr=(torch.arange(batch + 1, dtype=torch.int32) * q_len_per_req),
                kv_indptr=kv_indptr, kv_indices=kv_indices, kv_last_page_len=last,
                k_scale=ks, v_scale=vs, bmm1_scale=ks / math.sqrt(head_dim), bmm2_scale=vs,
                window_left=window_left, sinks=sinks, layout=HND)


def bulk_append(device="cpu", seed=6, batch=256, seq=(4096, 8192), rows=1024,
                num_kv_heads=8, head_dim=128, page_size=32,
                kv_dtype=torch.float8_e4m3fn, layout=HND):
    """A bandwidth-sized append (beyond the pages' examples, which are
    launch-bound): ``rows`` new K/V rows per request (a chunk of prefill)
    written at the end of each sequence (seq_lens ~ U{seq} are the lengths
    after the append), into a cache of exactly the pages the requests own, in
    random order, with the same layout as the speculative-decode workload.
    At the defaults 512 MiB is read and 512 MiB written, well beyond the
    chip's 256 MB last-level cache."""
    host, dev = _gens(seed, device)
    sl = _uniform_int(host, seq[0], seq[1], batch).to(torch.int64)
    bt, pool = _page_tables(sl.tolist(), page_size, None, host)
    n_pages = [(int(s) + page_size - 1) // page_size for s in sl]
    kv_indptr = torch.zeros(batch + 1, dtype=torch.int32)
    kv_indptr[1:] = torch.tensor(n_pages, dtype=torch.int32).cumsum(0)
    kv_indices = torch.cat([bt[b, :n_pages[b]] for b in range(batch)])
    last = ((sl - 1) % page_size + 1).to(torch.int32)
    shape = (pool, 2, num_kv_heads, page_size, head_dim) if layout == HND \
        else (pool, 2, page_size, num_kv_heads, head_dim)
    kv = _randn(shape, dev, device, kv_dtype)
    nnz = batch * rows
    k_append = _randn((nnz, num_kv_heads, head_dim), dev, device, kv_dtype)
    v_append = _randn((nnz, num_kv_heads, head_dim), dev, device, kv_dtype)
    return dict(kv_cache=kv, k_append=k_append, v_append=v_append, seq_lens=sl.to(torch.int32),
                append_indptr=(torch.arange(batch + 1, dtype=torch.int32) * rows),
                kv_indptr=kv_indptr, kv_indices=kv_indices, kv_last_page_len=last,
                block_tables=bt, page_size=page_size, num_kv_heads=num_kv_heads,
                head_dim=head_dim, layout=layout)


def append_sweep(device="cpu", nnz=4096, seed=1, num_kv_heads=32, head_dim=128, page_size=16,
                 dtype=torch.float16):
    """The append Example's shape family (fp16, 32 kv heads, d 128, NHD page
    16) at ``nnz`` rows, for a bandwidth sweep: max(4, nnz / 1024) requests
    each append their whole sequence (nnz split evenly, the remainder on the
    last), into a pool of exactly the pages they own, in random order.
    Values are filled in chunks so that no float32 copy of a large tensor is
    ever held."""
    host, dev = _gens(seed, device)
    batch = max(4, nnz // 1024)
    lens = torch.full((batch,), nnz // batch, dtype=torch.int64)
    lens[-1] += nnz - int(lens.sum())
    bt, pool = _page_tables(lens.tolist(), page_size, None, host)
    n_pages = [(int(s) + page_size - 1) // page_size for s in lens]
    kv_indptr = torch.zeros(batch + 1, dtype=torch.int32)
    kv_indptr[1:] = torch.tensor(n_pages, dtype=torch.int32).cumsum(0)
    kv_indices = torch.cat([bt[b, :n_pages[b]] for b in range(batch)])
    last = ((lens - 1) % page_size + 1).to(torch.int32)

    def filled(shape):
        t = torch.empty(shape, dtype=dtype, device=device)
        flat = t.view(-1)
        step = 1 << 26
        for i in range(0, flat.numel(), step):
            n = min(step, flat.numel() - i)
            flat[i:i + n] = torch.randn(n, generator=dev, device=device).to(dtype)
        return t

    kv = filled((pool, 2, page_size, num_kv_heads, head_dim))
    k_append = filled((nnz, num_kv_heads, head_dim))
    v_append = filled((nnz, num_kv_heads, head_dim))
    ai = torch.zeros(batch + 1, dtype=torch.int32)
    ai[1:] = lens.to(torch.int32).cumsum(0)
    return dict(kv_cache=kv, k_append=k_append, v_append=v_append,
                seq_lens=lens.to(torch.int32), append_indptr=ai, kv_indptr=kv_indptr,
                kv_indices=kv_indices, kv_last_page_len=last, page_size=page_size,
                num_kv_heads=num_kv_heads, head_dim=head_dim, layout=NHD)


def compact_pages(cache, block_tables, n_pages_used, page_axis=0):
    """Host copy of just the pages a batch uses, and block tables renumbered
    into it (so an oracle need not hold a multi-GB pool). ``cache`` is any
    tensor whose dim ``page_axis`` is the page index."""
    used = []
    for b in range(block_tables.shape[0]):
        used.extend(int(x) for x in block_tables[b, :n_pages_used[b]])
    uniq = sorted(set(used))
    remap = {p: i for i, p in enumerate(uniq)}
    idx = torch.tensor(uniq, dtype=torch.long, device=cache.device)
    sub = cache.index_select(page_axis, idx).cpu()
    bt = torch.full_like(block_tables, -1)
    for b in range(block_tables.shape[0]):
        for k in range(n_pages_used[b]):
            bt[b, k] = remap[int(block_tables[b, k])]
    return sub, bt
