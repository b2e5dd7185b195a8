"""Paged-KV attention for AMD MI355X: thin Python binding of libpkv.so.

The functions keep the names and argument order of FlashInfer's API pages
(flashinfer.page.append_paged_kv_cache with get_seq_lens /
get_batch_indices_positions from its Example;
flashinfer.prefill.cudnn_batch_prefill_with_kv_cache;
flashinfer.decode.trtllm_batch_decode_with_kv_cache). They only marshal
arguments -- shapes, strides, dtypes, the current HIP stream -- and call the C
ABI declared in include/pkv.h; every step of the computation runs in the HIP
kernels. torch supplies device memory and streams.

If libpkv.so is not built, every call raises: there is no fallback path.
"""

import torch

from . import _lib
from ._lib import NHD, HND, F16, BF16, E4M3, PkvError

__all__ = [
    "get_seq_lens",
    "get_batch_indices_positions",
    "csr_to_block_tables",
    "append_paged_kv_cache",
    "batch_prefill_with_kv_cache",
    "batch_decode_with_kv_cache",
    "batch_decode_with_kv_cache_no_alloc",
    "prefill_workspace_size",
    "decode_workspace_size",
    "PkvError",
]

_DTYPES = {torch.float16: F16, torch.bfloat16: BF16, torch.float8_e4m3fn: E4M3}
_LAYOUTS = {"NHD": NHD, "HND": HND}


def _dt(t):
    return _dtc(t.dtype)


def _dtc(dtype):
    try:
        return _DTYPES[dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {dtype}") from None


def _layout(name):
    try:
        return _LAYOUTS[name]
    except KeyError:
        raise ValueError(f"kv_layout must be 'NHD' or 'HND', got {name!r}") from None


def _stream(device):
    """Raw handle of the current HIP stream of ``device`` (what the library
    enqueues on)."""
    return torch._C._cuda_getCurrentRawStream(device.index)


def _call(device, fn, *args):
    """Call ``fn(*args)`` with ``device`` current (a launch on the null stream
    goes to the current device); skips the device switch when it already is."""
    if torch._C._cuda_getDevice() == device.index:
        return fn(*args)
    with torch.cuda.device(device):
        return fn(*args)


def _on_gpu(device, **tensors):
    """Raise unless ``device`` is a GPU and every given tensor lives on it:
    the library reads its pointer arguments as device memory."""
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {device}")
    idx = device.index
    for name, t in tensors.items():
        if t is not None and t.get_device() != idx:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _i32_on(t, device):
    """int32 contiguous device copy of a length / index tensor; the tensor
    itself when it already is one."""
    if isinstance(t, torch.Tensor):
        if t.dtype == torch.int32 and t.get_device() == device.index and t.is_contiguous():
            return t
    else:
        t = torch.as_tensor(t)
    if t.dtype != torch.int32:
        t = t.to(torch.int32)
    return t.to(device).contiguous()


class _Cache:
    """Base pointers, page strides (elements) and dims of a paged K/V cache
    given as a 5D tensor [pages, 2, ., ., head_dim] or a (k, v) pair of 4D
    tensors [pages, ., ., head_dim]; each page must be contiguous."""

    __slots__ = ("k_ptr", "v_ptr", "psk", "psv", "dims", "dtype", "device", "k_tensor",
                 "v_tensor")

    def __init__(self, paged_kv_cache):
        if isinstance(paged_kv_cache, (tuple, list)):
            k, v = paged_kv_cache
            for t in (k, v):
                if t.dim() != 4:
                    raise ValueError("k/v caches must be 4D [pages, ., ., head_dim]")
                _page_contiguous(t.shape[1:], t.stride())
            self.k_ptr, self.v_ptr = k.data_ptr(), v.data_ptr()
            self.psk, self.psv = k.stride(0), v.stride(0)
            self.dims = tuple(k.shape[1:])
            if v.dtype != k.dtype:
                raise ValueError("k and v caches must share one dtype")
            self.dtype, self.device = k.dtype, k.device
            self.k_tensor, self.v_tensor = k, v
        else:
            c = paged_kv_cache
            if c.dim() != 5 or c.shape[1] != 2:
                raise ValueError("a single paged_kv_cache tensor must be 5D with dim 1 == 2")
            st = c.stride()
            _page_contiguous(c.shape[2:], (st[0],) + st[2:])
            self.k_ptr = c.data_ptr()
            self.v_ptr = self.k_ptr + st[1] * c.element_size()
            self.psk = self.psv = st[0]
            self.dims = tuple(c.shape[2:])
            self.dtype, self.device = c.dtype, c.device
            self.k_tensor = self.v_tensor = c


def _page_contiguous(inner_shape, strides):
    a, b, d = inner_shape
    if (strides[3], strides[2], strides[1]) != (1, d, b * d) or strides[0] < a * b * d:
        raise ValueError("each page of the k/v cache must be contiguous")


def _cache_dims(dims, layout):
    """(page_size, num_kv_heads, head_dim) from a cache's per-page dims."""
    if layout == NHD:
        return dims[0], dims[1], dims[2]
    return dims[1], dims[0], dims[2]


def get_seq_lens(kv_indptr, kv_last_page_len, page_size):
    """Tokens of each request: (pages - 1) * page_size + last_page_len."""
    dev = kv_last_page_len.device
    _on_gpu(dev)
    indptr = _i32_on(kv_indptr, dev)
    last = _i32_on(kv_last_page_len, dev)
    out = torch.empty(last.shape[0], dtype=torch.int32, device=dev)
    _lib.check(_call(dev, _lib.load().pkv_get_seq_lens, _ptr(indptr), _ptr(last),
                     last.shape[0], int(page_size), _ptr(out), _stream(dev)), "get_seq_lens")
    return out


def get_batch_indices_positions(append_indptr, seq_lens, nnz):
    """(batch_indices, positions) of the appended rows; positions are the
    last append-length positions of each request."""
    dev = seq_lens.device
    _on_gpu(dev)
    ai = _i32_on(append_indptr, dev)
    seq = _i32_on(seq_lens, dev)
    bi = torch.empty(int(nnz), dtype=torch.int32, device=dev)
    pos = torch.empty(int(nnz), dtype=torch.int32, device=dev)
    _lib.check(_call(dev, _lib.load().pkv_get_batch_indices_positions, _ptr(ai), _ptr(seq),
                     seq.shape[0], int(nnz), _ptr(bi), _ptr(pos), _stream(dev)),
               "get_batch_indices_positions")
    return bi, pos


def csr_to_block_tables(kv_indptr, kv_indices, max_pages_per_seq):
    """Dense block_tables [batch, max_pages_per_seq] from kv_indptr/kv_indices
    (entries past a request's pages are -1)."""
    dev = kv_indices.device
    _on_gpu(dev)
    indptr = _i32_on(kv_indptr, dev)
    idx = _i32_on(kv_indices, dev)
    batch = indptr.shape[0] - 1
    bt = torch.empty(batch, int(max_pages_per_seq), dtype=torch.int32, device=dev)
    _lib.check(_call(dev, _lib.load().pkv_csr_to_block_tables, _ptr(indptr), _ptr(idx), batch,
                     int(max_pages_per_seq), _ptr(bt), _stream(dev)), "csr_to_block_tables")
    return bt


def append_paged_kv_cache(append_key, append_value, batch_indices, positions,
                          paged_kv_cache, kv_indices, kv_indptr, kv_last_page_len,
                          kv_layout="NHD"):
    """Scatter appended K/V rows into their pages (in place; returns None)."""
    layout = _layout(kv_layout)
    c = _Cache(paged_kv_cache)
    ps, hkv, d = _cache_dims(c.dims, layout)
    if append_key.dtype != c.dtype or append_value.dtype != c.dtype:
        raise ValueError("append rows and cache must share one dtype")
    if tuple(append_key.shape[1:]) != (hkv, d) or append_value.shape != append_key.shape:
        raise ValueError("append_key/append_value must be [nnz, num_kv_heads, head_dim]")
    dev = c.device
    _on_gpu(dev, v_cache=c.v_tensor, append_key=append_key, append_value=append_value)
    ak, av = append_key.contiguous(), append_value.contiguous()
    bi, pos = _i32_on(batch_indices, dev), _i32_on(positions, dev)
    idx, indptr = _i32_on(kv_indices, dev), _i32_on(kv_indptr, dev)
    _lib.check(_call(dev, _lib.load().pkv_append_paged_kv_cache, _ptr(ak), _ptr(av), _ptr(bi),
                     _ptr(pos), ak.shape[0], c.k_ptr, c.v_ptr, c.psk, c.psv, _ptr(idx),
                     _ptr(indptr), None, indptr.shape[0] - 1, hkv, d, ps, layout,
                     _dt(ak), _stream(dev)),
               "append_paged_kv_cache")


def prefill_workspace_size(batch_size):
    return int(_lib.load().pkv_prefill_workspace_size(int(batch_size)))


def _scale_ptr(x, device, keep):
    if x is None:
        return None
    if not isinstance(x, torch.Tensor):
        x = torch.tensor([float(x)], dtype=torch.float32, device=device)
    if x.dtype != torch.float32 or x.numel() != 1:
        raise ValueError("q/k/v scales must be float32 tensors with one element")
    x = x.to(device).contiguous()
    keep.append(x)
    return x.data_ptr()


def batch_prefill_with_kv_cache(q, k_cache, v_cache, scale, workspace_buffer, *,
                                max_token_per_sequence, max_sequence_kv,
                                actual_seq_lens_q, actual_seq_lens_kv, block_tables=None,
                                causal, return_lse=True, q_scale=None, k_scale=None,
                                v_scale=None, batch_offsets_q=None, batch_offsets_o=None,
                                batch_offsets_k=None, batch_offsets_v=None,
                                batch_offsets_stats=None, out=None, lse=None, o_data_type=None,
                                kv_layout="HND"):
    """Batch prefill; returns (out, lse).

    With block_tables, k_cache / v_cache are paged ([pages, H, ps, d] for HND,
    [pages, ps, H, d] for NHD). Without, they are [total_kv_rows, H_kv, d] and
    request b's keys start at row batch_offsets_k[b] (values at
    batch_offsets_v[b]). batch_offsets_q / _o / _stats give each request's
    first row in q, out and lse. Absent offsets mean rows packed in request
    order.
    """
    if not return_lse:
        raise ValueError("return_lse must be True")
    dev = q.device
    paged = block_tables is not None
    if paged:
        layout = _layout(kv_layout)
        for t in (k_cache, v_cache):
            if t.dim() != 4:
                raise ValueError("paged k_cache/v_cache must be 4D [pages, ., ., d]")
            _page_contiguous(t.shape[1:], t.stride())
        ps, hkv, d_qk = _cache_dims(k_cache.shape[1:], layout)
        _, _, d_vo = _cache_dims(v_cache.shape[1:], layout)
    else:
        layout, ps = NHD, 16
        for t in (k_cache, v_cache):
            if t.dim() != 3 or not t.is_contiguous():
                raise ValueError("without block_tables, k_cache/v_cache must be contiguous "
                                 "[total_kv_rows, num_heads_kv, d]")
        hkv, d_qk = k_cache.shape[1], k_cache.shape[2]
        d_vo = v_cache.shape[2]
        if v_cache.shape[1] != hkv:
            raise ValueError("k_cache and v_cache must have the same number of heads")
    if q.dim() != 3 or q.shape[2] != d_qk:
        raise ValueError("q must be [total_tokens, num_heads_qo, d_qk]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q, k_cache and v_cache must share one dtype")
    q = q.contiguous()
    h_qo = q.shape[1]
    if o_data_type is None:
        o_data_type = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    if out is None:
        out = torch.empty(q.shape[0], h_qo, d_vo, dtype=o_data_type, device=dev)
    if lse is None:
        lse = torch.empty(q.shape[0], h_qo, dtype=torch.float32, device=dev)
    if out.dtype != o_data_type or not out.is_contiguous() or out.dim() != 3 or \
            tuple(out.shape[1:]) != (h_qo, d_vo):
        raise ValueError("out must be a contiguous [rows, num_heads_qo, d_vo] tensor")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.dim() != 2 or \
            lse.shape[1] != h_qo:
        raise ValueError("lse must be a contiguous float32 [rows, num_heads_qo] tensor")
    _on_gpu(dev, k_cache=k_cache, v_cache=v_cache, workspace_buffer=workspace_buffer,
            out=out, lse=lse)
    lq = _i32_on(actual_seq_lens_q, dev)
    lkv = _i32_on(actual_seq_lens_kv, dev)
    bt = _i32_on(block_tables, dev) if paged else None
    offs = [None if x is None else _i32_on(x, dev) for x in
            (batch_offsets_q, batch_offsets_o, batch_offsets_k, batch_offsets_v,
             batch_offsets_stats)]
    for o in offs:
        if o is not None and o.shape[0] != lq.shape[0]:
            raise ValueError("batch offsets must have batch_size entries")
    keep = []
    scales = [_scale_ptr(x, dev, keep) for x in (q_scale, k_scale, v_scale)]
    _lib.check(_call(
        dev, _lib.load().pkv_batch_prefill_with_kv_cache, _ptr(q), _ptr(k_cache),
        _ptr(v_cache), k_cache.stride(0) if paged else 0, v_cache.stride(0) if paged else 0,
        float(scale), _ptr(workspace_buffer),
        workspace_buffer.numel() * workspace_buffer.element_size(),
        int(max_token_per_sequence), int(max_sequence_kv), _ptr(lq), _ptr(lkv),
        _ptr(bt) if paged else None, bt.shape[1] if paged else 0, lq.shape[0], h_qo, hkv,
        d_qk, d_vo, ps, layout, 1 if causal else 0, *scales, _ptr(out), _ptr(lse),
        _dt(q), _dt(out), *[None if o is None else _ptr(o) for o in offs], _stream(dev)),
        "batch_prefill_with_kv_cache")
    return out, lse


def decode_workspace_size(batch_size, q_len_per_req, num_heads_qo, num_heads_kv,
                          head_dim, max_seq_len, window_left=-1):
    return int(_lib.load().pkv_decode_workspace_size(
        int(batch_size), int(q_len_per_req), int(num_heads_qo), int(num_heads_kv),
        int(head_dim), int(max_seq_len), int(window_left)))


def batch_decode_with_kv_cache(query, kv_cache, workspace_buffer, block_tables, seq_lens,
                               max_seq_len, bmm1_scale=1.0, bmm2_scale=1.0, window_left=-1,
                               out=None, out_dtype=None, sinks=None, kv_layout="HND",
                               q_len_per_req=1, o_scale=1.0, mask=None, max_q_len=None,
                               cum_seq_lens_q=None):
    """Batch decode over block_tables; returns out [num_tokens, num_heads, head_dim].

    bmm1_scale / bmm2_scale are floats or one-element float32 device tensors
    (read by the kernels at run time). With out_dtype torch.float8_e4m3fn each
    stored code is e4m3fn(out / o_scale) (nearest, ties to even, saturating).
    cum_seq_lens_q ([batch + 1] int32) with max_q_len gives each request its
    own query count; mask ([batch, Q, Q] bool or uint8) lets draft t see
    draft i when mask[b, t, i] is set, in place of the causal rule.
    """
    return _decode(False, query, kv_cache, workspace_buffer, block_tables, seq_lens,
                   max_seq_len, bmm1_scale, bmm2_scale, window_left, out, out_dtype, sinks,
                   kv_layout, q_len_per_req, o_scale, mask, max_q_len, cum_seq_lens_q)


def batch_decode_with_kv_cache_no_alloc(query, kv_cache, block_tables, seq_lens, max_seq_len,
                                        *, out, bmm1_scale=1.0, bmm2_scale=1.0, window_left=-1,
                                        sinks=None, kv_layout="HND", q_len_per_req=1,
                                        o_scale=1.0, mask=None, max_q_len=None,
                                        cum_seq_lens_q=None):
    """batch_decode_with_kv_cache without a workspace, for callers that cannot
    allocate: the split partials go to the library's static scratch array
    (64 MiB per GPU; larger split plans raise ValueError). ``out`` is
    required and its dtype is the output type. Calls that overlap on one GPU
    share that array and race: serialise them."""
    return _decode(True, query, kv_cache, None, block_tables, seq_lens, max_seq_len,
                   bmm1_scale, bmm2_scale, window_left, out, out.dtype, sinks, kv_layout,
                   q_len_per_req, o_scale, mask, max_q_len, cum_seq_lens_q)


def _decode(no_alloc, query, kv_cache, workspace_buffer, block_tables, seq_lens, max_seq_len,
            bmm1_scale, bmm2_scale, window_left, out, out_dtype, sinks, kv_layout,
            q_len_per_req, o_scale, mask, max_q_len, cum_seq_lens_q):
    layout = _layout(kv_layout)
    dev = query.device
    c = _Cache(kv_cache)
    ps, hkv, d = _cache_dims(c.dims, layout)
    if query.dim() != 3 or query.shape[2] != d:
        raise ValueError("query must be [num_tokens, num_heads, head_dim]")
    query = query.contiguous()
    h_qo = query.shape[1]
    if (max_q_len is None) != (cum_seq_lens_q is None):
        raise ValueError("max_q_len and cum_seq_lens_q must be given together")
    cum = None
    if cum_seq_lens_q is not None:
        cum = _i32_on(cum_seq_lens_q, dev)
        batch = cum.shape[0] - 1
        q_max = int(max_q_len)
    else:
        if query.shape[0] % int(q_len_per_req):
            raise ValueError("num_tokens must be batch_size * q_len_per_req")
        batch = query.shape[0] // int(q_len_per_req)
        q_max = int(q_len_per_req)
    mask_ptr = None
    if mask is not None:
        if tuple(mask.shape) != (batch, q_max, q_max):
            raise ValueError("mask must be [batch_size, Q, Q] with Q the query count per request")
        if mask.dtype not in (torch.bool, torch.uint8) or mask.get_device() != dev.index \
                or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous bool or uint8 tensor on the "
                             "query's device")
        mask_ptr = mask.data_ptr()  # one byte per entry, nonzero = visible
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else query.dtype
    if out is None:
        out = torch.empty(query.shape[0], h_qo, d, dtype=out_dtype, device=dev)
    if out.dtype != out_dtype or not out.is_contiguous() or tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must be a contiguous tensor shaped like query")
    _on_gpu(dev, k_cache=c.k_tensor, v_cache=c.v_tensor, workspace_buffer=workspace_buffer,
            out=out)
    bt = _i32_on(block_tables, dev)
    seq = seq_lens
    if not (isinstance(seq, torch.Tensor) and seq.dtype in (torch.int32, torch.uint32)
            and seq.get_device() == dev.index and seq.is_contiguous()):
        seq = torch.as_tensor(seq).to(dev)
        if seq.dtype not in (torch.int32, torch.uint32):
            seq = seq.to(torch.int32)
        seq = seq.contiguous()
    if seq.shape[0] != batch:
        raise ValueError("seq_lens must have batch_size entries")
    sink_ptr = None
    if sinks is not None:
        if isinstance(sinks, (list, tuple)):
            sinks = torch.cat([s.reshape(-1) for s in sinks])
        if not (sinks.dtype == torch.float32 and sinks.get_device() == dev.index
                and sinks.is_contiguous()):
            sinks = sinks.to(device=dev, dtype=torch.float32).contiguous()
        if sinks.numel() != h_qo:
            raise ValueError("sinks must hold one value per qo head")
        sink_ptr = sinks.data_ptr()
    b1, b1_ptr = _scale_arg(bmm1_scale, dev, "bmm1_scale")
    b2, b2_ptr = _scale_arg(bmm2_scale, dev, "bmm2_scale")
    lib = _lib.load()
    if no_alloc:
        fn, name, ws = lib.pkv_batch_decode_with_kv_cache_no_alloc, \
            "batch_decode_with_kv_cache_no_alloc", ()
    else:
        fn, name = lib.pkv_batch_decode_with_kv_cache, "batch_decode_with_kv_cache"
        ws = (_ptr(workspace_buffer), workspace_buffer.numel() * workspace_buffer.element_size())
    _lib.check(_call(
        dev, fn, _ptr(query), c.k_ptr, c.v_ptr, c.psk, c.psv, *ws, _ptr(bt), bt.shape[1],
        _ptr(seq), batch, int(max_seq_len), b1, b2, int(window_left), _ptr(out), _dt(out),
        sink_ptr, layout, int(q_len_per_req), h_qo, hkv, d, ps, _dt(query), _dtc(c.dtype),
        b1_ptr, b2_ptr, float(o_scale), None if cum is None else cum.data_ptr(),
        0 if cum is None else q_max, mask_ptr, _stream(dev)), name)
    return out


def _scale_arg(x, dev, name):
    """(host float, device pointer or None) for a float or a one-element
    float32 device tensor."""
    if isinstance(x, torch.Tensor):
        if x.dtype != torch.float32 or x.numel() != 1 or x.get_device() != dev.index:
            raise ValueError(f"{name} tensor must be one float32 element on {dev}")
        return 1.0, x.data_ptr()
    return float(x), None
