"""Shared helpers of the tests: raw-bit views, tolerances, oracle calls."""

import numpy as np
import torch

import oracle
from oracle.paging import HND, NHD

_FMT = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float8_e4m3fn: "e4m3"}


def fmt(t):
    return _FMT[t.dtype]


def bits(t):
    """numpy array of the raw element bits of a tensor (any device)."""
    t = t.detach().contiguous().cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy()
    raise ValueError(t.dtype)


def half_ulp(ref, out_dtype):
    """Half a unit in the last place of each reference value in out_dtype."""
    mant = {torch.bfloat16: 7, torch.float16: 10}[out_dtype]
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 0.5 * 2.0 ** (e - mant)


def assert_out_close(got, ref, out_dtype, atol=2e-2, what="out"):
    """|got - ref| <= atol + half an output ulp of ref, elementwise."""
    got = got.detach().float().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    bound = atol + half_ulp(ref, out_dtype)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} elements off; max err "
                           f"{err.max():.4g} at {np.unravel_index(err.argmax(), err.shape)}")
    return float(err.max())


def assert_lse_close(got, ref, atol=1e-3):
    got = got.detach().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):  # -inf - -inf where both rows are empty
        err = np.where(both_inf, 0.0, np.abs(got - ref))
    assert not np.isnan(err).any(), "lse: NaN"
    assert err.max() <= atol, f"lse max err {err.max():.4g}"
    return float(err.max())


def n_pages(seq_lens, page_size):
    return [(int(s) + page_size - 1) // page_size for s in seq_lens]


def oracle_prefill(w, rows=None):
    """Oracle prefill of a workloads.batch_prefill / fp8_prefill dict."""
    ps = w["page_size"]
    used = n_pages(w["seq_lens_kv"], ps)
    from workloads import compact_pages
    kc, bt = compact_pages(w["k_cache"], w["block_tables"], used)
    vc, _ = compact_pages(w["v_cache"], w["block_tables"], used)
    sc = lambda x: 1.0 if x is None else float(x.reshape(-1)[0])
    return oracle.batch_prefill(
        bits(w["q"]), fmt(w["q"]), bits(kc), bits(vc), fmt(w["k_cache"]), bt.numpy(),
        w["seq_lens_q"].numpy(), w["seq_lens_kv"].numpy(), w["scale"], w["causal"],
        w["layout"], q_scale=sc(w["q_scale"]), k_scale=sc(w["k_scale"]),
        v_scale=sc(w["v_scale"]), rows=rows)


def oracle_decode(w, requests=None, kv_cache=None):
    """Oracle decode of a workloads.batch_decode / spec_decode dict."""
    ps = w["page_size"]
    kv = w["kv_cache"] if kv_cache is None else kv_cache
    seq = w["seq_lens"].to(torch.int64)
    reqs = list(range(seq.shape[0])) if requests is None else list(requests)
    used = [0] * seq.shape[0]
    for b in reqs:
        used[b] = n_pages([seq[b]], ps)[0]
    from workloads import compact_pages
    sub, bt = compact_pages(kv, w["block_tables"], used)
    sinks = None if w["sinks"] is None else w["sinks"].double().numpy()
    return oracle.batch_decode(
        bits(w["query"]), fmt(w["query"]), bits(sub[:, 0]), bits(sub[:, 1]), fmt(kv),
        bt.numpy(), seq.numpy(), w["bmm1_scale"], w["bmm2_scale"], w["window_left"],
        sinks, w["layout"], w["q_len_per_req"], requests=reqs)
