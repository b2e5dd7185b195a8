"""Pins for the oracle's attention against library routines, closed forms and
brute force (CPU only).

Each test fixes something a plausible slip in ``oracle/attention.py`` would
break: the scale or sign of the scores, the causal alignment, the window's
inclusive edge, the GQA head map, the sink term, the LSE, the fp8 scales.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.attention import attention, allowed_mask
from oracle.paging import HND, NHD


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa_reference(q, k, v, alpha, mask):
    """torch SDPA in float64 with KV heads expanded to the qo heads.

    mask: bool [L_q, L_kv] (True = attend), built by the caller from
    torch.tril / torch.triu, not from the oracle.
    """
    G = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)                    # [H, L_q, d]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1).permute(1, 0, 2)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask),
                                       scale=alpha)
    return o.permute(1, 0, 2).numpy()


def _br_causal(L_q, L_kv, window_left=-1):
    m = torch.ones(L_q, L_kv, dtype=torch.bool).tril(diagonal=L_kv - L_q)
    if window_left >= 0:
        m &= torch.ones(L_q, L_kv, dtype=torch.bool).triu(diagonal=L_kv - L_q - window_left)
    return m.numpy()


@pytest.mark.parametrize("L_q,L_kv,H_qo,H_kv,causal,w", [
    (5, 5, 2, 2, True, -1),
    (3, 9, 4, 2, True, -1),     # bottom-right: cached prefix of 6
    (7, 7, 8, 1, False, -1),
    (4, 13, 6, 3, True, 2),     # window of 3 keys including self
    (1, 17, 4, 4, True, 0),
    (6, 11, 4, 1, True, 5),
])
def test_attention_equals_torch_sdpa(L_q, L_kv, H_qo, H_kv, causal, w):
    rng = np.random.default_rng(L_q * 100 + L_kv)
    q, k, v = _rand(rng, L_q, H_qo, 16), _rand(rng, L_kv, H_kv, 16), _rand(rng, L_kv, H_kv, 8)
    alpha = 0.37
    mask = _br_causal(L_q, L_kv, w) if causal else np.ones((L_q, L_kv), dtype=bool)
    ref = _sdpa_reference(q, k, v, alpha, mask)
    out, _ = attention(q, k, v, alpha, 1.0, causal, window_left=w)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_mask_brute_force_tiny():
    # Enumerate by positions: the query row t of L_q rows sits at key
    # position L_kv - L_q + t; causal admits keys at or before it; the window
    # admits keys at most w positions before it.
    for L_q in range(1, 6):
        for L_kv in range(L_q, 9):
            for w in (-1, 0, 1, 2, 5):
                got = allowed_mask(np.arange(L_q), L_q, L_kv, True, w)
                for t in range(L_q):
                    pos = L_kv - L_q + t
                    expect = [j <= pos and (w < 0 or pos - j <= w) for j in range(L_kv)]
                    assert got[t].tolist() == expect


def test_causal_square_mask_is_lower_triangle_and_pair_count():
    m = allowed_mask(np.arange(9), 9, 9, True)
    assert np.array_equal(m, np.tril(np.ones((9, 9), dtype=bool)))
    # bottom-right causal pair count L_q*(L_kv-L_q) + L_q*(L_q+1)/2
    for L_q, L_kv in [(3, 10), (10, 10), (1, 5), (64, 300)]:
        assert oracle.allowed_pairs([L_q], [L_kv], True) == L_q * (L_kv - L_q) + L_q * (L_q + 1) // 2
    assert oracle.keys_read([100], 4, 10) == 14
    assert oracle.keys_read([5], 4, 10) == 5


def test_row_sample_equals_full_computation():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 9, 4, 8), _rand(rng, 20, 2, 8), _rand(rng, 20, 2, 8)
    full, lse = attention(q, k, v, 0.5, 1.0, True)
    rows = np.array([0, 4, 8])
    part, lse_p = attention(q[rows], k, v, 0.5, 1.0, True, row_index=rows, L_q=9)
    np.testing.assert_allclose(part, full[rows], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse_p, lse[rows], rtol=1e-14, atol=1e-15)


def test_masking_equals_slicing_the_keys():
    rng = np.random.default_rng(4)
    L_q, L_kv, w = 5, 23, 6
    q, k, v = _rand(rng, L_q, 2, 8), _rand(rng, L_kv, 1, 8), _rand(rng, L_kv, 1, 8)
    out, lse = attention(q, k, v, 0.8, 2.0, True, window_left=w)
    for t in range(L_q):
        pos = L_kv - L_q + t
        lo = max(0, pos - w)
        o1, l1 = attention(q[t:t + 1], k[lo:pos + 1], v[lo:pos + 1], 0.8, 2.0, False)
        np.testing.assert_allclose(out[t], o1[0], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[t], l1[0], rtol=1e-13, atol=1e-13)


def test_lse_merge_of_two_key_halves():
    # Attention over K1 u K2 from the halves: weights exp(lse_i).
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 3, 2, 8), _rand(rng, 30, 2, 8), _rand(rng, 30, 2, 8)
    o, lse = attention(q, k, v, 0.3, 1.0, False)
    for cut in (1, 11, 29):
        o1, l1 = attention(q, k[:cut], v[:cut], 0.3, 1.0, False)
        o2, l2 = attention(q, k[cut:], v[cut:], 0.3, 1.0, False)
        lm = np.logaddexp(l1, l2)
        om = (np.exp(l1 - lm)[..., None] * o1 + np.exp(l2 - lm)[..., None] * o2)
        np.testing.assert_allclose(o, om, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, lm, rtol=1e-13, atol=1e-13)


def test_lse_special_cases():
    rng = np.random.default_rng(6)
    k, v = _rand(rng, 12, 1, 8), _rand(rng, 12, 1, 8)
    # q = 0: uniform weights over the allowed keys
    q0 = np.zeros((4, 1, 8))
    o, lse = attention(q0, k, v, 1.0, 3.0, True)
    for t in range(4):
        n = 12 - 4 + t + 1
        np.testing.assert_allclose(o[t, 0], 3.0 * v[:n, 0].mean(axis=0), rtol=1e-13)
        np.testing.assert_allclose(lse[t, 0], np.log(n), rtol=1e-14)
    # window 0: one allowed key, the query's own position
    q = _rand(rng, 4, 1, 8)
    o, lse = attention(q, k, v, 0.7, 2.0, True, window_left=0)
    for t in range(4):
        pos = 8 + t
        np.testing.assert_allclose(o[t, 0], 2.0 * v[pos, 0], rtol=1e-14)
        np.testing.assert_allclose(lse[t, 0], 0.7 * q[t, 0] @ k[pos, 0], rtol=1e-13)


def test_empty_rows():
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 4, 1, 8), _rand(rng, 2, 1, 8), _rand(rng, 2, 1, 8)
    # L_kv < L_q under causal: the first two rows see nothing
    o, lse = attention(q, k, v, 1.0, 1.0, True)
    assert np.all(o[:2] == 0) and np.all(np.isneginf(lse[:2]))
    assert np.all(np.isfinite(lse[2:]))


def test_sinks_closed_form():
    # softmax with one extra logit sigma in the denominator only:
    # o_sink = o * Z / (Z + e^sigma) = o * sigmoid(lse - sigma)
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 4, 4, 8), _rand(rng, 40, 2, 8), _rand(rng, 40, 2, 8)
    sinks = rng.standard_normal(4) * 3
    o, lse = attention(q, k, v, 0.4, 1.5, True, window_left=9)
    o_s, lse_s = attention(q, k, v, 0.4, 1.5, True, window_left=9, sinks=sinks)
    sig = 1.0 / (1.0 + np.exp(-(lse - sinks[None, :])))
    np.testing.assert_allclose(o_s, o * sig[..., None], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(lse_s, lse)


def test_gqa_equals_replicated_kv_heads():
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 6, 8, 16), _rand(rng, 10, 2, 16), _rand(rng, 10, 2, 16)
    o, lse = attention(q, k, v, 0.25, 1.0, True)
    o2, lse2 = attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.25, 1.0, True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    # heads 0..3 read kv head 0: changing kv head 1 leaves them alone
    k3 = k.copy()
    k3[:, 1] += rng.standard_normal(k3[:, 1].shape)
    o3, _ = attention(q, k3, v, 0.25, 1.0, True)
    np.testing.assert_array_equal(o3[:, :4], o[:, :4])
    assert not np.allclose(o3[:, 4:], o[:, 4:])


def _paged(rng, seqs, H, D, ps, layout, fmt_bits):
    """Scatter contiguous sequences into random pages by hand."""
    n_pages = [-(-s // ps) for s in seqs]
    pool = sum(n_pages) + 5
    perm = rng.permutation(pool)
    shape = (pool, ps, H, D) if layout == NHD else (pool, H, ps, D)
    cache = rng.integers(0, 2 ** 8, size=shape).astype(fmt_bits)
    bt = np.full((len(seqs), max(n_pages)), -1, dtype=np.int32)
    data = []
    off = 0
    for b, s in enumerate(seqs):
        bt[b, :n_pages[b]] = perm[off:off + n_pages[b]]
        off += n_pages[b]
        x = rng.integers(0, 2 ** 8, size=(s, H, D)).astype(fmt_bits)
        for j in range(s):
            if layout == NHD:
                cache[bt[b, j // ps], j % ps] = x[j]
            else:
                cache[bt[b, j // ps], :, j % ps] = x[j]
        data.append(x)
    return cache, bt, data


def _bf16_bits(rng, *shape):
    x = torch.from_numpy(rng.standard_normal(shape)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("layout", [NHD, HND])
def test_batch_prefill_paged_equals_contiguous_sdpa_with_fp8_scales(layout):
    rng = np.random.default_rng(10)
    ps, H_qo, H_kv, d_qk, d_vo = 4, 4, 2, 16, 8
    Lq, Lkv = [3, 1, 6], [7, 1, 6]
    kc, bt, kseq = _paged(rng, Lkv, H_kv, d_qk, ps, layout, np.uint8)
    # V uses the same page list with its own contents
    vshape = (kc.shape[0], ps, H_kv, d_vo) if layout == NHD else (kc.shape[0], H_kv, ps, d_vo)
    vc = rng.integers(0, 256, size=vshape).astype(np.uint8)
    vc[..., :] &= 0x7E  # no NaN codes anywhere in V
    kc &= 0x7E
    q = (rng.integers(0, 256, size=(sum(Lq), H_qo, d_qk)) & 0x7E).astype(np.uint8)
    qs, ks, vs, scale = 1.5, 0.75, 1.25, 0.2
    out, lse = oracle.batch_prefill(q, "e4m3", kc, vc, "e4m3", bt, Lq, Lkv, scale, True,
                                    layout, q_scale=qs, k_scale=ks, v_scale=vs)
    cq = np.concatenate([[0], np.cumsum(Lq)])
    f8 = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    for b in range(3):
        kb = oracle.gather_pages(kc, bt[b], Lkv[b], layout)
        vb = oracle.gather_pages(vc, bt[b], Lkv[b], layout)
        ref = _sdpa_reference(f8(q[cq[b]:cq[b + 1]]) * qs, f8(kb) * ks, f8(vb) * vs,
                              scale, _br_causal(Lq[b], Lkv[b]))
        np.testing.assert_allclose(out[cq[b]:cq[b + 1]], ref, rtol=1e-12, atol=1e-12)
        # lse from the library's logsumexp of the scaled masked scores
        G = H_qo // H_kv
        s = torch.einsum("thd,jhd->htj", torch.from_numpy(f8(q[cq[b]:cq[b + 1]]) * qs),
                         torch.from_numpy(np.repeat(f8(kb) * ks, G, axis=1))) * scale
        s = s.masked_fill(~torch.from_numpy(_br_causal(Lq[b], Lkv[b])), float("-inf"))
        np.testing.assert_allclose(lse[cq[b]:cq[b + 1]], torch.logsumexp(s, -1).T.numpy(),
                                   rtol=1e-12, atol=1e-12)


def test_batch_prefill_row_sample_equals_full():
    rng = np.random.default_rng(11)
    kc, bt, _ = _paged(rng, [9, 5], 2, 8, 4, HND, np.uint16)
    kc = _bf16_bits(rng, *kc.shape)
    vc = _bf16_bits(rng, *kc.shape)
    q = _bf16_bits(rng, 8, 4, 8)
    out, lse = oracle.batch_prefill(q, "bf16", kc, vc, "bf16", bt, [5, 3], [9, 5], 0.3, True, HND)
    rows = [(1, 2), (0, 0), (0, 4)]
    o2, l2 = oracle.batch_prefill(q, "bf16", kc, vc, "bf16", bt, [5, 3], [9, 5], 0.3, True, HND,
                                  rows=rows)
    np.testing.assert_allclose(o2, out[[7, 0, 4]], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l2, lse[[7, 0, 4]], rtol=1e-14, atol=1e-15)


def test_batch_decode_equals_prefill_of_the_last_positions():
    rng = np.random.default_rng(12)
    seqs = [9, 17, 4]
    ql = 3
    kc, bt, _ = _paged(rng, seqs, 2, 8, 4, HND, np.uint16)
    kc = _bf16_bits(rng, *kc.shape)
    vc = _bf16_bits(rng, *kc.shape)
    q = _bf16_bits(rng, len(seqs) * ql, 4, 8)
    dec = oracle.batch_decode(q, "bf16", kc, vc, "bf16", bt, seqs, 0.3, 1.7, -1, None, HND, ql)
    pre, _ = oracle.batch_prefill(q, "bf16", kc, vc, "bf16", bt, [ql] * 3, seqs, 0.3, True, HND)
    np.testing.assert_allclose(dec, 1.7 * pre, rtol=1e-13, atol=1e-14)
    # window and sinks against the library routine, request by request
    sinks = rng.standard_normal(4)
    dec = oracle.batch_decode(q, "bf16", kc, vc, "bf16", bt, seqs, 0.3, 1.7, 5, sinks, HND, ql,
                              requests=[1])
    kb = oracle.decode_bits(oracle.gather_pages(kc, bt[1], 17, HND), "bf16")
    vb = oracle.decode_bits(oracle.gather_pages(vc, bt[1], 17, HND), "bf16")
    qb = oracle.decode_bits(q[3:6], "bf16")
    ref = _sdpa_reference(qb, kb, vb, 0.3, _br_causal(ql, 17, 5))
    _, lse = attention(qb, kb, vb, 0.3, 1.0, True, window_left=5)
    sig = 1.0 / (1.0 + np.exp(-(lse - sinks[None, :])))
    np.testing.assert_allclose(dec, 1.7 * ref * sig[..., None], rtol=1e-12, atol=1e-13)
