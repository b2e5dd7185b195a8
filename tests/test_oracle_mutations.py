"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of ``oracle/attention.py`` (the text
is edited in memory and loaded as a separate module; the oracle on disk is
untouched) and checks that at least one independent pin rejects the
mutant: torch's scaled-dot-product attention in float64 with a bottom-right
mask built from tril / triu, a brute-force loop over the mask definition,
or a closed form (sinks: o_sink = o * sigmoid(lse - sink); one allowed key:
o = beta * v_j, lse = s_j); for the speculative-decoding draft mask and
variable-length queries, reductions to the causal case, to key removal, and
to one uniform call per request.
"""

import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "attention.py")

MUTATIONS = {
    "top_left_causal": ("pos = t + (L_kv - L_q)", "pos = t"),
    "strict_causal": ("ok &= j <= pos", "ok &= j < pos"),
    "exclusive_window": ("ok &= j >= pos - window_left", "ok &= j > pos - window_left"),
    "gqa_modulo_map": ("kh = h // G", "kh = h % H_kv"),
    "dropped_score_scale": ("s = alpha * (q[:, h, :] @ k[:, kh, :].T)",
                            "s = (q[:, h, :] @ k[:, kh, :].T)"),
    "sink_dropped": ("z = p.sum(axis=1) + np.exp(sig - m)", "z = p.sum(axis=1)"),
    "sink_in_numerator": ("o = (p @ v[:, kh, :]) / z[:, None]",
                          "o = (p @ v[:, kh, :] + np.exp(sig - m)[:, None]) / z[:, None] "
                          "if sinks is not None else (p @ v[:, kh, :]) / z[:, None]"),
    "output_scale_dropped": ("beta * o, 0.0)", "o, 0.0)"),
    "lse_base_2": ("m_s + np.log(np.where", "m_s + np.log2(np.where"),
    "not_normalised": ("o = (p @ v[:, kh, :]) / z[:, None]", "o = (p @ v[:, kh, :])"),
    "draft_mask_transposed": ("seen = dm[t, np.clip(i, 0, L_q - 1)]",
                              "seen = dm[np.clip(i, 0, L_q - 1), t]"),
    "draft_mask_off_by_one": ("i = j - (L_kv - L_q)", "i = j - (L_kv - L_q) + 1"),
    "draft_mask_and_causal": ("ok &= ~in_drafts | seen", "ok &= (~in_drafts | seen) & (j <= pos)"),
    "draft_mask_hides_prefix": ("ok &= ~in_drafts | seen", "ok &= in_drafts & seen"),
    "window_skipped_with_mask": ("    if window_left >= 0:\n        ok &= j >= pos - window_left",
                                 "    if window_left >= 0 and draft_mask is None:\n"
                                 "        ok &= j >= pos - window_left"),
    "varlen_rows_uniform": ("qb = decode_bits(query[cum[b]:cum[b + 1]], q_fmt)",
                            "qb = decode_bits(query[b * ql:(b + 1) * ql], q_fmt)"),
    "varlen_mask_block": ("np.asarray(spec_mask)[b, :ql, :ql] != 0",
                          "np.asarray(spec_mask)[b, -ql:, -ql:] != 0"),
    "ragged_k_at_q_offsets": ("kb = decode_bits(k[ok_[b]:ok_[b] + L_kv], kv_fmt)",
                              "kb = decode_bits(k[oq[b]:oq[b] + L_kv], kv_fmt)"),
    "ragged_v_at_k_offsets": ("vb = decode_bits(v[ov[b]:ov[b] + L_kv], kv_fmt)",
                              "vb = decode_bits(v[ok_[b]:ok_[b] + L_kv], kv_fmt)"),
    "ragged_out_at_q_offsets": ("out[oo[b]:oo[b] + L_q] = o", "out[oq[b]:oq[b] + L_q] = o"),
    "ragged_lse_at_out_offsets": ("lse[os_[b]:os_[b] + L_q] = l", "lse[oo[b]:oo[b] + L_q] = l"),
    "ragged_kv_packed_by_q_lens": ("ck = _exclusive_cumsum(seq_lens_kv)",
                                   "ck = _exclusive_cumsum(seq_lens_q)"),
}


def load_mutant(old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, old
    mod = types.ModuleType("oracle._mutant")
    mod.__package__ = "oracle"
    mod.__file__ = SRC
    exec(compile(text.replace(old, new), SRC, "exec"), mod.__dict__)
    return mod


# ---- independent pins ---------------------------------------------------------

def br_mask(L_q, L_kv, w):
    m = torch.ones(L_q, L_kv, dtype=torch.bool).tril(diagonal=L_kv - L_q)
    if w >= 0:
        m &= torch.ones(L_q, L_kv, dtype=torch.bool).triu(diagonal=L_kv - L_q - w)
    return m


def pin_sdpa(mod):
    rng = np.random.default_rng(5)
    for (L_q, L_kv, H_qo, H_kv, w) in [(3, 9, 4, 2, -1), (4, 13, 6, 3, 2), (2, 6, 4, 1, 0)]:
        q = rng.standard_normal((L_q, H_qo, 16))
        k = rng.standard_normal((L_kv, H_kv, 16))
        v = rng.standard_normal((L_kv, H_kv, 8))
        G = H_qo // H_kv
        qt = torch.from_numpy(q).permute(1, 0, 2)
        kt = torch.from_numpy(k).repeat_interleave(G, dim=1).permute(1, 0, 2)
        vt = torch.from_numpy(v).repeat_interleave(G, dim=1).permute(1, 0, 2)
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=br_mask(L_q, L_kv, w),
                                             scale=0.37).permute(1, 0, 2).numpy() * 1.3
        out, lse = mod.attention(q, k, v, 0.37, 1.3, True, window_left=w)
        if not np.allclose(out, ref, rtol=1e-10, atol=1e-10):
            return False
        # natural-log LSE from logsumexp of the masked, scaled scores
        s = 0.37 * torch.einsum("qhd,khd->hqk", qt.permute(1, 0, 2), kt.permute(1, 0, 2))
        s = s.masked_fill(~br_mask(L_q, L_kv, w), float("-inf"))
        if not np.allclose(lse, torch.logsumexp(s, dim=-1).T.numpy(), rtol=1e-10, atol=1e-10):
            return False
    return True


def pin_brute_force_mask(mod):
    for L_q in range(1, 5):
        for L_kv in range(0, 7):
            for w in (-1, 0, 1, 3):
                got = mod.allowed_mask(np.arange(L_q), L_q, L_kv, True, w)
                for t in range(L_q):
                    pos = t + L_kv - L_q
                    for j in range(L_kv):
                        want = j <= pos and (w < 0 or j >= pos - w)
                        if bool(got[t, j]) != want:
                            return False
    return True


def pin_sinks_closed_form(mod):
    rng = np.random.default_rng(6)
    q = rng.standard_normal((3, 4, 16))
    k = rng.standard_normal((10, 2, 16))
    v = rng.standard_normal((10, 2, 8))
    sinks = rng.standard_normal(4)
    o0, lse = mod.attention(q, k, v, 0.5, 1.0, True)
    o1, _ = mod.attention(q, k, v, 0.5, 1.0, True, sinks=sinks)
    sig = 1.0 / (1.0 + np.exp(-(lse - sinks[None, :])))
    return np.allclose(o1, o0 * sig[:, :, None], rtol=1e-10, atol=1e-12)


def pin_one_key(mod):
    # window_left = 0 with causal: each query sees only its own position
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 2, 16))
    k = rng.standard_normal((5, 1, 16))
    v = rng.standard_normal((5, 1, 8))
    out, lse = mod.attention(q, k, v, 0.25, 2.0, True, window_left=0)
    for t in range(2):
        j = t + 3
        for h in range(2):
            if not np.allclose(out[t, h], 2.0 * v[j, 0], rtol=1e-12, atol=1e-12):
                return False
            if not np.isclose(lse[t, h], 0.25 * q[t, h] @ k[j, 0], rtol=1e-12, atol=1e-12):
                return False
    return True


def pin_draft_mask_lower_triangle_is_causal(mod):
    # a lower-triangular draft mask is the causal rule among the drafts
    rng = np.random.default_rng(8)
    for (L_q, L_kv, w) in [(4, 11, -1), (3, 9, 2), (4, 3, -1), (2, 7, 0)]:
        tril = np.tril(np.ones((L_q, L_q), dtype=bool))
        a = mod.allowed_mask(np.arange(L_q), L_q, L_kv, True, w, draft_mask=tril)
        b = mod.allowed_mask(np.arange(L_q), L_q, L_kv, True, w)
        if not np.array_equal(a, b):
            return False
        q = rng.standard_normal((L_q, 2, 16))
        k = rng.standard_normal((L_kv, 1, 16))
        v = rng.standard_normal((L_kv, 1, 8))
        o1, _ = mod.attention(q, k, v, 0.3, 1.0, True, window_left=w, draft_mask=tril)
        o2, _ = mod.attention(q, k, v, 0.3, 1.0, True, window_left=w)
        if not np.array_equal(o1, o2):
            return False
    return True


def pin_draft_mask_is_key_removal(mod):
    # masking keys is the same as removing them: draft t's output equals a
    # single unmasked query over the prefix plus the drafts its row allows
    # (no window); random masks, not only trees
    rng = np.random.default_rng(9)
    for (L_q, L_kv) in [(4, 12), (5, 6), (3, 3)]:
        dm = rng.random((L_q, L_q)) < 0.5
        q = rng.standard_normal((L_q, 2, 16))
        k = rng.standard_normal((L_kv, 1, 16))
        v = rng.standard_normal((L_kv, 1, 8))
        out, _ = mod.attention(q, k, v, 0.4, 1.5, True, draft_mask=dm)
        d0 = L_kv - L_q
        for t in range(L_q):
            keep = [j for j in range(L_kv) if j < d0 or dm[t, j - d0]]
            if not keep:
                if not np.all(out[t] == 0):
                    return False
                continue
            ref, _ = mod.attention(q[t:t + 1], k[keep], v[keep], 0.4, 1.5, False)
            if not np.allclose(out[t], ref[0], rtol=1e-12, atol=1e-12):
                return False
    return True


def pin_draft_mask_with_window_sdpa(mod):
    # torch's float64 scaled-dot-product attention with the explicit mask:
    # drafts by the draft mask, then the inclusive window on positions
    rng = np.random.default_rng(10)
    L_q, L_kv, w = 4, 10, 3
    dm = rng.random((L_q, L_q)) < 0.6
    np.fill_diagonal(dm, True)
    m = torch.ones(L_q, L_kv, dtype=torch.bool)
    m[:, L_kv - L_q:] = torch.from_numpy(dm)
    m &= torch.ones(L_q, L_kv, dtype=torch.bool).triu(diagonal=L_kv - L_q - w)
    q = rng.standard_normal((L_q, 1, 16))
    k = rng.standard_normal((L_kv, 1, 16))
    v = rng.standard_normal((L_kv, 1, 8))
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2), attn_mask=m, scale=0.5).permute(1, 0, 2).numpy()
    out, _ = mod.attention(q, k, v, 0.5, 1.0, True, window_left=w, draft_mask=dm)
    return np.allclose(out, ref, rtol=1e-10, atol=1e-10)


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def pin_varlen_rows(mod):
    # ragged cum_seq_lens_q equals one uniform call per request with
    # q_len_per_req = that request's query count; a spec_mask [B, Q, Q]
    # uses each request's leading ql x ql block
    rng = np.random.default_rng(11)
    ps, H, d = 4, 2, 8
    seq = np.array([9, 3, 6])
    ql = np.array([3, 1, 2])
    cum = np.concatenate([[0], np.cumsum(ql)])
    n_pages = (seq + ps - 1) // ps
    bt = np.full((3, int(n_pages.max())), -1, dtype=np.int64)
    perm = rng.permutation(int(n_pages.sum()))
    off = 0
    for b in range(3):
        bt[b, :n_pages[b]] = perm[off:off + n_pages[b]]
        off += n_pages[b]
    kc = _bf16_bits(rng.standard_normal((int(n_pages.sum()), H, ps, d)))
    vc = _bf16_bits(rng.standard_normal((int(n_pages.sum()), H, ps, d)))
    qry = _bf16_bits(rng.standard_normal((int(cum[-1]), 2 * H, d)))
    mask = rng.random((3, 3, 3)) < 0.5
    for b in range(3):
        np.fill_diagonal(mask[b], True)
    for sm in (None, mask):
        got = mod.batch_decode(qry, "bf16", kc, vc, "bf16", bt, seq, 0.3, 1.0, -1, None, "HND",
                               cum_seq_lens_q=cum, spec_mask=sm)
        for b in range(3):
            one = mod.batch_decode(qry[cum[b]:cum[b + 1]], "bf16", kc, vc, "bf16", bt[b:b + 1],
                                   seq[b:b + 1], 0.3, 1.0, -1, None, "HND",
                                   q_len_per_req=int(ql[b]),
                                   spec_mask=None if sm is None else sm[b:b + 1, :ql[b], :ql[b]])
            if not np.array_equal(got[cum[b]:cum[b + 1]], one):
                return False
    return True


def _ragged_case(rng):
    lq = np.array([5, 0, 3, 7])
    lkv = lq + np.array([4, 2, 0, 9])
    H_qo, H_kv, d = 4, 2, 8
    q = _bf16_bits(rng.standard_normal((int(lq.sum()), H_qo, d)))
    k = _bf16_bits(rng.standard_normal((int(lkv.sum()), H_kv, d)))
    v = _bf16_bits(rng.standard_normal((int(lkv.sum()), H_kv, d)))
    return lq, lkv, q, k, v


def pin_ragged_equals_paged(mod):
    # the packed non-paged layout is the paged one with its pages gathered:
    # scatter each request's rows into 4-token pages in shuffled order and the
    # paged prefill must return the same values
    rng = np.random.default_rng(12)
    lq, lkv, q, k, v = _ragged_case(rng)
    ps = 4
    n_pages = (lkv + ps - 1) // ps
    perm = rng.permutation(int(n_pages.sum()))
    bt = np.full((4, int(n_pages.max())), -1, dtype=np.int64)
    kc = np.zeros((int(n_pages.sum()), ps, 2, 8), dtype=np.uint16)
    vc = np.zeros_like(kc)
    ck = np.concatenate([[0], np.cumsum(lkv)])
    off = 0
    for b in range(4):
        for p in range(n_pages[b]):
            page = perm[off + p]
            bt[b, p] = page
            rows = range(p * ps, min((p + 1) * ps, int(lkv[b])))
            for j in rows:
                kc[page, j - p * ps] = k[ck[b] + j]
                vc[page, j - p * ps] = v[ck[b] + j]
        off += n_pages[b]
    o1, l1 = mod.batch_prefill_ragged(q, "bf16", k, v, "bf16", lq, lkv, 0.3, True)
    o2, l2 = mod.batch_prefill(q, "bf16", kc, vc, "bf16", bt, lq, lkv, 0.3, True, "NHD")
    return np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_ragged_offsets_move_rows(mod):
    # explicit offsets that store the requests in another order with gaps
    # between them give the packed result, moved to those rows
    rng = np.random.default_rng(13)
    lq, lkv, q, k, v = _ragged_case(rng)
    o_ref, l_ref = mod.batch_prefill_ragged(q, "bf16", k, v, "bf16", lq, lkv, 0.3, True)
    order = [2, 0, 3, 1]
    def place(lens, gap):
        offs, cur = np.zeros(4, dtype=np.int64), 0
        for b in order:
            offs[b] = cur
            cur += int(lens[b]) + gap
        return offs, cur
    oq, nq = place(lq, 2)
    oo, no = place(lq, 3)
    os_, ns = place(lq, 1)
    ok_, nk = place(lkv, 5)
    ov, nv = place(lkv, 1)
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lkv)])
    q2 = np.zeros((nq,) + q.shape[1:], dtype=q.dtype)
    k2 = np.zeros((nk,) + k.shape[1:], dtype=k.dtype)
    v2 = np.zeros((nv,) + v.shape[1:], dtype=v.dtype)
    for b in range(4):
        q2[oq[b]:oq[b] + lq[b]] = q[cq[b]:cq[b + 1]]
        k2[ok_[b]:ok_[b] + lkv[b]] = k[ck[b]:ck[b + 1]]
        v2[ov[b]:ov[b] + lkv[b]] = v[ck[b]:ck[b + 1]]
    o, _ = mod.batch_prefill_ragged(q2, "bf16", k2, v2, "bf16", lq, lkv, 0.3, True,
                                    offsets_q=oq, offsets_o=oo, offsets_k=ok_, offsets_v=ov,
                                    offsets_stats=os_, out_rows=max(no, ns))
    _, l = mod.batch_prefill_ragged(q2, "bf16", k2, v2, "bf16", lq, lkv, 0.3, True,
                                    offsets_q=oq, offsets_o=oo, offsets_k=ok_, offsets_v=ov,
                                    offsets_stats=os_, out_rows=max(no, ns))
    for b in range(4):
        if not np.array_equal(o[oo[b]:oo[b] + lq[b]], o_ref[cq[b]:cq[b + 1]]):
            return False
        if not np.array_equal(l[os_[b]:os_[b] + lq[b]], l_ref[cq[b]:cq[b + 1]]):
            return False
    written = sum(int(x) for x in lq)
    return int(np.isfinite(o[:, 0, 0]).sum()) == written


PINS = [pin_sdpa, pin_brute_force_mask, pin_sinks_closed_form, pin_one_key,
        pin_draft_mask_lower_triangle_is_causal, pin_draft_mask_is_key_removal,
        pin_draft_mask_with_window_sdpa, pin_varlen_rows, pin_ragged_equals_paged,
        pin_ragged_offsets_move_rows]


def test_pins_accept_the_oracle():
    mod = load_mutant("import numpy as np", "import numpy as np")
    for pin in PINS:
        assert pin(mod), pin.__name__


def passes(pin, mod):
    """A pin rejects a mutant by returning False or by the mutant raising."""
    try:
        return bool(pin(mod))
    except Exception:
        return False


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_mutant(name):
    mod = load_mutant(*MUTATIONS[name])
    failed = [p.__name__ for p in PINS if not passes(p, mod)]
    assert failed, f"no pin caught the mutation {name}"
