"""Masked softmax attention over a gathered paged cache, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources:
* ``flashinfer.prefill.cudnn_batch_prefill_with_kv_cache`` -- Parameters
  (q, k_cache, v_cache, scale, actual_seq_lens_q/kv, block_tables, causal,
  return_lse, q_scale/k_scale/v_scale), Returns (output and log-sum-exp),
  Note (num_heads_qo >= num_heads_kv; d_qk 128 or 192, d_vo 128).
* ``flashinfer.decode.trtllm_batch_decode_with_kv_cache`` -- Parameters
  (query, block_tables, seq_lens, bmm1_scale, bmm2_scale, window_left, sinks,
  q_len_per_req).

Readings taken where the pages are silent (each listed in the design notes):
* causal alignment is bottom-right: query row t of a request with L_q queries
  and L_kv keys sits at position t + L_kv - L_q;
* window_left w >= 0 keeps keys j with pos - w <= j (w + 1 keys including
  the query's own position); -1 keeps everything;
* qo head h reads kv head h // (H_qo / H_kv);
* a sink is one extra logit per qo head, in the same units as the scaled
  scores, that joins the softmax denominator only;
* fp8 scales dequantise by multiplication (x = scale * stored value);
* the log-sum-exp is natural-log of the scaled scores over allowed keys
  (sinks excluded); a row with no allowed key has output 0 and lse -inf.
"""

import numpy as np

from .formats import decode_bits
from .paging import gather_pages


def allowed_mask(row_index, L_q, L_kv, causal, window_left=-1, draft_mask=None):
    """allowed[r, j] for query rows ``row_index`` (0..L_q-1) and keys 0..L_kv-1.

    Bottom-right alignment: row t is at position pos = t + L_kv - L_q. With
    ``causal`` a key is allowed only if j <= pos; with window_left w >= 0 also
    only if j >= pos - w.

    ``draft_mask`` (decode page, Parameters: ``mask``, the attention mask for
    speculative decoding) is a boolean [L_q, L_q]: the L_q queries are drafts
    at the last L_q positions, and draft t may see the draft at position
    L_kv - L_q + i exactly when draft_mask[t, i]. It takes the place of the
    causal rule among the drafts; keys before the drafts stay visible, and
    the window still applies.
    """
    t = np.asarray(row_index, dtype=np.int64)[:, None]
    j = np.arange(L_kv, dtype=np.int64)[None, :]
    pos = t + (L_kv - L_q)
    ok = np.ones((t.shape[0], L_kv), dtype=bool)
    if draft_mask is not None:
        dm = np.asarray(draft_mask, dtype=bool)
        i = j - (L_kv - L_q)                     # draft index of key j
        in_drafts = i >= 0
        seen = dm[t, np.clip(i, 0, L_q - 1)]
        ok &= ~in_drafts | seen
    elif causal:
        ok &= j <= pos
    if window_left >= 0:
        ok &= j >= pos - window_left
    return ok


def attention(q, k, v, alpha, beta, causal, window_left=-1, sinks=None,
              row_index=None, L_q=None, draft_mask=None):
    """Softmax attention of one request.

    q [R, H_qo, d_qk], k [L_kv, H_kv, d_qk], v [L_kv, H_kv, d_vo], float64.
    ``row_index`` (default 0..R-1) names which of the request's L_q query rows
    the R rows of q are, so that a sample of rows can be computed alone.
    Returns out [R, H_qo, d_vo] = beta * softmax(alpha * q k^T + mask) v and
    lse [R, H_qo] = log(sum over allowed keys of exp(alpha * q.k)).
    """
    R, H_qo, _ = q.shape
    L_kv, H_kv, d_vo = v.shape
    if H_qo % H_kv:
        raise ValueError("num_heads_qo must be a multiple of num_heads_kv")
    G = H_qo // H_kv
    if row_index is None:
        row_index = np.arange(R)
    if L_q is None:
        L_q = R
    ok = allowed_mask(row_index, L_q, L_kv, causal, window_left, draft_mask)
    any_ok = ok.any(axis=1)
    out = np.zeros((R, H_qo, d_vo), dtype=np.float64)
    lse = np.full((R, H_qo), -np.inf, dtype=np.float64)
    for h in range(H_qo):
        kh = h // G
        s = alpha * (q[:, h, :] @ k[:, kh, :].T)            # [R, L_kv]
        s = np.where(ok, s, -np.inf)
        m_s = np.where(any_ok, s.max(axis=1, initial=-np.inf), 0.0)
        p_s = np.exp(s - m_s[:, None])                      # masked -> 0
        z_s = p_s.sum(axis=1)
        lse[:, h] = np.where(any_ok, m_s + np.log(np.where(any_ok, z_s, 1.0)), -np.inf)
        # softmax denominator, with the sink logit when one is given
        if sinks is not None:
            sig = float(sinks[h])
            m = np.where(any_ok, np.maximum(m_s, sig), sig)
            p = np.exp(s - m[:, None])
            z = p.sum(axis=1) + np.exp(sig - m)
        else:
            p, z = p_s, np.where(any_ok, z_s, 1.0)
        o = (p @ v[:, kh, :]) / z[:, None]
        out[:, h, :] = np.where(any_ok[:, None], beta * o, 0.0)
    return out, lse


def _exclusive_cumsum(x):
    c = np.zeros(len(x) + 1, dtype=np.int64)
    c[1:] = np.cumsum(np.asarray(x, dtype=np.int64))
    return c


def batch_prefill(q, q_fmt, k_cache, v_cache, kv_fmt, block_tables,
                  seq_lens_q, seq_lens_kv, scale, causal, kv_layout,
                  q_scale=1.0, k_scale=1.0, v_scale=1.0, rows=None):
    """Batch prefill over a paged cache (prefill page).

    q: raw bits [sum L_q, H_qo, d_qk]; request b owns rows
    cq[b] .. cq[b+1]-1 with cq the exclusive cumsum of ``seq_lens_q``.
    k_cache / v_cache: raw bits in ``kv_layout``. Values are dequantised as
    stored value * per-tensor scale, then attention with softmax scale
    ``scale``. ``rows``: optional list of (b, t) pairs to compute alone.
    Returns (out [sum L_q or len(rows), H_qo, d_vo], lse [.., H_qo]).
    """
    cq = _exclusive_cumsum(seq_lens_q)
    H_qo = q.shape[1]
    d_vo = v_cache.shape[-1]
    if rows is None:
        want = {b: np.arange(int(seq_lens_q[b])) for b in range(len(seq_lens_q))}
        n_out = int(cq[-1])
    else:
        want = {}
        for b, t in rows:
            want.setdefault(int(b), []).append(int(t))
        n_out = len(rows)
    out = np.zeros((n_out, H_qo, d_vo))
    lse = np.full((n_out, H_qo), -np.inf)
    for b, ts in want.items():
        ts = np.asarray(ts, dtype=np.int64)
        L_q, L_kv = int(seq_lens_q[b]), int(seq_lens_kv[b])
        kb = decode_bits(gather_pages(k_cache, block_tables[b], L_kv, kv_layout), kv_fmt) * k_scale
        vb = decode_bits(gather_pages(v_cache, block_tables[b], L_kv, kv_layout), kv_fmt) * v_scale
        qb = decode_bits(q[cq[b] + ts], q_fmt) * q_scale
        o, l = attention(qb, kb, vb, alpha=scale, beta=1.0, causal=causal,
                         row_index=ts, L_q=L_q)
        if rows is None:
            out[cq[b]:cq[b + 1]] = o
            lse[cq[b]:cq[b + 1]] = l
        else:
            idx = [i for i, (bb, _) in enumerate(rows) if int(bb) == b]
            out[idx] = o
            lse[idx] = l
    return out, lse


def batch_prefill_ragged(q, q_fmt, k, v, kv_fmt, seq_lens_q, seq_lens_kv, scale,
                         causal, q_scale=1.0, k_scale=1.0, v_scale=1.0,
                         offsets_q=None, offsets_o=None, offsets_k=None, offsets_v=None,
                         offsets_stats=None, out_rows=None):
    """Batch prefill without paging (prefill page: k_cache / v_cache of shape
    (total KV length, H_kv, d) when paging is off; batch_offsets_q/o/k/v/
    stats). Request b's L_q query rows start at row offsets_q[b] of q, its
    L_kv key and value rows at offsets_k[b] / offsets_v[b] of k / v, and its
    output and LSE rows at offsets_o[b] / offsets_stats[b]. An absent offset
    array is the exclusive prefix sum of the lengths (rows packed in request
    order). Offsets count rows (tokens). q, k, v are raw bits.
    Returns (out [out_rows, H_qo, d_vo], lse [out_rows, H_qo]); rows no
    request writes are NaN. out_rows defaults to sum L_q.
    """
    B = len(seq_lens_q)
    cq = _exclusive_cumsum(seq_lens_q)
    ck = _exclusive_cumsum(seq_lens_kv)
    pick = lambda off, dflt: dflt[:B] if off is None else np.asarray(off, dtype=np.int64)
    oq, oo = pick(offsets_q, cq), pick(offsets_o, cq)
    ok_, ov = pick(offsets_k, ck), pick(offsets_v, ck)
    os_ = pick(offsets_stats, cq)
    n = int(cq[-1]) if out_rows is None else int(out_rows)
    H_qo, d_vo = q.shape[1], v.shape[-1]
    out = np.full((n, H_qo, d_vo), np.nan)
    lse = np.full((n, H_qo), np.nan)
    for b in range(B):
        L_q, L_kv = int(seq_lens_q[b]), int(seq_lens_kv[b])
        if L_q == 0:
            continue
        qb = decode_bits(q[oq[b]:oq[b] + L_q], q_fmt) * q_scale
        kb = decode_bits(k[ok_[b]:ok_[b] + L_kv], kv_fmt) * k_scale
        vb = decode_bits(v[ov[b]:ov[b] + L_kv], kv_fmt) * v_scale
        o, l = attention(qb, kb, vb, alpha=scale, beta=1.0, causal=causal)
        out[oo[b]:oo[b] + L_q] = o
        lse[os_[b]:os_[b] + L_q] = l
    return out, lse


def batch_decode(query, q_fmt, k_cache, v_cache, kv_fmt, block_tables,
                 seq_lens, bmm1_scale, bmm2_scale, window_left, sinks,
                 kv_layout, q_len_per_req=1, requests=None, cum_seq_lens_q=None,
                 spec_mask=None):
    """Batch decode over ``block_tables`` (decode page).

    query: raw bits [num_tokens, H_qo, d]. Request b's queries are its last
    q_len_b positions, causal among themselves: rows b*q_len_per_req ..
    (q_len_b = q_len_per_req), or, with ``cum_seq_lens_q`` ([batch + 1],
    the page's variable-length form), rows cum_seq_lens_q[b] ..
    cum_seq_lens_q[b+1] - 1. ``spec_mask`` ([batch, Q, Q], Q the largest
    query count) replaces the causal rule among a request's drafts: draft t
    sees draft i when spec_mask[b, t, i] is nonzero (see ``allowed_mask``).
    Scores are bmm1_scale * q.k on the stored K values; the output is
    bmm2_scale * softmax(.) V with the per-head ``sinks`` logits in the
    denominator and the inclusive left window. ``requests``: optional subset
    of request indices (their rows, in order, are the output).
    Returns out [rows, H_qo, d].
    """
    B = len(seq_lens)
    if cum_seq_lens_q is None:
        cum = np.arange(B + 1, dtype=np.int64) * q_len_per_req
    else:
        cum = np.asarray(cum_seq_lens_q, dtype=np.int64)
    if requests is None:
        requests = range(B)
    requests = list(requests)
    H_qo = query.shape[1]
    d_vo = v_cache.shape[-1]
    n_out = sum(int(cum[b + 1] - cum[b]) for b in requests)
    out = np.zeros((n_out, H_qo, d_vo))
    r = 0
    for b in requests:
        ql = int(cum[b + 1] - cum[b])
        L_kv = int(seq_lens[b])
        kb = decode_bits(gather_pages(k_cache, block_tables[b], L_kv, kv_layout), kv_fmt)
        vb = decode_bits(gather_pages(v_cache, block_tables[b], L_kv, kv_layout), kv_fmt)
        qb = decode_bits(query[cum[b]:cum[b + 1]], q_fmt)
        dm = None if spec_mask is None else np.asarray(spec_mask)[b, :ql, :ql] != 0
        o, _ = attention(qb, kb, vb, alpha=bmm1_scale, beta=bmm2_scale,
                         causal=True, window_left=window_left, sinks=sinks,
                         draft_mask=dm)
        out[r:r + ql] = o
        r += ql
    return out


def allowed_pairs(seq_lens_q, seq_lens_kv, causal, window_left=-1):
    """Number of allowed (query row, key) pairs summed over the batch."""
    total = 0
    for L_q, L_kv in zip(seq_lens_q, seq_lens_kv):
        total += int(allowed_mask(np.arange(int(L_q)), int(L_q), int(L_kv),
                                  causal, window_left).sum())
    return total


def keys_read(seq_lens, q_len_per_req, window_left):
    """Keys that at least one query of a decode request may attend to."""
    total = 0
    for L_kv in seq_lens:
        ok = allowed_mask(np.arange(q_len_per_req), q_len_per_req, int(L_kv),
                          True, window_left)
        total += int(ok.any(axis=0).sum())
    return total
