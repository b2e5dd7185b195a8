"""Long contexts and large tensors, checked on sampled outputs against the
float64 oracle.

* decode over requests of up to 261k tokens: several hundred splits per (request,
  kv head) and a long merge;
* one prefill request of 16384 queries over 65536 keys;
* a prefill batch whose q and out tensors pass 2^31 bytes, so the row
  offsets of the last requests need 64-bit address arithmetic.
"""

import numpy as np
import pytest
import torch

import workloads
from tests.helpers import assert_lse_close, assert_out_close, oracle_decode, oracle_prefill
from tests.test_gpu_decode import run_decode
from tests.test_gpu_prefill import _rows_of, run_prefill

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def pkv():
    import attention_paged_kv_cache_amd as m
    return m


@pytest.mark.parametrize("kv_dtype,ps,ql,window,sinks", [
    (torch.bfloat16, 16, 1, -1, False),
    (torch.float8_e4m3fn, 64, 4, 100000, True),
])
def test_decode_256k_tokens(pkv, kv_dtype, ps, ql, window, sinks):
    # seed 118 draws 261019, 229886 and 152231 tokens
    w = workloads.batch_decode(DEV, seed=118, batch=3, seq=(150000, 262144), num_qo_heads=8,
                               num_kv_heads=2, page_size=ps, q_len_per_req=ql,
                               kv_dtype=kv_dtype, window_left=window, sinks=sinks)
    print(f"decode seq {w['seq_lens'].tolist()} {kv_dtype} page {ps} q_len {ql} "
          f"window {window}", flush=True)
    out = run_decode(pkv, w)
    assert_out_close(out, oracle_decode(w), out.dtype)


def _sampled(w, picks):
    """(b, t) rows: the first and last row of each picked request plus
    seeded interior rows."""
    rng = np.random.default_rng(91)
    lq = w["seq_lens_q"].numpy()
    rows = []
    for b in picks:
        rows += [(b, 0), (b, int(lq[b]) - 1)]
        rows += [(b, int(t)) for t in rng.integers(0, lq[b], 6)]
    return rows


def test_prefill_one_request_64k_keys(pkv):
    w = workloads.batch_prefill(DEV, seed=92, batch=2, q_len=(16384, 16384),
                                prefix=(49152, 49152), pool_pages=2 * 4096 + 16)
    w["seq_lens_q"][1] = 700  # and a short one beside it
    w["seq_lens_kv"][1] = 900
    w["q"] = w["q"][:16384 + 700]
    print(f"prefill lens_q {w['seq_lens_q'].tolist()} lens_kv {w['seq_lens_kv'].tolist()}",
          flush=True)
    out, lse = run_prefill(pkv, w)
    rows = _sampled(w, [0, 0, 0, 1])
    ref_o, ref_l = oracle_prefill(w, rows=rows)
    assert_out_close(_rows_of(out, w, rows), ref_o, out.dtype)
    assert_lse_close(_rows_of(lse, w, rows), ref_l)


def test_prefill_q_and_out_past_2gib(pkv):
    # 520 requests of 512 tokens, 32 qo heads: q and out hold
    # 266240 * 32 * 128 bf16 = 2.18e9 bytes each
    B = 520
    w = workloads.batch_prefill(DEV, seed=93, batch=B, q_len=(512, 512), prefix=(0, 0),
                                pool_pages=B * 32 + 8)
    assert w["q"].numel() * 2 > 2 ** 31
    print(f"prefill {B} x 512 tokens, q {w['q'].numel() * 2 / 2 ** 30:.2f} GiB", flush=True)
    out, lse = run_prefill(pkv, w)
    # the last requests sit past the 2 GiB mark in q and out
    rows = _sampled(w, [0, B - 40, B - 2, B - 1])
    ref_o, ref_l = oracle_prefill(w, rows=rows)
    assert_out_close(_rows_of(out, w, rows), ref_o, out.dtype)
    assert_lse_close(_rows_of(lse, w, rows), ref_l)
    assert torch.isfinite(out[-512:].float()).all()
