"""GPU parity of batch decode (and append followed by decode) against the
float64 oracle. Bar: |out - ref| <= 2e-2 + half an output ulp of ref."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import assert_out_close, bits, fmt, oracle_decode

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def pkv():
    import attention_paged_kv_cache_amd as m
    return m


def run_decode(pkv, w, kv_cache=None, out_dtype=None):
    kv = w["kv_cache"] if kv_cache is None else kv_cache
    ws = torch.zeros(max(pkv.decode_workspace_size(
        w["seq_lens"].shape[0], w["q_len_per_req"], w["num_qo_heads"], w["num_kv_heads"],
        w["head_dim"], w["max_seq_len"], w["window_left"]), 16), dtype=torch.uint8, device=DEV)
    sinks = None if w["sinks"] is None else w["sinks"].to(DEV)
    out = pkv.batch_decode_with_kv_cache(
        w["query"], kv, ws, w["block_tables"].to(DEV), w["seq_lens"].to(DEV), w["max_seq_len"],
        bmm1_scale=w["bmm1_scale"], bmm2_scale=w["bmm2_scale"], window_left=w["window_left"],
        sinks=sinks, kv_layout=w["layout"], q_len_per_req=w["q_len_per_req"],
        out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def check(pkv, w, requests=None):
    out = run_decode(pkv, w)
    ref = oracle_decode(w, requests)
    if requests is not None:
        ql = w["q_len_per_req"]
        idx = torch.tensor([b * ql + i for b in requests for i in range(ql)], device=DEV)
        out = out.index_select(0, idx)
    err = assert_out_close(out, ref, out.dtype)
    print(f"max |out err| {err:.3g}", flush=True)
    return out


def small(**kw):
    args = dict(device=DEV, seed=40, batch=5, seq=(1, 700))
    args.update(kw)
    return workloads.batch_decode(**args)


@pytest.mark.parametrize("hqo,hkv", [(32, 8), (8, 8), (16, 1)])
def test_bf16(pkv, hqo, hkv):
    check(pkv, small(num_qo_heads=hqo, num_kv_heads=hkv, seed=hqo + hkv))


@pytest.mark.parametrize("ps,layout", [(16, "NHD"), (32, "HND"), (64, "NHD")])
def test_layouts_and_pages(pkv, ps, layout):
    check(pkv, small(page_size=ps, layout=layout, seed=ps))


@pytest.mark.parametrize("ps,layout,kv", [(16, "HND", "bf16"), (16, "NHD", "e4m3"),
                                          (32, "NHD", "bf16"), (32, "HND", "e4m3"),
                                          (64, "HND", "bf16"), (64, "NHD", "e4m3")])
@pytest.mark.parametrize("ql,hqo,hkv", [(1, 8, 2), (4, 16, 2)])
def test_steps_per_wave(pkv, ps, layout, kv, ql, hqo, hkv):
    # One plan for the batch (its chunk, 640 keys here, comes from the
    # longest request), so each wave streams 0 to 5 32-key steps: odd and
    # even counts (steps go in pairs; an odd last pair skips its second
    # compute), a partial last step, waves with no keys, and sequence ends
    # in either half of a 16-token page (whose second half is another page).
    lens = [max(ql, 1), 20, 33, 64, 95, 130, 161, 300, 371, 517]
    kv_dtype = torch.float8_e4m3fn if kv == "e4m3" else torch.bfloat16
    w = workloads.batch_decode(device=DEV, seed=70 + ps + ql, batch=len(lens), seq=(517, 517),
                               num_qo_heads=hqo, num_kv_heads=hkv, page_size=ps,
                               q_len_per_req=ql, kv_dtype=kv_dtype, layout=layout)
    w["seq_lens"] = torch.tensor(lens, dtype=torch.uint32)
    w["max_seq_len"] = max(lens)
    assert pkv.decode_workspace_size(len(lens), ql, hqo, hkv, 128, max(lens), -1) == 0
    check(pkv, w)


def test_long_sequences_split_kv(pkv):
    # long enough that every request needs several splits
    check(pkv, small(batch=3, seq=(3000, 9000), seed=41))


@pytest.mark.parametrize("window", [-1, 6000])
def test_many_rows_split_kv_with_sinks(pkv, window):
    # 32 query rows per kv head and sequences long enough for several splits:
    # the merge combines partials and the sink term
    check(pkv, small(batch=2, seq=(9000, 20000), q_len_per_req=4, num_qo_heads=16,
                     num_kv_heads=2, window_left=window, sinks=True, seed=60))


@pytest.mark.parametrize("ql,window,sinks", [(4, 100, True), (2, -1, True), (4, 0, False),
                                             (3, 37, False), (1, 5000, True)])
def test_multi_query_window_sinks(pkv, ql, window, sinks):
    check(pkv, small(q_len_per_req=ql, window_left=window, sinks=sinks, num_qo_heads=16,
                     num_kv_heads=2, seq=(1, 900), seed=50 + ql))


def test_fp8_kv(pkv):
    w = small(kv_dtype=torch.float8_e4m3fn, q_len_per_req=4, window_left=200, sinks=True,
              num_qo_heads=16, num_kv_heads=2, page_size=32, seed=42)
    w["bmm1_scale"], w["bmm2_scale"] = 0.7 / np.sqrt(128), 1.3
    check(pkv, w)


def test_rows_64(pkv):
    # q_len * G = 64, the largest supported row count per kv head
    check(pkv, small(q_len_per_req=4, num_qo_heads=16, num_kv_heads=1, seq=(100, 2000),
                     seed=43))


def test_seq_shorter_than_q_len(pkv):
    w = small(q_len_per_req=4, num_qo_heads=4, num_kv_heads=4, seed=44, batch=3, seq=(1, 3))
    check(pkv, w)


# ---- fp16 queries, output types other than the query's, empty requests ------

def _merged(pkv, w):
    """True when a decode call's plan has several splits per (request, kv
    head): partials go to the workspace and the merge kernel writes the
    output. False: each unit writes its output directly."""
    return (pkv.decode_workspace_size(w["seq_lens"].shape[0], w["q_len_per_req"],
                                      w["num_qo_heads"], w["num_kv_heads"], 128,
                                      w["max_seq_len"], w["window_left"]) > 0)


@pytest.mark.parametrize("kv_dtype", [torch.float16, torch.float8_e4m3fn])
@pytest.mark.parametrize("seq,window,seed,merged", [((1, 900), -1, 130, False),
                                                    ((3000, 9000), 2500, 131, True)])
def test_f16_query(pkv, kv_dtype, seq, window, seed, merged):
    # an fp16 query over an fp16 or e4m3 cache (e4m3 widened exactly to
    # fp16), fp16 output; short sequences take the direct write, long ones
    # the split partials and the merge kernel
    w = small(seed=seed, seq=seq, batch=4, q_len_per_req=2, window_left=window, sinks=True,
              num_qo_heads=16, num_kv_heads=2, kv_dtype=kv_dtype, q_dtype=torch.float16,
              page_size=32)
    assert _merged(pkv, w) == merged
    out = check(pkv, w)
    assert out.dtype == torch.float16


@pytest.mark.parametrize("q_dtype,kv_dtype,out_dtype", [
    (torch.bfloat16, torch.bfloat16, torch.float16),
    (torch.bfloat16, torch.float8_e4m3fn, torch.float16),
    (torch.float16, torch.float16, torch.bfloat16),
    (torch.float16, torch.float8_e4m3fn, torch.bfloat16),
])
@pytest.mark.parametrize("seq,seed,merged", [((1, 900), 132, False), ((3000, 9000), 133, True)])
def test_output_dtype_other_than_query(pkv, q_dtype, kv_dtype, out_dtype, seq, seed, merged):
    # out_dtype picks the output's 16-bit type independently of the query;
    # both writers (direct and merge) round to it
    w = small(seed=seed, seq=seq, batch=4, q_len_per_req=3, window_left=-1, sinks=True,
              num_qo_heads=8, num_kv_heads=2, kv_dtype=kv_dtype, q_dtype=q_dtype)
    assert _merged(pkv, w) == merged
    out = run_decode(pkv, w, out_dtype=out_dtype)
    assert out.dtype == out_dtype
    err = assert_out_close(out, oracle_decode(w), out_dtype)
    print(f"max |out err| {err:.3g}", flush=True)


@pytest.mark.parametrize("seq,out_dtype,merged", [((300, 900), torch.bfloat16, False),
                                                  ((4000, 9000), torch.float16, True),
                                                  ((300, 900), torch.float8_e4m3fn, False),
                                                  ((4000, 9000), torch.float8_e4m3fn, True)])
def test_zero_length_request(pkv, seq, out_dtype, merged):
    # a request whose sequence is empty: its query rows see no key and come
    # back zero, whether the batch's plan writes outputs directly (one
    # split) or through the merge kernel; the other requests are unaffected
    w = small(seed=134, batch=4, seq=seq, q_len_per_req=2, sinks=True, num_qo_heads=8,
              num_kv_heads=2, window_left=-1)
    sl = w["seq_lens"].to(torch.int64)
    sl[1] = 0
    w = dict(w, seq_lens=sl.to(torch.uint32))
    assert _merged(pkv, w) == merged
    ws = torch.zeros(max(pkv.decode_workspace_size(4, 2, 8, 2, 128, w["max_seq_len"], -1), 16),
                     dtype=torch.uint8, device=DEV)
    out = torch.full(w["query"].shape, float("nan"), dtype=torch.float32,
                     device=DEV).to(out_dtype)
    pkv.batch_decode_with_kv_cache(
        w["query"], w["kv_cache"], ws, w["block_tables"].to(DEV), w["seq_lens"].to(DEV),
        w["max_seq_len"], bmm1_scale=w["bmm1_scale"], bmm2_scale=w["bmm2_scale"],
        sinks=w["sinks"].to(DEV), kv_layout=w["layout"], q_len_per_req=2, out=out,
        out_dtype=out_dtype)
    torch.cuda.synchronize()
    if out_dtype == torch.float8_e4m3fn:
        raw = out.view(torch.uint8)
        assert torch.all((raw[2:4] & 0x7F) == 0), "empty request's rows must be zero"
        ref = oracle_decode(w)
        check_fp8_out(out, ref, 1.0)
    else:
        assert torch.all(out[2:4].float() == 0), "empty request's rows must be zero"
        assert_out_close(out, oracle_decode(w), out_dtype)


def test_e4m3_decode_table_exhaustive(pkv):
    # seq_len 1 and q = 0: the output is bmm2 * v[0] exactly, so V rows
    # holding all 256 codes read back the GPU's e4m3fn decode (bf16 holds
    # every e4m3fn value exactly). NaN codes must come back NaN.
    B, H, D, ps = 2, 1, 128, 16
    kv = torch.zeros(B, 2, H, ps, D, dtype=torch.uint8, device=DEV)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(2, 128)
    kv[:, 1, 0, 0, :] = codes.to(DEV)
    kv = kv.view(torch.float8_e4m3fn)
    q = torch.zeros(B, H, D, dtype=torch.bfloat16, device=DEV)
    bt = torch.arange(B, dtype=torch.int32).reshape(B, 1)
    w = dict(query=q, kv_cache=kv, block_tables=bt,
             seq_lens=torch.ones(B, dtype=torch.int32).to(torch.uint32), max_seq_len=1,
             page_size=ps, num_qo_heads=H, num_kv_heads=H, head_dim=D, q_len_per_req=1,
             bmm1_scale=1.0, bmm2_scale=1.0, window_left=-1, sinks=None, layout="HND")
    out = run_decode(pkv, w).float().cpu().numpy().reshape(256).astype(np.float64)
    tab = oracle.e4m3fn_table()
    assert np.array_equal(np.isnan(out), np.isnan(tab))
    ok = ~np.isnan(tab)
    assert np.array_equal(out[ok], tab[ok])


def test_deterministic(pkv):
    w = small(seed=45, seq=(2000, 5000), q_len_per_req=2, sinks=True)
    a = run_decode(pkv, w)
    b = run_decode(pkv, w)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_full_size_bf16_sampled(pkv):
    w = workloads.batch_decode(DEV)
    out = run_decode(pkv, w)
    assert torch.isfinite(out.float()).all()
    reqs = [0, 7, 100, int(torch.argmax(w["seq_lens"].to(torch.int64))),
            int(torch.argmin(w["seq_lens"].to(torch.int64)))]
    ref = oracle_decode(w, reqs)
    assert_out_close(out.index_select(0, torch.tensor(reqs, device=DEV)), ref, out.dtype)


def test_full_size_append_then_spec_decode_sampled(pkv):
    w = workloads.spec_decode(DEV)
    kv = w["kv_cache"]
    seq = w["seq_lens"].to(torch.int32).to(DEV)
    bi, pos = pkv.get_batch_indices_positions(w["append_indptr"].to(DEV), seq,
                                              w["k_append"].shape[0])
    pkv.append_paged_kv_cache(w["k_append"], w["v_append"], bi, pos, kv,
                              w["kv_indices"].to(DEV), w["kv_indptr"].to(DEV),
                              w["kv_last_page_len"].to(DEV), kv_layout="HND")
    out = run_decode(pkv, w)
    assert torch.isfinite(out.float()).all()
    reqs = [0, 9, 33, 63]
    ref = oracle_decode(w, reqs)
    idx = torch.tensor([b * 4 + i for b in reqs for i in range(4)], device=DEV)
    assert_out_close(out.index_select(0, idx), ref, out.dtype)
    # the appended rows are what the last 4 positions of each request hold
    b = 9
    L = int(w["seq_lens"][b])
    ps = w["page_size"]
    for i in range(4):
        p = L - 4 + i
        page = int(w["block_tables"][b, p // ps])
        assert torch.equal(kv[page, 0, :, p % ps].view(torch.uint8),
                           w["k_append"][b * 4 + i].view(torch.uint8))


@pytest.mark.parametrize("kv_dtype", [torch.bfloat16, torch.float8_e4m3fn])
def test_poisoned_unused_memory_is_never_read(pkv, kv_dtype):
    # NaN in every byte decode must not read: pool pages no request uses,
    # tail slots past each sequence in its last page, and block-table padding
    # pointing at a NaN page. The output must be bit-identical.
    w = small(seed=47, batch=6, seq=(1, 900), q_len_per_req=3, window_left=150, sinks=True,
              num_qo_heads=8, num_kv_heads=2, kv_dtype=kv_dtype)
    kv = w["kv_cache"]
    extra = 3
    k8 = kv.view(torch.uint8)
    pad = torch.zeros((extra,) + tuple(k8.shape[1:]), dtype=torch.uint8, device=DEV)
    kv = torch.cat([k8, pad]).view(kv_dtype)
    w = dict(w, kv_cache=kv)
    out0 = run_decode(pkv, w)
    nan = 0x7F if kv_dtype == torch.float8_e4m3fn else 0x7FC0
    kvp = kv.clone()
    raw = kvp.view(torch.uint8) if kv_dtype == torch.float8_e4m3fn else kvp.view(torch.int16)
    n_pages = kv.shape[0] - extra
    raw[n_pages:] = nan
    ps = w["page_size"]
    for b in range(w["block_tables"].shape[0]):
        L = int(w["seq_lens"][b])
        if L % ps:
            p = int(w["block_tables"][b, L // ps])
            raw[p, :, :, L % ps:] = nan  # HND: [page][K/V][head][slot][d]
    bt = w["block_tables"].clone()
    bt[bt < 0] = n_pages
    out1 = run_decode(pkv, dict(w, kv_cache=kvp, block_tables=bt))
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))


# ---- fp8 output with o_scale, device-tensor scales ---------------------------

def _bf16_exact(vals):
    """float64 values -> the bf16 values torch rounds them to (as float64)."""
    return torch.tensor(vals, dtype=torch.float64).to(torch.bfloat16).double().numpy()


def _encode_cases():
    tab = oracle.e4m3fn_table()
    mags = tab[:127]
    mid = (mags[:-1] + mags[1:]) / 2
    # the bf16 neighbours of each midpoint: one bf16 ulp either side
    bits16 = torch.tensor(mid, dtype=torch.bfloat16).view(torch.int16)
    below = (bits16 - 1).view(torch.bfloat16).double().numpy()
    above = (bits16 + 1).view(torch.bfloat16).double().numpy()
    extra = [448.0, 450.0, 464.0, 480.0, 1000.0, 2.0 ** 127, 0.0, 2.0 ** -12, 2.0 ** -10]
    v = np.concatenate([mags, mid, below, above, extra])
    v = np.concatenate([v, -v])
    assert np.array_equal(_bf16_exact(v), v)  # every case is a bf16 value
    return v


@pytest.mark.parametrize("bmm2,o_scale", [(1.0, 1.0), (0.5, 4.0), (2.0, 0.25)])
def test_fp8_output_encoding_exact(pkv, bmm2, o_scale):
    # one key per request and q = 0: out = bmm2 * v[0] exactly, so the stored
    # codes must be the oracle's encoding of bmm2 * v / o_scale, bit for bit
    # (powers of two keep the scaling exact); NaN rows must come back NaN
    v = _encode_cases()
    v = np.concatenate([v, [np.nan, -np.nan]])
    n_req = (v.size + 127) // 128
    vals = np.zeros(n_req * 128)
    vals[:v.size] = v
    B, H, D, ps = n_req, 1, 128, 16
    kv = torch.zeros(B, 2, H, ps, D, dtype=torch.bfloat16)
    kv[:, 1, 0, 0, :] = torch.tensor(vals.reshape(B, D), dtype=torch.float64).to(torch.bfloat16)
    q = torch.zeros(B, H, D, dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(16, dtype=torch.uint8, device=DEV)
    out = pkv.batch_decode_with_kv_cache(
        q, kv.to(DEV), ws, torch.arange(B, dtype=torch.int32).reshape(B, 1).to(DEV),
        torch.ones(B, dtype=torch.int32).to(DEV), 1, bmm1_scale=1.0, bmm2_scale=bmm2,
        out_dtype=torch.float8_e4m3fn, o_scale=o_scale)
    torch.cuda.synchronize()
    got = out.view(torch.uint8).cpu().numpy().reshape(-1)
    want = oracle.encode_e4m3fn(vals * bmm2 / o_scale)
    # the accumulation starts from +0, so a zero comes back as +0 whatever
    # the sign of v: zeros compare by value
    nan, zero = np.isnan(vals), vals == 0
    exact = ~nan & ~zero
    bad = np.nonzero(got[exact] != want[exact])[0]
    for i in bad[:8]:
        print(f"v {vals[exact][i]!r}: got 0x{got[exact][i]:02x} want 0x{want[exact][i]:02x}")
    assert bad.size == 0
    assert np.all((got[zero] & 0x7F) == 0)
    assert np.all((got[nan] & 0x7F) == 0x7F)


def _e4m3_ulp(y):
    """Spacing of e4m3fn values at magnitude y (subnormal spacing below 2^-6)."""
    y = np.maximum(np.abs(y), 2.0 ** -6)
    return np.exp2(np.floor(np.log2(y)) - 3)


def check_fp8_out(out, ref, o_scale, atol=2e-2):
    """Stored codes against the oracle: the unquantised values may differ by
    atol, and the code then lies within one e4m3 spacing of the larger
    magnitude (nearest rounding of a value at most atol away); references
    beyond the format's range compare against the saturated value."""
    dec = oracle.decode_bits(out.view(torch.uint8).cpu().numpy(), oracle.formats.E4M3) * o_scale
    ref = np.clip(np.asarray(ref, dtype=np.float64), -448.0 * o_scale, 448.0 * o_scale)
    tol = atol + _e4m3_ulp((np.abs(ref) + atol) / o_scale) * o_scale
    err = np.abs(dec - ref)
    assert np.all(err <= tol), float((err - tol).max())
    return float(err.max())


@pytest.mark.parametrize("seq,seed", [((1, 900), 80), ((3000, 9000), 81)])
def test_fp8_output_against_oracle(pkv, seq, seed):
    # short sequences take the single-split write, long ones the merge kernel
    w = small(seed=seed, seq=seq, batch=4, q_len_per_req=3, window_left=2000, sinks=True,
              num_qo_heads=8, num_kv_heads=2)
    o_scale = 0.37
    ws = torch.zeros(max(pkv.decode_workspace_size(4, 3, 8, 2, 128, w["max_seq_len"], 2000), 16),
                     dtype=torch.uint8, device=DEV)
    out = pkv.batch_decode_with_kv_cache(
        w["query"], w["kv_cache"], ws, w["block_tables"].to(DEV), w["seq_lens"].to(DEV),
        w["max_seq_len"], bmm1_scale=w["bmm1_scale"], bmm2_scale=1.7, window_left=2000,
        sinks=w["sinks"].to(DEV), kv_layout=w["layout"], q_len_per_req=3,
        out_dtype=torch.float8_e4m3fn, o_scale=o_scale)
    torch.cuda.synchronize()
    ref = oracle_decode(dict(w, bmm2_scale=1.7))
    err = check_fp8_out(out, ref, o_scale)
    print(f"max |dec(code) * o_scale - ref| {err:.3g}", flush=True)


def test_device_tensor_scales_equal_float_scales(pkv):
    w = small(seed=82, seq=(500, 6000), q_len_per_req=2, sinks=True, num_qo_heads=8,
              num_kv_heads=2, kv_dtype=torch.float8_e4m3fn, page_size=32)
    b1, b2 = 0.071, 1.9
    a = run_decode(pkv, dict(w, bmm1_scale=b1, bmm2_scale=b2))
    t1 = torch.tensor([b1], dtype=torch.float32, device=DEV)
    t2 = torch.tensor([b2], dtype=torch.float32, device=DEV)
    b = run_decode(pkv, dict(w, bmm1_scale=t1, bmm2_scale=t2))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # a negative device bmm1 flips the query's sign inside the kernel
    c = run_decode(pkv, dict(w, bmm1_scale=-b1, bmm2_scale=b2))
    d = run_decode(pkv, dict(w, bmm1_scale=torch.tensor([-b1], device=DEV), bmm2_scale=t2))
    assert torch.equal(c.view(torch.int16), d.view(torch.int16))
    assert_out_close(d, oracle_decode(dict(w, bmm1_scale=-b1, bmm2_scale=b2)), d.dtype)


# ---- variable-length queries and the speculative-decoding mask ----------------

def oracle_decode_ragged(w, cum, mask=None):
    from workloads import compact_pages
    seq = w["seq_lens"].to(torch.int64)
    used = [(int(s) + w["page_size"] - 1) // w["page_size"] for s in seq]
    sub, bt = compact_pages(w["kv_cache"], w["block_tables"], used)
    sinks = None if w["sinks"] is None else w["sinks"].double().numpy()
    return oracle.batch_decode(
        bits(w["query"]), fmt(w["query"]), bits(sub[:, 0]), bits(sub[:, 1]), fmt(w["kv_cache"]),
        bt.numpy(), seq.numpy(), w["bmm1_scale"], w["bmm2_scale"], w["window_left"], sinks,
        w["layout"], cum_seq_lens_q=cum, spec_mask=None if mask is None else mask.cpu().numpy())


def run_ragged(pkv, w, cum, q_max, mask=None, out=None):
    B = w["seq_lens"].shape[0]
    ws = torch.zeros(max(pkv.decode_workspace_size(
        B, q_max, w["num_qo_heads"], w["num_kv_heads"], 128, w["max_seq_len"],
        w["window_left"]), 16), dtype=torch.uint8, device=DEV)
    sinks = None if w["sinks"] is None else w["sinks"].to(DEV)
    r = pkv.batch_decode_with_kv_cache(
        w["query"], w["kv_cache"], ws, w["block_tables"].to(DEV), w["seq_lens"].to(DEV),
        w["max_seq_len"], bmm1_scale=w["bmm1_scale"], bmm2_scale=w["bmm2_scale"],
        window_left=w["window_left"], sinks=sinks, kv_layout=w["layout"], out=out,
        mask=mask, max_q_len=None if cum is None else q_max,
        cum_seq_lens_q=None if cum is None else torch.tensor(cum, dtype=torch.int32, device=DEV),
        q_len_per_req=w["q_len_per_req"] if cum is None else 1)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("seq,kv_dtype,window,seed", [
    ((1, 900), torch.bfloat16, -1, 90),
    ((3000, 9000), torch.bfloat16, 2500, 91),
    ((200, 5000), torch.float8_e4m3fn, 300, 92),
])
def test_variable_length_queries(pkv, seq, kv_dtype, window, seed):
    # ragged query counts 0..4 per request (empty requests included); the
    # rows past the last query are never written
    q_max = 4
    w = small(seed=seed, seq=seq, batch=7, q_len_per_req=q_max, window_left=window, sinks=True,
              num_qo_heads=16, num_kv_heads=4, kv_dtype=kv_dtype, page_size=32)
    counts = np.random.default_rng(seed).integers(0, q_max + 1, size=7)
    counts[2] = 0
    cum = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    out = torch.full_like(w["query"], float("nan"))
    got = run_ragged(pkv, w, cum, q_max, out=out)
    n = int(cum[-1])
    ref = oracle_decode_ragged(w, cum)
    err = assert_out_close(got[:n], ref, got.dtype)
    assert torch.isnan(got[n:].float()).all()
    print(f"counts {counts.tolist()} max |out err| {err:.3g}", flush=True)


def test_uniform_offsets_equal_fixed_query_count(pkv):
    w = small(seed=93, seq=(100, 6000), batch=5, q_len_per_req=3, window_left=1000, sinks=True,
              num_qo_heads=8, num_kv_heads=2)
    a = run_decode(pkv, w)
    cum = (np.arange(6) * 3).astype(np.int32)
    b = run_ragged(pkv, w, cum, 3)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _tree_mask(B, Q, rng):
    # each draft's parent is an earlier draft (or the prefix); a draft sees
    # itself and its ancestors
    m = np.zeros((B, Q, Q), dtype=bool)
    for b in range(B):
        parent = [-1] + [int(rng.integers(-1, i)) for i in range(1, Q)]
        for t in range(Q):
            a = t
            while a >= 0:
                m[b, t, a] = True
                a = parent[a]
    return m


@pytest.mark.parametrize("kind,window,seed", [("tree", -1, 94), ("random", 40, 95),
                                              ("tree", 3, 96)])
def test_spec_mask(pkv, kind, window, seed):
    Q = 4
    w = small(seed=seed, seq=(2, 3000), batch=6, q_len_per_req=Q, window_left=window,
              sinks=True, num_qo_heads=16, num_kv_heads=2)
    rng = np.random.default_rng(seed)
    m = _tree_mask(6, Q, rng) if kind == "tree" else rng.random((6, Q, Q)) < 0.5
    mask = torch.from_numpy(m).to(DEV)
    got = run_ragged(pkv, w, None, Q, mask=mask)
    cum = (np.arange(7) * Q).astype(np.int32)
    ref = oracle_decode_ragged(w, cum, mask)
    err = assert_out_close(got, ref, got.dtype)
    print(f"{kind} mask max |out err| {err:.3g}", flush=True)


def test_lower_triangular_mask_equals_causal(pkv):
    Q = 4
    w = small(seed=97, seq=(50, 7000), batch=5, q_len_per_req=Q, window_left=-1, sinks=True,
              num_qo_heads=8, num_kv_heads=2)
    tril = torch.ones(5, Q, Q, dtype=torch.bool).tril().to(DEV)
    a = run_decode(pkv, w)
    b = run_ragged(pkv, w, None, Q, mask=tril)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_spec_mask_with_variable_length_queries(pkv):
    q_max = 4
    w = small(seed=98, seq=(5, 4000), batch=6, q_len_per_req=q_max, window_left=500, sinks=True,
              num_qo_heads=8, num_kv_heads=2, kv_dtype=torch.float8_e4m3fn, page_size=16)
    rng = np.random.default_rng(98)
    counts = rng.integers(1, q_max + 1, size=6)
    cum = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    m = rng.random((6, q_max, q_max)) < 0.5
    mask = torch.from_numpy(m).to(DEV)
    got = run_ragged(pkv, w, cum, q_max, mask=mask)
    n = int(cum[-1])
    ref = oracle_decode_ragged(w, cum, mask)
    assert_out_close(got[:n], ref, got.dtype)


@pytest.mark.parametrize("ql,hqo,seq,window,seed", [
    (3, 16, (3000, 12000), 5000, 120),   # 48 rows: a full and a half group, split KV
    (4, 16, (1, 900), -1, 121),          # 64 rows: two full groups, one split
    (2, 24, (2000, 9000), -1, 122),      # 48 rows with GQA 24
])
def test_row_groups(pkv, ql, hqo, seq, window, seed):
    # more than 32 rows per kv head run as groups of 32 rows, one workgroup each
    hkv = 1 if hqo == 16 else 2
    check(pkv, small(seed=seed, seq=seq, batch=4, q_len_per_req=ql, num_qo_heads=hqo,
                     num_kv_heads=hkv, window_left=window, sinks=True))


def test_row_groups_with_ragged_queries_and_mask(pkv):
    # 4 x 16 = 64 rows at most: ragged counts leave the second group partial
    # or empty; the draft mask spans both groups
    q_max = 4
    w = small(seed=123, seq=(500, 7000), batch=6, q_len_per_req=q_max, window_left=900,
              sinks=True, num_qo_heads=16, num_kv_heads=1, kv_dtype=torch.float8_e4m3fn,
              page_size=32)
    rng = np.random.default_rng(123)
    counts = np.array([4, 1, 2, 0, 3, 4])
    cum = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    mask = torch.from_numpy(_tree_mask(6, q_max, rng)).to(DEV)
    out = torch.full_like(w["query"], float("nan"))
    got = run_ragged(pkv, w, cum, q_max, mask=mask, out=out)
    n = int(cum[-1])
    assert_out_close(got[:n], oracle_decode_ragged(w, cum, mask), got.dtype)
    assert torch.isnan(got[n:].float()).all()


def test_full_size_spec_decode_mask_and_offsets_reproduce_causal(pkv):
    # the speculative-decoding workload: a lower-triangular draft mask and
    # explicit uniform query offsets each reproduce the implicit causal
    # decode bitwise
    w = workloads.spec_decode(DEV)
    a = run_decode(pkv, w)
    tril = torch.ones(64, 4, 4, dtype=torch.bool).tril().to(DEV)
    b = run_ragged(pkv, w, None, 4, mask=tril)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    cum = (np.arange(65) * 4).astype(np.int32)
    c = run_ragged(pkv, w, cum, 4)
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("ql,hqo,hkv,seq,window,masked,seed", [
    (16, 64, 8, (1, 900), -1, False, 160),        # 128 rows: 16 drafts x GQA 8, one split
    (16, 64, 8, (20000, 40000), -1, True, 161),   # 128 rows, split partials, tree mask
    (32, 64, 8, (100, 3000), 500, False, 162),    # 256 rows
    (64, 16, 1, (50, 700), -1, True, 163),        # 1024 rows: 64 drafts x GQA 16, mask
])
def test_more_than_64_rows(pkv, ql, hqo, hkv, seq, window, masked, seed):
    # more query rows per kv head than one 64-bit mask word: groups of 32
    # rows, one workgroup each, on one XCD; the draft mask stays one word
    # per row (at most 64 drafts)
    w = small(seed=seed, seq=seq, batch=3, q_len_per_req=ql, num_qo_heads=hqo,
              num_kv_heads=hkv, window_left=window, sinks=True,
              kv_dtype=torch.float8_e4m3fn if seed % 2 else torch.bfloat16, page_size=32)
    cum = (np.arange(4) * ql).astype(np.int32)
    mask = None
    if masked:
        mask = torch.from_numpy(_tree_mask(3, ql, np.random.default_rng(seed))).to(DEV)
    got = run_ragged(pkv, w, None, ql, mask=mask)
    err = assert_out_close(got, oracle_decode_ragged(w, cum, mask), got.dtype)
    print(f"{ql * hqo // hkv} rows: max |out err| {err:.3g}", flush=True)
