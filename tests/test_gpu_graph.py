"""The path under HIP graph capture (torch.cuda.CUDAGraph).

Every entry point only enqueues kernels on the caller's stream and reads no
device memory on the host; grid sizes come from host bounds
(max_token_per_sequence, max_sequence_kv, max_seq_len, nnz), so a captured
call replays correctly after the device-resident lengths and values change
within those bounds. Each test replays several times, with eager work and
synchronisations between replays, and checks every replay bitwise against an
eager call on the same inputs, and one replay against the float64 oracle.
"""

import numpy as np
import pytest
import torch

import workloads
from tests.helpers import assert_lse_close, assert_out_close, oracle_decode, oracle_prefill

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def pkv():
    import attention_paged_kv_cache_amd as m
    return m


def capture(fn):
    fn()  # warm-up outside the graph
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_prefill_replays_with_new_lengths(pkv):
    w = workloads.batch_prefill(DEV, seed=70, batch=4, q_len=(40, 300), prefix=(0, 300),
                                pool_pages=256)
    lq0, lkv0 = w["seq_lens_q"].clone(), w["seq_lens_kv"].clone()
    mq, mk = int(lq0.max()), int(lkv0.max())
    lq_d, lkv_d = lq0.to(DEV), lkv0.to(DEV)
    bt = w["block_tables"].to(DEV)
    ws = torch.zeros(pkv.prefill_workspace_size(4), dtype=torch.uint8, device=DEV)
    n_rows, h = w["q"].shape[0], w["num_qo_heads"]
    out_g = torch.empty(n_rows, h, 128, dtype=torch.bfloat16, device=DEV)
    lse_g = torch.empty(n_rows, h, dtype=torch.float32, device=DEV)

    def call(out, lse):
        pkv.batch_prefill_with_kv_cache(
            w["q"], w["k_cache"], w["v_cache"], w["scale"], ws, max_token_per_sequence=mq,
            max_sequence_kv=mk, actual_seq_lens_q=lq_d, actual_seq_lens_kv=lkv_d,
            block_tables=bt, causal=True, out=out, lse=lse, kv_layout=w["layout"])

    g = capture(lambda: call(out_g, lse_g))
    rng = np.random.default_rng(70)
    trials = [(lq0, lkv0),
              (torch.clamp(lq0 // 2, min=1), torch.clamp(lq0 // 2, min=1) + lkv0 // 3),
              (torch.tensor([0, 17, int(lq0[2]), 1], dtype=torch.int32),
               torch.tensor([5, 17, int(lkv0[2]), int(lkv0[3])], dtype=torch.int32))]
    for i, (lq, lkv) in enumerate(trials):
        lq, lkv = lq.to(torch.int32), torch.minimum(lkv.to(torch.int32), lkv0)
        lq_d.copy_(lq)
        lkv_d.copy_(lkv)
        w["q"].copy_(torch.from_numpy(rng.standard_normal(w["q"].shape, dtype=np.float32))
                     .to(torch.bfloat16))
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        out_e, lse_e = torch.empty_like(out_g), torch.empty_like(lse_g)
        call(out_e, lse_e)
        torch.cuda.synchronize()
        n = int(lq.sum())
        print(f"replay {i}: lens_q {lq.tolist()} lens_kv {lkv.tolist()}", flush=True)
        assert torch.equal(out_g[:n].view(torch.int16), out_e[:n].view(torch.int16))
        assert torch.equal(lse_g[:n].view(torch.int32), lse_e[:n].view(torch.int32))
        if i == 1:
            w2 = dict(w, q=w["q"][:n], seq_lens_q=lq, seq_lens_kv=lkv)
            ref_o, ref_l = oracle_prefill(w2)
            assert_out_close(out_g[:n], ref_o, torch.bfloat16)
            assert_lse_close(lse_g[:n], ref_l)


def test_decode_replays_with_new_lengths(pkv):
    w = workloads.batch_decode(DEV, seed=71, batch=8, seq=(100, 3000), q_len_per_req=2,
                               num_qo_heads=16, num_kv_heads=4, window_left=700, sinks=True)
    seq0 = w["seq_lens"].to(torch.int64)
    seq_d = w["seq_lens"].to(DEV)
    bt = w["block_tables"].to(DEV)
    sinks = w["sinks"].to(DEV)
    ws = torch.zeros(max(pkv.decode_workspace_size(8, 2, 16, 4, 128, w["max_seq_len"], 700), 16),
                     dtype=torch.uint8, device=DEV)
    out_g = torch.empty_like(w["query"])
    # bmm2 as a device tensor (the page's tensor form): its value changes
    # between replays too
    bmm2_d = torch.tensor([0.8], dtype=torch.float32, device=DEV)

    def call(out, bmm2):
        pkv.batch_decode_with_kv_cache(w["query"], w["kv_cache"], ws, bt, seq_d,
                                       w["max_seq_len"], bmm1_scale=w["bmm1_scale"],
                                       bmm2_scale=bmm2, window_left=700, out=out, sinks=sinks,
                                       kv_layout="HND", q_len_per_req=2)

    g = capture(lambda: call(out_g, bmm2_d))
    gen = torch.Generator().manual_seed(71)
    for i, bmm2 in enumerate((0.8, 1.25, 0.5)):
        seq = seq0 if i == 0 else torch.randint(1, int(seq0.min()) + 1, (8,), generator=gen)
        seq_d.copy_(seq.to(torch.uint32))
        bmm2_d.fill_(bmm2)
        w["query"].copy_(torch.randn(w["query"].shape, generator=gen).to(torch.bfloat16))
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        out_e = torch.empty_like(out_g)
        call(out_e, bmm2)
        torch.cuda.synchronize()
        print(f"replay {i}: seq {seq.tolist()} bmm2 {bmm2}", flush=True)
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16))
        if i == 1:
            w2 = dict(w, seq_lens=seq.to(torch.uint32), bmm2_scale=bmm2)
            assert_out_close(out_g, oracle_decode(w2), torch.bfloat16)


def test_append_then_decode_step_replays(pkv):
    w = workloads.spec_decode(DEV, seed=72, batch=6, seq=(100, 2000))
    kv = w["kv_cache"]
    seq32 = w["seq_lens"].to(torch.int32).to(DEV)
    seq = w["seq_lens"].to(DEV)
    ai, idx = w["append_indptr"].to(DEV), w["kv_indices"].to(DEV)
    indptr, last = w["kv_indptr"].to(DEV), w["kv_last_page_len"].to(DEV)
    bt, sinks = w["block_tables"].to(DEV), w["sinks"].to(DEV)
    nnz = w["k_append"].shape[0]
    ws = torch.zeros(max(pkv.decode_workspace_size(6, 4, 64, 8, 128, w["max_seq_len"], 4095), 16),
                     dtype=torch.uint8, device=DEV)
    out_g = torch.empty_like(w["query"])

    def step(out):
        bi, pos = pkv.get_batch_indices_positions(ai, seq32, nnz)
        pkv.append_paged_kv_cache(w["k_append"], w["v_append"], bi, pos, kv, idx, indptr, last,
                                  kv_layout="HND")
        pkv.batch_decode_with_kv_cache(w["query"], kv, ws, bt, seq, w["max_seq_len"],
                                       bmm1_scale=w["bmm1_scale"], bmm2_scale=w["bmm2_scale"],
                                       window_left=4095, out=out, sinks=sinks, kv_layout="HND",
                                       q_len_per_req=4)

    g = capture(lambda: step(out_g))
    gen = torch.Generator(device=DEV).manual_seed(72)
    ps = w["page_size"]
    for i in range(3):
        for t in (w["k_append"], w["v_append"]):
            t.copy_(torch.randn(t.shape, generator=gen, device=DEV).to(t.dtype))
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # the replay wrote this replay's rows at each request's last 4 positions
        for b in (0, 5):
            L = int(w["seq_lens"][b])
            for r in range(4):
                p = L - 4 + r
                page = int(w["block_tables"][b, p // ps])
                assert torch.equal(kv[page, 0, :, p % ps].view(torch.uint8),
                                   w["k_append"][b * 4 + r].view(torch.uint8))
                assert torch.equal(kv[page, 1, :, p % ps].view(torch.uint8),
                                   w["v_append"][b * 4 + r].view(torch.uint8))
        out_e = torch.empty_like(out_g)
        step(out_e)
        torch.cuda.synchronize()
        print(f"replay {i}", flush=True)
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16))
        if i == 2:
            assert_out_close(out_g, oracle_decode(w), torch.bfloat16)
