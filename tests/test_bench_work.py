"""The benchmark's algorithmic work (CPU only): the closed forms bench.py
divides by agree with counting allowed pairs / keys from the oracle's mask
definition, on the workloads' own length draws and on edge cases."""

import numpy as np

import bench
import oracle
import workloads


def test_prefill_flops_equal_oracle_pair_count():
    for lq, lkv in [([1, 5, 7], [1, 9, 7]), ([4], [2]), ([0, 3], [5, 3]), ([64, 130], [64, 500])]:
        pairs = oracle.allowed_pairs(lq, lkv, True)
        assert bench.prefill_flops(lq, lkv, 8, 128, 128) == 2 * 256 * 8 * pairs


def test_prefill_flops_on_the_workload_lengths():
    # the headline workload's drawn lengths (drawn before, and independent
    # of, the tensor shapes, so small heads keep this CPU draw cheap)
    w = workloads.batch_prefill("cpu", num_qo_heads=1, num_kv_heads=1, d_qk=16, d_vo=16)
    lq, lkv = w["seq_lens_q"].tolist(), w["seq_lens_kv"].tolist()
    pairs = oracle.allowed_pairs(lq, lkv, True)
    assert bench.prefill_flops(lq, lkv, 32, 128, 128) == 2 * 256 * 32 * pairs


def test_decode_bytes_count_the_keys_the_oracle_allows():
    seq = [1, 3, 100, 4099, 5000]
    for q_len, window in [(1, -1), (4, 4095), (4, 10), (2, 0)]:
        keys = oracle.keys_read(seq, q_len, window)
        pages = 0
        for s in seq:
            n = min(s, window + q_len) if window >= 0 else s
            pages += (n + 31) // 32
        got = bench.decode_bytes(seq, q_len, window, 64, 8, 128, 1, 2, 2, 32)
        want = keys * 8 * 2 * 128 * 1 + len(seq) * q_len * 64 * 128 * 4 + pages * 4 + len(seq) * 4
        assert got == want, (q_len, window)


def test_append_bytes():
    # read and write both K and V rows, plus batch index and position per row
    assert bench.append_bytes(10, 8, 128, 1) == 4 * 10 * 8 * 128 + 80
    assert bench.append_bytes(0, 8, 128, 2) == 0


def test_roofline_fields():
    r = bench.roofline("hbm", 4000.0, 8000.0, "GB/s", None)
    assert r == {"bound": "hbm", "achieved": 4000.0, "peak": 8000.0, "unit": "GB/s",
                 "frac": 0.5, "traffic": None}
    assert np.isclose(bench.rate(1e12, 1.0, 1e12), 1000.0)
