"""The Python binding rejects tensors that are not on a GPU before it calls
the library: the C ABI reads its pointer arguments as device memory, so a
host pointer reaching a kernel would be a memory fault, not an error."""

import pytest
import torch

import attention_paged_kv_cache_amd as pkv


def _i32(*xs):
    return torch.tensor(xs, dtype=torch.int32)


def test_index_helpers_reject_host_tensors():
    with pytest.raises(ValueError, match="GPU"):
        pkv.get_seq_lens(_i32(0, 3), _i32(5), 16)
    with pytest.raises(ValueError, match="GPU"):
        pkv.get_batch_indices_positions(_i32(0, 3), _i32(37), 3)
    with pytest.raises(ValueError, match="GPU"):
        pkv.csr_to_block_tables(_i32(0, 3), _i32(0, 1, 2), 3)


def test_append_rejects_host_tensors():
    cache = torch.zeros(4, 2, 2, 16, 128, dtype=torch.bfloat16)
    rows = torch.zeros(3, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        pkv.append_paged_kv_cache(rows, rows, _i32(0, 0, 0), _i32(0, 1, 2), cache,
                                  _i32(0), _i32(0, 1), _i32(3), kv_layout="HND")


def test_prefill_rejects_host_tensors():
    q = torch.zeros(5, 4, 128, dtype=torch.bfloat16)
    k = torch.zeros(2, 2, 16, 128, dtype=torch.bfloat16)
    ws = torch.zeros(1 << 12, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        pkv.batch_prefill_with_kv_cache(
            q, k, k, 0.1, ws, max_token_per_sequence=5, max_sequence_kv=5,
            actual_seq_lens_q=_i32(5), actual_seq_lens_kv=_i32(5),
            block_tables=_i32(0).reshape(1, 1), causal=True)


def test_decode_rejects_host_tensors():
    q = torch.zeros(2, 4, 128, dtype=torch.bfloat16)
    kv = torch.zeros(2, 2, 2, 16, 128, dtype=torch.bfloat16)
    ws = torch.zeros(1 << 12, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        pkv.batch_decode_with_kv_cache(q, kv, ws, _i32(0, 1).reshape(2, 1),
                                       torch.tensor([5, 9], dtype=torch.int32), 9)
