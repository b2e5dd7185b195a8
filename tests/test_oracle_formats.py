"""Pins for the oracle's element decoders against library conversions (CPU)."""

import numpy as np
import torch

from oracle.formats import decode_bits, e4m3fn_table, F16, BF16, E4M3


def test_e4m3fn_table_equals_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    tab = e4m3fn_table()
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(tab[ok], ref[ok])
    # format facts: max finite 448, smallest subnormal 2^-9, two NaN codes
    assert np.nanmax(tab) == 448.0 and np.nanmin(tab) == -448.0
    assert tab[1] == 2.0 ** -9
    assert np.isnan(tab).sum() == 2


def test_f16_decode_equals_numpy_for_all_codes():
    codes = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = decode_bits(codes, F16)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_bf16_decode_equals_torch_for_all_codes():
    codes = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = decode_bits(codes, BF16)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_decode_dispatch_keeps_shape():
    x = np.arange(24, dtype=np.uint8).reshape(2, 3, 4)
    assert decode_bits(x, E4M3).shape == (2, 3, 4)
    assert decode_bits(x.astype(np.uint16), BF16).shape == (2, 3, 4)
