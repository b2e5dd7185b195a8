"""Pins for the oracle's element decoders against library conversions (CPU)."""

import numpy as np
import torch

from oracle.formats import decode_bits, e4m3fn_table, encode_e4m3fn, F16, BF16, E4M3


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


def test_e4m3fn_encode_round_trips_every_finite_code():
    tab = e4m3fn_table()
    codes = np.arange(256)
    fin = ~np.isnan(tab)
    assert np.array_equal(encode_e4m3fn(tab[fin]), codes[fin].astype(np.uint8))


def test_e4m3fn_encode_equals_torch_in_range():
    # torch's float32 -> float8_e4m3fn conversion rounds to nearest even; on
    # every float32 value with |x| <= 464 (where it has not overflowed to NaN)
    # the two must agree: a dense sweep, every midpoint between neighbouring
    # codes (the ties) and the float32 values on either side of each midpoint
    mags = e4m3fn_table()[:127]
    mid = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(1e9))
    xs = np.concatenate([np.linspace(-464, 464, 200001).astype(np.float32),
                         mid, -mid, below, above, -below, -above])
    ours = encode_e4m3fn(xs.astype(np.float64))
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3fn_encode_ties_go_to_even_codes():
    mags = e4m3fn_table()[:127]
    mid = (mags[:-1] + mags[1:]) / 2
    got = encode_e4m3fn(mid).astype(np.int64)
    assert np.all(got % 2 == 0)
    assert np.all((got == np.arange(126)) | (got == np.arange(1, 127)))


def test_e4m3fn_encode_saturates_and_keeps_nan_and_signed_zero():
    got = encode_e4m3fn([448.0, 449.0, 464.0, 1e30, np.inf, -1e30, -np.inf,
                         np.nan, -np.nan, 0.0, -0.0, 2.0 ** -10, 2.0 ** -30])
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE,
                            0x7F, 0xFF, 0x00, 0x80, 0x00, 0x00]
