"""Element formats of the paged cache, decoded from raw bits to float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The prefill page (``cudnn_batch_prefill_with_kv_cache``, Parameters:
q_scale / k_scale / v_scale) accepts fp8 inputs with per-tensor scales; the
cache dtypes in use are fp16, bf16 and fp8 e4m3. The e4m3 variant taken here is
the OCP "fn" encoding (no infinities, bias 7, max +-448, S.1111.111 is NaN).

Each decoder is written from the format's definition, not from a library.
"""

import numpy as np

F16, BF16, E4M3 = "f16", "bf16", "e4m3"

_BITS_DTYPE = {F16: np.uint16, BF16: np.uint16, E4M3: np.uint8}


def bits_dtype(fmt):
    """numpy integer type that holds one element of ``fmt`` as raw bits."""
    return _BITS_DTYPE[fmt]


def _decode_f16(bits):
    """IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits."""
    b = bits.astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    m = (b & 0x3FF).astype(np.float64)
    normal = sign * (1.0 + m / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    sub = sign * (m / 1024.0) * 2.0 ** -14
    out = np.where(e == 0, sub, normal)
    special = np.where(m == 0, sign * np.inf, np.nan)
    return np.where(e == 0x1F, special, out)


def _decode_bf16(bits):
    """bfloat16: the upper 16 bits of an IEEE binary32 word."""
    b32 = bits.astype(np.uint32) << np.uint32(16)
    return b32.view(np.float32).astype(np.float64)


def e4m3fn_table():
    """All 256 e4m3fn codes as float64, built from the format definition.

    Layout S.EEEE.MMM, exponent bias 7. Exponent field 0 is subnormal
    (value m/8 * 2^-6). There are no infinities; S.1111.111 is NaN, so the
    largest finite magnitude is 1.75 * 2^8 = 448.
    """
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = np.nan
        elif e == 0:
            tab[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            tab[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


_E4M3_TABLE = e4m3fn_table()


def encode_e4m3fn(x):
    """float64 values (any shape) -> e4m3fn codes (uint8), from the format's
    definition: the nearest finite e4m3fn value, a tie going to the code whose
    mantissa is even; magnitudes above 448 saturate to +-448; NaN gives the
    NaN code of its sign; -0.0 keeps its sign bit.

    Decode page, Parameters: ``o_scale`` is the output scale for fp8 output.
    The reading taken here mirrors how the per-tensor k/v scales dequantise
    (value = scale * stored code), so a stored output code is
    ``encode_e4m3fn(out / o_scale)``; saturating rather than producing NaN
    on overflow is the reading for values beyond the format's range.
    """
    x = np.asarray(x, dtype=np.float64)
    mags = _E4M3_TABLE[:127]              # codes 0x00..0x7E: 0 .. 448, ascending
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(mags, a, side="left")   # first magnitude >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == mags[hi], hi, code)
    sign = np.where(np.signbit(x), 0x80, 0x00)
    out = (code | sign).astype(np.uint8)
    return np.where(np.isnan(x), (sign | 0x7F).astype(np.uint8), out)


def decode_bits(bits, fmt):
    """Raw bits (any shape) -> float64 values of format ``fmt``."""
    bits = np.asarray(bits)
    if fmt == F16:
        return _decode_f16(bits.astype(np.uint16))
    if fmt == BF16:
        return _decode_bf16(bits.astype(np.uint16))
    if fmt == E4M3:
        return _E4M3_TABLE[bits.astype(np.uint8)]
    raise ValueError(f"unknown format {fmt!r}")

