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

