"""Loading of libpkv.so and its C signatures (ctypes).

torch is imported before the library is opened so that the HIP runtime
torch already holds (same soname) is the one libpkv.so binds to: device
pointers and streams from torch are then valid in the library's calls.
"""

import ctypes
import os

import torch  # noqa: F401  (must come first, see module docstring)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
STATUS_NAMES = {
    0: "PKV_OK",
    1: "PKV_ERR_INVALID_ARG",
    2: "PKV_ERR_UNSUPPORTED",
    3: "PKV_ERR_WORKSPACE_TOO_SMALL",
    4: "PKV_ERR_HIP",
}
NHD, HND = 0, 1
F16, BF16, E4M3 = 0, 1, 2

# exported name -> (restype, argtypes); mirrors include/pkv.h
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t
SIGNATURES = {
    "pkv_abi_version": (ctypes.c_int, []),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_get_seq_lens": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P]),
    "pkv_get_batch_indices_positions": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P, _P]),
    "pkv_csr_to_block_tables": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P]),
    "pkv_append_paged_kv_cache": (ctypes.c_int, [
        _P, _P, _P, _P, _I32, _P, _P, _I64, _I64, _P, _P, _P, _I32, _I32, _I32, _I32,
        ctypes.c_int, ctypes.c_int, _P]),
    "pkv_prefill_workspace_size": (_SZ, [_I32]),
    "pkv_batch_prefill_with_kv_cache": (ctypes.c_int, [
        _P, _P, _P, _I64, _I64, _F, _P, _SZ, _I32, _I32, _P, _P, _P, _I32, _I32,
        _I32, _I32, _I32, _I32, _I32, ctypes.c_int, _I32, _P, _P, _P, _P, _P,
        ctypes.c_int, ctypes.c_int, _P, _P, _P, _P, _P, _P]),
    "pkv_decode_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_batch_decode_with_kv_cache": (ctypes.c_int, [
        _P, _P, _P, _I64, _I64, _P, _SZ, _P, _I32, _P, _I32, _I32, _F, _F, _I32,
        _P, ctypes.c_int, _P, ctypes.c_int, _I32, _I32, _I32, _I32, _I32,
        ctypes.c_int, ctypes.c_int, _P, _P, _F, _P, _I32, _P, _P]),
    "pkv_batch_decode_with_kv_cache_no_alloc": (ctypes.c_int, [
        _P, _P, _P, _I64, _I64, _P, _I32, _P, _I32, _I32, _F, _F, _I32,
        _P, ctypes.c_int, _P, ctypes.c_int, _I32, _I32, _I32, _I32, _I32,
        ctypes.c_int, ctypes.c_int, _P, _P, _F, _P, _I32, _P, _P]),
}

# bytes of the no-alloc decode's static scratch array (PKV_DECODE_SCRATCH_BYTES)
DECODE_SCRATCH_BYTES = 64 << 20

_lib = None


class PkvError(RuntimeError):
    pass


def load(path=None):
    """Open libpkv.so (once) and attach its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise PkvError(
            f"{p} is missing: build it first (python -m attention_paged_kv_cache_amd.build)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def check(status, what):
    if status != PKV_OK:
        msg = load().pkv_last_error().decode(errors="replace")
        err = ValueError if status in (1, 2, 3) else PkvError
        raise err(f"{what} failed with {STATUS_NAMES.get(status, status)}: {msg}")
