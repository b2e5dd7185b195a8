"""The C ABI library loads, exports every symbol include/pkv.h declares, and
rejects bad arguments on the host before any HIP call (no GPU needed)."""

import ctypes
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

from attention_paged_kv_cache_amd import _lib

HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libpkv.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 11, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_abi_version(lib):
    assert lib.pkv_abi_version() == 4


def _err(lib):
    return lib.pkv_last_error().decode()


# Pointers below are never dereferenced: every call must fail validation.
FAKE = ctypes.c_void_p(0x1000)


def _prefill(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, psk=16 * 8 * 128, psv=16 * 8 * 128, scale=0.1,
             ws=FAKE, ws_bytes=4096, max_q=10, max_kv=10, lq=FAKE, lkv=FAKE, bt=FAKE,
             max_pages=1, batch=1, hqo=32, hkv=8, dqk=128, dvo=128, ps=16, layout=1,
             causal=1, qs=None, ks=None, vs=None, out=FAKE, lse=FAKE, qdt=1, odt=1,
             off_q=None, off_o=None, off_k=None, off_v=None, off_stats=None, stream=None)
    a.update(over)
    return lib.pkv_batch_prefill_with_kv_cache(*a.values())


@pytest.mark.parametrize("over,needle", [
    (dict(dqk=64), "128 or 192"),
    (dict(dvo=192), "must be 128"),
    (dict(hqo=4, hkv=8), ">= num_heads_kv"),
    (dict(hqo=12, hkv=8), "multiple"),
    (dict(lse=None), "lse is required"),
    (dict(layout=7), "NHD or HND"),
    (dict(ps=8), "page_size"),
    (dict(ws_bytes=0), "workspace"),
    (dict(odt=2), "output dtype"),
    (dict(batch=-1), "batch_size"),
    (dict(psk=100), "page stride"),
    (dict(max_kv=17), "too narrow"),
    (dict(off_k=FAKE), "only without block_tables"),
    (dict(off_v=FAKE), "only without block_tables"),
    (dict(bt=None, qdt=7), "dtype"),
    (dict(bt=None, dqk=64), "128 or 192"),
])
def test_prefill_validation(lib, over, needle):
    st = _prefill(lib, **over)
    assert st in (1, 2, 3)
    assert needle in _err(lib)


def _decode(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, psk=2 * 16 * 8 * 128, psv=2 * 16 * 8 * 128, ws=FAKE,
             ws_bytes=1 << 30, bt=FAKE, max_pages=64, seq=FAKE, batch=4, max_seq=1024,
             bmm1=0.1, bmm2=1.0, window=-1, out=FAKE, odt=1, sinks=None, layout=1, ql=1,
             hqo=32, hkv=8, d=128, ps=16, qdt=1, kvdt=1, bmm1_dev=None, bmm2_dev=None,
             o_scale=1.0, cum_q=None, max_q=0, mask=None, stream=None)
    a.update(over)
    return lib.pkv_batch_decode_with_kv_cache(*a.values())


@pytest.mark.parametrize("over,needle", [
    (dict(window=-2), "window_left"),
    (dict(ql=0), "q_len_per_req"),
    (dict(d=64), "head_dim"),
    (dict(ql=33, hqo=32, hkv=1), "<= 1024"),
    (dict(ql=65, hqo=8, hkv=8, mask=FAKE), "spec_mask"),
    (dict(qdt=2), "query dtype"),
    (dict(kvdt=0), "kv dtype"),
    (dict(ws_bytes=0, max_seq=100000, max_pages=10000), "workspace"),
    (dict(layout=3), "NHD or HND"),
    (dict(max_pages=1), "too narrow"),
    (dict(hqo=8, hkv=16), ">= num_heads_kv"),
    (dict(odt=2, o_scale=0.0), "o_scale"),
    (dict(odt=2, o_scale=-1.0), "o_scale"),
    (dict(odt=2, o_scale=float("inf")), "o_scale"),
    (dict(odt=2, o_scale=float("nan")), "o_scale"),
    (dict(odt=7), "output dtype"),
    (dict(cum_q=FAKE, max_q=0), "max_q_len"),
    (dict(cum_q=None, max_q=3), "max_q_len"),
    (dict(cum_q=FAKE, max_q=257, hqo=32, hkv=8), "<= 1024"),
])
def test_decode_validation(lib, over, needle):
    st = _decode(lib, **over)
    assert st in (1, 2, 3)
    assert needle in _err(lib)


def _decode_no_alloc(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, psk=2 * 16 * 8 * 128, psv=2 * 16 * 8 * 128, bt=FAKE,
             max_pages=64, seq=FAKE, batch=4, max_seq=1024, bmm1=0.1, bmm2=1.0, window=-1,
             out=FAKE, odt=1, sinks=None, layout=1, ql=1, hqo=32, hkv=8, d=128, ps=16, qdt=1,
             kvdt=1, bmm1_dev=None, bmm2_dev=None, o_scale=1.0, cum_q=None, max_q=0, mask=None,
             stream=None)
    a.update(over)
    return lib.pkv_batch_decode_with_kv_cache_no_alloc(*a.values())


@pytest.mark.parametrize("over,needle", [
    (dict(window=-2), "window_left"),
    (dict(d=64), "head_dim"),
    (dict(ql=33, hqo=32, hkv=1), "<= 1024"),
    (dict(kvdt=0), "kv dtype"),
    (dict(max_pages=1), "too narrow"),
    # a split plan larger than the static scratch array
    (dict(batch=64, ql=4, hqo=64, hkv=8, max_seq=1 << 20, max_pages=1 << 16), "static scratch"),
])
def test_decode_no_alloc_validation(lib, over, needle):
    # every check runs on host scalars before any HIP call, the scratch
    # size check included
    st = _decode_no_alloc(lib, **over)
    assert st in (1, 2, 3)
    msg = _err(lib)
    assert needle in msg and "pkv_batch_decode_with_kv_cache_no_alloc" in msg


def test_decode_no_alloc_scratch_limit(lib):
    # the batch-decode workload's plan fits the static scratch array; a
    # plan just over it is refused with PKV_ERR_WORKSPACE_TOO_SMALL
    assert _lib.DECODE_SCRATCH_BYTES == 64 << 20
    assert lib.pkv_decode_workspace_size(256, 1, 32, 8, 128, 8192, -1) <= _lib.DECODE_SCRATCH_BYTES
    st = _decode_no_alloc(lib, batch=64, ql=4, hqo=64, hkv=8, max_seq=1 << 20, max_pages=1 << 16)
    assert st == 3
    assert lib.pkv_decode_workspace_size(64, 4, 64, 8, 128, 1 << 20, -1) > \
        _lib.DECODE_SCRATCH_BYTES


def test_append_validation(lib):
    st = lib.pkv_append_paged_kv_cache(FAKE, FAKE, FAKE, FAKE, 10, FAKE, FAKE, 100, 100, FAKE,
                                       FAKE, None, 1, 32, 128, 16, 0, 0, None)
    assert st == 1 and "page stride" in _err(lib)
    st = lib.pkv_append_paged_kv_cache(FAKE, FAKE, FAKE, FAKE, 10, FAKE, FAKE, 1 << 20, 1 << 20,
                                       FAKE, FAKE, None, 1, 32, 4, 16, 0, 0, None)
    assert st == 2 and "16 bytes" in _err(lib)
    st = lib.pkv_append_paged_kv_cache(FAKE, FAKE, FAKE, FAKE, -1, FAKE, FAKE, 1 << 20, 1 << 20,
                                       FAKE, FAKE, None, 1, 32, 128, 16, 0, 0, None)
    assert st == 1 and "nnz" in _err(lib)


def test_index_validation(lib):
    assert lib.pkv_get_seq_lens(FAKE, FAKE, 4, 0, FAKE, None) == 1
    assert lib.pkv_get_batch_indices_positions(FAKE, FAKE, 4, -3, FAKE, FAKE, None) == 1
    assert lib.pkv_csr_to_block_tables(FAKE, FAKE, 4, 0, FAKE, None) == 1
    # empty work is not an error and enqueues nothing
    assert lib.pkv_get_seq_lens(None, None, 0, 16, None, None) == 0


def test_workspace_sizes(lib):
    assert lib.pkv_prefill_workspace_size(16) >= 17 * 4
    # cfg-like decode sizes stay within the 128 MB the prefill page suggests
    assert 0 < lib.pkv_decode_workspace_size(256, 1, 32, 8, 128, 8192, -1) < 128 << 20
    # many query rows per kv head: one chunk per request, no partials
    assert lib.pkv_decode_workspace_size(64, 4, 64, 8, 128, 32768, 4095) == 0
    assert 0 < lib.pkv_decode_workspace_size(64, 4, 64, 8, 128, 32768, -1) < 128 << 20
    assert lib.pkv_decode_workspace_size(4, 0, 32, 8, 128, 1024, -1) == 0


def test_ceiling_library_exports_and_validates():
    # the chip-ceiling kernels the benchmark reads rates against
    path = os.path.join(ROOT, "attention_paged_kv_cache_amd", "libpkv_ceiling.so")
    if not os.path.exists(path):
        pytest.fail("libpkv_ceiling.so is not built (run __graft_entry__.build())")
    c = ctypes.CDLL(path)
    c.pkv_ceiling_mfma_bf16_flop.restype = ctypes.c_double
    c.pkv_ceiling_mfma_bf16_flop.argtypes = [ctypes.c_int32, ctypes.c_int32]
    # 2 blocks x 4 waves x 3 rounds x 8 chains x 32x32x16 MACs x 2
    assert c.pkv_ceiling_mfma_bf16_flop(2, 3) == 2 * 4 * 3 * 8 * 32 * 32 * 16 * 2
    c.pkv_ceiling_read.restype = ctypes.c_int
    c.pkv_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p]
    c.pkv_ceiling_mfma_bf16.restype = ctypes.c_int
    c.pkv_ceiling_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p]
    # rejected on the host before any launch: a span that does not divide
    # evenly, an unaligned buffer, null outputs, empty grids
    dummy = ctypes.c_void_p(4096)
    assert c.pkv_ceiling_read(dummy, 1000, 4, dummy, None) != 0
    assert c.pkv_ceiling_read(ctypes.c_void_p(4100), 4 * 32768, 4, dummy, None) != 0
    assert c.pkv_ceiling_read(dummy, 4 * 32768, 4, None, None) != 0
    assert c.pkv_ceiling_mfma_bf16(0, 1, dummy, None) != 0
    assert c.pkv_ceiling_mfma_bf16(1, 1, None, None) != 0
    c.pkv_ceiling_copy.restype = ctypes.c_int
    c.pkv_ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p]
    dst = ctypes.c_void_p(1 << 30)
    assert c.pkv_ceiling_copy(dummy, dst, 4 * 16384, 4, 1, 3, None) != 0  # unroll 4 or 8
    assert c.pkv_ceiling_copy(dummy, dst, 1000, 4, 1, 4, None) != 0       # span
    assert c.pkv_ceiling_copy(dummy, dummy, 4 * 16384, 4, 1, 4, None) != 0  # overlap
    assert c.pkv_ceiling_copy(ctypes.c_void_p(4100), dst, 4 * 16384, 4, 1, 4, None) != 0


def test_header_compiles_as_c99_and_cpp17(tmp_path):
    """include/pkv.h is a plain C header (C99, pedantic, warnings as errors)
    and the same text compiles as C++17."""
    for cc, std, lang in (("gcc", "-std=c99", "c"), ("g++", "-std=c++17", "c++")):
        r = subprocess.run([cc, std, "-Wall", "-Wextra", "-Werror", "-pedantic",
                            "-fsyntax-only", "-x", lang, HEADER],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr


def test_c_program_links_and_gets_statuses(lib, tmp_path):
    """tests/c/abi_from_c.c, built with gcc as C99 against include/pkv.h and
    linked to libpkv.so, checks the ABI version, validation statuses and
    messages, and the workspace-size queries, all on the host."""
    exe = str(tmp_path / "abi_from_c")
    libdir = os.path.dirname(_lib.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        f"-I{os.path.dirname(HEADER)}", os.path.join(ROOT, "tests", "c",
                                                                      "abi_from_c.c"),
                        "-o", exe, f"-L{libdir}", "-l:libpkv.so", f"-Wl,-rpath,{libdir}"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
