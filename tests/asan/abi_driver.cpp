// Host-side check of the C ABI under AddressSanitizer: every entry point's
// argument validation (which returns before any HIP call, so no GPU is
// needed), the error messages and the size queries. Built and run by
// tests/test_abi_asan.py; exits non-zero on an unexpected status or message.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "pkv.h"

namespace {

int failures = 0;
// Never dereferenced: every call below fails validation first.
const void *F = reinterpret_cast<const void *>(0x1000);
int32_t *FI = reinterpret_cast<int32_t *>(0x1000);
float *FF = reinterpret_cast<float *>(0x1000);

void expect(pkv_status st, pkv_status want, const char *needle, const char *what) {
  const char *m = pkv_last_error();
  if (st != want || m == nullptr || std::strstr(m, needle) == nullptr) {
    std::printf("FAIL %s: status %d (want %d), message '%s'\n", what, (int)st, (int)want,
                m ? m : "(null)");
    ++failures;
  }
}

struct Prefill {
  const void *q = F, *k = F, *v = F;
  int64_t psk = 16 * 8 * 128, psv = 16 * 8 * 128;
  float scale = 0.1f;
  void *ws = const_cast<void *>(F);
  size_t ws_bytes = 4096;
  int32_t max_q = 10, max_kv = 10;
  const int32_t *lq = FI, *lkv = FI, *bt = FI;
  int32_t max_pages = 1, batch = 1, hqo = 32, hkv = 8, dqk = 128, dvo = 128, ps = 16;
  pkv_layout layout = PKV_HND;
  int32_t causal = 1;
  const float *qs = nullptr, *ks = nullptr, *vs = nullptr;
  void *out = const_cast<void *>(F);
  float *lse = FF;
  pkv_dtype qdt = PKV_BF16, odt = PKV_BF16;
  const int32_t *oq = nullptr, *oo = nullptr, *ok = nullptr, *ov = nullptr, *os = nullptr;
  pkv_status call() const {
    return pkv_batch_prefill_with_kv_cache(q, k, v, psk, psv, scale, ws, ws_bytes, max_q, max_kv,
                                           lq, lkv, bt, max_pages, batch, hqo, hkv, dqk, dvo, ps,
                                           layout, causal, qs, ks, vs, out, lse, qdt, odt, oq, oo,
                                           ok, ov, os, nullptr);
  }
};

struct Decode {
  const void *q = F, *k = F, *v = F;
  int64_t psk = 2 * 16 * 8 * 128, psv = 2 * 16 * 8 * 128;
  void *ws = const_cast<void *>(F);
  size_t ws_bytes = size_t(1) << 30;
  const int32_t *bt = FI;
  int32_t max_pages = 64;
  const uint32_t *seq = reinterpret_cast<const uint32_t *>(F);
  int32_t batch = 4, max_seq = 1024;
  float bmm1 = 0.1f, bmm2 = 1.0f;
  int32_t window = -1;
  void *out = const_cast<void *>(F);
  pkv_dtype odt = PKV_BF16;
  const float *sinks = nullptr;
  pkv_layout layout = PKV_HND;
  int32_t ql = 1, hqo = 32, hkv = 8, d = 128, ps = 16;
  pkv_dtype qdt = PKV_BF16, kvdt = PKV_BF16;
  const float *b1 = nullptr, *b2 = nullptr;
  float o_scale = 1.0f;
  const int32_t *cum = nullptr;
  int32_t max_q = 0;
  const uint8_t *mask = nullptr;
  pkv_status call() const {
    return pkv_batch_decode_with_kv_cache(q, k, v, psk, psv, ws, ws_bytes, bt, max_pages, seq,
                                          batch, max_seq, bmm1, bmm2, window, out, odt, sinks,
                                          layout, ql, hqo, hkv, d, ps, qdt, kvdt, b1, b2, o_scale,
                                          cum, max_q, mask, nullptr);
  }
};

}  // namespace

int main() {
  if (pkv_abi_version() != PKV_ABI_VERSION) {
    std::printf("FAIL abi version %d\n", pkv_abi_version());
    ++failures;
  }
  // ---- prefill ----------------------------------------------------------------
  {
    Prefill p;
    Prefill a = p; a.dqk = 64; expect(a.call(), PKV_ERR_UNSUPPORTED, "128 or 192", "prefill dqk");
    a = p; a.dvo = 192; expect(a.call(), PKV_ERR_UNSUPPORTED, "must be 128", "prefill dvo");
    a = p; a.hqo = 4; expect(a.call(), PKV_ERR_INVALID_ARG, ">= num_heads_kv", "prefill heads");
    a = p; a.hqo = 12; expect(a.call(), PKV_ERR_UNSUPPORTED, "multiple", "prefill gqa");
    a = p; a.lse = nullptr; expect(a.call(), PKV_ERR_INVALID_ARG, "lse is required", "prefill lse");
    a = p; a.layout = (pkv_layout)7; expect(a.call(), PKV_ERR_INVALID_ARG, "NHD or HND", "prefill layout");
    a = p; a.ps = 8; expect(a.call(), PKV_ERR_UNSUPPORTED, "page_size", "prefill ps");
    a = p; a.ws_bytes = 0; expect(a.call(), PKV_ERR_WORKSPACE_TOO_SMALL, "workspace", "prefill ws");
    a = p; a.odt = PKV_E4M3; expect(a.call(), PKV_ERR_UNSUPPORTED, "output dtype", "prefill odt");
    a = p; a.psk = 100; expect(a.call(), PKV_ERR_INVALID_ARG, "page stride", "prefill stride");
    a = p; a.max_kv = 17; expect(a.call(), PKV_ERR_INVALID_ARG, "too narrow", "prefill narrow");
    a = p; a.ok = FI; expect(a.call(), PKV_ERR_INVALID_ARG, "only without block_tables", "prefill offs k");
    a = p; a.bt = nullptr; a.qdt = (pkv_dtype)7; expect(a.call(), PKV_ERR_INVALID_ARG, "dtype", "unpaged dtype");
    a = p; a.batch = 0; if (a.call() != PKV_OK) { std::printf("FAIL prefill empty\n"); ++failures; }
  }
  // ---- decode -----------------------------------------------------------------
  {
    Decode p;
    Decode a = p; a.window = -2; expect(a.call(), PKV_ERR_INVALID_ARG, "window_left", "decode window");
    a = p; a.ql = 0; expect(a.call(), PKV_ERR_INVALID_ARG, "q_len_per_req", "decode ql");
    a = p; a.d = 64; expect(a.call(), PKV_ERR_UNSUPPORTED, "head_dim", "decode d");
    a = p; a.ql = 33; a.hkv = 1; expect(a.call(), PKV_ERR_UNSUPPORTED, "<= 1024", "decode rows");
    a = p; a.ql = 65; a.hqo = 8; a.mask = reinterpret_cast<const uint8_t *>(F);
    expect(a.call(), PKV_ERR_UNSUPPORTED, "spec_mask", "decode mask drafts");
    a = p; a.qdt = PKV_E4M3; expect(a.call(), PKV_ERR_UNSUPPORTED, "query dtype", "decode qdt");
    a = p; a.kvdt = PKV_F16; expect(a.call(), PKV_ERR_UNSUPPORTED, "kv dtype", "decode kvdt");
    a = p; a.odt = PKV_E4M3; a.o_scale = 0.0f; expect(a.call(), PKV_ERR_INVALID_ARG, "o_scale", "decode o_scale");
    a = p; a.odt = PKV_E4M3; a.o_scale = std::numeric_limits<float>::quiet_NaN();
    expect(a.call(), PKV_ERR_INVALID_ARG, "o_scale", "decode o_scale nan");
    a = p; a.cum = FI; expect(a.call(), PKV_ERR_INVALID_ARG, "max_q_len", "decode cum");
    a = p; a.max_q = 3; expect(a.call(), PKV_ERR_INVALID_ARG, "max_q_len", "decode max_q");
    a = p; a.ws_bytes = 0; a.max_seq = 100000; a.max_pages = 10000;
    expect(a.call(), PKV_ERR_WORKSPACE_TOO_SMALL, "workspace", "decode ws");
    a = p; a.layout = (pkv_layout)3; expect(a.call(), PKV_ERR_INVALID_ARG, "NHD or HND", "decode layout");
    a = p; a.max_pages = 1; expect(a.call(), PKV_ERR_INVALID_ARG, "too narrow", "decode narrow");
    a = p; a.batch = 0; if (a.call() != PKV_OK) { std::printf("FAIL decode empty\n"); ++failures; }
    // the no-alloc variant: the same checks, plus the static scratch limit,
    // all before any HIP call
    auto no_alloc = [](const Decode &d) {
      return pkv_batch_decode_with_kv_cache_no_alloc(
          d.q, d.k, d.v, d.psk, d.psv, d.bt, d.max_pages, d.seq, d.batch, d.max_seq, d.bmm1,
          d.bmm2, d.window, d.out, d.odt, d.sinks, d.layout, d.ql, d.hqo, d.hkv, d.d, d.ps,
          d.qdt, d.kvdt, d.b1, d.b2, d.o_scale, d.cum, d.max_q, d.mask, nullptr);
    };
    a = p; a.window = -2;
    expect(no_alloc(a), PKV_ERR_INVALID_ARG, "window_left", "no-alloc window");
    a = p; a.d = 64; expect(no_alloc(a), PKV_ERR_UNSUPPORTED, "head_dim", "no-alloc d");
    a = p; a.batch = 64; a.ql = 4; a.hqo = 64; a.max_seq = 1 << 20; a.max_pages = 1 << 16;
    expect(no_alloc(a), PKV_ERR_WORKSPACE_TOO_SMALL, "static scratch", "no-alloc scratch");
    a = p; a.batch = 0;
    if (no_alloc(a) != PKV_OK) { std::printf("FAIL no-alloc empty\n"); ++failures; }
  }
  // ---- append and index math ------------------------------------------------------
  expect(pkv_append_paged_kv_cache(F, F, FI, FI, 10, const_cast<void *>(F), const_cast<void *>(F),
                                   100, 100, FI, FI, nullptr, 1, 32, 128, 16, PKV_NHD, PKV_F16,
                                   nullptr),
         PKV_ERR_INVALID_ARG, "page stride", "append stride");
  expect(pkv_append_paged_kv_cache(F, F, FI, FI, -1, const_cast<void *>(F), const_cast<void *>(F),
                                   1 << 20, 1 << 20, FI, FI, nullptr, 1, 32, 128, 16, PKV_NHD,
                                   PKV_F16, nullptr),
         PKV_ERR_INVALID_ARG, "nnz", "append nnz");
  expect(pkv_get_seq_lens(FI, FI, 4, 0, FI, nullptr), PKV_ERR_INVALID_ARG, "page_size", "seq_lens ps");
  expect(pkv_get_batch_indices_positions(FI, FI, 4, -3, FI, FI, nullptr), PKV_ERR_INVALID_ARG, "nnz",
         "indices nnz");
  if (pkv_get_seq_lens(nullptr, nullptr, 0, 16, nullptr, nullptr) != PKV_OK) {
    std::printf("FAIL empty seq_lens\n");
    ++failures;
  }
  // ---- size queries -------------------------------------------------------------------
  if (pkv_prefill_workspace_size(16) < 17 * 4 || pkv_prefill_workspace_size(-1) != 0 ||
      pkv_decode_workspace_size(64, 4, 64, 8, 128, 32768, 4095) != 0) {
    std::printf("FAIL workspace sizes\n");
    ++failures;
  }
  std::printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
