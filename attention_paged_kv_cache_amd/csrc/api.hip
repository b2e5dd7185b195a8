// C ABI of the paged-KV library: argument validation and kernel launch.
//
// Every entry point checks its host-side arguments first and returns an
// error before any HIP call if one is out of range, so the checks run (and
// can be tested) on a machine without a GPU. The library never allocates,
// never synchronises and never reads device memory on the host. The
// no-alloc decode entry point uses a static device array of the library's
// own (at the end of this file) instead of a workspace.

#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "launch.h"
#include "pkv.h"

#define PKV_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status st, const char *fn, const char *msg) {
  g_last_error = std::string(fn) + ": " + msg;
  return st;
}

pkv_status from_hip(hipError_t e, const char *fn) {
  if (e == hipSuccess) return PKV_OK;
  g_last_error = std::string(fn) + ": HIP error: " + hipGetErrorString(e);
  return PKV_ERR_HIP;
}

int elem_bytes(int dt) { return dt == PKV_E4M3 ? 1 : 2; }

bool aligned(const void *p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool page_size_ok(int32_t ps) { return ps == 16 || ps == 32 || ps == 64; }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

#define CHECK(cond, st, msg)                      \
  do {                                            \
    if (!(cond)) return fail((st), __func__, (msg)); \
  } while (0)

PKV_API int pkv_abi_version(void) { return PKV_ABI_VERSION; }

PKV_API const char *pkv_last_error(void) { return g_last_error.c_str(); }

PKV_API pkv_status pkv_get_seq_lens(const int32_t *kv_indptr,
                                    const int32_t *kv_last_page_len,
                                    int32_t batch_size, int32_t page_size,
                                    int32_t *seq_lens, void *stream) {
  CHECK(batch_size >= 0, PKV_ERR_INVALID_ARG, "batch_size < 0");
  CHECK(page_size > 0, PKV_ERR_INVALID_ARG, "page_size <= 0");
  if (batch_size == 0) return PKV_OK;
  CHECK(kv_indptr && kv_last_page_len && seq_lens, PKV_ERR_INVALID_ARG,
        "null pointer");
  return from_hip(pkv::launch_get_seq_lens(kv_indptr, kv_last_page_len,
                                           batch_size, page_size, seq_lens,
                                           as_stream(stream)),
                  __func__);
}

PKV_API pkv_status pkv_get_batch_indices_positions(
    const int32_t *append_indptr, const int32_t *seq_lens, int32_t batch_size,
    int32_t nnz, int32_t *batch_indices, int32_t *positions, void *stream) {
  CHECK(batch_size >= 0, PKV_ERR_INVALID_ARG, "batch_size < 0");
  CHECK(nnz >= 0, PKV_ERR_INVALID_ARG, "nnz < 0");
  if (batch_size == 0 || nnz == 0) return PKV_OK;
  CHECK(append_indptr && seq_lens && batch_indices && positions,
        PKV_ERR_INVALID_ARG, "null pointer");
  return from_hip(pkv::launch_batch_indices_positions(
                      append_indptr, seq_lens, batch_size, nnz, batch_indices,
                      positions, as_stream(stream)),
                  __func__);
}

PKV_API pkv_status pkv_csr_to_block_tables(const int32_t *kv_indptr,
                                           const int32_t *kv_indices,
                                           int32_t batch_size,
                                           int32_t max_pages_per_seq,
                                           int32_t *block_tables,
                                           void *stream) {
  CHECK(batch_size >= 0, PKV_ERR_INVALID_ARG, "batch_size < 0");
  CHECK(max_pages_per_seq > 0, PKV_ERR_INVALID_ARG, "max_pages_per_seq <= 0");
  if (batch_size == 0) return PKV_OK;
  CHECK(kv_indptr && kv_indices && block_tables, PKV_ERR_INVALID_ARG,
        "null pointer");
  return from_hip(pkv::launch_csr_to_block_tables(kv_indptr, kv_indices,
                                                  batch_size, max_pages_per_seq,
                                                  block_tables,
                                                  as_stream(stream)),
                  __func__);
}

PKV_API pkv_status pkv_append_paged_kv_cache(
    const void *append_key, const void *append_value,
    const int32_t *batch_indices, const int32_t *positions, int32_t nnz,
    void *k_cache, void *v_cache, int64_t page_stride_k, int64_t page_stride_v,
    const int32_t *kv_indices, const int32_t *kv_indptr,
    const int32_t *kv_last_page_len, int32_t batch_size, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size, pkv_layout kv_layout, pkv_dtype dtype,
    void *stream) {
  (void)kv_last_page_len;
  CHECK(nnz >= 0, PKV_ERR_INVALID_ARG, "nnz < 0");
  CHECK(batch_size >= 0, PKV_ERR_INVALID_ARG, "batch_size < 0");
  CHECK(num_kv_heads > 0, PKV_ERR_INVALID_ARG, "num_kv_heads <= 0");
  CHECK(head_dim > 0, PKV_ERR_INVALID_ARG, "head_dim <= 0");
  CHECK(page_size > 0, PKV_ERR_INVALID_ARG, "page_size <= 0");
  CHECK(kv_layout == PKV_NHD || kv_layout == PKV_HND, PKV_ERR_INVALID_ARG,
        "kv_layout must be NHD or HND");
  CHECK(dtype == PKV_F16 || dtype == PKV_BF16 || dtype == PKV_E4M3,
        PKV_ERR_INVALID_ARG, "unknown dtype");
  const int es = elem_bytes(dtype);
  CHECK((head_dim * es) % 16 == 0, PKV_ERR_UNSUPPORTED,
        "head_dim * element size must be a multiple of 16 bytes");
  const int64_t page_elems = (int64_t)page_size * num_kv_heads * head_dim;
  CHECK(page_stride_k >= page_elems && page_stride_v >= page_elems,
        PKV_ERR_INVALID_ARG, "page stride smaller than one page");
  CHECK((page_stride_k * es) % 16 == 0 && (page_stride_v * es) % 16 == 0,
        PKV_ERR_UNSUPPORTED, "page strides must be multiples of 16 bytes");
  if (nnz == 0) return PKV_OK;
  CHECK(append_key && append_value && batch_indices && positions && k_cache &&
            v_cache && kv_indices && kv_indptr,
        PKV_ERR_INVALID_ARG, "null pointer");
  CHECK(aligned(append_key, 16) && aligned(append_value, 16) &&
            aligned(k_cache, 16) && aligned(v_cache, 16),
        PKV_ERR_UNSUPPORTED, "K/V pointers must be 16-byte aligned");
  pkv::AppendArgs a{};
  a.key = append_key;
  a.value = append_value;
  a.batch_indices = batch_indices;
  a.positions = positions;
  a.nnz = nnz;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_stride_k = page_stride_k * es;
  a.page_stride_v = page_stride_v * es;
  if (kv_layout == PKV_NHD) {
    a.slot_stride = (int64_t)num_kv_heads * head_dim * es;
    a.head_stride = (int64_t)head_dim * es;
  } else {
    a.slot_stride = (int64_t)head_dim * es;
    a.head_stride = (int64_t)page_size * head_dim * es;
  }
  a.kv_indices = kv_indices;
  a.kv_indptr = kv_indptr;
  a.num_heads = num_kv_heads;
  a.row_bytes_per_head = head_dim * es;
  a.page_size = page_size;
  return from_hip(pkv::launch_append(a, as_stream(stream)), __func__);
}

// Two 256-byte-aligned regions of batch_size + 1 int32: the query-row and
// key-row prefix sums used when offsets are not given.
static size_t prefill_region_bytes(int32_t batch_size) {
  return ((size_t)(batch_size + 1) * sizeof(int32_t) + 255) / 256 * 256;
}

PKV_API size_t pkv_prefill_workspace_size(int32_t batch_size) {
  if (batch_size < 0) return 0;
  return 2 * prefill_region_bytes(batch_size);
}

PKV_API pkv_status pkv_batch_prefill_with_kv_cache(
    const void *q, const void *k_cache, const void *v_cache,
    int64_t page_stride_k, int64_t page_stride_v, float scale, void *workspace,
    size_t workspace_bytes, int32_t max_token_per_sequence,
    int32_t max_sequence_kv, const int32_t *actual_seq_lens_q,
    const int32_t *actual_seq_lens_kv, const int32_t *block_tables,
    int32_t max_pages_per_seq, int32_t batch_size, int32_t num_heads_qo,
    int32_t num_heads_kv, int32_t d_qk, int32_t d_vo, int32_t page_size,
    pkv_layout kv_layout, int32_t causal, const float *q_scale,
    const float *k_scale, const float *v_scale, void *out, float *lse,
    pkv_dtype qkv_dtype, pkv_dtype o_dtype, const int32_t *batch_offsets_q,
    const int32_t *batch_offsets_o, const int32_t *batch_offsets_k,
    const int32_t *batch_offsets_v, const int32_t *batch_offsets_stats, void *stream) {
  const bool paged = block_tables != nullptr;
  CHECK(batch_size >= 0, PKV_ERR_INVALID_ARG, "batch_size < 0");
  CHECK(!paged || (batch_offsets_k == nullptr && batch_offsets_v == nullptr),
        PKV_ERR_INVALID_ARG, "batch_offsets_k / batch_offsets_v apply only without block_tables");
  CHECK(num_heads_kv > 0 && num_heads_qo > 0, PKV_ERR_INVALID_ARG,
        "head counts must be positive");
  CHECK(num_heads_qo >= num_heads_kv, PKV_ERR_INVALID_ARG,
        "num_heads_qo must be >= num_heads_kv");
  CHECK(num_heads_qo % num_heads_kv == 0, PKV_ERR_UNSUPPORTED,
        "num_heads_qo must be a multiple of num_heads_kv");
  CHECK(d_qk == 128 || d_qk == 192, PKV_ERR_UNSUPPORTED,
        "query/key head dim must be 128 or 192");
  CHECK(d_vo == 128, PKV_ERR_UNSUPPORTED, "value/output head dim must be 128");
  CHECK(kv_layout == PKV_NHD || kv_layout == PKV_HND, PKV_ERR_INVALID_ARG,
        "kv_layout must be NHD or HND");
  CHECK(qkv_dtype == PKV_F16 || qkv_dtype == PKV_BF16 || qkv_dtype == PKV_E4M3,
        PKV_ERR_INVALID_ARG, "unknown q/k/v dtype");
  CHECK(o_dtype == PKV_F16 || o_dtype == PKV_BF16, PKV_ERR_UNSUPPORTED,
        "output dtype must be F16 or BF16");
  CHECK(max_token_per_sequence >= 0 && max_sequence_kv >= 0,
        PKV_ERR_INVALID_ARG, "negative maximum length");
  CHECK(lse != nullptr, PKV_ERR_INVALID_ARG,
        "lse is required (the log-sum-exp must be returned)");
  const int es = elem_bytes(qkv_dtype);
  if (paged) {
    CHECK(page_size_ok(page_size), PKV_ERR_UNSUPPORTED,
          "page_size must be 16, 32 or 64");
    CHECK(max_pages_per_seq > 0, PKV_ERR_INVALID_ARG, "max_pages_per_seq <= 0");
    CHECK((int64_t)max_pages_per_seq * page_size >= max_sequence_kv,
          PKV_ERR_INVALID_ARG, "block_tables too narrow for max_sequence_kv");
    const int64_t pk = (int64_t)page_size * num_heads_kv * d_qk;
    const int64_t pv = (int64_t)page_size * num_heads_kv * d_vo;
    CHECK(page_stride_k >= pk && page_stride_v >= pv, PKV_ERR_INVALID_ARG,
          "page stride smaller than one page");
    CHECK((page_stride_k * es) % 16 == 0 && (page_stride_v * es) % 16 == 0,
          PKV_ERR_UNSUPPORTED, "page strides must be multiples of 16 bytes");
  }
  CHECK(workspace_bytes >= pkv_prefill_workspace_size(batch_size),
        PKV_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than "
        "pkv_prefill_workspace_size(batch_size)");
  if (batch_size == 0 || max_token_per_sequence == 0) return PKV_OK;
  CHECK(q && k_cache && v_cache && workspace && actual_seq_lens_q &&
            actual_seq_lens_kv && out,
        PKV_ERR_INVALID_ARG, "null pointer");
  CHECK(aligned(q, 16) && aligned(k_cache, 16) && aligned(v_cache, 16) &&
            aligned(out, 16) && aligned(workspace, 16),
        PKV_ERR_UNSUPPORTED, "q/k/v/out/workspace must be 16-byte aligned");

  pkv::PrefillArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.page_stride_k = page_stride_k;
  a.page_stride_v = page_stride_v;
  if (kv_layout == PKV_NHD || !paged) {  // unpaged rows are [row][head][d]
    a.slot_stride_k = (int64_t)num_heads_kv * d_qk;
    a.head_stride_k = d_qk;
    a.slot_stride_v = (int64_t)num_heads_kv * d_vo;
    a.head_stride_v = d_vo;
  } else {
    a.slot_stride_k = d_qk;
    a.head_stride_k = (int64_t)page_size * d_qk;
    a.slot_stride_v = d_vo;
    a.head_stride_v = (int64_t)page_size * d_vo;
  }
  a.lens_q = actual_seq_lens_q;
  a.lens_kv = actual_seq_lens_kv;
  int32_t *cum_q = reinterpret_cast<int32_t *>(workspace);
  int32_t *cum_kv = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(workspace) +
                                                prefill_region_bytes(batch_size));
  // Absent offsets mean packed rows: small batches leave them null and the
  // kernel sums the lengths itself; larger ones get a prefix-sum launch.
  const bool inline_offsets = batch_size <= pkv::kInlineOffsetBatch;
  int32_t *packed_q = inline_offsets ? nullptr : cum_q;
  int32_t *packed_kv = inline_offsets ? nullptr : cum_kv;
  a.off_q = batch_offsets_q ? batch_offsets_q : packed_q;
  a.off_o = batch_offsets_o ? batch_offsets_o : packed_q;
  a.off_lse = batch_offsets_stats ? batch_offsets_stats : packed_q;
  a.block_tables = block_tables;
  a.off_k = batch_offsets_k ? batch_offsets_k : packed_kv;
  a.off_v = batch_offsets_v ? batch_offsets_v : packed_kv;
  a.max_pages = max_pages_per_seq;
  a.batch = batch_size;
  a.num_heads_qo = num_heads_qo;
  a.num_heads_kv = num_heads_kv;
  a.d_qk = d_qk;
  a.d_vo = d_vo;
  a.page_size = paged ? page_size : 16;  // unpaged: 16-row groups per wave
  a.max_q = max_token_per_sequence;
  a.max_kv = max_sequence_kv;
  a.causal = causal ? 1 : 0;
  a.scale = scale;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.out = out;
  a.lse = lse;
  a.qkv_dtype = qkv_dtype;
  a.o_dtype = o_dtype;
  hipStream_t s = as_stream(stream);
  if (!inline_offsets && (!batch_offsets_q || !batch_offsets_o || !batch_offsets_stats)) {
    const hipError_t e = pkv::launch_exclusive_cumsum(actual_seq_lens_q, batch_size, cum_q, s);
    if (e != hipSuccess) return from_hip(e, __func__);
  }
  if (!inline_offsets && !paged && (!batch_offsets_k || !batch_offsets_v)) {
    const hipError_t e =
        pkv::launch_exclusive_cumsum(actual_seq_lens_kv, batch_size, cum_kv, s);
    if (e != hipSuccess) return from_hip(e, __func__);
  }
  return from_hip(pkv::launch_prefill(a, s), __func__);
}

PKV_API size_t pkv_decode_workspace_size(int32_t batch_size,
                                         int32_t q_len_per_req,
                                         int32_t num_heads_qo,
                                         int32_t num_heads_kv, int32_t head_dim,
                                         int32_t max_seq_len,
                                         int32_t window_left) {
  if (batch_size < 0 || q_len_per_req < 1 || num_heads_kv <= 0 ||
      num_heads_qo < num_heads_kv || head_dim <= 0 || max_seq_len < 0)
    return 0;
  return pkv::plan_decode(batch_size, q_len_per_req, num_heads_qo,
                          num_heads_kv, head_dim, max_seq_len, window_left)
      .workspace_bytes;
}

// ---- decode ---------------------------------------------------------------
//
// The no-alloc entry point's split partials live in this file-scope device
// array instead of a caller's workspace. Host code never uses the array's
// name as an address: on the host it is only a stand-in for the symbol. The
// device address comes from hipGetSymbolAddress, taken once per device (on
// the first call that needs it on that device, with the device current) and
// kept in g_scratch_addr.
static __device__ __align__(256) char scratch[PKV_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the device `stream` runs on, which must be
// the current device.
pkv_status scratch_address(hipStream_t stream, void **addr, const char *fn) {
  int cur = -1, sdev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return from_hip(e, fn);
  e = hipStreamGetDevice(stream, &sdev);
  if (e != hipSuccess) return from_hip(e, fn);
  if (sdev != cur)
    return fail(PKV_ERR_INVALID_ARG, fn, "the stream's device must be the current device");
  if (cur < 0 || cur >= kMaxDevices)
    return fail(PKV_ERR_UNSUPPORTED, fn, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[cur]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return from_hip(e, fn);
    if (!p) return fail(PKV_ERR_HIP, fn, "hipGetSymbolAddress gave a null address");
    g_scratch_addr[cur] = p;
  }
  *addr = g_scratch_addr[cur];
  return PKV_OK;
}

#define CHECKF(cond, st, msg)                 \
  do {                                        \
    if (!(cond)) return fail((st), fn, (msg)); \
  } while (0)

// Both decode entry points: every argument check on host scalars first,
// then (no-alloc only) the scratch array's address, then the launch.
pkv_status decode_entry(
    const char *fn, bool use_scratch, const void *query, const void *k_cache,
    const void *v_cache, int64_t page_stride_k, int64_t page_stride_v, void *workspace,
    size_t workspace_bytes, const int32_t *block_tables, int32_t max_pages_per_seq,
    const uint32_t *seq_lens, int32_t batch_size, int32_t max_seq_len, float bmm1_scale,
    float bmm2_scale, int32_t window_left, void *out, pkv_dtype out_dtype,
    const float *sinks, pkv_layout kv_layout, int32_t q_len_per_req, int32_t num_heads_qo,
    int32_t num_heads_kv, int32_t head_dim, int32_t page_size, pkv_dtype q_dtype,
    pkv_dtype kv_dtype, const float *bmm1_scale_dev, const float *bmm2_scale_dev,
    float o_scale, const int32_t *cum_seq_lens_q, int32_t max_q_len,
    const uint8_t *spec_mask, void *stream) {
  CHECKF(batch_size >= 0, PKV_ERR_INVALID_ARG, "batch_size < 0");
  CHECKF(q_len_per_req >= 1, PKV_ERR_INVALID_ARG, "q_len_per_req < 1");
  CHECKF(cum_seq_lens_q ? max_q_len >= 1 : max_q_len == 0, PKV_ERR_INVALID_ARG,
         "max_q_len must be >= 1 with cum_seq_lens_q and 0 without it");
  // queries per request, or their maximum with variable-length queries
  const int32_t q_max = cum_seq_lens_q ? max_q_len : q_len_per_req;
  CHECKF(window_left >= -1, PKV_ERR_INVALID_ARG, "window_left < -1");
  CHECKF(num_heads_kv > 0 && num_heads_qo > 0, PKV_ERR_INVALID_ARG,
         "head counts must be positive");
  CHECKF(num_heads_qo >= num_heads_kv, PKV_ERR_INVALID_ARG,
         "num_heads_qo must be >= num_heads_kv");
  CHECKF(num_heads_qo % num_heads_kv == 0, PKV_ERR_UNSUPPORTED,
         "num_heads_qo must be a multiple of num_heads_kv");
  CHECKF(head_dim == 128, PKV_ERR_UNSUPPORTED, "head_dim must be 128");
  CHECKF((int64_t)q_max * (num_heads_qo / num_heads_kv) <= pkv::kDecodeMaxRows,
         PKV_ERR_UNSUPPORTED,
         "q_len_per_req (or max_q_len) * num_heads_qo / num_heads_kv must be <= 1024");
  CHECKF(!spec_mask || q_max <= 64, PKV_ERR_UNSUPPORTED,
         "with a spec_mask, q_len_per_req (or max_q_len) must be <= 64");
  CHECKF(kv_layout == PKV_NHD || kv_layout == PKV_HND, PKV_ERR_INVALID_ARG,
         "kv_layout must be NHD or HND");
  CHECKF(q_dtype == PKV_F16 || q_dtype == PKV_BF16, PKV_ERR_UNSUPPORTED,
         "query dtype must be F16 or BF16");
  CHECKF(kv_dtype == q_dtype || kv_dtype == PKV_E4M3, PKV_ERR_UNSUPPORTED,
         "kv dtype must equal the query dtype or be E4M3");
  CHECKF(out_dtype == PKV_F16 || out_dtype == PKV_BF16 || out_dtype == PKV_E4M3,
         PKV_ERR_UNSUPPORTED, "output dtype must be F16, BF16 or E4M3");
  CHECKF(out_dtype != PKV_E4M3 || (o_scale > 0.0f && o_scale <= 3.4e38f),
         PKV_ERR_INVALID_ARG, "o_scale must be finite and > 0");
  CHECKF(page_size_ok(page_size), PKV_ERR_UNSUPPORTED, "page_size must be 16, 32 or 64");
  CHECKF(max_seq_len >= 0, PKV_ERR_INVALID_ARG, "max_seq_len < 0");
  CHECKF(max_pages_per_seq > 0, PKV_ERR_INVALID_ARG, "max_pages_per_seq <= 0");
  CHECKF((int64_t)max_pages_per_seq * page_size >= max_seq_len, PKV_ERR_INVALID_ARG,
         "block_tables too narrow for max_seq_len");
  const int es = elem_bytes(kv_dtype);
  const int64_t pe = (int64_t)page_size * num_heads_kv * head_dim;
  CHECKF(page_stride_k >= pe && page_stride_v >= pe, PKV_ERR_INVALID_ARG,
         "page stride smaller than one page");
  CHECKF((page_stride_k * es) % 16 == 0 && (page_stride_v * es) % 16 == 0,
         PKV_ERR_UNSUPPORTED, "page strides must be multiples of 16 bytes");
  const pkv::DecodePlan plan =
      pkv::plan_decode(batch_size, q_max, num_heads_qo, num_heads_kv, head_dim,
                       max_seq_len, window_left);
  if (use_scratch) {
    if (plan.workspace_bytes > PKV_DECODE_SCRATCH_BYTES) {
      char msg[192];
      snprintf(msg, sizeof msg,
               "the split plan needs %zu bytes of workspace; the static scratch holds %zu "
               "(use pkv_batch_decode_with_kv_cache with a workspace)",
               plan.workspace_bytes, (size_t)PKV_DECODE_SCRATCH_BYTES);
      return fail(PKV_ERR_WORKSPACE_TOO_SMALL, fn, msg);
    }
  } else {
    CHECKF(workspace_bytes >= plan.workspace_bytes, PKV_ERR_WORKSPACE_TOO_SMALL,
           "workspace smaller than pkv_decode_workspace_size(...)");
  }
  if (batch_size == 0) return PKV_OK;
  CHECKF(query && k_cache && v_cache && block_tables && seq_lens && out,
         PKV_ERR_INVALID_ARG, "null pointer");
  CHECKF(use_scratch || plan.workspace_bytes == 0 || workspace, PKV_ERR_INVALID_ARG,
         "null workspace");
  CHECKF(aligned(query, 16) && aligned(k_cache, 16) && aligned(v_cache, 16) &&
             aligned(out, 16) && aligned(workspace, 16),
         PKV_ERR_UNSUPPORTED, "query/k/v/out/workspace must be 16-byte aligned");
  if (use_scratch) {
    workspace = nullptr;
    if (plan.workspace_bytes > 0) {
      const pkv_status st = scratch_address(as_stream(stream), &workspace, fn);
      if (st != PKV_OK) return st;
    }
  }

  pkv::DecodeArgs a{};
  a.q = query;
  a.k = k_cache;
  a.v = v_cache;
  a.page_stride_k = page_stride_k;
  a.page_stride_v = page_stride_v;
  if (kv_layout == PKV_NHD) {
    a.slot_stride = (int64_t)num_heads_kv * head_dim;
    a.head_stride = head_dim;
  } else {
    a.slot_stride = head_dim;
    a.head_stride = (int64_t)page_size * head_dim;
  }
  a.block_tables = block_tables;
  a.max_pages = max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.batch = batch_size;
  a.max_seq_len = max_seq_len;
  a.bmm1_scale = bmm1_scale;
  a.bmm1_ptr = bmm1_scale_dev;
  a.bmm2_ptr = bmm2_scale_dev;
  a.o_scale = out_dtype == PKV_E4M3 ? o_scale : 1.0f;
  a.bmm2_scale = bmm2_scale;
  a.window_left = window_left;
  a.out = out;
  a.sinks = sinks;
  a.q_len = q_max;
  a.cum_q = cum_seq_lens_q;
  a.mask = spec_mask;
  a.num_heads_qo = num_heads_qo;
  a.num_heads_kv = num_heads_kv;
  a.head_dim = head_dim;
  a.page_size = page_size;
  a.q_dtype = q_dtype;
  a.kv_dtype = kv_dtype;
  a.out_dtype = out_dtype;
  a.workspace = workspace;
  return from_hip(pkv::launch_decode(a, plan, as_stream(stream)), fn);
}

#undef CHECKF

}  // namespace

PKV_API pkv_status pkv_batch_decode_with_kv_cache(
    const void *query, const void *k_cache, const void *v_cache,
    int64_t page_stride_k, int64_t page_stride_v, void *workspace,
    size_t workspace_bytes, const int32_t *block_tables,
    int32_t max_pages_per_seq, const uint32_t *seq_lens, int32_t batch_size,
    int32_t max_seq_len, float bmm1_scale, float bmm2_scale,
    int32_t window_left, void *out, pkv_dtype out_dtype, const float *sinks,
    pkv_layout kv_layout, int32_t q_len_per_req, int32_t num_heads_qo,
    int32_t num_heads_kv, int32_t head_dim, int32_t page_size,
    pkv_dtype q_dtype, pkv_dtype kv_dtype, const float *bmm1_scale_dev,
    const float *bmm2_scale_dev, float o_scale, const int32_t *cum_seq_lens_q,
    int32_t max_q_len, const uint8_t *spec_mask, void *stream) {
  return decode_entry(__func__, false, query, k_cache, v_cache, page_stride_k, page_stride_v,
                      workspace, workspace_bytes, block_tables, max_pages_per_seq, seq_lens,
                      batch_size, max_seq_len, bmm1_scale, bmm2_scale, window_left, out,
                      out_dtype, sinks, kv_layout, q_len_per_req, num_heads_qo, num_heads_kv,
                      head_dim, page_size, q_dtype, kv_dtype, bmm1_scale_dev, bmm2_scale_dev,
                      o_scale, cum_seq_lens_q, max_q_len, spec_mask, stream);
}

PKV_API pkv_status pkv_batch_decode_with_kv_cache_no_alloc(
    const void *query, const void *k_cache, const void *v_cache,
    int64_t page_stride_k, int64_t page_stride_v, const int32_t *block_tables,
    int32_t max_pages_per_seq, const uint32_t *seq_lens, int32_t batch_size,
    int32_t max_seq_len, float bmm1_scale, float bmm2_scale,
    int32_t window_left, void *out, pkv_dtype out_dtype, const float *sinks,
    pkv_layout kv_layout, int32_t q_len_per_req, int32_t num_heads_qo,
    int32_t num_heads_kv, int32_t head_dim, int32_t page_size,
    pkv_dtype q_dtype, pkv_dtype kv_dtype, const float *bmm1_scale_dev,
    const float *bmm2_scale_dev, float o_scale, const int32_t *cum_seq_lens_q,
    int32_t max_q_len, const uint8_t *spec_mask, void *stream) {
  return decode_entry(__func__, true, query, k_cache, v_cache, page_stride_k, page_stride_v,
                      nullptr, 0, block_tables, max_pages_per_seq, seq_lens, batch_size,
                      max_seq_len, bmm1_scale, bmm2_scale, window_left, out, out_dtype, sinks,
                      kv_layout, q_len_per_req, num_heads_qo, num_heads_kv, head_dim,
                      page_size, q_dtype, kv_dtype, bmm1_scale_dev, bmm2_scale_dev, o_scale,
                      cum_seq_lens_q, max_q_len, spec_mask, stream);
}
