/*
 * pkv.h -- C ABI of the paged-KV attention library for AMD MI355X (gfx950).
 *
 * Three operations over a paged key/value cache, following FlashInfer's API
 * pages:
 *   - flashinfer.page.append_paged_kv_cache (and the helpers get_seq_lens /
 *     get_batch_indices_positions used in its Example);
 *   - flashinfer.prefill.cudnn_batch_prefill_with_kv_cache;
 *   - flashinfer.decode.trtllm_batch_decode_with_kv_cache.
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless the argument name starts with h_.
 *   - The caller owns every buffer (caches, page tables, outputs, workspace).
 *     The library allocates nothing, keeps no state between calls, never
 *     synchronises and never reads device memory from the host. The one
 *     exception is pkv_batch_decode_with_kv_cache_no_alloc, which uses a
 *     fixed device array of the library's own instead of a workspace.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     null stream). A call returns once the work is enqueued.
 *   - Validation uses host scalars and pointer non-nullness only. On any
 *     violation the call returns an error before enqueueing anything, and
 *     pkv_last_error() describes it. Device-side values that break a stated
 *     precondition (a position outside its request, a page id outside the
 *     pool) are not checked and give undefined results.
 *   - Element sizes: PKV_F16 and PKV_BF16 are 2 bytes, PKV_E4M3 (OCP e4m3fn,
 *     max 448, no infinities) is 1 byte. Strides are in ELEMENTS.
 *
 * Cache layout (append page, Parameters "paged_kv_cache"; decode page,
 * Parameters "kv_cache"): K and V are passed as two base pointers, each
 * addressing pages of `page_stride` elements:
 *   NHD  page = [page_size][num_kv_heads][head_dim]
 *   HND  page = [num_kv_heads][page_size][head_dim]
 * A single 5D tensor [max_num_pages, 2, ...] is K = &t[0,0], V = &t[0,1] with
 * page_stride = 2 * page elements; a (k_cache, v_cache) tuple has
 * page_stride = page elements (K and V may differ in head_dim).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 4

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,        /* argument out of its documented range */
  PKV_ERR_UNSUPPORTED = 2,        /* legal on the pages, not built here   */
  PKV_ERR_WORKSPACE_TOO_SMALL = 3,
  PKV_ERR_HIP = 4                 /* a HIP runtime call failed            */
} pkv_status;

typedef enum { PKV_NHD = 0, PKV_HND = 1 } pkv_layout;

typedef enum { PKV_F16 = 0, PKV_BF16 = 1, PKV_E4M3 = 2 } pkv_dtype;

/* Version of this header's ABI (PKV_ABI_VERSION). */
int pkv_abi_version(void);

/* Message for the last non-OK status returned on the calling thread. */
const char *pkv_last_error(void);

/*
 * Tokens held by each request's pages (append page, Example: each length is
 * (pages - 1) * page_size + kv_last_page_len, e.g. 45 = (3 - 1) * 16 + 13).
 *   kv_indptr        [batch_size + 1] int32, page-list offsets per request
 *   kv_last_page_len [batch_size]     int32, entries in each last page
 *   seq_lens         [batch_size]     int32, output
 * A request with no pages gets 0. Errors: batch_size < 0, page_size <= 0,
 * null pointer with batch_size > 0.
 */
pkv_status pkv_get_seq_lens(const int32_t *kv_indptr,
                            const int32_t *kv_last_page_len,
                            int32_t batch_size, int32_t page_size,
                            int32_t *seq_lens, void *stream);

/*
 * Request index and absolute position of each appended row (append page,
 * Example and Note). The page table already includes the appended rows, so
 * the n_b = append_indptr[b+1] - append_indptr[b] rows of request b are its
 * last n_b positions: row append_indptr[b] + k gets batch index b and
 * position seq_lens[b] - n_b + k.
 *   append_indptr  [batch_size + 1] int32, append_indptr[batch_size] == nnz
 *   seq_lens       [batch_size]     int32, lengths INCLUDING the new rows
 *   batch_indices  [nnz] int32, output
 *   positions      [nnz] int32, output
 * Errors: batch_size < 0, nnz < 0, null pointers with nnz > 0.
 */
pkv_status pkv_get_batch_indices_positions(const int32_t *append_indptr,
                                           const int32_t *seq_lens,
                                           int32_t batch_size, int32_t nnz,
                                           int32_t *batch_indices,
                                           int32_t *positions, void *stream);

/*
 * CSR page list -> dense block table. The append page describes pages by
 * kv_indptr / kv_indices; the prefill and decode pages take block_tables
 * [batch_size, num_pages_per_seq]. Entry k of request b is
 * kv_indices[kv_indptr[b] + k]; entries past a request's page count are -1.
 *   block_tables [batch_size, max_pages_per_seq] int32, output (row-major)
 * Errors: batch_size < 0, max_pages_per_seq <= 0, null pointers.
 */
pkv_status pkv_csr_to_block_tables(const int32_t *kv_indptr,
                                   const int32_t *kv_indices,
                                   int32_t batch_size,
                                   int32_t max_pages_per_seq,
                                   int32_t *block_tables, void *stream);

/*
 * append_paged_kv_cache (append page, Parameters and Note).
 * Row i of append_key / append_value ([nnz, num_kv_heads, head_dim],
 * contiguous, `dtype`) is copied bit for bit into request
 * batch_indices[i]'s page kv_indices[kv_indptr[b] + positions[i] / page_size]
 * at slot positions[i] % page_size, for K and V. Nothing else is written.
 *   k_cache / v_cache  cache base pointers, pages of page_stride_k / _v elems
 *   kv_last_page_len   accepted for signature parity; not read (may be NULL)
 * Precondition (Note of the page): the pages already cover the appended
 * positions. Errors: nnz < 0, batch_size < 0, num_kv_heads <= 0,
 * head_dim <= 0 or head_dim * element size not a multiple of 16 bytes,
 * page_size <= 0, page strides smaller than one page, unknown layout/dtype,
 * null pointers with nnz > 0.
 */
pkv_status pkv_append_paged_kv_cache(const void *append_key,
                                     const void *append_value,
                                     const int32_t *batch_indices,
                                     const int32_t *positions, int32_t nnz,
                                     void *k_cache, void *v_cache,
                                     int64_t page_stride_k,
                                     int64_t page_stride_v,
                                     const int32_t *kv_indices,
                                     const int32_t *kv_indptr,
                                     const int32_t *kv_last_page_len,
                                     int32_t batch_size, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t page_size,
                                     pkv_layout kv_layout, pkv_dtype dtype,
                                     void *stream);

/* Workspace bytes pkv_batch_prefill_with_kv_cache needs for batch_size. */
size_t pkv_prefill_workspace_size(int32_t batch_size);

/*
 * Batch prefill over a paged cache (prefill page, Parameters, Returns, Note).
 * For each request b with L_q = actual_seq_lens_q[b] queries and
 * L_kv = actual_seq_lens_kv[b] keys:
 *   out[t, h] = v_scale * softmax_j(scale * q_scale * k_scale * q[t,h].k[j,h/G]
 *                                   + mask(t, j)) . v[j, h/G]
 *   lse[t, h] = natural log of the softmax denominator (log-sum-exp of the
 *               scaled scores over allowed keys)
 * with G = num_heads_qo / num_heads_kv, and with causal=1 the mask aligned
 * bottom-right: query t sees keys j <= t + L_kv - L_q. Token j of request b
 * is slot j % page_size of page block_tables[b * max_pages_per_seq +
 * j / page_size].
 * Without paging (block_tables NULL; the page's non-paged k_cache / v_cache
 * of shape (total KV length, H_kv, d)), token j of request b is row
 * batch_offsets_k[b] + j of k_cache and batch_offsets_v[b] + j of v_cache;
 * page_size, page strides, max_pages_per_seq and kv_layout are then ignored.
 * batch_offsets_q / _o / _k / _v / _stats ([batch_size] int32 on the device,
 * the page's batch offsets, counted in rows) give the first row of each
 * request in q, out, k_cache, v_cache and lse; each may be NULL, meaning the
 * exclusive prefix sum of the request lengths (rows packed in request order).
 * _k and _v apply only without paging (PKV_ERR_INVALID_ARG otherwise).
 *   q    [sum L_q, num_heads_qo, d_qk] contiguous, qkv_dtype; request b's
 *        rows start at the exclusive prefix sum of actual_seq_lens_q
 *   out  [sum L_q, num_heads_qo, d_vo], o_dtype (PKV_F16 or PKV_BF16)
 *   lse  [sum L_q, num_heads_qo] float32 (required: the page says the
 *        log-sum-exp must be returned)
 *   q_scale/k_scale/v_scale  device float32 scalars or NULL (= 1.0); the
 *        page's per-tensor (1,1,1,1) scales for fp8 inputs
 *   actual_seq_lens_q/_kv    [batch_size] int32 on the device
 *   max_token_per_sequence   >= every L_q; max_sequence_kv >= every L_kv
 *   workspace  >= pkv_prefill_workspace_size(batch_size) bytes
 * Supported (page Note): d_qk in {128, 192}, d_vo == 128,
 * num_heads_qo % num_heads_kv == 0; qkv_dtype F16, BF16 or E4M3 (E4M3 takes
 * a BF16 output); page_size in {16, 32, 64}. A row with no allowed key gets
 * out = 0 and lse = -inf.
 */
pkv_status pkv_batch_prefill_with_kv_cache(
    const void *q, const void *k_cache, const void *v_cache,
    int64_t page_stride_k, int64_t page_stride_v, float scale,
    void *workspace, size_t workspace_bytes, int32_t max_token_per_sequence,
    int32_t max_sequence_kv, const int32_t *actual_seq_lens_q,
    const int32_t *actual_seq_lens_kv, const int32_t *block_tables,
    int32_t max_pages_per_seq, int32_t batch_size, int32_t num_heads_qo,
    int32_t num_heads_kv, int32_t d_qk, int32_t d_vo, int32_t page_size,
    pkv_layout kv_layout, int32_t causal, const float *q_scale,
    const float *k_scale, const float *v_scale, void *out, float *lse,
    pkv_dtype qkv_dtype, pkv_dtype o_dtype, const int32_t *batch_offsets_q,
    const int32_t *batch_offsets_o, const int32_t *batch_offsets_k,
    const int32_t *batch_offsets_v, const int32_t *batch_offsets_stats, void *stream);

/* Workspace bytes pkv_batch_decode_with_kv_cache needs for these sizes. */
size_t pkv_decode_workspace_size(int32_t batch_size, int32_t q_len_per_req,
                                 int32_t num_heads_qo, int32_t num_heads_kv,
                                 int32_t head_dim, int32_t max_seq_len,
                                 int32_t window_left);

/*
 * Batch decode over block_tables (decode page, Parameters).
 * Request b has seq_lens[b] keys; its q_len_per_req queries
 * (query rows b*q_len_per_req ..) are its last q_len_per_req positions,
 * causal among themselves. For query row t at position
 * pos = seq_lens[b] - q_len_per_req + t and qo head h:
 *   s_j   = bmm1_scale * q[t,h] . k[j, h/G]     for allowed keys j
 *   allowed: j <= pos and (window_left < 0 or j >= pos - window_left)
 *   out   = bmm2_scale * sum_j e^{s_j} v[j, h/G] / (sum_j e^{s_j} + e^{sinks[h]})
 * (the sink term only when sinks != NULL). window_left is inclusive; -1
 * means the whole sequence.
 *   query [batch_size * q_len_per_req, num_heads_qo, head_dim], q_dtype BF16
 *         or F16
 *   out   [batch_size * q_len_per_req, num_heads_qo, head_dim], out_dtype
 *         BF16, F16 or E4M3. For E4M3 (the page's fp8 output with o_scale)
 *         each stored code is e4m3fn(out / o_scale): nearest value, ties to
 *         the even code, saturating at +-448, NaN kept; o_scale must be
 *         finite and > 0 (it is ignored for the other output types).
 *   kv_dtype BF16, F16 or E4M3 (E4M3 values are used as stored: fold a
 *         per-tensor k scale into bmm1_scale and a v scale into bmm2_scale)
 *   bmm1_scale_dev / bmm2_scale_dev  device float32 scalars or NULL; when
 *         given they replace bmm1_scale / bmm2_scale (the page's tensor form
 *         of the two scales), read by the kernels at run time
 *   seq_lens [batch_size] uint32; max_seq_len >= every entry
 *   sinks    [num_heads_qo] float32 logits or NULL
 *   cum_seq_lens_q, max_q_len  variable-length queries (decode page,
 *         Parameters): when cum_seq_lens_q ([batch_size + 1] int32 on the
 *         device) is given, request b's queries are query/out rows
 *         cum_seq_lens_q[b] .. cum_seq_lens_q[b+1] - 1 (its last that many
 *         positions, any count from 0 to max_q_len >= 1) and q_len_per_req
 *         is ignored; otherwise max_q_len must be 0
 *   spec_mask  the speculative-decoding mask (decode page, Parameters) or
 *         NULL: uint8 [batch_size][Q][Q] on the device, Q = max_q_len with
 *         cum_seq_lens_q, else q_len_per_req. Draft t of request b sees the
 *         draft at position seq_lens[b] - q_b + i when
 *         spec_mask[b][t][i] != 0 (q_b its query count); this replaces the
 *         causal rule among the drafts. Keys before the drafts stay visible,
 *         and window_left still applies (to positions).
 *   workspace >= pkv_decode_workspace_size(...) bytes (contents ignored)
 * Supported: head_dim == 128, num_heads_qo % num_heads_kv == 0,
 * Q * num_heads_qo / num_heads_kv <= 1024 (query rows per kv head), Q <= 64
 * when spec_mask is given, page_size in {16, 32, 64}.
 */
pkv_status pkv_batch_decode_with_kv_cache(
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
    int32_t max_q_len, const uint8_t *spec_mask, void *stream);

/* Largest split-KV workspace pkv_batch_decode_with_kv_cache_no_alloc can
 * serve from its static scratch array (bytes). */
#define PKV_DECODE_SCRATCH_BYTES ((size_t)64 << 20)

/* pkv_batch_decode_with_kv_cache without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. It calls no allocating
 * routine. Arguments, results and errors are those of
 * pkv_batch_decode_with_kv_cache; the split partials go to a file-scope
 * device array of PKV_DECODE_SCRATCH_BYTES bytes inside the library instead
 * of a caller's workspace (each GPU the library runs on holds its own copy
 * until the process ends). Nothing in it needs clearing: the kernels read
 * back only what the same call wrote.
 *   - The array is shared by every call on one GPU: calls that overlap on
 *     one GPU (on different streams, or from several threads) race on it
 *     and give wrong results. Serialise them.
 *   - The stream's device must be the current device (NULL stream: the
 *     current device), since the array's address is per device.
 *   - A call whose split plan needs more than PKV_DECODE_SCRATCH_BYTES
 *     (pkv_decode_workspace_size(...) larger than that) returns
 *     PKV_ERR_WORKSPACE_TOO_SMALL before any HIP call.
 */
pkv_status pkv_batch_decode_with_kv_cache_no_alloc(
    const void *query, const void *k_cache, const void *v_cache,
    int64_t page_stride_k, int64_t page_stride_v, const int32_t *block_tables,
    int32_t max_pages_per_seq, const uint32_t *seq_lens, int32_t batch_size,
    int32_t max_seq_len, float bmm1_scale, float bmm2_scale,
    int32_t window_left, void *out, pkv_dtype out_dtype, const float *sinks,
    pkv_layout kv_layout, int32_t q_len_per_req, int32_t num_heads_qo,
    int32_t num_heads_kv, int32_t head_dim, int32_t page_size,
    pkv_dtype q_dtype, pkv_dtype kv_dtype, const float *bmm1_scale_dev,
    const float *bmm2_scale_dev, float o_scale, const int32_t *cum_seq_lens_q,
    int32_t max_q_len, const uint8_t *spec_mask, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
