// Host-side launchers of the HIP kernels. Declared here, defined next to
// their kernels, called from the C ABI layer after validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

hipError_t launch_get_seq_lens(const int32_t *kv_indptr, const int32_t *last,
                               int32_t batch, int32_t page_size,
                               int32_t *seq_lens, hipStream_t s);

hipError_t launch_batch_indices_positions(const int32_t *append_indptr,
                                          const int32_t *seq_lens,
                                          int32_t batch, int32_t nnz,
                                          int32_t *batch_indices,
                                          int32_t *positions, hipStream_t s);

hipError_t launch_csr_to_block_tables(const int32_t *kv_indptr,
                                      const int32_t *kv_indices, int32_t batch,
                                      int32_t max_pages, int32_t *bt,
                                      hipStream_t s);

struct AppendArgs {
  const void *key, *value;
  const int32_t *batch_indices, *positions;
  int32_t nnz;
  void *k_cache, *v_cache;
  int64_t page_stride_k, page_stride_v;  // bytes
  int64_t slot_stride, head_stride;      // bytes
  const int32_t *kv_indices, *kv_indptr;
  int32_t num_heads, row_bytes_per_head;  // bytes of one head's head_dim run
  int32_t page_size;
};
hipError_t launch_append(const AppendArgs &a, hipStream_t s);

// Exclusive prefix sum of lens[0..batch) into out[0..batch].
hipError_t launch_exclusive_cumsum(const int32_t *lens, int32_t batch,
                                   int32_t *out, hipStream_t s);

// Batches up to this size get packed row offsets summed inside the prefill
// kernel (at most this many scalar loads per workgroup) instead of a
// separate prefix-sum launch.
constexpr int32_t kInlineOffsetBatch = 64;

struct PrefillArgs {
  const void *q, *k, *v;
  int64_t page_stride_k, page_stride_v;  // elements
  int64_t slot_stride_k, head_stride_k;  // elements
  int64_t slot_stride_v, head_stride_v;  // elements
  const int32_t *lens_q, *lens_kv;
  // first row of each request in q, out and lse ([batch] int32 each);
  // null: packed rows, the kernel sums lens_q of the requests before it
  // (used for batches of at most kInlineOffsetBatch)
  const int32_t *off_q, *off_o, *off_lse;
  // null: K/V are not paged; request b's key / value rows start at row
  // off_k[b] / off_v[b] of [rows, H_kv, d] tensors (null offsets: packed,
  // summed from lens_kv as above)
  const int32_t *block_tables;
  const int32_t *off_k, *off_v;
  int32_t max_pages;
  int32_t batch, num_heads_qo, num_heads_kv, d_qk, d_vo, page_size;
  int32_t max_q;
  int32_t causal;
  float scale;
  const float *q_scale, *k_scale, *v_scale;
  void *out;
  float *lse;
  int32_t qkv_dtype, o_dtype;  // pkv_dtype values
};
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);

struct DecodeArgs {
  const void *q, *k, *v;
  int64_t page_stride_k, page_stride_v;  // elements
  int64_t slot_stride, head_stride;      // elements
  const int32_t *block_tables;
  int32_t max_pages;
  const uint32_t *seq_lens;
  int32_t batch, max_seq_len;
  float bmm1_scale, bmm2_scale;
  const float *bmm1_ptr, *bmm2_ptr;  // device scalars replacing the floats, or null
  float o_scale;                     // e4m3 output: stored code = e4m3(out / o_scale)
  int32_t window_left;
  void *out;
  const float *sinks;
  // q_len: queries per request, or their maximum when cum_q is given
  int32_t q_len, num_heads_qo, num_heads_kv, head_dim, page_size;
  int32_t q_dtype, kv_dtype, out_dtype;  // pkv_dtype values
  const int32_t *cum_q;  // [batch + 1] query row offsets, or null (uniform q_len)
  const uint8_t *mask;   // [batch][q_len][q_len] draft mask, or null (causal)
  void *workspace;
};
// Split plan shared by the workspace-size query and the launcher.
struct DecodePlan {
  int32_t rows;        // q_len * G, rows per (request, kv head)
  int32_t chunk;       // keys per split
  int32_t max_splits;  // splits per (request, kv head), upper bound
  size_t workspace_bytes;
};
DecodePlan plan_decode(int32_t batch, int32_t q_len, int32_t num_heads_qo,
                       int32_t num_heads_kv, int32_t head_dim,
                       int32_t max_seq_len, int32_t window_left);
hipError_t launch_decode(const DecodeArgs &a, const DecodePlan &plan,
                         hipStream_t s);

}  // namespace pkv
