// Host-side launcher of the prefill kernels and its argument block.
// Declared here, defined next to the kernels, called from the C ABI layer
// after validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

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
  int32_t max_kv;  // >= every L_kv (sizes the tile dispatch batches)
  int32_t causal;
  float scale;
  const float *q_scale, *k_scale, *v_scale;
  void *out;
  float *lse;
  int32_t qkv_dtype, o_dtype;  // pkv_dtype values
};
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);

}  // namespace pkv
