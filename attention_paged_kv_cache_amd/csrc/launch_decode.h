// Host-side launcher of the decode kernels and its argument block.
// Declared here, defined next to the kernels, called from the C ABI layer
// after validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Query rows (queries x GQA group) per (request, kv head) the decode takes:
// groups of 32 rows, one workgroup each, up to 32 groups.
constexpr int32_t kDecodeMaxRows = 1024;

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
