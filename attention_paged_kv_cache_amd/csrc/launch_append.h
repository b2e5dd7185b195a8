// Host-side launcher of the append and index-math kernels and its argument block.
// Declared here, defined next to the kernels, called from the C ABI layer
// after validation.
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

}  // namespace pkv
