// Page-table index math and the append scatter.
//
// Source: flashinfer.page.append_paged_kv_cache -- Parameters (append_key,
// append_value, batch_indices, positions, paged_kv_cache, kv_indices,
// kv_indptr, kv_last_page_len, kv_layout), Example (get_seq_lens and
// get_batch_indices_positions), Note (pages already cover appended rows).
//
// The append is a bit copy, bound by HBM bandwidth: every thread moves
// 16-byte vectors, and a token's run of head_dim elements per head is
// contiguous in both layouts (NHD and HND differ only in the head / slot
// strides), so rows are copied as runs of 16-byte chunks.

#include "launch.h"
#include "pkv_common.h"

namespace pkv {

// seq_len[b] = (pages_b - 1) * page_size + last_page_len[b]
__global__ void get_seq_lens_kernel(const int32_t *__restrict__ indptr,
                                    const int32_t *__restrict__ last,
                                    int32_t batch, int32_t page_size,
                                    int32_t *__restrict__ out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int pages = indptr[b + 1] - indptr[b];
  out[b] = pages > 0 ? (pages - 1) * page_size + last[b] : 0;
}

// One workgroup per request writes that request's rows: row k of n_b is at
// absolute position seq_len - n_b + k (the last n_b positions).
__global__ void batch_indices_positions_kernel(const int32_t *__restrict__ ai,
                                               const int32_t *__restrict__ seq,
                                               int32_t nnz,
                                               int32_t *__restrict__ bidx,
                                               int32_t *__restrict__ pos) {
  const int b = blockIdx.x;
  const int start = ai[b], n = ai[b + 1] - start, len = seq[b];
  for (int k = threadIdx.x; k < n; k += blockDim.x) {
    const int i = start + k;
    if (i < nnz) {
      bidx[i] = b;
      pos[i] = len - n + k;
    }
  }
}

__global__ void csr_to_block_tables_kernel(const int32_t *__restrict__ indptr,
                                           const int32_t *__restrict__ indices,
                                           int32_t max_pages,
                                           int32_t *__restrict__ bt) {
  const int b = blockIdx.y;
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= max_pages) return;
  const int start = indptr[b], n = indptr[b + 1] - start;
  bt[(int64_t)b * max_pages + k] = k < n ? indices[start + k] : -1;
}

// Flattened over (row, K|V, 16-byte chunk). chunks_per_row = heads *
// row_bytes_per_head / 16. Consecutive threads take consecutive chunks of
// one row, so both the read of the appended row and the write into the page
// are 16-byte coalesced runs.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a,
                                                     int32_t chunks_per_head,
                                                     int32_t chunks_per_row,
                                                     int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int32_t c = (int32_t)(gid % chunks_per_row);
  const int64_t rk = gid / chunks_per_row;  // row * 2 + (0: K, 1: V)
  const int32_t which = (int32_t)(rk & 1);
  const int64_t row = rk >> 1;
  const int32_t b = a.batch_indices[row];
  const int32_t p = a.positions[row];
  const int32_t page = a.kv_indices[a.kv_indptr[b] + p / a.page_size];
  const int32_t slot = p % a.page_size;
  const int32_t head = c / chunks_per_head;
  const int32_t off = (c % chunks_per_head) * 16;
  const char *src = (const char *)(which ? a.value : a.key) +
                    row * (int64_t)chunks_per_row * 16 + (int64_t)c * 16;
  char *dst = (char *)(which ? a.v_cache : a.k_cache) +
              (int64_t)page * (which ? a.page_stride_v : a.page_stride_k) +
              (int64_t)slot * a.slot_stride + (int64_t)head * a.head_stride +
              off;
  st16(dst, ld16(src));
}

__global__ void exclusive_cumsum_kernel(const int32_t *__restrict__ lens,
                                        int32_t batch,
                                        int32_t *__restrict__ out) {
  // One workgroup of 256 threads; running carry across 256-wide chunks.
  __shared__ int32_t buf[256];
  int32_t carry = 0;
  for (int base = 0; base < batch; base += 256) {
    const int i = base + threadIdx.x;
    buf[threadIdx.x] = i < batch ? lens[i] : 0;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int32_t v = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
      __syncthreads();
      buf[threadIdx.x] += v;
      __syncthreads();
    }
    const int32_t incl = buf[threadIdx.x];
    if (i < batch) out[i] = carry + incl - (i < batch ? lens[i] : 0);
    carry += buf[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[batch] = carry;
}

hipError_t launch_get_seq_lens(const int32_t *kv_indptr, const int32_t *last,
                               int32_t batch, int32_t page_size,
                               int32_t *seq_lens, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(get_seq_lens_kernel, dim3((batch + 255) / 256), dim3(256),
                     0, s, kv_indptr, last, batch, page_size, seq_lens);
  return hipGetLastError();
}

hipError_t launch_batch_indices_positions(const int32_t *ai,
                                          const int32_t *seq, int32_t batch,
                                          int32_t nnz, int32_t *bidx,
                                          int32_t *pos, hipStream_t s) {
  if (batch == 0 || nnz == 0) return hipSuccess;
  hipLaunchKernelGGL(batch_indices_positions_kernel, dim3(batch), dim3(256), 0,
                     s, ai, seq, nnz, bidx, pos);
  return hipGetLastError();
}

hipError_t launch_csr_to_block_tables(const int32_t *indptr,
                                      const int32_t *indices, int32_t batch,
                                      int32_t max_pages, int32_t *bt,
                                      hipStream_t s) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(csr_to_block_tables_kernel,
                     dim3((max_pages + 255) / 256, batch), dim3(256), 0, s,
                     indptr, indices, max_pages, bt);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  if (a.nnz == 0) return hipSuccess;
  const int32_t chunks_per_head = a.row_bytes_per_head / 16;
  const int32_t chunks_per_row = chunks_per_head * a.num_heads;
  const int64_t total = (int64_t)a.nnz * 2 * chunks_per_row;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(append_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, a,
                     chunks_per_head, chunks_per_row, total);
  return hipGetLastError();
}

hipError_t launch_exclusive_cumsum(const int32_t *lens, int32_t batch,
                                   int32_t *out, hipStream_t s) {
  hipLaunchKernelGGL(exclusive_cumsum_kernel, dim3(1), dim3(256), 0, s, lens,
                     batch, out);
  return hipGetLastError();
}

}  // namespace pkv
