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
// strides), so rows are copied as runs of 16-byte chunks. K and V share
// each row's page lookup.

#include "launch_append.h"
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

// One thread per (row, group of C 16-byte chunks): it resolves the row's
// page once (batch index -> position -> page id through
// kv_indptr/kv_indices, and the slot) and moves the group's bytes of both K
// and V, so 2C 16-byte loads are in flight behind one lookup. Chunks
// c, c + groups, ... of a row go to one thread, so consecutive threads read
// consecutive 16-byte pieces of the appended rows and write consecutive
// pieces of each head's run. A chunk is 16 bytes of one head's head_dim
// run, so a write never straddles a head (or a page slot) in either layout.
//
// C by layout (TB/s by C = 1 / 2 / 4 / 8, one MI355X, same process):
//   HND, e4m3 1 KB rows:  5.43 / 5.49 / 5.65 / 5.64
//   HND, fp16 2 KB rows:  5.64 / 5.54 / 5.77 / 5.48
//   NHD, e4m3 1 KB rows:  5.88 / 5.90 / 5.74 / 5.23
//   NHD, fp16 8 KB rows:  5.75 / 5.31 / 5.42 / 5.25
// A token's heads are adjacent in NHD (one contiguous run per row): many
// threads of one chunk each stream it best. In HND each head's run goes to
// its own place in the page, and four chunks per thread do best.
constexpr int kChunksHnd = 4;
constexpr int kChunksNhd = 1;

// Bytes of appended rows (K and V) from which the append streams: the
// chip's 256 MB last-level cache.
constexpr int64_t kAppendStreamBytes = (int64_t)256 << 20;

// NTL / NTS: non-temporal (streaming) loads of the appended rows / stores
// into the pages.
template <bool NTL, bool NTS, int C>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a, int32_t chunks_per_head,
                                                     int32_t chunks_per_row, int32_t groups,
                                                     int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int32_t g = (int32_t)(gid % groups);
  const int64_t row = gid / groups;
  const int32_t b = a.batch_indices[row];
  const int32_t p = a.positions[row];
  const int32_t page = a.kv_indices[a.kv_indptr[b] + p / a.page_size];
  const int64_t slot = (int64_t)(p % a.page_size) * a.slot_stride;
  const char *ks = (const char *)a.key + row * chunks_per_row * 16;
  const char *vs = (const char *)a.value + row * chunks_per_row * 16;
  char *kd = (char *)a.k_cache + (int64_t)page * a.page_stride_k + slot;
  char *vd = (char *)a.v_cache + (int64_t)page * a.page_stride_v + slot;
  u32x4 kv[2][C];
#pragma unroll
  for (int u = 0; u < C; ++u) {
    const int32_t c = g + u * groups;
    if (c < chunks_per_row) {
      if constexpr (NTL) {
        kv[0][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ks + c * 16));
        kv[1][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vs + c * 16));
      } else {
        kv[0][u] = ld16(ks + c * 16);
        kv[1][u] = ld16(vs + c * 16);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < C; ++u) {
    const int32_t c = g + u * groups;
    if (c < chunks_per_row) {
      const int32_t head = c / chunks_per_head;
      const int64_t o = (int64_t)head * a.head_stride + (c - head * chunks_per_head) * 16;
      if constexpr (NTS) {
        __builtin_nontemporal_store(kv[0][u], reinterpret_cast<u32x4 *>(kd + o));
        __builtin_nontemporal_store(kv[1][u], reinterpret_cast<u32x4 *>(vd + o));
      } else {
        st16(kd + o, kv[0][u]);
        st16(vd + o, kv[1][u]);
      }
    }
  }
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

template <int C>
static void launch_append_c(const AppendArgs &a, int32_t chunks_per_head, int32_t chunks_per_row,
                            hipStream_t s) {
  const int32_t groups = (chunks_per_row + C - 1) / C;
  const int64_t total = (int64_t)a.nnz * groups;
  const int64_t blocks = (total + 255) / 256;
  // Appends that read at least kAppendStreamBytes of rows use non-temporal
  // loads and stores: they stream through the chip's 256 MB last-level
  // cache anyway, and keeping them out of its normal allocation measured
  // faster (1.07 GB moved: 5.08 -> 5.52 TB/s; 2.1 GB: 5.20 -> 5.31).
  // Smaller ones keep plain accesses, so that the written pages stay cached
  // for the attention call that reads them next (and the rows, freshly
  // produced, are read from the cache: at 269 MB moved, streaming loads
  // measured 6.26 -> 5.40 TB/s).
  const int64_t src_bytes = 2 * (int64_t)a.nnz * chunks_per_row * 16;
  if (src_bytes >= kAppendStreamBytes)
    hipLaunchKernelGGL((append_kernel<true, true, C>), dim3((uint32_t)blocks), dim3(256), 0, s, a,
                       chunks_per_head, chunks_per_row, groups, total);
  else
    hipLaunchKernelGGL((append_kernel<false, false, C>), dim3((uint32_t)blocks), dim3(256), 0, s,
                       a, chunks_per_head, chunks_per_row, groups, total);
}

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  if (a.nnz == 0) return hipSuccess;
  const int32_t chunks_per_head = a.row_bytes_per_head / 16;
  const int32_t chunks_per_row = chunks_per_head * a.num_heads;
  // NHD: a slot's heads are adjacent (the head stride is one head's run)
  if (a.head_stride == a.row_bytes_per_head)
    launch_append_c<kChunksNhd>(a, chunks_per_head, chunks_per_row, s);
  else
    launch_append_c<kChunksHnd>(a, chunks_per_head, chunks_per_row, s);
  return hipGetLastError();
}

hipError_t launch_exclusive_cumsum(const int32_t *lens, int32_t batch,
                                   int32_t *out, hipStream_t s) {
  hipLaunchKernelGGL(exclusive_cumsum_kernel, dim3(1), dim3(256), 0, s, lens,
                     batch, out);
  return hipGetLastError();
}

}  // namespace pkv
