// Measured ceilings of the chip, against which the attention kernels' rates
// are read beside the datasheet peaks: a bf16 matrix-core loop with no
// memory traffic, a streaming HBM read and a streaming HBM copy (read plus
// write, the traffic of an append). Measurement only: nothing in the
// attention path calls these. Built into its own library.
//
// Each call validates its sizes on the host and launches one kernel on the
// given stream; all buffers are the caller's device memory.

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CEIL_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kChains = 8;  // independent accumulators per wave

// Each wave runs `iters` rounds of kChains independent 32x32x16 bf16 MFMAs
// (32768 FLOP each); one float per lane is written so nothing is dropped.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int32_t iters, float *__restrict__ out) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((threadIdx.x + e) & 7);
    b[e] = (__bf16)(float)((threadIdx.x * 3 + e) & 7);
  }
  f32x16 acc[kChains];
  for (int k = 0; k < kChains; ++k)
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  for (int32_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
  for (int k = 0; k < kChains; ++k)
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

constexpr int kReadUnroll = 8;

// Each workgroup reads its own contiguous span of per_wg16 16-byte vectors
// with non-temporal (streaming) loads, which read faster than plain loads
// on this chip (4 GiB: about 6.9 against 6.2 TB/s), kReadUnroll loads in
// flight per thread (per_wg16 is a multiple of
// 256 * kReadUnroll); one xor-folded word per thread is written so nothing is
// dropped.
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4 *__restrict__ p,
                                                          int64_t per_wg16,
                                                          uint32_t *__restrict__ out) {
  const u32x4 *q = p + (int64_t)blockIdx.x * per_wg16 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i = 0; i < per_wg16; i += 256 * kReadUnroll) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(q + i + 256 * u);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Each workgroup copies its own contiguous span of per_wg16 16-byte vectors
// from src to dst, U loads in flight per thread before their stores; NT
// selects non-temporal (streaming) loads and stores.
template <bool NT, int U>
__global__ __launch_bounds__(256) void copy_stream_kernel(const u32x4 *__restrict__ src,
                                                          u32x4 *__restrict__ dst,
                                                          int64_t per_wg16) {
  const int64_t base = (int64_t)blockIdx.x * per_wg16 + threadIdx.x;
  const u32x4 *q = src + base;
  u32x4 *d = dst + base;
  for (int64_t i = 0; i < per_wg16; i += 256 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = NT ? __builtin_nontemporal_load(q + i + 256 * u) : q[i + 256 * u];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (NT)
        __builtin_nontemporal_store(v[u], d + i + 256 * u);
      else
        d[i + 256 * u] = v[u];
    }
  }
}

}  // namespace

// `out` holds blocks * 256 floats. Returns a hipError_t value (0 = success).
CEIL_API int pkv_ceiling_mfma_bf16(int32_t blocks, int32_t iters, float *out, void *stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters,
                     out);
  return (int)hipGetLastError();
}

// FLOP one pkv_ceiling_mfma_bf16 call performs.
CEIL_API double pkv_ceiling_mfma_bf16_flop(int32_t blocks, int32_t iters) {
  return (double)blocks * 4 * iters * kChains * 32768.0;
}

// Reads `bytes` from `buf` (16-byte aligned; bytes a multiple of
// blocks * 32 KiB, each workgroup taking an equal contiguous span); `out`
// holds blocks * 256 words.
CEIL_API int pkv_ceiling_read(const void *buf, int64_t bytes, int32_t blocks, uint32_t *out,
                              void *stream) {
  const int64_t span = (int64_t)blocks * 256 * kReadUnroll * 16;
  if (blocks <= 0 || bytes <= 0 || bytes % span || buf == nullptr || out == nullptr ||
      (uintptr_t)buf % 16)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4 *)buf, bytes / 16 / blocks, out);
  return (int)hipGetLastError();
}

// Copies `bytes` from `src` to `dst` (both 16-byte aligned, not
// overlapping; bytes a multiple of blocks * unroll * 4 KiB, each workgroup
// taking an equal contiguous span), `unroll` (4 or 8) 16-byte loads in
// flight per thread, with non-temporal loads and stores when `nontemporal`
// is nonzero.
CEIL_API int pkv_ceiling_copy(const void *src, void *dst, int64_t bytes, int32_t blocks,
                              int32_t nontemporal, int32_t unroll, void *stream) {
  if (unroll != 4 && unroll != 8) return (int)hipErrorInvalidValue;
  const int64_t span = (int64_t)blocks * 256 * unroll * 16;
  if (blocks <= 0 || bytes <= 0 || bytes % span || src == nullptr || dst == nullptr ||
      (uintptr_t)src % 16 || (uintptr_t)dst % 16)
    return (int)hipErrorInvalidValue;
  const char *s = (const char *)src;
  const char *d = (const char *)dst;
  if (s < d + bytes && d < s + bytes) return (int)hipErrorInvalidValue;
  const int64_t per = bytes / 16 / blocks;
  const hipStream_t st = (hipStream_t)stream;
  const u32x4 *si = (const u32x4 *)src;
  u32x4 *di = (u32x4 *)dst;
  if (nontemporal && unroll == 8)
    hipLaunchKernelGGL((copy_stream_kernel<true, 8>), dim3(blocks), dim3(256), 0, st, si, di, per);
  else if (nontemporal)
    hipLaunchKernelGGL((copy_stream_kernel<true, 4>), dim3(blocks), dim3(256), 0, st, si, di, per);
  else if (unroll == 8)
    hipLaunchKernelGGL((copy_stream_kernel<false, 8>), dim3(blocks), dim3(256), 0, st, si, di, per);
  else
    hipLaunchKernelGGL((copy_stream_kernel<false, 4>), dim3(blocks), dim3(256), 0, st, si, di, per);
  return (int)hipGetLastError();
}
