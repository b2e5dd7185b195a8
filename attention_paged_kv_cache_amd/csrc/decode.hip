// Batch decode over a block_tables page table: split-KV on MFMA, LSE merge.
//
// Source: flashinfer.decode.trtllm_batch_decode_with_kv_cache -- Parameters
// (query, kv_cache, workspace_buffer, block_tables, seq_lens, max_seq_len,
// bmm1_scale, bmm2_scale, window_left, sinks, kv_layout, q_len_per_req).
// Request b's q_len queries are its last q_len positions, causal among
// themselves; window_left is an inclusive left window (-1: whole sequence);
// a sink is a per-qo-head logit that joins only the softmax denominator.
//
// The kernel is bound by HBM reads of the K/V pages: every K and V element
// of a kv head is read once and serves all G * q_len query rows of that
// head (G = num_heads_qo / num_heads_kv). Those rows form the N side of
// 16x16x32 MFMAs, so the arithmetic stays far below the matrix-core roof
// and the loads decide the time.
//
// Work decomposition
//   A unit is (request, kv head, split): `chunk` consecutive keys of the
//   request's key range (only keys some query may see: with a window, the
//   range starts at seq - q_len - window_left). A workgroup of 4 waves owns
//   one unit; each wave streams chunk/4 keys, 32 at a time:
//     K: 1 KB LDS DMAs of whole key rows into the wave's own LDS rows (two
//        stages), then per lane = (key, d run) 16-byte operand reads (8 d
//        of one MFMA k-step, or 16 e4m3 d feeding two k-steps, widened
//        exactly to the query's 16-bit type in registers).
//     V: lane = (8 keys, 8-element d run): 16-byte (e4m3: 8-byte) loads
//        straight into registers, each load instruction reading whole
//        rows, then an 8x8 transpose in registers gives V^T operands whose
//        k-run is 8 consecutive keys.
//     S^T = K Q^T, online softmax in fp32 (base 2; the reference maximum
//     is raised lazily, so most steps skip rescaling O), O^T += V^T P^T.
//   With one row group per unit the K/V loads are non-temporal (streaming):
//   each byte is read once per call.
//   The four waves' (m, l, O) are merged in LDS. A request that fits one
//   unit writes its output directly; otherwise the unit writes its partial
//   (m, l, O) to the workspace and a merge kernel combines the splits and
//   the sink term.

#include <math.h>

#include <algorithm>
#include <type_traits>

#include "launch_decode.h"
#include "pkv_common.h"

namespace pkv {

namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;  // workgroups are dispatched round-robin over 8 XCDs
constexpr int kWaves = 4;
constexpr int kD = 128;
constexpr float kLazy = 8.0f;  // see the online softmax in decode_kernel

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c, BF16Tag) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c, F16Tag) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(
      __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Eight e4m3fn codes -> eight 16-bit values of the query's type (exact).
__device__ __forceinline__ u32x4 widen8(u32x2 w, BF16Tag) {
  const u32x2 lo = e4m3x4_to_bf16x4(w[0]);
  const u32x2 hi = e4m3x4_to_bf16x4(w[1]);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}
__device__ __forceinline__ u32x4 widen8(u32x2 w, F16Tag) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, true));
  return r;
}

// K/V loads (V loads, and the cache policy of the K DMAs). With one row
// group per unit every K/V byte is read once per call, and non-temporal
// (streaming) loads measured faster than plain ones
// (bit-identical outputs; batch decode 5.74 -> 5.82 TB/s, speculative decode
// (e4m3) 5.12 -> 5.77 TB/s, 5.18 -> 5.61 with cold caches). With several row
// groups the later groups re-read the unit's K/V from L2, which streaming
// loads evict early (64-row speculative decode 3.37 -> 3.07 TB/s), so those
// keep plain loads.
template <bool STREAM>
__device__ __forceinline__ u32x4 ld16_kv(const void *p) {
  if constexpr (STREAM)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  else
    return ld16(p);
}

// First key a unit range may start at: the window's left edge (if any),
// rounded down to a multiple of 32 so that every 32-key step starts on a
// page boundary for page sizes 16, 32 and 64. Keys below the true left edge
// are masked like any other key outside the window.
__device__ __forceinline__ int key_origin(const DecodeArgs &a, int seq, int ql) {
  int lo = 0;
  if (a.window_left >= 0) lo = max(0, seq - ql - a.window_left);
  return lo & ~31;
}

// Request b's query count and first query row: uniform q_len, or from the
// variable-length offsets.
__device__ __forceinline__ void request_rows(const DecodeArgs &a, int b, int &ql, int &row0) {
  if (a.cum_q) {
    row0 = a.cum_q[b];
    ql = a.cum_q[b + 1] - row0;
  } else {
    row0 = b * a.q_len;
    ql = a.q_len;
  }
}

// Raw V of one 32-key step as loaded: 8 keys x 8 d per lane, as 16-byte
// loads of 16-bit values (v) or 8-byte loads of e4m3 bytes (v8); each load
// instruction reads whole rows (4 rows). Loading e4m3 V 16 bytes per lane
// (4 keys x 16 d) and swapping halves between the lanes of a pair issued
// half the loads but cost a DPP move and selects per dword: speculative
// decode 5.87 vs 5.93 TB/s once K went through LDS. K goes through LDS.
template <bool FP8>
struct RawKV {
  u32x4 v[FP8 ? 1 : 8];
  u32x2 v8[FP8 ? 8 : 1];
};

template <bool STREAM>
__device__ __forceinline__ u32x2 ld8_kv(const void *p) {
  if constexpr (STREAM)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
  else
    return ld8(p);
}

// K of a 32-key step is staged in LDS, one wave's 32 rows in [row][d]
// order. A K operand (16 rows x 16 bytes of d per lane group) read
// straight from global memory touches 16 rows x 64 bytes per load
// instruction, and such loads measured 5.66 TB/s against 6.73 for 1 KB
// contiguous pieces (random 4 KB pages, same kernel shape). So each
// 1 KB LDS DMA instead takes whole rows (4 rows of 256 B, or 8 of 128 B
// for e4m3), and the operand is read back from LDS. The 16-byte chunk c of
// row r sits at chunk slot c ^ kswz(r): the 16 rows one operand read
// touches then fall in distinct banks.
template <bool FP8>
__device__ __forceinline__ int kswz(int row) {
  return FP8 ? ((((row >> 3) << 1) | ((row >> 1) & 1)) & 7) : (((row >> 1) & 12) | (row & 3));
}

// Buffer resource over `bytes` bytes from `base` (raw, untyped access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, bytes, 0x00020000);
}

// 16 bytes from LDS (p points into a __shared__ array).
__device__ __forceinline__ u32x4 lds16(const char *p) {
  return *(const __attribute__((address_space(3))) u32x4 *)p;
}

// 16 bytes at rsrc + voff straight into LDS: lane l's bytes land at
// lds_base + 16 * l (lds_base the same for every lane); STREAM: the
// non-temporal cache policy. Loads past the resource's range write zeros.
template <bool STREAM>
__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t r, int voff, char *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_base,
                                           16, voff, 0, 0, STREAM ? 2 : 0);
}

// d offset of the 8 query elements lane group g4 feeds to k-step t. For
// e4m3 K a lane reads 16 consecutive d (one 16-byte LDS read) and feeds its
// two halves to k-steps 2u and 2u + 1; Q uses the same assignment. Any
// assignment that covers every d once per kv head gives the same dot
// product.
template <bool FP8>
__device__ __forceinline__ int kstep_d(int t, int g4) {
  return FP8 ? 64 * (t >> 1) + 16 * g4 + 8 * (t & 1) : 32 * t + 8 * g4;
}

// NB: number of 16-row blocks a workgroup takes of the (q_len x G) query
// rows of a kv head (1 or 2). More than 32 rows are split into n_groups
// groups of 32, one workgroup each.
// STREAM: non-temporal K/V loads (one row group per unit).
template <int NB, class QT, bool FP8, bool STREAM>
__global__ __launch_bounds__(kThreads, (NB == 1 || FP8) ? 2 : 1) void decode_kernel(
    DecodeArgs a, int32_t chunk, int32_t max_splits, int32_t n_groups,
    float *__restrict__ ws_o, float *__restrict__ ws_ml) {
  constexpr int ES = FP8 ? 1 : 2;
  constexpr int R = NB * 16;
  __shared__ float sh_m[kWaves][R];
  __shared__ float sh_l[kWaves][R];
  // each row's draft mask as bits (bit i: draft i visible), when a mask is
  // given; read only on the steps that reach the drafts
  __shared__ uint64_t sh_mbits[R];
  // each wave's K of a step, two stages (two arrays, so that the compiler
  // sees that a DMA into one never aliases the reads of the other)
  constexpr int KROWB = kD * ES;      // bytes of one K row
  constexpr int LPR = KROWB / 16;     // DMA lanes per K row
  constexpr int RPI = 64 / LPR;       // K rows per 1 KB DMA
  constexpr int NKI = 32 / RPI;       // DMAs per step
  // After the loop the four waves' O^T rows go to four buffers, one per
  // wave, in the two K stages (waves 0-1 in the first, 2-3 in the second):
  // every wave has left the loop (and drained its DMAs) by the merge's
  // first barrier.
  constexpr int KSTAGE = kWaves * 32 * KROWB;
  constexpr int SHO = R * (kD + 4) * 4;  // one wave's rows (padded by 4 floats)
  constexpr int SKB = KSTAGE > 2 * SHO ? KSTAGE : 2 * SHO;
  __shared__ __attribute__((aligned(16))) char sk_a[SKB];
  __shared__ __attribute__((aligned(16))) char sk_b[SKB];
  // per wave and row: the factor that brings its O to the common maximum;
  // per row: the output scale (one split) -- see the merge
  __shared__ float sh_fw[kWaves][R];
  __shared__ float sh_sc[R];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;
  const int r16 = lane & 15;

  // Block -> (unit u = (split, request, kv head), row group). Blocks are
  // dealt to the 8 XCDs in turn (block i on XCD i % 8).
  //  * One row group: the kv heads of one (split, request) go to one XCD as
  //    consecutive blocks, so the pages' K (then V) runs of all heads, which
  //    are adjacent in an HND page, are read by one XCD close in time.
  //  * Several row groups: the groups of one unit sit 8 blocks apart, so
  //    they run on the same XCD, close in time, and the second streams the
  //    unit's K/V from that XCD's L2.
  const int bh = a.batch * a.num_heads_kv;
  int u, grp = 0;
  if (n_groups == 1) {
    const int H = a.num_heads_kv;
    const int slot = blockIdx.x / kXcds;
    u = ((slot / H) * kXcds + blockIdx.x % kXcds) * H + slot % H;
    if (u >= bh * max_splits) return;
  } else {
    const int rest = blockIdx.x / kXcds;
    grp = rest % n_groups;
    u = (rest / n_groups) * kXcds + blockIdx.x % kXcds;
    if (u >= bh * max_splits) return;
  }
  const int split = u / bh;
  const int b = (u / a.num_heads_kv) % a.batch;
  const int kvh = u % a.num_heads_kv;
  const int seq = (int)a.seq_lens[b];
  int ql, qrow0;
  request_rows(a, b, ql, qrow0);
  const int G = a.num_heads_qo / a.num_heads_kv;
  const int row_base = grp * R;                // this group's first row
  const int rows = min(R, ql * G - row_base);  // its rows of this request
  if (rows <= 0) return;
  const int lo = key_origin(a, seq, ql);
  const int k_begin = lo + split * chunk;
  if (k_begin >= seq) {
    // Only an empty sequence leaves split 0 without keys. Its rows see no
    // key, so their output is zero; split 0 writes it (the merge kernel
    // skips such rows), whatever the batch's split plan.
    if (seq == 0 && split == 0) {
      const int ob = a.out_dtype == 2 ? 1 : 2;  // bytes per output element
      for (int idx = tid; idx < rows * (kD / 8); idx += kThreads) {
        const int ng = row_base + idx / (kD / 8);
        const int qi = ng / G, g = ng - qi * G;
        const int64_t orow = (int64_t)(qrow0 + qi) * a.num_heads_qo + kvh * G + g;
        char *op = (char *)a.out + (orow * kD + (idx % (kD / 8)) * 8) * ob;
        if (ob == 2)
          st16(op, u32x4{0u, 0u, 0u, 0u});
        else
          st8(op, u32x2{0u, 0u});
      }
    }
    return;
  }
  const int k_end = min(seq, k_begin + chunk);
  const int n_splits = (seq - lo + chunk - 1) / chunk;
  const int cw = chunk / kWaves;
  const int w_begin = k_begin + wave * cw;
  const int w_end = min(k_end, w_begin + cw);

  const int rows_ws = a.q_len * G;  // workspace rows per unit (the maximum)
  // With a draft mask, keys from the first draft on are allowed by the
  // mask; keys before it only by the window.
  const int dstart = seq - ql;
  const int mask_from = a.mask ? dstart : 0x7fffffff;
  const float bmm1 = a.bmm1_ptr ? a.bmm1_ptr[0] : a.bmm1_scale;
  const float c_raw = bmm1 * kLog2e;
  const bool negate = c_raw < 0.0f;
  const float c = fmaxf(fabsf(c_raw), 1e-30f);

  // ---- Q^T operands: row n = 16*nb + r16 -> (query qi, head g) ------------
  u32x4 qop[NB][4];
  int pos[NB], wlo[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + r16;
    const int ng = row_base + n;
    const int qi = ng / G, g = ng - qi * G;
    const bool ok = n < rows;
    const int qpos = seq - ql + qi;  // the query's position
    // last allowed key (padding rows: none); with a mask every key up to
    // the end is a candidate and the mask decides among the drafts
    pos[nb] = ok ? (a.mask ? seq - 1 : qpos) : -1;
    wlo[nb] = (a.window_left >= 0) ? qpos - a.window_left : 0;
    const char *qp = (const char *)a.q +
                     ((int64_t)(qrow0 + qi) * a.num_heads_qo + kvh * G + g) * kD * 2;
    const uint32_t flip = negate ? 0x80008000u : 0u;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = ld16(qp + kstep_d<FP8>(s, g4) * 2);
      v[0] ^= flip; v[1] ^= flip; v[2] ^= flip; v[3] ^= flip;
      qop[nb][s] = v;
    }
  }
  if (a.mask) {  // uniform: every thread takes the barrier or none does
    if (tid < R) {
      uint64_t bits = 0;
      if (tid < rows) {  // ql <= 64 whenever a mask is given
        const uint8_t *mrow = a.mask + ((int64_t)b * a.q_len + (row_base + tid) / G) * a.q_len;
        for (int i = 0; i < ql; ++i)
          if (mrow[i]) bits |= 1ull << i;
      }
      sh_mbits[tid] = bits;
    }
    __syncthreads();
  }

  // bounds over the real rows only (padding rows have pos = -1)
  int pos_min = 0x7fffffff, wlo_max = -0x7fffffff;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (nb * 16 + r16 < rows) {
      pos_min = min(pos_min, pos[nb]);
      wlo_max = max(wlo_max, wlo[nb]);
    }
  }
  // wave-uniform bounds of the mask-free region
  for (int off = 1; off < 64; off <<= 1) {
    pos_min = min(pos_min, __shfl_xor(pos_min, off));
    wlo_max = max(wlo_max, __shfl_xor(wlo_max, off));
  }
  pos_min = __builtin_amdgcn_readfirstlane(pos_min);
  wlo_max = __builtin_amdgcn_readfirstlane(wlo_max);

  // block table row through the constant address space: scalar loads, so
  // that the next step's page ids do not queue behind (and wait for) this
  // step's K/V loads
  const __attribute__((address_space(4))) int32_t *bt =
      (const __attribute__((address_space(4))) int32_t *)(a.block_tables) +
      (int64_t)b * a.max_pages;
  const int log2ps = __builtin_ctz(a.page_size);
  const int ps_mask = a.page_size - 1;
  const int last_pg = (seq - 1) >> log2ps;
  const char *kbase = (const char *)a.k + (int64_t)kvh * a.head_stride * ES;
  const char *vbase = (const char *)a.v + (int64_t)kvh * a.head_stride * ES;
  const int64_t psk = a.page_stride_k * ES, psv = a.page_stride_v * ES;
  const int64_t sstr = a.slot_stride * ES;

  // Per-lane key offsets inside a 32-key step (loop invariant).
  //   K, m-block mb: offset 8*(r16/4) + 4*mb + r16%4 (the lane's MFMA row)
  //   V: offsets 8*g4 .. 8*g4+7 (the lane's 8-key run)
  int koff[2];
  koff[0] = 8 * (r16 >> 2) + (r16 & 3);
  koff[1] = koff[0] + 4;
  const int voff = 8 * g4;

  // K DMA q, lane l: row q * RPI + l / LPR of the step, LDS chunk slot
  // l % LPR, which holds global chunk slot ^ kswz(row). The row's offset in
  // its page is taken modulo 16 for 16-token pages (rows 16..31 of a step
  // are the second page's first 16). Loop invariant.
  int kdma_off[NKI];
#pragma unroll
  for (int q = 0; q < NKI; ++q) {
    const int row = q * RPI + lane / LPR;
    const int c = (lane % LPR) ^ kswz<FP8>(row);
    kdma_off[q] = (row & (a.page_size == 16 ? 15 : 31)) * (int)sstr + c * 16;
  }
  // With 16-bit K the resources end at the sequence's last key: rows past
  // it load zeros (their scores are masked) and cost no memory traffic
  // (batch decode 6.36 -> 6.42 TB/s). The e4m3 kernel, bound by its
  // instruction stream rather than by its loads, measured slower with the
  // per-DMA bound (5.93 vs 5.88 TB/s) and maps the whole page. rows_from:
  // the step's rows before this DMA's page part (16 for the second page of
  // a 16-token page step).
  const int kpage_bytes = (int)((a.page_size - 1) * sstr + KROWB);
  auto dma_bytes = [&](int kg0, int rows_from, bool live) {
    if constexpr (FP8) return live ? kpage_bytes : 0;
    const int n = live ? min(32, seq - kg0 - rows_from) : 0;
    return n > 0 ? (int)((n - 1) * sstr + KROWB) : 0;
  };
  // operand reads: m-block mb, 16-byte piece u (16-bit: k-step u; e4m3:
  // k-steps 2u and 2u + 1) of the lane's key row koff[mb]
  constexpr int KU = FP8 ? 2 : 4;
  int kld[2][KU];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int row = koff[mb];
      kld[mb][u] = wave * (32 * KROWB) + row * KROWB + ((4 * u + g4) ^ kswz<FP8>(row)) * 16;
    }

  // The two pages a 32-key step can touch (the second differs only for
  // 16-token pages); indices are clamped into the sequence so that no
  // padding entry of the block table is ever followed.
  auto step_pages = [&](int kg0, int &p0, int &p1) {
    p0 = bt[min(kg0 >> log2ps, last_pg)];
    p1 = bt[min((kg0 + 16) >> log2ps, last_pg)];
  };
  // Loads of one step. Every step issues the next one unconditionally, so
  // that the compiler's wait before a step's compute counts exactly the
  // next step's loads (a conditional issue left a join at which it waited
  // for all loads). Past the wave's last step (live = false) the K DMAs get
  // an empty range (no memory access; they write zeros into the unused
  // stage) and the V loads all read the same 256 bytes of the query.
  auto issue = [&](RawKV<FP8> &r, int kg0, int p0, int p1, char *stage, bool live) {
    // K: NKI DMAs of RPI whole rows each into this wave's LDS rows; the
    // rows of one DMA lie in one page (RPI divides 16)
    const int64_t kin = (int64_t)(kg0 & ps_mask) * sstr;  // step's first row in its page
#pragma unroll
    for (int q = 0; q < NKI; ++q) {
      const bool second = (q * RPI) >> log2ps;
      const int p = second ? p1 : p0;
      dma16b<STREAM>(make_rsrc(kbase + (int64_t)p * psk + kin, dma_bytes(kg0, second ? 16 : 0, live)),
                     kdma_off[q], stage + wave * (32 * KROWB) + q * 1024);
    }
    const char *vb0 = vbase + (int64_t)p0 * psv, *vb1 = vbase + (int64_t)p1 * psv;
    const int64_t vstr = live ? sstr : 0;
    const char *vdummy = (const char *)a.q + (lane & 15) * 16;
    if constexpr (FP8) {
      // keys voff .. voff+7, d 8*r16 .. 8*r16+7 (8 bytes of each row)
      const char *vp =
          ((voff >> log2ps) ? vb1 : vb0) + ((kg0 + voff) & ps_mask) * sstr + r16 * 8;
      if (!live) vp = vdummy;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) r.v8[jj] = ld8_kv<STREAM>(vp + jj * vstr);
    } else {
      const char *vp =
          ((voff >> log2ps) ? vb1 : vb0) + ((kg0 + voff) & ps_mask) * sstr + r16 * 8 * ES;
      if (!live) vp = vdummy;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) r.v[jj] = ld16_kv<STREAM>(vp + jj * vstr);
    }
  };

  f32x4 o[8][NB];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[cc][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.0f;
  }

  auto compute = [&](const RawKV<FP8> &r, int kg0, const char *stage) {
    // ---- S^T = K Q^T (e4m3 K widened one k-step at a time, right before
    // its MFMAs; V is widened and transposed after the softmax, so neither
    // holds registers across the other's work) --------------------------------
    f32x4 sacc[2][NB];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sacc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 kop;
        if constexpr (FP8) {
          const u32x4 w = lds16(stage + kld[mb][s >> 1]);
          kop = widen8((s & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]}, QT{});
        } else {
          kop = lds16(stage + kld[mb][s]);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sacc[mb][nb] = mfma16(kop, qop[nb][s], sacc[mb][nb], QT{});
      }

    // ---- mask where the step crosses a boundary ----------------------------
    // lane holds keys kg0 + 8*g4 + 4*mb + i for its row
    const bool clean = (kg0 + 32 <= w_end) && (kg0 >= w_begin) && (kg0 >= wlo_max) &&
                       (kg0 + 31 <= pos_min) && (kg0 + 32 <= mask_from);
    if (!clean) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        // the row's draft bits, read once (no load inside the per-key
        // selects, so they stay branch-free)
        const uint64_t bits = a.mask ? sh_mbits[nb * 16 + r16] : ~0ull;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kg0 + 8 * g4 + 4 * mb + i;
            // a draft key (key >= mask_from, so 0 <= key - dstart < ql for
            // keys inside the sequence) must have its mask bit set
            const uint32_t di = (uint32_t)(key - dstart);
            const bool shown = di < 64u && ((bits >> (di & 63)) & 1ull);
            const bool hidden = key >= mask_from && !shown;
            if (key >= w_end || key < w_begin || key > pos[nb] || key < wlo[nb] || hidden)
              sacc[mb][nb][i] = -INFINITY;
          }
      }
    }

    // ---- online softmax per row ----------------------------------------------
    u32x4 pop[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float mloc = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, sacc[mb][nb][i]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      // The reference maximum m_run is raised lazily: only when this step's
      // maximum exceeds it by more than kLazy (log2 units), so most steps
      // skip rescaling O and exponentials stay <= 2^kLazy.
      const float m_tile = mloc * c;  // -inf when every key of the row is masked
      const bool need = m_tile > m_run[nb] + kLazy;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? m_tile : m_run[nb];
        const float alpha = need ? fast_exp2(m_run[nb] - m_new) : 1.0f;
        m_run[nb] = m_new;
        l_run[nb] *= alpha;
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) o[cc][nb] *= alpha;
      }
      const float m_use = (m_run[nb] == -INFINITY) ? 0.0f : m_run[nb];
      float ps = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const float p0 = fast_exp2(fmaf(sacc[mb][nb][0], c, -m_use));
        const float p1 = fast_exp2(fmaf(sacc[mb][nb][1], c, -m_use));
        const float p2 = fast_exp2(fmaf(sacc[mb][nb][2], c, -m_use));
        const float p3 = fast_exp2(fmaf(sacc[mb][nb][3], c, -m_use));
        ps += (p0 + p1) + (p2 + p3);
        pop[nb][2 * mb] = pack2(p0, p1, QT{});
        pop[nb][2 * mb + 1] = pack2(p2, p3, QT{});
      }
      l_run[nb] += ps;
    }

    // ---- O^T += V^T P^T --------------------------------------------------------
    u32x4 vrow[8];
    if constexpr (FP8) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) vrow[jj] = widen8(r.v8[jj], QT{});
    } else {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) vrow[jj] = r.v[jj];
    }
    // keys past the sequence end hold whatever the last page's tail holds:
    // zero them so that p = 0 meets v = 0, never NaN
    if (kg0 + 32 > seq) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (kg0 + voff + jj >= seq) vrow[jj] = u32x4{0u, 0u, 0u, 0u};
    }

    u32x4 vt[8];
    transpose8x8_b16(vrow, vt);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[cc][nb] = mfma16(vt[cc], pop[nb], o[cc][nb], QT{});
  };

  // ---- stream the wave's keys: loads of step i+1 fly during step i --------
  // Two named buffers (no register copies); page ids are fetched one step
  // ahead of the loads that use them.
  if (w_begin < w_end) {
    RawKV<FP8> buf_a, buf_b;
    int p0, p1, n0, n1;
    step_pages(w_begin, p0, p1);
    issue(buf_a, w_begin, p0, p1, sk_a, true);
    step_pages(w_begin + 32, n0, n1);
    // Steps go in pairs (buffers a then b), with the loop's only exit at
    // its test: a second exit after the first step of a pair became a path
    // from that step back to the loop head in the compiler's structured
    // control flow, on which the first step's loads were pending, so the
    // loop head waited for every load. An odd last pair skips its second
    // compute (its loads were the empty ones).
    const int n_steps = (w_end - w_begin + 31) >> 5;
    // Before a step's compute, wait until only the next step's loads (NKI
    // DMAs and NV V loads, issued after this step's) are outstanding: the
    // wait for this step's K DMAs (LDS writes) is explicit rather than left
    // to the compiler, whose tracking of DMA writes into LDS dropped it
    // across the loop's back edge.
    constexpr int NV = 8;  // V loads per step
    constexpr int kWaitStep = NKI + NV;
    constexpr int kWaitImm = 0x0F70 | (kWaitStep & 15) | ((kWaitStep >> 4) << 14);
    for (int i = 0; i < n_steps; i += 2) {
      const int kg = w_begin + 32 * i;
      issue(buf_b, kg + 32, n0, n1, sk_b, i + 1 < n_steps);
      step_pages(kg + 64, n0, n1);
      __builtin_amdgcn_s_waitcnt(kWaitImm);
      // nothing crosses: this step's LDS reads stay after the wait, the
      // next step's loads before it
      __builtin_amdgcn_sched_barrier(0);
      compute(buf_a, kg, sk_a);
      issue(buf_a, kg + 64, n0, n1, sk_a, i + 2 < n_steps);
      step_pages(kg + 96, n0, n1);
      __builtin_amdgcn_s_waitcnt(kWaitImm);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < n_steps) compute(buf_b, kg + 32, sk_b);
    }
    // the last, empty issue's DMAs write LDS: drain them before the
    // workgroup can end
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }

  // ---- merge the four waves ------------------------------------------------------
  // lane (r16, g4) holds, for row 16*nb + r16: l partial over its keys and
  // O^T at d = 8*(4*g4 + i) + cc.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float l = l_run[nb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    l_run[nb] = l;
    if (g4 == 0) {
      sh_m[wave][nb * 16 + r16] = m_run[nb];
      sh_l[wave][nb * 16 + r16] = l;
    }
  }
  __syncthreads();
  float fw[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + r16;
    float M = sh_m[0][n];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh_m[w][n]);
    const float M_use = (M == -INFINITY) ? 0.0f : M;
    fw[nb] = fast_exp2(m_run[nb] - M_use);
    if (g4 == 0) sh_fw[wave][n] = fw[nb];
  }
  // Each wave writes its O^T rows into its own buffer, all at once (wave 0
  // already rescaled, the others as they are); the output pass then forms
  // ((o0 fw0 + o1 fw1) + o2 fw2) + o3 fw3 with one rounding per step, the
  // result of a one-wave-at-a-time accumulation into one buffer with a
  // barrier per wave, which this replaces (bit-identical; speculative
  // decode 5.94 -> 6.03 TB/s, batch decode level).
  typedef float RowsO[kD + 4];
  RowsO *const mine = reinterpret_cast<RowsO *>((wave < 2 ? sk_a : sk_b) + (wave & 1) * SHO);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mine[nb * 16 + r16][8 * (4 * g4 + i) + cc] =
            wave == 0 ? o[cc][nb][i] * fw[nb] : o[cc][nb][i];

  // Per row, once: the softmax denominator over the four waves and the sink,
  // and from it the output scale (one split), or the partial's (m, l).
  const int n_rows = rows;  // only this request's rows are written
  const bool direct = n_splits == 1;
  if (tid < n_rows) {
    const int n = tid;
    float M = sh_m[0][n];
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh_m[w][n]);
    const float M_use = (M == -INFINITY) ? 0.0f : M;
    float L = 0.0f;
    for (int w = 0; w < kWaves; ++w) L += sh_l[w][n] * fast_exp2(sh_m[w][n] - M_use);
    const int ng = row_base + n;
    if (direct) {
      const int qi = ng / G, g = ng - qi * G;
      float den = L;
      if (a.sinks) den += fast_exp2(a.sinks[kvh * G + g] * kLog2e - M_use);
      const float bmm2 = a.bmm2_ptr ? a.bmm2_ptr[0] : a.bmm2_scale;
      if (a.out_dtype == 2)
        sh_sc[n] = den > 0.0f ? bmm2 / (den * a.o_scale) : 0.0f;
      else
        sh_sc[n] = den > 0.0f ? bmm2 / den : 0.0f;
    } else {
      const int64_t unit = ((int64_t)b * a.num_heads_kv + kvh) * max_splits + split;
      ws_ml[(unit * rows_ws + ng) * 2 + 0] = M;
      ws_ml[(unit * rows_ws + ng) * 2 + 1] = L;
    }
  }
  __syncthreads();

  // ---- write: final output (single split) or partial ------------------------------
  const RowsO *const o0 = reinterpret_cast<const RowsO *>(sk_a);
  const RowsO *const o1 = reinterpret_cast<const RowsO *>(sk_a + SHO);
  const RowsO *const o2 = reinterpret_cast<const RowsO *>(sk_b);
  const RowsO *const o3 = reinterpret_cast<const RowsO *>(sk_b + SHO);
  for (int idx = tid; idx < n_rows * (kD / 4); idx += kThreads) {
    const int n = idx / (kD / 4);
    const int d4 = (idx % (kD / 4)) * 4;
    const f32x4 s0 = *reinterpret_cast<const f32x4 *>(&o0[n][d4]);
    const f32x4 s1 = *reinterpret_cast<const f32x4 *>(&o1[n][d4]);
    const f32x4 s2 = *reinterpret_cast<const f32x4 *>(&o2[n][d4]);
    const f32x4 s3 = *reinterpret_cast<const f32x4 *>(&o3[n][d4]);
    const float f1 = sh_fw[1][n], f2 = sh_fw[2][n], f3 = sh_fw[3][n];
    float src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) src[i] = fmaf(s3[i], f3, fmaf(s2[i], f2, fmaf(s1[i], f1, s0[i])));
    const int ng = row_base + n;
    if (direct) {
      const int qi = ng / G, g = ng - qi * G;
      const int head = kvh * G + g;
      const int64_t orow = (int64_t)(qrow0 + qi) * a.num_heads_qo + head;
      const float scale = sh_sc[n];
      if (a.out_dtype == 2) {
        const uint32_t w = e4m3_encode(src[0] * scale) | (e4m3_encode(src[1] * scale) << 8) |
                           (e4m3_encode(src[2] * scale) << 16) |
                           (e4m3_encode(src[3] * scale) << 24);
        *reinterpret_cast<uint32_t *>((char *)a.out + orow * kD + d4) = w;
      } else {
        char *op = (char *)a.out + orow * kD * 2;
        u32x2 w;
        if (a.out_dtype == 0) {
          w[0] = pack2(src[0] * scale, src[1] * scale, F16Tag{});
          w[1] = pack2(src[2] * scale, src[3] * scale, F16Tag{});
        } else {
          w[0] = pack2(src[0] * scale, src[1] * scale, BF16Tag{});
          w[1] = pack2(src[2] * scale, src[3] * scale, BF16Tag{});
        }
        st8(op + d4 * 2, w);
      }
    } else {
      const int64_t unit = ((int64_t)b * a.num_heads_kv + kvh) * max_splits + split;
      float *dst = ws_o + (unit * rows_ws + ng) * kD + d4;
      *reinterpret_cast<f32x4 *>(dst) = f32x4{src[0], src[1], src[2], src[3]};
    }
  }
}

// One wave per (request, kv head, row); lanes cover d in pairs.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a,
                                                           int32_t chunk,
                                                           int32_t max_splits,
                                                           const float *__restrict__ ws_o,
                                                           const float *__restrict__ ws_ml) {
  const int G = a.num_heads_qo / a.num_heads_kv;
  const int rows = a.q_len * G;  // workspace rows per unit (the maximum)
  const int gw = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int total = a.batch * a.num_heads_kv * rows;
  if (gw >= total) return;
  const int n = gw % rows;
  const int kvh = (gw / rows) % a.num_heads_kv;
  const int b = gw / (rows * a.num_heads_kv);
  int ql, qrow0;
  request_rows(a, b, ql, qrow0);
  if (n >= ql * G) return;
  const int seq = (int)a.seq_lens[b];
  const int lo = key_origin(a, seq, ql);
  const int n_splits = seq > lo ? (seq - lo + chunk - 1) / chunk : 0;
  const int qi = n / G, g = n - qi * G;
  const int head = kvh * G + g;
  const int64_t orow = (int64_t)(qrow0 + qi) * a.num_heads_qo + head;
  if (n_splits <= 1) return;  // written by the split kernel (empty sequences too)
  const int64_t unit0 = ((int64_t)b * a.num_heads_kv + kvh) * max_splits;
  // One pass over the splits with a running maximum M (starting at the
  // sink logit), four splits' loads in flight at a time: L and O are
  // rescaled by 2^(M_old - M_new) whenever M rises.
  const float sink = a.sinks ? a.sinks[head] * kLog2e : -INFINITY;
  float M = sink, L = 0.0f, o0 = 0.0f, o1 = 0.0f;
  int s = 0;
  for (; s + 4 <= n_splits; s += 4) {
    f32x2 ml[4], v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t u = (unit0 + s + i) * rows + n;
      ml[i] = *reinterpret_cast<const f32x2 *>(ws_ml + u * 2);
      v[i] = *reinterpret_cast<const f32x2 *>(ws_o + u * kD + lane * 2);
    }
    const float Mn = fmaxf(fmaxf(M, fmaxf(ml[0][0], ml[1][0])), fmaxf(ml[2][0], ml[3][0]));
    const float Mu = Mn == -INFINITY ? 0.0f : Mn;
    const float r = fast_exp2(M - Mu);
    L *= r;
    o0 *= r;
    o1 *= r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f = fast_exp2(ml[i][0] - Mu);
      L += f * ml[i][1];
      o0 += f * v[i][0];
      o1 += f * v[i][1];
    }
    M = Mn;
  }
  for (; s < n_splits; ++s) {
    const int64_t u = (unit0 + s) * rows + n;
    const f32x2 ml = *reinterpret_cast<const f32x2 *>(ws_ml + u * 2);
    const f32x2 v = *reinterpret_cast<const f32x2 *>(ws_o + u * kD + lane * 2);
    const float Mn = fmaxf(M, ml[0]);
    const float Mu = Mn == -INFINITY ? 0.0f : Mn;
    const float r = fast_exp2(M - Mu), f = fast_exp2(ml[0] - Mu);
    L = L * r + f * ml[1];
    o0 = o0 * r + f * v[0];
    o1 = o1 * r + f * v[1];
    M = Mn;
  }
  const float M_use = (M == -INFINITY) ? 0.0f : M;
  if (a.sinks) L += fast_exp2(sink - M_use);
  const float bmm2 = a.bmm2_ptr ? a.bmm2_ptr[0] : a.bmm2_scale;
  if (a.out_dtype == 2) {
    const float scale = L > 0.0f ? bmm2 / (L * a.o_scale) : 0.0f;
    const uint32_t w = e4m3_encode(o0 * scale) | (e4m3_encode(o1 * scale) << 8);
    *reinterpret_cast<uint16_t *>((char *)a.out + orow * kD + lane * 2) = (uint16_t)w;
    return;
  }
  const float scale = L > 0.0f ? bmm2 / L : 0.0f;
  uint32_t w = (a.out_dtype == 0) ? pack2(o0 * scale, o1 * scale, F16Tag{})
                                  : pack2(o0 * scale, o1 * scale, BF16Tag{});
  *reinterpret_cast<uint32_t *>((char *)a.out + orow * kD * 2 + lane * 4) = w;
}

template <int NB, class QT, bool FP8>
hipError_t launch_nb(const DecodeArgs &a, const DecodePlan &p, hipStream_t s) {
  float *ws = reinterpret_cast<float *>(a.workspace);
  const int64_t units = (int64_t)a.batch * a.num_heads_kv;
  float *ws_o = ws;
  float *ws_ml = ws + units * p.max_splits * p.rows * kD;
  const int64_t n_units = units * p.max_splits;
  if (n_units == 0) return hipSuccess;
  // rows beyond 32 per kv head: groups of 32, each unit's groups on one XCD
  const int n_groups = (p.rows + 31) / 32;
  // whole rounds of 8 XCDs x (kv heads or row groups); blocks past the last
  // unit return at once
  const int64_t per_round = n_groups == 1 ? (int64_t)kXcds * a.num_heads_kv : kXcds;
  const int64_t blocks = (n_units + per_round - 1) / per_round * per_round * n_groups;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (n_groups == 1)
    hipLaunchKernelGGL((decode_kernel<NB, QT, FP8, true>), dim3((uint32_t)blocks),
                       dim3(kThreads), 0, s, a, p.chunk, p.max_splits, n_groups, ws_o,
                       ws_ml);
  else if constexpr (NB == 2)
    hipLaunchKernelGGL((decode_kernel<NB, QT, FP8, false>), dim3((uint32_t)blocks),
                       dim3(kThreads), 0, s, a, p.chunk, p.max_splits, n_groups, ws_o,
                       ws_ml);
  else
    return hipErrorInvalidConfiguration;  // 16-row blocks never need groups
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_splits == 1) return e;
  const int64_t waves = units * p.rows;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((uint32_t)((waves + 3) / 4)),
                     dim3(256), 0, s, a, p.chunk, p.max_splits, ws_o, ws_ml);
  return hipGetLastError();
}

template <class QT, bool FP8>
hipError_t launch_q(const DecodeArgs &a, const DecodePlan &p, hipStream_t s) {
  // up to 16 rows: one 16-row block; more: 32-row workgroups
  if (p.rows <= 16) return launch_nb<1, QT, FP8>(a, p, s);
  return launch_nb<2, QT, FP8>(a, p, s);
}

}  // namespace

DecodePlan plan_decode(int32_t batch, int32_t q_len, int32_t num_heads_qo,
                       int32_t num_heads_kv, int32_t head_dim,
                       int32_t max_seq_len, int32_t window_left) {
  DecodePlan p{};
  const int G = num_heads_qo / num_heads_kv;
  p.rows = q_len * G;
  const int64_t max_keys =
      window_left >= 0 ? (int64_t)std::min<int64_t>(max_seq_len, (int64_t)window_left + q_len)
                       : (int64_t)max_seq_len;
  const int64_t units = (int64_t)batch * num_heads_kv;
  // About 8192 workgroups at the longest request (32 per CU: enough to
  // balance ragged lengths; more, shorter chunks measured slower), but
  // chunks long enough that the partial (m, l, O) rows, written once and
  // read once by the merge, stay within 3% of the K/V bytes a chunk streams
  // (at one byte per element; bf16 caches halve that share). With many
  // query rows per kv head (drafts x GQA group) this leaves one chunk per
  // request: no merge.
  int64_t c_bal = units > 0 ? (max_keys * units + 8191) / 8192 : max_keys;
  const int64_t kv_bytes_per_key = 2 * (int64_t)head_dim;
  int64_t c_min = 2 * (int64_t)p.rows * (head_dim + 2) * 4 * 100 / (3 * kv_bytes_per_key);
  int64_t chunk = std::max<int64_t>(c_bal, c_min);
  chunk = std::max<int64_t>(chunk, 128);
  chunk = (chunk + 127) / 128 * 128;
  const int64_t cap = (max_keys + 127) / 128 * 128;
  if (chunk > cap) chunk = std::max<int64_t>(cap, 128);
  p.chunk = (int32_t)chunk;
  // range starts are rounded down to 32 keys: up to 31 extra keys
  const int64_t span = window_left >= 0 ? max_keys + 31 : max_keys;
  p.max_splits = span > 0 ? (int32_t)((span + chunk - 1) / chunk) : 1;
  p.workspace_bytes = p.max_splits > 1
                          ? (size_t)units * p.max_splits * p.rows * (kD + 2) * sizeof(float)
                          : 0;
  return p;
}

hipError_t launch_decode(const DecodeArgs &a, const DecodePlan &p, hipStream_t s) {
  const bool fp8 = a.kv_dtype == 2;
  const bool f16 = a.q_dtype == 0;
  if (fp8) return f16 ? launch_q<F16Tag, true>(a, p, s) : launch_q<BF16Tag, true>(a, p, s);
  return f16 ? launch_q<F16Tag, false>(a, p, s) : launch_q<BF16Tag, false>(a, p, s);
}

}  // namespace pkv
