// Batch prefill attention over a paged KV cache, MFMA on gfx950.
//
// Source: flashinfer.prefill.cudnn_batch_prefill_with_kv_cache --
// Parameters (q, k_cache, v_cache, scale, actual_seq_lens_q/kv,
// block_tables, causal, return_lse, q_scale/k_scale/v_scale), Returns (output
// and log-sum-exp per token and head), Note (num_heads_qo >= num_heads_kv;
// d_qk 128 or 192, d_vo 128). The causal mask is aligned bottom-right:
// query t of a request with L_q queries and L_kv keys may attend to keys
// j <= t + L_kv - L_q.
//
// Work decomposition
//   One workgroup (4 waves, 256 threads) owns a tile of 128 query rows that
//   share one kv head: T tokens x Gc qo heads of that kv head's group
//   (GQA packing: T = 128 / Gc), so each K/V tile staged in LDS serves every
//   qo head of the group. Each wave owns 32 rows.
//
// Per kv tile of 64 keys
//   K and V go from HBM straight into LDS with buffer_load_dwordx4 ... lds
//   (no staging registers): each wave gathers 16 keys of the tile, all in
//   one page, through the block table, with a buffer resource that starts
//   at the wave's first key and ends at the sequence's last key. Every DMA
//   instruction is a full one: lanes whose rows lie past the sequence end
//   fall outside the resource and write zeros into LDS (their scores are
//   masked). The loads carry no branches and no per-tile address math, and
//   are spread between the MFMAs of the previous tile instead of arriving
//   as one burst. So that the 16 K rows one read
//   touches fall in distinct banks, 256-byte K rows (16-bit d 128) keep
//   their 16-byte chunks XOR-swizzled by row (16 rows fill exactly 4 KB);
//   other K rows are padded by 16 bytes, and each wave's 16 K rows occupy a
//   whole number of KB. V rows stay in the
//   cache's [key][d] order with a 16-byte-chunk XOR swizzle, and the PV
//   operand (V^T, keys along k) is read with the LDS transpose reads
//   ds_read_b64_tr_b16 (ds_read_b64_tr_b8 for e4m3, widened after the read).
//   S^T = K Q^T on 32x32 MFMA (A = K rows from LDS, B = Q from registers).
//       In the S^T output a lane holds one query row and 32 of the tile's 64
//       keys, so row max / sum are lane-local plus one exchange across the
//       two half-waves.
//   Online softmax in fp32 registers, exponent base 2 with log2(e) folded
//       into the score scale; the row maximum used for the exponentials is
//       raised lazily, so most tiles do not rescale O.
//   O^T += V^T P^T on 32x32 MFMA (B = P^T straight from the S^T registers).
//   The rows of the S^T MFMA are fed keys in the order pi(m) (bits 2 and 3
//   of m swapped) so that a lane's 8 consecutive accumulator registers
//   hold 8 consecutive keys: exactly the k-run of a PV B operand.
//   Two LDS stages: tile j + 1 lands while tile j is computed; one barrier
//   per tile.
//
// fp8 (e4m3fn) inputs: QK^T runs on the 32x32x64 f8f6f4 MFMA; V is widened
// exactly to bf16 after the transpose read, P is rounded to bf16, PV runs on
// bf16 MFMA. q_scale * k_scale folds into the score scale, v_scale into the
// epilogue.

#include <math.h>

#include <algorithm>
#include <type_traits>

#include "launch_prefill.h"
#include "pkv_common.h"

namespace pkv {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 128;  // query rows per workgroup
constexpr int kKeys = 64;   // keys per kv tile
constexpr int kDvo = 128;   // value / output head dim
constexpr int kXcds = 8;    // MI355X accelerator complex dies

#define PKV_LDS __attribute__((address_space(3)))

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

template <class ET>
struct PvTag {  // 16-bit type of P and V^T for the PV MFMA
  using type = BF16Tag;
};
template <>
struct PvTag<F16Tag> {
  using type = F16Tag;
};

template <class ET, int DQK>
struct Geo {
  static constexpr int ES = ET::bytes;
  static constexpr int ROWB = DQK * ES;                 // bytes of one K row
  // 256-byte K rows: unpadded, 16-byte chunks XOR-swizzled by row (16 rows
  // fill exactly 4 KB: four DMAs per wave); other widths: padded by 16 B
  static constexpr bool KSWZ = ROWB == 256;
  static constexpr int KRB = KSWZ ? ROWB : ROWB + 16;   // K row in LDS
  static constexpr int VRB = kDvo * ES;                 // V row (unpadded, swizzled)
  static constexpr int KB = (ES == 1) ? 32 : 16;        // k bytes per lane per MFMA
  static constexpr int KSTEPS = ROWB / (2 * KB);        // MFMA k-steps for QK^T
  static constexpr int NQ = ROWB / 32;                  // 16-B Q chunks per lane
  static constexpr int WKB = (16 * KRB + 1023) / 1024 * 1024;  // a wave's K block
  static constexpr int K_BYTES = 4 * WKB;
  static constexpr int V_BYTES = kKeys * VRB;
  static constexpr int STAGE = K_BYTES + V_BYTES;       // one LDS stage
  static constexpr int K_INSTR = WKB / 1024;            // 1 KB DMA writes per wave
  static constexpr int V_INSTR = 16 * VRB / 1024;
};

// pi(m): swap bits 2 and 3 (an involution on 0..31).
__device__ __forceinline__ int key_perm(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// XOR applied to the 16-byte chunk index of V row `key` in LDS. It spreads
// the rows one transpose read touches over distinct banks.
template <int ES>
__device__ __forceinline__ int vswz(int key) {
  return ES == 2 ? 4 * (key & 3) : 2 * ((key >> 1) & 3);
}

__device__ __forceinline__ f32x16 mfma_qk(const u32x4 *a, const u32x4 *b,
                                          f32x16 c, BF16Tag) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8, a[0]), __builtin_bit_cast(bf16x8, b[0]), c, 0,
      0, 0);
}
__device__ __forceinline__ f32x16 mfma_qk(const u32x4 *a, const u32x4 *b,
                                          f32x16 c, F16Tag) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(
      __builtin_bit_cast(f16x8, a[0]), __builtin_bit_cast(f16x8, b[0]), c, 0,
      0, 0);
}
__device__ __forceinline__ f32x16 mfma_qk(const u32x4 *a, const u32x4 *b,
                                          f32x16 c, E4M3Tag) {
  i32x8 av, bv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    av[i] = (int)a[0][i];
    av[4 + i] = (int)a[1][i];
    bv[i] = (int)b[0][i];
    bv[4 + i] = (int)b[1][i];
  }
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 0,
                                                         0, 0);
}

__device__ __forceinline__ f32x16 mfma_pv(u32x4 a, u32x4 b, f32x16 c,
                                          BF16Tag) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_pv(u32x4 a, u32x4 b, f32x16 c,
                                          F16Tag) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(
      __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Buffer resource over `bytes` bytes from `base` (raw, untyped access).
// Loads past the range return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, bytes, 0x00020000);
}

// 16 bytes at rsrc + voff straight into LDS: lane l's bytes land at
// lds_base + 16 * l (lds_base must be the same for every lane). The buffer
// form, unlike the flat global_load_lds, is not modelled by the compiler as
// a flat access that may touch LDS, which would make every later LDS read
// wait for all outstanding loads.
__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t r, int voff, char *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (PKV_LDS void *)lds_base, 16, voff, 0, 0, 0);
}

// Wait until this wave's outstanding global loads (LDS DMA included) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <class ET, int DQK, class OT, bool PAGED>
__global__ __launch_bounds__(kThreads, (DQK * ET::bytes > 256) ? 1 : 2) void prefill_kernel(
    PrefillArgs a, int32_t T, int32_t Gc, int32_t head_chunks,
    int32_t n_qtiles, int32_t S) {
  using G_ = Geo<ET, DQK>;
  using PT = typename PvTag<ET>::type;
  constexpr int ES = G_::ES;
  // Two LDS stages of [K rows | V rows]: tile j is read from one while tile
  // j + 1 lands in the other. Two distinct arrays (not one buffer indexed by
  // j % 2) let the compiler see that the DMA into one stage never aliases
  // the reads of the other, so it does not wait for the DMA before them.
  __shared__ __attribute__((aligned(16))) char lds_s0[G_::STAGE];
  __shared__ __attribute__((aligned(16))) char lds_s1[G_::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- which tile -------------------------------------------------------
  // Workgroups are dispatched round-robin over the 8 XCDs (block i runs on
  // XCD i % 8), each with its own L2. A "pair" (request, kv head, head
  // chunk) owns one K/V stream; all query tiles of a pair are mapped to the
  // same XCD, so the pair's K/V pages are fetched from HBM about once and
  // re-read from L2. An XCD's pairs are taken S at a time (a batch sized
  // so that its K/V streams fit the XCD's L2); within a batch the tiles go
  // by query-tile index from the last (the heaviest under the causal mask)
  // down, cycling over the batch's pairs. Dispatching heavy tiles first
  // keeps the grid's tail made of light tiles.
  const int n_pairs = a.batch * a.num_heads_kv * head_chunks;
  const int xcd = blockIdx.x % kXcds;
  const int slot_in_xcd = blockIdx.x / kXcds;
  const int per_batch = S * n_qtiles;
  const int batch_i = slot_in_xcd / per_batch;
  const int r_in = slot_in_xcd - batch_i * per_batch;
  const int pair = xcd + kXcds * (batch_i * S + r_in % S);
  if (pair >= n_pairs) return;
  const int qtile = n_qtiles - 1 - r_in / S;
  const int b = pair / (a.num_heads_kv * head_chunks);
  const int kvh = (pair / head_chunks) % a.num_heads_kv;
  const int hc = pair % head_chunks;
  const int L_q = a.lens_q[b];
  const int L_kv = a.lens_kv[b];
  const int tok0 = qtile * T;
  if (tok0 >= L_q) return;
  const int G = a.num_heads_qo / a.num_heads_kv;
  const int tok_last = min(L_q, tok0 + T) - 1;
  // First rows of request b: given offsets, or packed rows (null offsets,
  // small batches): the sum of the lengths of the requests before b.
  auto packed_row = [&](const int32_t *lens) {
    int r0 = 0;
    for (int i = 0; i < b; ++i) r0 += lens[i];
    return r0;
  };
  const bool any_packed_q = !a.off_q || !a.off_o || !a.off_lse;
  const int packed_q = any_packed_q ? packed_row(a.lens_q) : 0;
  const int row_q = a.off_q ? a.off_q[b] : packed_q;
  const int row_o = a.off_o ? a.off_o[b] : packed_q;
  const int row_lse = a.off_lse ? a.off_lse[b] : packed_q;
  const int shift = L_kv - L_q;  // bottom-right alignment

  // ---- this lane's query row ---------------------------------------------
  const int r = wave * 32 + l32;
  const int g = r / T;
  const int t = r - g * T;
  const int qh = hc * Gc + g;  // head index inside the kv head's group
  const int tok = tok0 + t;
  const bool row_ok = (g < Gc) && (qh < G) && (tok < L_q);
  const int head = kvh * G + qh;
  int lim = 0;  // keys [0, lim) allowed for this row
  if (row_ok) lim = a.causal ? min(L_kv, shift + tok + 1) : L_kv;
  if (lim < 0) lim = 0;

  // ---- scales ------------------------------------------------------------
  float qs = a.q_scale ? *a.q_scale : 1.0f;
  float ks = a.k_scale ? *a.k_scale : 1.0f;
  float vs = a.v_scale ? *a.v_scale : 1.0f;
  float c = a.scale * qs * ks * kLog2e;
  const bool negate = c < 0.0f;
  c = fmaxf(fabsf(c), 1e-30f);

  // ---- Q^T operand in registers -------------------------------------------
  u32x4 qreg[G_::NQ];
  {
    const int64_t qrow = (int64_t)(row_q + tok) * a.num_heads_qo + head;
    const char *qp = (const char *)a.q + qrow * G_::ROWB;
    const uint32_t flip = negate ? (ES == 1 ? 0x80808080u : 0x80008000u) : 0u;
#pragma unroll
    for (int s = 0; s < G_::KSTEPS; ++s) {
#pragma unroll
      for (int u = 0; u < G_::KB / 16; ++u) {
        const int off = s * 2 * G_::KB + half * G_::KB + 16 * u;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row_ok) v = ld16(qp + off);
        v[0] ^= flip; v[1] ^= flip; v[2] ^= flip; v[3] ^= flip;
        qreg[s * (G_::KB / 16) + u] = v;
      }
    }
  }

  // ---- kv range of the tile ------------------------------------------------
  const int kv_end = a.causal ? min(L_kv, shift + tok_last + 1) : L_kv;
  const int kv_clean = a.causal ? min(L_kv, shift + tok0 + 1) : L_kv;
  const int n_tiles = kv_end > 0 ? (kv_end + kKeys - 1) / kKeys : 0;

  // block table row through the constant address space: scalar loads
  const __attribute__((address_space(4))) int32_t *bt =
      (const __attribute__((address_space(4))) int32_t *)(a.block_tables) +
      (int64_t)b * a.max_pages;
  const int log2ps = __builtin_ctz(a.page_size);
  const int ps_mask = a.page_size - 1;
  const int last_pg = L_kv > 0 ? (L_kv - 1) >> log2ps : 0;
  const char *kbase = (const char *)a.k + (int64_t)kvh * a.head_stride_k * ES;
  const char *vbase = (const char *)a.v + (int64_t)kvh * a.head_stride_v * ES;
  const int64_t psk = a.page_stride_k * ES, psv = a.page_stride_v * ES;
  const int64_t ssk = a.slot_stride_k * ES, ssv = a.slot_stride_v * ES;

  // Each wave gathers keys r0 .. r0+15 of every tile; they share one page
  // (page sizes 16, 32, 64). The page index is clamped into the sequence so
  // that padding entries of the block table are never followed.
  const int r0 = 16 * wave;
  auto wave_page = [&](int j) {
    if constexpr (PAGED) return bt[min((j * kKeys + r0) >> log2ps, last_pg)];
    else return 0;  // rows are addressed directly (dma_prep)
  };
  // Without paging each wave's 16 keys are 16 consecutive rows from
  // off_k[b] + key (off_v[b] + key for values).
  int row_k = 0, row_v = 0;
  if constexpr (!PAGED) {
    const int packed_kv = (!a.off_k || !a.off_v) ? packed_row(a.lens_kv) : 0;
    row_k = a.off_k ? a.off_k[b] : packed_kv;
    row_v = a.off_v ? a.off_v[b] : packed_kv;
  }

  // Per-lane source rows / columns of each 1 KB LDS DMA of this wave's 16 K
  // rows (a whole number of KB per wave: lanes that fall in the row padding
  // or past the 16th row load a duplicate into unused LDS bytes) and 16 V
  // rows.
  int k_row[G_::K_INSTR], k_col[G_::K_INSTR], v_row[G_::V_INSTR], v_col[G_::V_INSTR];
#pragma unroll
  for (int q = 0; q < G_::K_INSTR; ++q) {
    const int byte = q * 1024 + lane * 16;
    int row = byte / G_::KRB, col = byte - row * G_::KRB;
    if constexpr (G_::KSWZ) {
      col = (((col >> 4) ^ row) & 15) * 16;  // LDS chunk c of row r holds chunk c ^ r
    } else {
      if (row > 15) { row = 15; col = 0; }
      if (col >= G_::ROWB) col = G_::ROWB - 16;
    }
    k_row[q] = row;
    k_col[q] = col;
  }
#pragma unroll
  for (int q = 0; q < G_::V_INSTR; ++q) {
    const int byte = q * 1024 + lane * 16;
    const int row = byte / G_::VRB;
    const int pc = (byte - row * G_::VRB) >> 4;
    v_row[q] = row;
    v_col[q] = (pc ^ vswz<ES>(row)) * 16;
  }
  // DMA state of the tile being loaded: buffer resources over the wave's 16
  // K and V rows, cut at the sequence end. Rows past it lie outside the
  // range, and a buffer load out of range returns zeros, which the DMA
  // writes into LDS like any other data (zero rows: their scores are masked
  // and their probabilities are exactly zero, so they add nothing). The
  // per-lane offsets inside the 16 rows are the same for every tile.
  struct Dma {
    __amdgpu_buffer_rsrc_t rk, rv;
    char *kl, *vl;
  };
  int k_off[G_::K_INSTR], v_off[G_::V_INSTR];
#pragma unroll
  for (int q = 0; q < G_::K_INSTR; ++q) k_off[q] = k_row[q] * (int)ssk + k_col[q];
#pragma unroll
  for (int q = 0; q < G_::V_INSTR; ++q) v_off[q] = v_row[q] * (int)ssv + v_col[q];
  auto dma_prep = [&](int j, int page, char *stage) {
    Dma d;
    const int key0 = j * kKeys + r0;
    const int valid = min(16, max(L_kv - key0, 0));  // rows inside the sequence
    int64_t ok, ov;  // byte offsets of the block's first row
    if constexpr (PAGED) {
      ok = (int64_t)page * psk + (int64_t)(key0 & ps_mask) * ssk;
      ov = (int64_t)page * psv + (int64_t)(key0 & ps_mask) * ssv;
    } else {
      ok = (int64_t)(row_k + key0) * ssk;
      ov = (int64_t)(row_v + key0) * ssv;
    }
    if (valid == 0) ok = ov = 0;
    d.rk = make_rsrc(kbase + ok, valid > 0 ? (int)((valid - 1) * ssk + G_::ROWB) : 0);
    d.rv = make_rsrc(vbase + ov, valid > 0 ? (int)((valid - 1) * ssv + G_::VRB) : 0);
    d.kl = stage + wave * G_::WKB;
    d.vl = stage + G_::K_BYTES + r0 * G_::VRB;
    return d;
  };
  auto dma_k = [&](const Dma &d, int q) { dma16b(d.rk, k_off[q], d.kl + q * 1024); };
  auto dma_v = [&](const Dma &d, int q) { dma16b(d.rv, v_off[q], d.vl + q * 1024); };
  auto issue_tile = [&](int j, int page, char *stage) {
    const Dma d = dma_prep(j, page, stage);
#pragma unroll
    for (int q = 0; q < G_::K_INSTR; ++q) dma_k(d, q);
#pragma unroll
    for (int q = 0; q < G_::V_INSTR; ++q) dma_v(d, q);
  };

  // Per-lane parts of the V^T transpose-read addresses (see vswz).
  const int li = lane & 15, lg = (lane >> 4) & 1, lt4 = (li >> 2) & 3;
  int v_lane, v_md[4];
  if constexpr (ES == 2) {
    v_lane = (8 * half + (li >> 2)) * G_::VRB + 32 * lg + 16 * ((li & 3) >> 1) + 8 * (li & 1);
#pragma unroll
    for (int md = 0; md < 4; ++md) v_md[md] = 64 * (md ^ lt4);
  } else {
    v_lane = (8 * half + (li >> 1)) * G_::VRB + 16 * lg + 8 * (li & 1);
#pragma unroll
    for (int md = 0; md < 4; ++md) v_md[md] = 32 * (md ^ lt4);
  }

  f32x16 o[4];
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[md][i] = 0.0f;
  // m_ref: the row's reference maximum (log2 units of the scaled score).
  // It is raised lazily, only when a tile's maximum exceeds it by more than
  // kLazy, so most tiles skip rescaling O; exponentials stay <= 2^kLazy.
  constexpr float kLazy = 8.0f;
  float m_ref = -INFINITY;
  float l_run = 0.0f;

  int pg_next = 0;
  if (n_tiles > 0) {
    issue_tile(0, wave_page(0), lds_s0);
    pg_next = wave_page(1);
    wait_vmem();
    __syncthreads();
  }

  // One kv tile: compute from `cur` while tile j + 1 lands in `nxt`.
  auto tile_step = [&](int j, const char *cur, char *nxt) {
    const char *lds_k = cur;
    const char *lds_v = cur + G_::K_BYTES;
    // Tile j + 1 (past the end: zero-range loads that only write zeros) is
    // loaded into `nxt` by DMAs spread over this tile's MFMAs.
    const Dma dn = dma_prep(j + 1, pg_next, nxt);

    // ---- S^T = K Q^T -------------------------------------------------------
    // The two 32-key m-blocks form two independent MFMA chains; their K
    // fragment reads are issued a few steps ahead of the MFMAs that use them.
    f32x16 sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[mb][i] = 0.0f;
    {
      const int kr = key_perm(l32);
      const char *krow0 = lds_k + (kr >> 4) * G_::WKB + (kr & 15) * G_::KRB;
      // swizzled rows: logical chunk 2s + half sits at chunk (2s) ^ kx
      const int kx = half ^ (kr & 15);
#pragma unroll
      for (int s = 0; s < G_::KSTEPS; ++s) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          u32x4 av[2];
          if constexpr (G_::KSWZ) {
            av[0] = ld16(krow0 + mb * 2 * G_::WKB + 16 * ((2 * s) ^ kx));
          } else {
#pragma unroll
            for (int u = 0; u < G_::KB / 16; ++u)
              av[u] = ld16(krow0 + mb * 2 * G_::WKB + s * 2 * G_::KB + half * G_::KB + 16 * u);
          }
          sacc[mb] = mfma_qk(av, &qreg[s * (G_::KB / 16)], sacc[mb], ET{});
        }
      }
#pragma unroll
      for (int q = 0; q < G_::K_INSTR; ++q) dma_k(dn, q);
      // The next tile's V DMAs are issued here too, among this tile's S^T
      // MFMAs (the V stage they fill was last read before the previous
      // barrier): they then have the whole tile to land before the
      // end-of-tile wait. Bit-identical outputs; bf16 974 -> 1004 TFLOP/s
      // against issuing them in the PV phase, e4m3 (six S^T MFMAs) 1378 ->
      // 1393 and 1401 -> 1405 on two boxes.
#pragma unroll
      for (int q = 0; q < G_::V_INSTR; ++q) dma_v(dn, q);
      constexpr int kRd = G_::KB / 16;             // LDS reads per MFMA
      constexpr int kMf = 2 * G_::KSTEPS;          // MFMAs
      constexpr int kAhead = 2;                    // MFMAs of look-ahead
      __builtin_amdgcn_sched_group_barrier(0x100, kRd * kAhead, 0);
#pragma unroll
      for (int i = 0; i < kMf - kAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kRd, 0);
        if (i % 2 == 1 && i / 2 < G_::K_INSTR + G_::V_INSTR)
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
    }

    // ---- mask (boundary tiles only) ----------------------------------------
    const int kv0 = j * kKeys;
    if (kv0 + kKeys > kv_clean) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kv0 + mb * 32 + (i >> 3) * 16 + half * 8 + (i & 7);
          if (key >= lim) sacc[mb][i] = -INFINITY;
        }
    }

    // ---- online softmax ------------------------------------------------------
    float mloc = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, sacc[mb][i]);
    mloc = wave_max_xor32(mloc);
    const float m_tile = mloc * c;  // -inf when every key of the row is masked
    const bool need = m_tile > m_ref + kLazy;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? m_tile : m_ref;
      const float alpha = need ? fast_exp2(m_ref - m_new) : 1.0f;
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int md = 0; md < 4; ++md)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[md][i] *= alpha;
    }
    const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;

    // ---- P and O^T += V^T P^T, one 16-key k-step at a time ------------------
    // The exponentials of k-step k+1 run on the VALU while the MFMAs of
    // k-step k execute. V^T comes from LDS transpose reads. The wave runs
    // this phase at raised issue priority, so that a SIMD's arbiter serves a
    // wave in its PV MFMA chain before waves in their softmax (e4m3 prefill
    // 1341 -> 1385 TFLOP/s, bf16 unchanged; raised over the S^T phase or the
    // softmax instead, it gained nothing).
    float psum = 0.0f;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      const int mb = kstep >> 1, hh = kstep & 1;
      u32x4 pb;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const float p0 = fast_exp2(fmaf(sacc[mb][hh * 8 + 2 * w2], c, -m_use));
        const float p1 = fast_exp2(fmaf(sacc[mb][hh * 8 + 2 * w2 + 1], c, -m_use));
        psum += p0 + p1;
        pb[w2] = pack2(p0, p1, PT{});
      }
#pragma unroll
      for (int md = 0; md < 4; ++md) {
        const char *vptr = lds_v + kstep * 16 * G_::VRB + v_lane + v_md[md];
        u32x4 av;
        if constexpr (ES == 2) {
          const i16x4 r0v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_LDS i16x4 *)vptr);
          const i16x4 r1v =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_LDS i16x4 *)(vptr + 4 * G_::VRB));
          const u32x2 w0 = __builtin_bit_cast(u32x2, r0v), w1 = __builtin_bit_cast(u32x2, r1v);
          av = u32x4{w0[0], w0[1], w1[0], w1[1]};
        } else {
          const i32x2 r8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PKV_LDS i32x2 *)vptr);
          const u32x2 lo = e4m3x4_to_bf16x4((uint32_t)r8[0]);
          const u32x2 hi = e4m3x4_to_bf16x4((uint32_t)r8[1]);
          av = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
        o[md] = mfma_pv(av, pb, o[md], PT{});
      }
    }
    __builtin_amdgcn_s_setprio(0);
    l_run += psum;
    // the page of tile j + 2 (read here, where its latency overlaps the wait)
    pg_next = wave_page(j + 2);

    // tile j + 1 has landed (this wave's DMA) and every wave is done with
    // `cur` after this barrier
    wait_vmem();
    __syncthreads();
  };

  for (int j = 0; j < n_tiles; j += 2) {
    tile_step(j, lds_s0, lds_s1);
    if (j + 1 < n_tiles) tile_step(j + 1, lds_s1, lds_s0);
  }

  // ---- epilogue ----------------------------------------------------------------
  const float l_tot = wave_sum_xor32(l_run);
  const float inv = l_tot > 0.0f ? vs / l_tot : 0.0f;
  if (row_ok && half == 0)
    a.lse[(int64_t)(row_lse + tok) * a.num_heads_qo + head] =
        l_tot > 0.0f ? m_ref * kLn2 + __logf(l_tot) : -INFINITY;
  // The output rows go through LDS so that every store writes whole rows. A
  // lane's O^T registers hold 4-element runs of one row, and the rows of a
  // wave's lanes lie far apart in memory (consecutive tokens of a head are
  // num_heads_qo rows apart), so stores straight from the registers write
  // each 256-byte row as sixteen 16-byte pieces (those stores cost 5% of the
  // batch-prefill time: 1000 vs 1052 TFLOP/s with them left out). Staged, 16
  // lanes write one row with 16-byte stores, non-temporal since nothing here
  // reads the output again: bf16 996 -> 1026 TFLOP/s, e4m3 1423 -> 1440
  // (1020 and 1434 with plain stores), bit-identical. The tile loop ended at
  // a barrier after every wave's last LDS read and DMA, so both stages are
  // free: each wave takes its own 32 padded rows (waves 0-1 in the first
  // stage, 2-3 in the second).
  constexpr int ORB = kDvo * 2 + 16;  // bytes per staged row (padded by 16)
  static_assert(2 * 32 * ORB <= G_::STAGE, "output staging exceeds an LDS stage");
  char *so = (wave < 2 ? lds_s0 : lds_s1) + (wave & 1) * 32 * ORB;
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = md * 32 + q4 * 8 + half * 4;
      u32x2 w;
      w[0] = pack2(o[md][q4 * 4 + 0] * inv, o[md][q4 * 4 + 1] * inv, OT{});
      w[1] = pack2(o[md][q4 * 4 + 2] * inv, o[md][q4 * 4 + 3] * inv, OT{});
      *(PKV_LDS u32x2 *)(so + l32 * ORB + d * 2) = w;
    }
  __syncthreads();
  // 32 rows x 16 chunks of 16 bytes: four rows per pass, 16 lanes per row
  const int c16 = lane & 15;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int rr = it * 4 + (lane >> 4);  // the wave's row
    const int rg = wave * 32 + rr;        // the workgroup's row
    const int g2 = rg / T, t2 = rg - g2 * T;
    const int qh2 = hc * Gc + g2, tok2 = tok0 + t2;
    const u32x4 v = *(const PKV_LDS u32x4 *)(so + rr * ORB + c16 * 16);
    if (g2 < Gc && qh2 < G && tok2 < L_q) {
      const int64_t orow = (int64_t)(row_o + tok2) * a.num_heads_qo + kvh * G + qh2;
      __builtin_nontemporal_store(v, (u32x4 *)((char *)a.out + orow * kDvo * 2 + c16 * 16));
    }
  }
}

// Pairs per dispatch batch of one XCD: the largest power of two (at most 8)
// of K/V streams of the longest request that fits three quarters of the
// XCD's 4 MB L2 (the rest holds the tiles' Q, output and DMA traffic).
// Measured on one MI355X (TFLOP/s by pairs per batch 1 / 2 / 4 / 8):
// batch prefill bf16, 2 MB streams: 966 / 839 / 751 / 761 (a second
// stream overflows the L2); fp8 prefill d_qk 192, 1.3 MB streams of 4096
// tokens: 1300 / 1349 / 1392 / 1384 (interleaving identical long causal
// streams ends the grid on light tiles). 3 pairs per batch measured 1294 on
// the fp8 workload (16 pairs per XCD leave a lone last pair, whose heavy
// tiles then end the grid), hence powers of two.
constexpr int64_t kStreamBytesPerXcd = (int64_t)3 << 20;

template <class ET, int DQK, class OT>
hipError_t launch_typed(const PrefillArgs &a, hipStream_t s) {
  const int G = a.num_heads_qo / a.num_heads_kv;
  const int Gc = G < kRows ? G : kRows;
  const int head_chunks = (G + Gc - 1) / Gc;
  const int T = kRows / Gc;
  const int n_qtiles = (a.max_q + T - 1) / T;
  const int64_t n_pairs = (int64_t)a.batch * a.num_heads_kv * head_chunks;
  const int64_t stream_bytes =
      std::max<int64_t>((int64_t)a.max_kv * (DQK + kDvo) * ET::bytes, 1);
#ifdef PKV_PREFILL_S
  const int S = PKV_PREFILL_S;
#else
  int S = 1;
  while (S < 8 && 2 * S * stream_bytes <= kStreamBytesPerXcd) S *= 2;
#endif
  const int64_t per_xcd = (n_pairs + kXcds - 1) / kXcds;
  const int64_t blocks = (int64_t)kXcds * ((per_xcd + S - 1) / S) * S * n_qtiles;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.block_tables)
    hipLaunchKernelGGL((prefill_kernel<ET, DQK, OT, true>), dim3((uint32_t)blocks),
                       dim3(kThreads), 0, s, a, T, Gc, head_chunks, n_qtiles, S);
  else
    hipLaunchKernelGGL((prefill_kernel<ET, DQK, OT, false>), dim3((uint32_t)blocks),
                       dim3(kThreads), 0, s, a, T, Gc, head_chunks, n_qtiles, S);
  return hipGetLastError();
}

template <class ET, class OT>
hipError_t launch_dqk(const PrefillArgs &a, hipStream_t s) {
  if (a.d_qk == 128) return launch_typed<ET, 128, OT>(a, s);
  return launch_typed<ET, 192, OT>(a, s);
}

}  // namespace

// pkv_dtype values: 0 = F16, 1 = BF16, 2 = E4M3
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
  const bool o_f16 = a.o_dtype == 0;
  switch (a.qkv_dtype) {
    case 0:
      return o_f16 ? launch_dqk<F16Tag, F16Tag>(a, s)
                   : launch_dqk<F16Tag, BF16Tag>(a, s);
    case 1:
      return o_f16 ? launch_dqk<BF16Tag, F16Tag>(a, s)
                   : launch_dqk<BF16Tag, BF16Tag>(a, s);
    default:
      return o_f16 ? launch_dqk<E4M3Tag, F16Tag>(a, s)
                   : launch_dqk<E4M3Tag, BF16Tag>(a, s);
  }
}

}  // namespace pkv
