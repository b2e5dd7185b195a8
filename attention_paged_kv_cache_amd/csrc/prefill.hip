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
//   K:  gathered through the block table (16-byte loads per lane) into LDS
//       as [key][d]; V: gathered 8 keys x 8 d per lane, transposed in
//       registers, stored as V^T [d][key] so that the PV operand reads are
//       16-byte runs along the key axis.
//   S^T = K Q^T on 32x32 MFMA (A = K rows from LDS, B = Q from registers).
//       In the S^T output a lane holds one query row and 32 of the tile's 64
//       keys, so row max / sum are lane-local plus one exchange across the
//       two half-waves.
//   Online softmax in fp32 registers, exponent base 2 with log2(e) folded
//       into the score scale.
//   O^T += V^T P^T on 32x32 MFMA (B = P^T straight from the S^T registers).
//   The rows of the S^T MFMA are fed keys in the order pi(m) (bits 2 and 3
//   of m swapped) so that a lane's 8 consecutive accumulator registers
//   hold 8 consecutive keys: exactly the k-run of a PV B operand.
//   Global loads of tile j+1 are issued before the MFMAs of tile j.
//
// fp8 (e4m3fn) inputs: QK^T runs on the 32x32x64 f8f6f4 MFMA; V is widened
// exactly to bf16 in the transpose, P is rounded to bf16, PV runs on bf16
// MFMA. q_scale * k_scale folds into the score scale, v_scale into the
// epilogue.

#include <math.h>

#include <type_traits>

#include "launch.h"
#include "pkv_common.h"

namespace pkv {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 128;  // query rows per workgroup
constexpr int kKeys = 64;   // keys per kv tile
constexpr int kDvo = 128;   // value / output head dim
constexpr int kVtRow = kKeys * 2 + 16;  // bytes per V^T row in LDS (padded)

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
  static constexpr int KROW = ROWB + 16;                // padded LDS row
  static constexpr int CPK = ROWB / 16;                 // 16-B chunks per K row
  static constexpr int NKCH = kKeys * CPK / 128;        // chunks per K loader
  static constexpr int KB = (ES == 1) ? 32 : 16;        // k bytes per lane per MFMA
  static constexpr int KSTEPS = ROWB / (2 * KB);        // MFMA k-steps for QK^T
  static constexpr int NQ = ROWB / 32;                  // 16-B Q chunks per lane
  static constexpr int LDS = kKeys * KROW + kDvo * kVtRow;
  static constexpr int NST = NKCH > 8 ? NKCH : 8;       // staging registers
};

// pi(m): swap bits 2 and 3 (an involution on 0..31).
__device__ __forceinline__ int key_perm(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
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

template <class ET, int DQK, class OT>
__global__ __launch_bounds__(kThreads, (DQK * ET::bytes > 256) ? 1 : 2) void prefill_kernel(
    PrefillArgs a, int32_t T, int32_t Gc, int32_t head_chunks,
    int32_t n_qtiles) {
  using G_ = Geo<ET, DQK>;
  using PT = typename PvTag<ET>::type;
  constexpr int ES = G_::ES;
  // Two LDS stages: tile j is read from stage j % 2 while tile j + 1 is
  // written into the other one.
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- which tile -------------------------------------------------------
  const int bhc = a.batch * a.num_heads_kv * head_chunks;
  const int bid = blockIdx.x;
  const int qtile = n_qtiles - 1 - bid / bhc;
  const int rem = bid % bhc;
  const int b = rem / (a.num_heads_kv * head_chunks);
  const int kvh = (rem / head_chunks) % a.num_heads_kv;
  const int hc = rem % head_chunks;
  const int L_q = a.lens_q[b];
  const int L_kv = a.lens_kv[b];
  const int tok0 = qtile * T;
  if (tok0 >= L_q) return;
  const int G = a.num_heads_qo / a.num_heads_kv;
  const int tok_last = min(L_q, tok0 + T) - 1;
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
    const int64_t qrow = (int64_t)(a.cum_q[b] + tok) * a.num_heads_qo + head;
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

  const int32_t *__restrict__ bt = a.block_tables + (int64_t)b * a.max_pages;
  const int log2ps = __builtin_ctz(a.page_size);
  const int ps_mask = a.page_size - 1;
  const int last_pg = L_kv > 0 ? (L_kv - 1) >> log2ps : 0;
  const char *kbase = (const char *)a.k + (int64_t)kvh * a.head_stride_k * ES;
  const char *vbase = (const char *)a.v + (int64_t)kvh * a.head_stride_v * ES;
  const int64_t psk = a.page_stride_k * ES, psv = a.page_stride_v * ES;
  const int64_t ssk = a.slot_stride_k * ES, ssv = a.slot_stride_v * ES;

  // Loader roles: waves 2..3 stage K, waves 0..1 stage V (transposed).
  const bool k_loader = wave >= 2;
  const int lt = tid & 127;
  // One register array serves both roles (a wave is either a K or a V
  // loader): K loaders keep their chunks of the next tile, V loaders 8 keys
  // x 8 d (e4m3 in the low half of each entry).
  u32x4 stage[G_::NST];

  // Page ids of the (up to) four pages a 64-key tile spans. Indices are
  // clamped into the sequence, so padding entries are never followed; keys
  // past the end read the last page's tail and are masked (K) or zeroed (V).
  auto tile_pages = [&](int j, int *p) {
    const int pg0 = (j * kKeys) >> log2ps;
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = bt[min(pg0 + i, last_pg)];
  };
  auto pick = [](const int *p, int idx) {  // p[idx] for idx in 0..3, branch-free
    const int lo = (idx & 1) ? p[1] : p[0];
    const int hi = (idx & 1) ? p[3] : p[2];
    return (idx & 2) ? hi : lo;
  };

  // Issue the global loads of tile j (no waits: the data is consumed by
  // store_tile one tile of compute later).
  auto load_tile = [&](const int *p) {
    if (k_loader) {
#pragma unroll
      for (int i = 0; i < G_::NKCH; ++i) {
        const int ch = lt + 128 * i;
        const int key = ch / G_::CPK, part = ch % G_::CPK;
        const int page = pick(p, key >> log2ps);
        stage[i] = ld16(kbase + (int64_t)page * psk + (key & ps_mask) * ssk + part * 16);
      }
    } else {
      const int kg = lt & 7, dg = lt >> 3;
      const int page = pick(p, (kg * 8) >> log2ps);
      const char *vp = vbase + (int64_t)page * psv + ((kg * 8) & ps_mask) * ssv + dg * 8 * ES;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (ES == 1) {
          const u32x2 w = ld8(vp + i * ssv);
          stage[i] = u32x4{w[0], w[1], 0u, 0u};
        } else {
          stage[i] = ld16(vp + i * ssv);
        }
      }
    }
  };

  auto store_tile = [&](int j) {
    char *lds_k = smem + (j & 1) * G_::LDS;
    char *lds_vt = lds_k + kKeys * G_::KROW;
    if (k_loader) {
#pragma unroll
      for (int i = 0; i < G_::NKCH; ++i) {
        const int ch = lt + 128 * i;
        const int key = ch / G_::CPK, part = ch % G_::CPK;
        st16(lds_k + key * G_::KROW + part * 16, stage[i]);
      }
    } else {
      const int kg = lt & 7, dg = lt >> 3;
      u32x4 rows[8], tr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (ES == 1) {
          const u32x2 lo = e4m3x4_to_bf16x4(stage[i][0]);
          const u32x2 hi = e4m3x4_to_bf16x4(stage[i][1]);
          rows[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          rows[i] = stage[i];
        }
      }
      // keys past the sequence end: zero, so that p = 0 meets v = 0
      const int kbeg = j * kKeys + kg * 8;
      if (kbeg + 8 > L_kv) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (kbeg + i >= L_kv) rows[i] = u32x4{0u, 0u, 0u, 0u};
      }
      transpose8x8_b16(rows, tr);
#pragma unroll
      for (int cidx = 0; cidx < 8; ++cidx)
        st16(lds_vt + (dg * 8 + cidx) * kVtRow + kg * 16, tr[cidx]);
    }
  };

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

  int pn[4];  // page ids of the next tile to load
  if (n_tiles > 0) {
    tile_pages(0, pn);
    load_tile(pn);
    store_tile(0);
    if (n_tiles > 1) {
      tile_pages(1, pn);
      load_tile(pn);
      if (n_tiles > 2) tile_pages(2, pn);
    }
    __syncthreads();
  }

  for (int j = 0; j < n_tiles; ++j) {
    const char *lds_k = smem + (j & 1) * G_::LDS;
    const char *lds_vt = lds_k + kKeys * G_::KROW;

    // ---- S^T = K Q^T -------------------------------------------------------
    f32x16 sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[mb][i] = 0.0f;
      const char *krow = lds_k + (mb * 32 + key_perm(l32)) * G_::KROW;
#pragma unroll
      for (int s = 0; s < G_::KSTEPS; ++s) {
        u32x4 av[2];
#pragma unroll
        for (int u = 0; u < G_::KB / 16; ++u)
          av[u] = ld16(krow + s * 2 * G_::KB + half * G_::KB + 16 * u);
        sacc[mb] = mfma_qk(av, &qreg[s * (G_::KB / 16)], sacc[mb], ET{});
      }
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
    float psum = 0.0f;
    u32x4 pb[4];  // P^T B operands, one per 16-key k-step
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          const float p0 = fast_exp2(fmaf(sacc[mb][hh * 8 + 2 * w2], c, -m_use));
          const float p1 = fast_exp2(fmaf(sacc[mb][hh * 8 + 2 * w2 + 1], c, -m_use));
          psum += p0 + p1;
          pb[mb * 2 + hh][w2] = pack2(p0, p1, PT{});
        }
    l_run += psum;

    // ---- O^T += V^T P^T --------------------------------------------------------
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
#pragma unroll
      for (int md = 0; md < 4; ++md) {
        const u32x4 av =
            ld16(lds_vt + (md * 32 + l32) * kVtRow + (kstep * 16 + half * 8) * 2);
        o[md] = mfma_pv(av, pb[kstep], o[md], PT{});
      }
    }

    // ---- stage tile j + 1 (its loads flew during this tile) -------------------
    if (j + 1 < n_tiles) {
      store_tile(j + 1);
      if (j + 2 < n_tiles) {
        load_tile(pn);
        if (j + 3 < n_tiles) tile_pages(j + 3, pn);
      }
    }
    __syncthreads();
  }

  // ---- epilogue ----------------------------------------------------------------
  const float l_tot = wave_sum_xor32(l_run);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? vs / l_tot : 0.0f;
  const int64_t orow = (int64_t)(a.cum_q[b] + tok) * a.num_heads_qo + head;
  char *op = (char *)a.out + orow * kDvo * 2;
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = md * 32 + q4 * 8 + half * 4;
      u32x2 w;
      w[0] = pack2(o[md][q4 * 4 + 0] * inv, o[md][q4 * 4 + 1] * inv, OT{});
      w[1] = pack2(o[md][q4 * 4 + 2] * inv, o[md][q4 * 4 + 3] * inv, OT{});
      st8(op + d * 2, w);
    }
  if (half == 0)
    a.lse[orow] = l_tot > 0.0f ? m_ref * kLn2 + __logf(l_tot) : -INFINITY;
}

template <class ET, int DQK, class OT>
hipError_t launch_typed(const PrefillArgs &a, hipStream_t s) {
  using G_ = Geo<ET, DQK>;
  const int G = a.num_heads_qo / a.num_heads_kv;
  const int Gc = G < kRows ? G : kRows;
  const int head_chunks = (G + Gc - 1) / Gc;
  const int T = kRows / Gc;
  const int n_qtiles = (a.max_q + T - 1) / T;
  const int64_t blocks =
      (int64_t)n_qtiles * a.batch * a.num_heads_kv * head_chunks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  static bool lds_opt_in = false;  // two LDS stages exceed the 64 KB default
  if (!lds_opt_in) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&prefill_kernel<ET, DQK, OT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 2 * G_::LDS);
    if (e != hipSuccess) return e;
    lds_opt_in = true;
  }
  hipLaunchKernelGGL((prefill_kernel<ET, DQK, OT>), dim3((uint32_t)blocks),
                     dim3(kThreads), 2 * G_::LDS, s, a, T, Gc, head_chunks,
                     n_qtiles);
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
