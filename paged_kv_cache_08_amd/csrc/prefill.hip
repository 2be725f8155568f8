// Chunked (paged) prefill attention for gfx950.
//
// The last m_s of the n_s tokens of sequence s are new: their K/V are
// already in the paged cache (kv_append), and each is a query.  Query i sits
// at position p = n_s - m_s + i and attends causally to positions 0 .. p (the
// last `window` of them when window > 0) through the block table: exact
// scaled-score softmax attention, evaluated blockwise with running max / sum
// statistics («Servicio…presupuesto de memoria» §6), grouped-query heads
// sharing one KV head («¿Cuánta memoria reservar para la caché KV?», "Emplear
// las cabezas KV").  Prefill work has many queries per KV token, so unlike
// decode it is bound by the matrix cores, not by HBM.
//
// One workgroup = 4 waves = 256 query rows of one (sequence, KV head).  A row
// is one (query position, query head of the group) pair, position-major, so
// the group's heads share every K/V tile.  Each wave owns 64 rows (four
// 16-row blocks).  K/V are streamed in tiles of 64 tokens (four 16-token
// blocks gathered through the block table) into LDS:
//   K  [64 tokens][D + 8]   (token rows, 16 bytes of padding against bank
//                            conflicts),
//   Vt [D][64 + 4]          (value-column rows, tokens fastest, padded).
// Per tile and wave, with lane l = 16*g + c (g = l/16, c = l%16):
//   S^T = K · Q^T   v_mfma_f32_16x16x32_bf16, A = K (row = token c of a
//                   16-token block, k = head-dim values 32kc+8g..+7),
//                   B = Q^T (column = row c of a row block; held in
//                   registers); lane l gets tokens 4g..4g+3 of row c.
//   O^T += Vt · P   v_mfma_f32_16x16x32_bf16 over 32 tokens (two 16-token
//                   blocks b0, b1): k-slot 8g+j is token 16*b0+4g+j (j < 4)
//                   or 16*b1+4g+j-4, so B = P is the lane's own eight
//                   probabilities and A = two 8-byte runs of a Vt row.
//                   Lane l accumulates value columns 16t+4g..+3 of row c.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "device_util.hpp"
#include "kernels.hpp"

namespace pkv {
namespace {

constexpr int kTok = 16;                 // tokens per cache block
constexpr int kTile = 64;                // tokens per K/V tile
constexpr int kWaves = 4;
constexpr int kRB = 4;                   // 16-row blocks per wave
constexpr int kRowsWG = kWaves * kRB * 16;

template <int D>
struct PrefillShape {
  static constexpr int kRow = D + 8;                     // K row, bf16 elements
  static constexpr int vRow = kTile + 4;                 // Vt row, bf16 elements
  static constexpr int kElems = kTile * kRow;
  static constexpr int vElems = D * vRow;
  static constexpr size_t bytes = static_cast<size_t>(kElems + vElems) * 2;
};

template <int D>
__device__ __forceinline__ void write_nan_rows(const PrefillParams& p, int q0, int m, int row_lo, int row_hi,
                                               int kvh) {
  __bf16* out = static_cast<__bf16*>(p.out);
  for (int r = row_lo + static_cast<int>(threadIdx.x) / (D / 8); r < row_hi; r += 256 / (D / 8)) {
    const int qi = r / p.G, g = r - (r / p.G) * p.G;
    if (qi >= m) continue;
    __bf16* o = out + (static_cast<size_t>(q0 + qi) * p.Hq + kvh * p.G + g) * D + (threadIdx.x % (D / 8)) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(NAN);
  }
}

template <int D>
__global__ __launch_bounds__(256) void prefill_bf16(PrefillParams p) {
  using Sh = PrefillShape<D>;
  constexpr int KC = D / 32;             // QK k-steps
  constexpr int VT = D / 16;             // value-column tiles
  extern __shared__ __bf16 lds[];
  __bf16* Kl = lds;
  __bf16* Vl = lds + Sh::kElems;

  const int s = blockIdx.y;
  const int kvh = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;

  const int q0 = p.query_start[s];
  const int m = p.query_start[s + 1] - q0;
  const int n = p.seq_lens[s];
  const int G = p.G;
  if (m < 1) return;
  const int tiles = (m * G + kRowsWG - 1) / kRowsWG;
  if (static_cast<int>(blockIdx.x) >= tiles) return;
  const int tile = tiles - 1 - static_cast<int>(blockIdx.x);   // the longest (last) rows first
  const int wg_row0 = tile * kRowsWG;
  const int wg_row1 = min(m * G, wg_row0 + kRowsWG);
  if (n < m || n > p.max_seq_len || n > p.max_blocks * kTok) {
    write_nan_rows<D>(p, q0, m, wg_row0, wg_row1, kvh);
    return;
  }
  const int c = n - m;                                         // cached context

  // Positions covered by the workgroup and by this wave.
  const int wg_pos_lo = c + wg_row0 / G;
  const int wg_pos_hi = c + (wg_row1 - 1) / G;
  const int w_row0 = wg_row0 + wave * kRB * 16;
  const int w_row_last = min(wg_row1, w_row0 + kRB * 16) - 1;
  const bool wave_active = w_row0 < wg_row1;
  const int w_pos_lo = c + w_row0 / G;
  const int w_pos_hi = c + max(w_row0, w_row_last) / G;

  // Rows of this lane (one per row block) and their Q^T operands.
  int pos[kRB];
  bool row_ok[kRB];
  bf16x8 qreg[kRB][KC];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int r = w_row0 + rb * 16 + c16;
    const int qi = r / G, g = r - (r / G) * G;
    row_ok[rb] = r < wg_row1;
    pos[rb] = row_ok[rb] ? c + qi : wg_pos_hi;
    const __bf16* q = static_cast<const __bf16*>(p.q) +
                      (static_cast<size_t>(q0 + (row_ok[rb] ? qi : 0)) * p.Hq + kvh * G + (row_ok[rb] ? g : 0)) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 v = {0, 0, 0, 0};
      if (row_ok[rb]) v = *reinterpret_cast<const u32x4*>(q + 32 * kc + 8 * g4);
      qreg[rb][kc] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Key range of the workgroup: [key_lo, wg_pos_hi].
  const int key_lo = p.window > 0 ? max(0, wg_pos_lo - p.window + 1) : 0;
  const int kt_first = key_lo / kTile;
  const int kt_last = wg_pos_hi / kTile;

  f32x4 acc[kRB][VT];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int t = 0; t < VT; ++t) acc[rb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[kRB], l_run[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }

  const size_t tile_elems = static_cast<size_t>(kTok) * D;                // one (block, head) tile
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * tile_elems;
  const __bf16* kc_base = static_cast<const __bf16*>(p.k_cache) + kvh * tile_elems;
  const __bf16* vc_base = static_cast<const __bf16*>(p.v_cache) + kvh * tile_elems;
  const int32_t* table = p.block_tables + static_cast<size_t>(s) * p.max_blocks;

  for (int kt = kt_first; kt <= kt_last; ++kt) {
    // ---- gather the tile's four blocks into LDS (all 256 threads) ----
    __syncthreads();                                   // the previous tile is consumed
    const int tb = tid >> 6;                           // block of the tile this thread copies
    const int bi = kt * (kTile / kTok) + tb;           // logical block
    const int tok0 = bi * kTok;
    bool bad = false;
    const bool needed = tok0 < n && tok0 + kTok > key_lo;
    int b = 0;
    if (needed) {
      b = table[bi];
      bad = static_cast<unsigned>(b) >= static_cast<unsigned>(p.num_blocks);
    }
    if (__syncthreads_or(bad)) {
      write_nan_rows<D>(p, q0, m, wg_row0, wg_row1, kvh);
      return;
    }
    const __bf16* kb = kc_base + static_cast<size_t>(b) * blk_stride;
    const __bf16* vb = vc_base + static_cast<size_t>(b) * blk_stride;
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      const int ci = lane + 64 * u;                    // 16-byte chunk of the block's K / V tile
      u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (needed) {
        kv = *reinterpret_cast<const u32x4*>(kb + static_cast<size_t>(ci) * 8);
        vv = *reinterpret_cast<const u32x4*>(vb + static_cast<size_t>(ci) * 8);
      }
      // K chunk ci = (head-dim chunk ci / 16, token ci % 16)
      const int kt_tok = ci & 15, kt_c = ci >> 4;
      if (tok0 + kt_tok >= n) kv = u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(Kl + (tb * kTok + kt_tok) * Sh::kRow + 8 * kt_c) = kv;
      // V chunk ci = (value column ci / 2, tokens 8 (ci % 2) .. +7)
      const int ve = ci >> 1, vh = ci & 1;
      const int vtok = tok0 + 8 * vh;
      if (vtok + 8 > n) {
        // zero the tokens at or past the sequence end (free or poisoned slots)
        uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (vtok + 2 * e < n) ? 0x0000FFFFu : 0u;
          const uint32_t hi = (vtok + 2 * e + 1 < n) ? 0xFFFF0000u : 0u;
          w[e] &= lo | hi;
        }
        vv = u32x4{w[0], w[1], w[2], w[3]};
      }
      *reinterpret_cast<u32x2*>(Vl + ve * Sh::vRow + tb * kTok + 8 * vh) = u32x2{vv.x, vv.y};
      *reinterpret_cast<u32x2*>(Vl + ve * Sh::vRow + tb * kTok + 8 * vh + 4) = u32x2{vv.z, vv.w};
    }
    __syncthreads();

    // ---- this wave's rows against the tile ----
    const int t_lo = kt * kTile, t_hi = t_lo + kTile - 1;
    if (!wave_active || t_lo > w_pos_hi) continue;
    if (p.window > 0 && t_hi < w_pos_lo - p.window + 1) continue;
    const bool masked = t_hi > w_pos_lo || (p.window > 0 && t_lo < w_pos_hi - p.window + 1);

    f32x4 S[kRB][4];
#pragma unroll
    for (int tb2 = 0; tb2 < 4; ++tb2) {
      bf16x8 ka[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        ka[kc] = *reinterpret_cast<const bf16x8*>(Kl + (tb2 * kTok + c16) * Sh::kRow + 32 * kc + 8 * g4);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kc], qreg[rb][kc], sc, 0, 0, 0);
        S[rb][tb2] = sc;
      }
    }

    bf16x8 pb[kRB][2];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      float x[4][4];
#pragma unroll
      for (int tb2 = 0; tb2 < 4; ++tb2)
#pragma unroll
        for (int j = 0; j < 4; ++j) x[tb2][j] = S[rb][tb2][j] * p.scale_log2;
      if (masked) {
        const int lo = p.window > 0 ? pos[rb] - p.window + 1 : 0;
#pragma unroll
        for (int tb2 = 0; tb2 < 4; ++tb2)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = t_lo + tb2 * kTok + 4 * g4 + j;
            if (t > pos[rb] || t < lo) x[tb2][j] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int tb2 = 0; tb2 < 4; ++tb2)
        mx = fmaxf(mx, fmaxf(fmaxf(x[tb2][0], x[tb2][1]), fmaxf(x[tb2][2], x[tb2][3])));
      mx = max_over_rows(mx);
      const float m_new = fmaxf(m_run[rb], mx);
      if (__any(m_new > m_run[rb])) {
        // Rows of one block have different masks: a row whose maximum did not
        // grow keeps alpha = 1 (also when it has seen no key yet, m = -inf).
        const float alpha = m_new > m_run[rb] ? exp2_fast(m_run[rb] - m_new) : 1.f;
        l_run[rb] *= alpha;
#pragma unroll
        for (int t = 0; t < VT; ++t) acc[rb][t] *= alpha;
        m_run[rb] = m_new;
      }
      // A row with no key in this tile yet keeps m = -inf: its terms are 0.
      const float m_use = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
      float ps = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const __bf16 e = static_cast<__bf16>(exp2_fast(x[2 * ks + (j >> 2)][j & 3] - m_use));
          v[j] = e;
          ps += static_cast<float>(e);
        }
        pb[rb][ks] = v;
      }
      l_run[rb] += ps;
    }

#pragma unroll
    for (int t = 0; t < VT; ++t) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const __bf16* vr = Vl + (16 * t + c16) * Sh::vRow + 32 * ks + 4 * g4;
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(vr);
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(vr + kTok);
        const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y});
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          acc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rb][ks], acc[rb][t], 0, 0, 0);
      }
    }
  }

  if (!wave_active) return;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float l_tot = sum_over_rows(l_run[rb]);
    if (!row_ok[rb]) continue;
    const int r = w_row0 + rb * 16 + c16;
    const int qi = r / G, g = r - (r / G) * G;
    const float inv = 1.f / l_tot;
    __bf16* o = static_cast<__bf16*>(p.out) + (static_cast<size_t>(q0 + qi) * p.Hq + kvh * G + g) * D + 4 * g4;
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      bf16x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = static_cast<__bf16>(acc[rb][t][j] * inv);
      *reinterpret_cast<bf16x4*>(o + 16 * t) = v;
    }
  }
}

}  // namespace

bool prefill_shape_supported(int head_dim, int block_size) {
  return block_size == kTok && (head_dim == 64 || head_dim == 128);
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.S <= 0 || p.max_query_len <= 0) return hipSuccess;
  const long long tiles = (static_cast<long long>(p.max_query_len) * p.G + kRowsWG - 1) / kRowsWG;
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(p.S), static_cast<unsigned>(p.Hkv));
  if (p.d == 128)
    hipLaunchKernelGGL(prefill_bf16<128>, grid, dim3(256), PrefillShape<128>::bytes, stream, p);
  else if (p.d == 64)
    hipLaunchKernelGGL(prefill_bf16<64>, grid, dim3(256), PrefillShape<64>::bytes, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
