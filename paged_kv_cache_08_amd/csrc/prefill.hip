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
// One workgroup = 8 waves = 256 query rows of one (sequence, KV head).  A row
// is one (query position, query head of the group) pair, position-major, so
// the group's heads share every K/V tile.  Each wave owns 32 rows (two
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
constexpr int kTile = 64;                // tokens per K/V tile (four blocks)

// 8 waves of 32 rows: 166 registers, no accumulator traffic between AGPRs
// and VGPRs, two waves per SIMD so one wave's softmax overlaps another's
// MFMAs (4 waves of 64 rows measured 40% slower).
#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 8
#endif
#ifndef PKV_PREFILL_RB
#define PKV_PREFILL_RB 2
#endif
constexpr int kWaves = PKV_PREFILL_WAVES;   // waves per workgroup
constexpr int kRB = PKV_PREFILL_RB;         // 16-row blocks per wave
constexpr int kRowsWG = kWaves * kRB * 16;

// LDS holds two tiles (double buffer).  A tile is four K block tiles in the
// cache's own order ([D/8][16 tokens][8]: a lane's A operand is one 16-byte
// chunk, 16 lanes read 16 consecutive chunks) and four V block tiles stored
// half-major ([2 token halves][D columns][8 tokens]: 16 lanes read 8 bytes
// from 16 consecutive chunks).  Both are filled by direct global-to-LDS
// loads (lane i writes bytes 16i..16i+15 of each 1 KiB run).
template <int D>
struct PrefillShape {
  static constexpr int blk = kTok * D;                   // bf16 elements of one block tile
  static constexpr int tile = 8 * blk;                   // K and V of four blocks
  static constexpr size_t bytes = static_cast<size_t>(2 * tile) * 2;
};

template <int D>
__device__ __forceinline__ void write_nan_rows(const PrefillParams& p, int q0, int m, int row_lo, int row_hi,
                                               int kvh) {
  __bf16* out = static_cast<__bf16*>(p.out);
  constexpr int per_row = D / 8;
  for (int r = row_lo + static_cast<int>(threadIdx.x) / per_row; r < row_hi; r += kWaves * 64 / per_row) {
    const int qi = r / p.G, g = r - (r / p.G) * p.G;
    if (qi >= m) continue;
    __bf16* o = out + (static_cast<size_t>(q0 + qi) * p.Hq + kvh * p.G + g) * D + (threadIdx.x % per_row) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(NAN);
  }
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void prefill_bf16(PrefillParams p) {
  using Sh = PrefillShape<D>;
  constexpr int KC = D / 32;             // QK k-steps
  constexpr int VT = D / 16;             // value-column tiles
  constexpr int kPieces = 8 / kWaves;    // block tiles (K or V) each wave loads per tile
  extern __shared__ __bf16 lds[];

  // blockIdx.x = (sequence, KV head), blockIdx.y = row tile counted from the
  // last one: workgroups are dispatched x first, so the longest causal row
  // tiles of every (sequence, KV head) start before any shorter one.
  const int s = blockIdx.x / p.Hkv;
  const int kvh = blockIdx.x - s * p.Hkv;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;

  const int q0 = p.query_start[s];
  const int m = p.query_start[s + 1] - q0;
  const int n = p.seq_lens[s];
  const int G = p.G;
  if (m < 1) return;
  const int tiles = (m * G + kRowsWG - 1) / kRowsWG;
  if (static_cast<int>(blockIdx.y) >= tiles) return;
  const int tile = tiles - 1 - static_cast<int>(blockIdx.y);   // the longest (last) rows first
  const int wg_row0 = tile * kRowsWG;
  const int wg_row1 = min(m * G, wg_row0 + kRowsWG);
  if (n < m || n > p.max_seq_len || n > p.max_blocks * kTok) {
    write_nan_rows<D>(p, q0, m, wg_row0, wg_row1, kvh);
    return;
  }
  const int c = n - m;                                         // cached context

  const int wg_pos_lo = c + wg_row0 / G;
  const int wg_pos_hi = c + (wg_row1 - 1) / G;
  const int w_row0 = wg_row0 + wave * kRB * 16;
  const int w_row_last = min(wg_row1, w_row0 + kRB * 16) - 1;
  const bool wave_active = w_row0 < wg_row1;
  const int w_pos_lo = c + w_row0 / G;
  const int w_pos_hi = c + max(w_row0, w_row_last) / G;

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

  const int key_lo = p.window > 0 ? max(0, wg_pos_lo - p.window + 1) : 0;
  const int kt_first = key_lo / kTile;
  const int kt_last = wg_pos_hi / kTile;

  const size_t tile_elems = static_cast<size_t>(kTok) * D;
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * tile_elems;
  const __bf16* kc_base = static_cast<const __bf16*>(p.k_cache) + kvh * tile_elems;
  const __bf16* vc_base = static_cast<const __bf16*>(p.v_cache) + kvh * tile_elems;
  const int32_t* table = p.block_tables + static_cast<size_t>(s) * p.max_blocks;
  bool bad = false;                                            // wave-uniform

  // Start the loads of tile kt into buffer `buf`: this wave's pieces.
  auto issue = [&](int kt, int buf) {
    __bf16* base = lds + buf * Sh::tile;
#pragma unroll
    for (int pc = 0; pc < kPieces; ++pc) {
      const int piece = wave * kPieces + pc;                   // 0..3: K of block piece; 4..7: V of block piece-4
      const bool is_v = piece >= 4;
      const int tb = piece & 3;
      const int bi = kt * (kTile / kTok) + tb;
      const int tok0 = bi * kTok;
      __bf16* dst = base + (is_v ? 4 * Sh::blk : 0) + tb * Sh::blk;
      const bool needed = tok0 < n && tok0 + kTok > key_lo;
      int b = needed ? table[bi] : 0;
      if (static_cast<unsigned>(b) >= static_cast<unsigned>(p.num_blocks)) {
        bad = true;
        b = 0;
      }
      if (!needed) {                                           // nothing to read: zeros
#pragma unroll
        for (int u = 0; u < D / 32; ++u)
          *reinterpret_cast<u32x4*>(dst + (64 * u + lane) * 8) = u32x4{0, 0, 0, 0};
        continue;
      }
      const __bf16* src = (is_v ? vc_base : kc_base) + static_cast<size_t>(b) * blk_stride;
#pragma unroll
      for (int u = 0; u < D / 32; ++u) {
        const int ci = 64 * u + lane;                          // LDS chunk of this lane
        // K keeps the cache order; V chunk ci holds (half ci / D, column ci % D),
        // which is cache chunk 2 * column + half
        const int gi = is_v ? 2 * (ci % D) + ci / D : ci;
        __builtin_amdgcn_global_load_lds(src + static_cast<size_t>(gi) * 8, dst + 64 * u * 8, 16, 0, 0);
      }
    }
  };
  // After this wave's loads of tile kt landed: zero V tokens at or past n
  // (free or poisoned slots) in the block that holds token n - 1.
  auto fix_tail = [&](int kt, int buf) {
#pragma unroll
    for (int pc = 0; pc < kPieces; ++pc) {
      const int piece = wave * kPieces + pc;
      if (piece < 4) continue;
      const int tb = piece & 3;
      const int tok0 = (kt * (kTile / kTok) + tb) * kTok;
      if (tok0 >= n || tok0 + kTok <= n) continue;
      __bf16* dst = lds + buf * Sh::tile + 4 * Sh::blk + tb * Sh::blk;
      for (int e = lane; e < D; e += 64)
        for (int t = n - tok0; t < kTok; ++t) dst[((t >> 3) * D + e) * 8 + (t & 7)] = static_cast<__bf16>(0.f);
    }
  };

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

  issue(kt_first, 0);
  int buf = 0;
  for (int kt = kt_first; kt <= kt_last; ++kt) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    fix_tail(kt, buf);
    __syncthreads();                   // tile kt is in LDS; tile kt-1 is consumed by every wave
    if (kt < kt_last) issue(kt + 1, buf ^ 1);
    const __bf16* Kt = lds + buf * Sh::tile;
    const __bf16* Vt = Kt + 4 * Sh::blk;
    buf ^= 1;
    if (!wave_active) continue;

#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {                           // 32-token halves of the tile
      const int t_lo = kt * kTile + 32 * hh, t_hi = t_lo + 31;
      if (t_lo > w_pos_hi) break;
      if (p.window > 0 && t_hi < w_pos_lo - p.window + 1) continue;
      const bool masked = t_hi > w_pos_lo || (p.window > 0 && t_lo < w_pos_hi - p.window + 1);

      f32x4 S[kRB][2];
#pragma unroll
      for (int tl = 0; tl < 2; ++tl) {
        const __bf16* kb = Kt + (2 * hh + tl) * Sh::blk;
        bf16x8 ka[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          ka[kc] = *reinterpret_cast<const bf16x8*>(kb + ((4 * kc + g4) * kTok + c16) * 8);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kc], qreg[rb][kc], sc, 0, 0, 0);
          S[rb][tl] = sc;
        }
      }

      // Scores stay in raw units; exp2(x * scale_log2 - m * scale_log2) is
      // one fused multiply-add per score (scale_log2 > 0 keeps the max).
      bf16x8 pb[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = S[rb][j >> 2][j & 3];
        if (masked) {
          const int lo = p.window > 0 ? pos[rb] - p.window + 1 : 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int t = t_lo + (j >> 2) * kTok + 4 * g4 + (j & 3);
            if (t > pos[rb] || t < lo) x[j] = -INFINITY;
          }
        }
        float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        mx = max_over_rows(mx);
        const float m_new = fmaxf(m_run[rb], mx);
        if (__any(m_new > m_run[rb])) {
          // Rows of one block have different masks: a row whose maximum did
          // not grow keeps alpha = 1 (also with no key yet, m = -inf).
          const float alpha = m_new > m_run[rb] ? exp2_fast((m_run[rb] - m_new) * p.scale_log2) : 1.f;
          l_run[rb] *= alpha;
#pragma unroll
          for (int t = 0; t < VT; ++t) acc[rb][t] *= alpha;
          m_run[rb] = m_new;
        }
        // A row with no key yet keeps m = -inf: its terms are 0.
        const float neg_m = m_run[rb] == -INFINITY ? 0.f : -m_run[rb] * p.scale_log2;
        float ps = 0.f;
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float e = exp2_fast(__builtin_fmaf(x[j], p.scale_log2, neg_m));
          v[j] = static_cast<__bf16>(e);
          ps += e;
        }
        pb[rb] = v;
        l_run[rb] += ps;
      }

      const __bf16* v0 = Vt + (2 * hh) * Sh::blk + ((g4 >> 1) * D + c16) * 8 + 4 * (g4 & 1);
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(v0 + 16 * t * 8);
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(v0 + Sh::blk + 16 * t * 8);
        const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y});
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          acc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rb], acc[rb][t], 0, 0, 0);
      }
    }
  }

  if (__syncthreads_or(bad)) {
    write_nan_rows<D>(p, q0, m, wg_row0, wg_row1, kvh);
    return;
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
  dim3 grid(static_cast<unsigned>(p.S * p.Hkv), static_cast<unsigned>(tiles));
  if (p.d == 128)
    hipLaunchKernelGGL(prefill_bf16<128>, grid, dim3(kWaves * 64), PrefillShape<128>::bytes, stream, p);
  else if (p.d == 64)
    hipLaunchKernelGGL(prefill_bf16<64>, grid, dim3(kWaves * 64), PrefillShape<64>::bytes, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
