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
// One workgroup = 12 waves = 384 query rows of one (sequence, KV head).  A row
// is one (query position, query head of the group) pair, position-major, so
// the group's heads share every K/V tile.  Each wave owns 32 rows (two
// 16-row blocks).  K/V are streamed in tiles of 64 tokens (four 16-token
// blocks gathered through the block table) into LDS (see PrefillShape).
// Per 32-token half tile (cache blocks b0, b1) and wave, with lane
// l = 16*g + c (g = l/16, c = l%16), lane group g owns the eight tokens
// tau(g, j) = 16*(g/2) + 8*(g%2) + j, j = 0..7 (block g/2, half g%2):
//   S^T = K · Q^T   two v_mfma_f32_16x16x32_bf16 (m = 0, 1) per head-dim
//                   slice, A = K rows permuted so that output row 4g+i is
//                   token tau(g, 4m+i) (A row c = token 16*(c/8) +
//                   8*((c/4)%2) + 4m + c%4, k = head-dim values 32kc+8g..+7),
//                   B = Q^T (column = row c of a row block; in registers);
//                   lane l gets tokens tau(g, 4m..4m+3) of row c.
//   O^T += Vt · P   v_mfma_f32_16x16x32_bf16 over the 32 tokens, k-slot
//                   8g+j = token tau(g, j): B = P is the lane's own eight
//                   probabilities and A is one 16-byte chunk of V (value
//                   column 16t+c, half g%2 of block g/2).
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

// 12 waves of 32 rows: 168 registers, no accumulator traffic between AGPRs
// and VGPRs, three waves per SIMD so that the others' MFMAs overlap one
// wave's softmax, and each K/V tile in LDS serves 384 rows.  (8 waves, two
// per SIMD: 7-14% slower; 4 waves of 64 rows: 40% slower.)  The workgroup's
// LDS ring (three tiles, 99 KiB at d = 128) allows one workgroup per CU.
#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 12
#endif
#ifndef PKV_PREFILL_RB
#define PKV_PREFILL_RB 2
#endif
#ifndef PKV_PREFILL_BUFS
#define PKV_PREFILL_BUFS 3
#endif
constexpr int kWaves = PKV_PREFILL_WAVES;   // waves per workgroup
constexpr int kBufs = PKV_PREFILL_BUFS;     // K/V tiles in LDS: loads run kBufs - 1 tiles ahead
constexpr int kRB = PKV_PREFILL_RB;         // 16-row blocks per wave
constexpr int kRowsWG = kWaves * kRB * 16;

// LDS holds kBufs tiles (a ring: tile kt + kBufs - 1 is loaded while tile
// kt is consumed).  A tile is four K block tiles in the cache's own order
// ([D/8][16 tokens][8]: a lane's A operand is one 16-byte chunk) and four V
// block tiles stored half-major ([2 token halves][D columns][8 tokens]: a
// lane's A operand is one 16-byte chunk, 16 lanes read 16 consecutive
// chunks).  Block tiles sit 64 bytes apart beyond their 4 KiB (D = 128), so
// the 16 lanes of a K read (eight tokens from each block of a pair) fall on
// distinct banks.  Both arrive by direct global-to-LDS loads (lane i writes
// bytes 16i..16i+15 of each 1 KiB run) in the cache's order; the wave that
// loaded a V block tile then reorders it in place (the cache keeps four
// tokens of a column together, [4 token groups][D/4][4 columns][4 tokens]).
template <int D>
struct PrefillShape {
  static constexpr int blk = kTok * D;                   // bf16 elements of one block tile
  static constexpr int blk_stride = blk + 32;            // + 64 bytes between block tiles
  static constexpr int tile = 8 * blk_stride;            // K and V of four blocks
  static constexpr size_t bytes = static_cast<size_t>(kBufs * tile) * 2;
};

template <int D>
__device__ __forceinline__ void write_nan_rows(const PrefillParams& p, int q0, int m, int row_lo, int row_hi,
                                               int kvh) {
  uint16_t* out = static_cast<uint16_t*>(p.out);        // bf16 bit patterns: 0x7FC0 is a quiet NaN
  constexpr int per_row = D / 8;
  for (int r = row_lo + static_cast<int>(threadIdx.x) / per_row; r < row_hi; r += kWaves * 64 / per_row) {
    const int qi = r / p.G, g = r - (r / p.G) * p.G;
    if (qi >= m) continue;
    uint16_t* o = out + (static_cast<size_t>(q0 + qi) * p.Hq + kvh * p.G + g) * D + (threadIdx.x % per_row) * 8;
    *reinterpret_cast<u32x4*>(o) = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  }
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void prefill_bf16(PrefillParams p) {
  using Sh = PrefillShape<D>;
  constexpr int KC = D / 32;             // QK k-steps
  constexpr int VT = D / 16;             // value-column tiles
  static_assert(kWaves >= 8, "waves 0..7 load the eight block tiles (K and V of four blocks) of a tile");
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

  // The Q loads complete here, before the tile loop: read first inside the
  // loop, they would make the compiler wait for every load in flight there
  // (the next tiles' loads included) on each tile.
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, qreg[rb][kc])));

  const int key_lo = p.window > 0 ? max(0, wg_pos_lo - p.window + 1) : 0;
  const int kt_first = key_lo / kTile;
  const int kt_last = wg_pos_hi / kTile;

  const size_t tile_elems = static_cast<size_t>(kTok) * D;
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * tile_elems;
  const __bf16* kc_base = static_cast<const __bf16*>(p.k_cache) + kvh * tile_elems;
  const __bf16* vc_base = static_cast<const __bf16*>(p.v_cache) + kvh * tile_elems;
  const int32_t* table = p.block_tables + static_cast<size_t>(s) * p.max_blocks;
  bool bad = false;                                            // wave-uniform

  // Waves 0..7 load one piece of every tile: the K (waves 0..3) or V (waves
  // 4..7) block tile of block slot tb = wave % 4; further waves only compute.
  // Block ids are read with scalar loads (the table is read-only here): they
  // complete under lgkmcnt, so no table read sits among the tile loads that
  // vmcnt counts.
  const bool loader = wave < 8;
  const int tb = wave & 3;
  const bool is_v = wave >= 4;
  const __attribute__((address_space(4))) int32_t* table_s =
      (const __attribute__((address_space(4))) int32_t*)table;

  // Start the loads of tile kt into buffer `buf`: this wave's piece.
  // Returns whether a global load was issued (a piece outside the sequence
  // or window is zero-filled instead).
  auto issue = [&](int kt, int buf) {
    if (!loader) return false;
    const int bi = kt * (kTile / kTok) + tb;
    const int tok0 = bi * kTok;
    __bf16* dst = lds + buf * Sh::tile + (is_v ? 4 * Sh::blk_stride : 0) + tb * Sh::blk_stride;
    const bool needed = tok0 < n && tok0 + kTok > key_lo;
    int b = needed ? table_s[bi] : 0;
    if (static_cast<unsigned>(b) >= static_cast<unsigned>(p.num_blocks)) {
      bad = true;
      b = 0;
    }
    if (!needed) {                                             // nothing to read: zeros
#pragma unroll
      for (int u = 0; u < D / 32; ++u)
        *reinterpret_cast<u32x4*>(dst + (64 * u + lane) * 8) = u32x4{0, 0, 0, 0};
      return false;
    }
    const __bf16* src = (is_v ? vc_base : kc_base) + static_cast<size_t>(b) * blk_stride;
    const int t_end = n - tok0;                                // written slots of this block (>= 1)
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      const int ci = 64 * u + lane;                            // LDS chunk of this lane
      // Both land in the cache order, except that a K slot past the end (K
      // chunk ci holds token ci % 16) is read from slot 0 of the same
      // head-dimension chunk (a written token) instead of whatever the free
      // slot holds.
      const int gi = is_v ? ci : ((ci & 15) < t_end ? ci : (ci & ~15));
      __builtin_amdgcn_global_load_lds(src + static_cast<size_t>(gi) * 8, dst + 64 * u * 8, 16, 0, 0);
    }
    return true;
  };
  // After this wave's loads of tile kt landed, a V loader puts its block
  // tile into the half-major order.  In the cache order, 16-byte chunk
  // (D/2) u + p holds columns 2p and 2p + 1 of tokens 4u .. 4u + 3; the
  // half-major chunk D h + c holds tokens 8h .. 8h + 7 of column c.  So the
  // chunks of token groups 2h and 2h + 1 of one column pair give the two
  // half-major chunks of those columns.  Every chunk is read before any is
  // written (the writes use the reads), so the reorder works in place.
  // Tokens at or past n (free slots, which may hold anything, NaN included)
  // become zeros; with the K redirect in issue(), every value the matrix
  // cores read is a cached token or zero.
  auto reorder_v = [&](int kt, int buf) {
    if (!loader || !is_v) return;
    const int tok0 = (kt * (kTile / kTok) + tb) * kTok;
    if (tok0 >= n || tok0 + kTok <= key_lo) return;       // zero-filled
    u32x4* blk = reinterpret_cast<u32x4*>(lds + buf * Sh::tile + 4 * Sh::blk_stride + tb * Sh::blk_stride);
    const int t_end = n - tok0;
    constexpr int kItems = D / 64;                          // (half, column pair) items per lane
    u32x4 a[kItems], b[kItems];
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
      const int i = lane + 64 * k, h = i / (D / 2), pc = i % (D / 2);
      a[k] = blk[h * D + pc];                               // token group 2h
      b[k] = blk[h * D + D / 2 + pc];                       // token group 2h + 1
    }
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
      const int i = lane + 64 * k, h = i / (D / 2), pc = i % (D / 2);
      uint32_t keep[4];                                     // 16-bit lanes of token 8h + 2j (+1) kept
#pragma unroll
      for (int j = 0; j < 4; ++j)
        keep[j] = (8 * h + 2 * j < t_end ? 0xFFFFu : 0u) | (8 * h + 2 * j + 1 < t_end ? 0xFFFF0000u : 0u);
      blk[h * D + 2 * pc] = u32x4{a[k].x & keep[0], a[k].y & keep[1], b[k].x & keep[2], b[k].y & keep[3]};
      blk[h * D + 2 * pc + 1] = u32x4{a[k].z & keep[0], a[k].w & keep[1], b[k].z & keep[2], b[k].w & keep[3]};
    }
  };

  f32x4 acc[kRB][VT];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int t = 0; t < VT; ++t) acc[rb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Per 16-row block: running maxima (raw score units), -m * scale_log2 for
  // the exp's fused multiply-add, and the maxima at which the next rescale is
  // due.  Row sums come from one more MFMA per half tile, of the
  // probabilities against an all-ones A operand: every element of acc_l is
  // its row's sum of the same bf16 probabilities that weight V.
  f32x4 acc_l[kRB];
  float m_run[kRB], neg_ms[kRB], thr[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    acc_l[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[rb] = -INFINITY;
    neg_ms[rb] = 0.f;
    thr[rb] = -INFINITY;
  }
  // Conditional rescale: the running maxima move only when some row's
  // maximum grew by more than 8 in exp2 units.  Until then a term
  // exp2((x - m) * scale_log2) is at most 2^8, which the fp32 sums and the
  // bf16 probabilities hold with the same relative precision as terms below
  // 1; the final division by the sum cancels the offset.
  const float thr_gap = 8.f / p.scale_log2;
  bf16x8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = static_cast<__bf16>(1.f);

  // Loads in flight are this wave's pieces of the next kBufs - 1 tiles; a
  // loading wave issues the same piece for every tile, so a wait for all but
  // the younger tiles' loads (one piece of D/32 loads per wave and tile, when
  // it was loaded and not zero-filled) leaves exactly tile kt complete.  The
  // barrier after it makes every piece visible to every wave.
  static_assert(kBufs == 3, "the wait counts below assume three buffers");
  constexpr int kLoadsPerTile = D / 32;
  bool ahead = false;                  // whether tile kt + 1 issued loads (issued before the wait below)
  issue(kt_first, 0);
  if (kt_first < kt_last) ahead = issue(kt_first + 1, 1);
  int buf = 0;
  for (int kt = kt_first; kt <= kt_last; ++kt) {
    if (ahead) {
      if constexpr (kLoadsPerTile == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    reorder_v(kt, buf);
    // Tile kt is in LDS (every wave waited for its own loads of it above,
    // and for its LDS writes here); tile kt-1 is consumed by every wave.  A
    // plain barrier: __syncthreads() would also wait for the loads of the
    // next tile, which must stay in flight.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    ahead = kt + 2 <= kt_last ? issue(kt + 2, buf == 0 ? 2 : buf - 1) : false;
    const __bf16* Kt = lds + buf * Sh::tile;
    const __bf16* Vt = Kt + 4 * Sh::blk_stride;
    buf = buf == kBufs - 1 ? 0 : buf + 1;
    if (!wave_active) continue;

#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {                           // 32-token halves of the tile
      const int t_lo = kt * kTile + 32 * hh, t_hi = t_lo + 31;
      if (t_lo > w_pos_hi) break;
      if (p.window > 0 && t_hi < w_pos_lo - p.window + 1) continue;
      const bool masked = t_hi > w_pos_lo || (p.window > 0 && t_lo < w_pos_hi - p.window + 1);
      f32x4 S[kRB][2];
      // A row c of MFMA mm: token 8*((c/4)%2) + 4*mm + c%4 of block 2*hh + c/8
      const __bf16* kb = Kt + (2 * hh + (c16 >> 3)) * Sh::blk_stride + (8 * ((c16 >> 2) & 1) + (c16 & 3)) * 8;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        bf16x8 ka[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          ka[kc] = *reinterpret_cast<const bf16x8*>(kb + ((4 * kc + g4) * kTok + 4 * mm) * 8);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kc], qreg[rb][kc], sc, 0, 0, 0);
          S[rb][mm] = sc;
        }
      }

      // Scores stay in raw units; exp2(x * scale_log2 - m * scale_log2) is
      // one fused multiply-add per score (scale_log2 > 0 keeps the max).
      bf16x8 pb[kRB];
      const int tok_x0 = t_lo + 16 * (g4 >> 1) + 8 * (g4 & 1);        // token of x[0]; x[j] is tok_x0 + j
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = S[rb][j >> 2][j & 3];
        if (masked) {
          const int hi = pos[rb] - tok_x0;                           // keys j <= hi are at or before the row
          if (p.window > 0) {
            const int lo = pos[rb] - p.window + 1 - tok_x0;          // and j >= lo inside its window
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (j > hi || j < lo) x[j] = -INFINITY;
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (j > hi) x[j] = -INFINITY;
          }
        }
        // IEEE maximum (v_maximum3_f32): the scores are never NaN here (every
        // key the cores read is a cached token or zero), and unlike fmaxf it
        // needs no canonicalisation of the matrix cores' results first.  The
        // eight scores take four three-input maxima when grouped this way.
        // Each lane tests its own maximum against its row's threshold; the
        // row maxima across the row's four lanes are formed only when some
        // score exceeds it (the same maxima, so the same rescale): the
        // softmax issue, not the matrix cores, sets this kernel's pace, and
        // the common path saves the cross-lane steps.
        const float m012 = fmax_ieee(fmax_ieee(x[0], x[1]), x[2]);
        const float m345 = fmax_ieee(fmax_ieee(x[3], x[4]), x[5]);
        float mx = fmax_ieee(fmax_ieee(fmax_ieee(m012, m345), x[6]), x[7]);
        if (__any(mx > thr[rb])) {
          mx = max_over_rows_ieee(mx);
          // Rows of one block have different masks: a row whose maximum did
          // not grow keeps alpha = 1 (also with no key yet, m = -inf).
          const float m_new = fmax_ieee(m_run[rb], mx);
          const float alpha = m_new > m_run[rb] ? exp2_fast((m_run[rb] - m_new) * p.scale_log2) : 1.f;
          acc_l[rb] *= alpha;
#pragma unroll
          for (int t = 0; t < VT; ++t) acc[rb][t] *= alpha;
          m_run[rb] = m_new;
          neg_ms[rb] = m_new == -INFINITY ? 0.f : -m_new * p.scale_log2;   // no key yet: terms are 0
          thr[rb] = m_new + thr_gap;
        }
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = static_cast<__bf16>(exp2_fast(__builtin_fmaf(x[j], p.scale_log2, neg_ms[rb])));
        pb[rb] = v;
      }

      const __bf16* v0 = Vt + (2 * hh + (g4 >> 1)) * Sh::blk_stride + ((g4 & 1) * D + c16) * 8;
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(v0 + 16 * t * 8);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          acc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rb], acc[rb][t], 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        acc_l[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[rb], acc_l[rb], 0, 0, 0);
    }
  }

  if (__syncthreads_or(bad)) {
    write_nan_rows<D>(p, q0, m, wg_row0, wg_row1, kvh);
    return;
  }
  if (!wave_active) return;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float l_tot = acc_l[rb][0];
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
