// HIP kernels of the paged KV cache for gfx950 (MI355X, wave64, MFMA).
//
//  kv_append      — write each new token's K and V into its slot
//                   («¿Cómo gestiona Paged Attention la caché KV…?», blocks
//                   filled as tokens arrive).
//  copy_blocks    — copy-on-write: a block a writer shares is copied whole,
//                   in every layer («Paged Attention optimiza el uso de
//                   memoria», copy-on-write paragraph).
//  decode_partial — exact attention of every query head over its sequence's
//                   blocks gathered through the block table, blockwise with
//                   running max / sum statistics («Servicio…presupuesto de
//                   memoria» §6), grouped-query heads sharing one KV head
//                   («¿Cuánta memoria reservar para la caché KV?», "Emplear
//                   las cabezas KV"); one wave per (sequence, KV head,
//                   partition of tokens, group of up to 16 query heads).
//  decode_reduce  — merges the partitions' (max, sum, accumulator) triples.
//
// Pool layout of one layer (B = 16 tokens per block for the decode kernels,
// x = 16 bytes / element size):
//   K [block][kv_head][d/x][B][x]    V [block][kv_head][B/4][d/4][4][4]
// The K layout makes one 16-byte load per lane, 64 lanes wide, read 1 KiB of
// contiguous memory that is already in the MFMA A-operand order (lane l:
// token l%16, 16-byte chunk l/16 of the head dimension slice).  The V layout
// keeps runs of four consecutive tokens of one value column together (value
// column j of token o at [o/4][j/4][j%4][o%4]), the PV product's operand
// order, and one token's values within a quarter of the tile: an append
// touches a quarter of the tile's 32-byte sectors.
//
// Scores are kept in base-2 units (score * scale * log2 e) so the softmax
// uses the hardware exp2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "device_util.hpp"
#include "kernels.hpp"

namespace pkv {
namespace {

constexpr int kBlock = 16;   // tokens per block on the decode path
// Partitions are merged in groups of kMergeGroup consecutive ones (numbered
// from 0, the window's first with a window), then the groups: one fixed
// order of operations whatever wave or kernel does each merge.
constexpr int kMergeGroup = 4;
// Blocks in flight per wave.  Two streaming waves on one SIMD do not share
// it evenly: the arbiter favours the older wave (about 3.5 : 1 in measured
// per-wave end times), so with equal work the younger wave streams alone for
// the second half of a launch.  The deep variant keeps twice the bytes in
// flight from a single wave per SIMD (the register file it needs allows no
// second one), which has no partner to wait for.  The bf16 cache uses it
// for batches with at least four partitions per deep wave slot (per the
// caller's length hint): there most bytes stream from HBM.  Smaller batches,
// and batches whose shared prefix is read from the caches, measured as fast
// or faster with two shallow waves per SIMD, which overlap one wave's
// arithmetic with the other's.  The 8-bit cache does more conversion work per
// byte and measured faster with two shallow waves per SIMD throughout.
#ifndef PKV_DEPTH
#define PKV_DEPTH 3
#endif
#ifndef PKV_DEPTH_DEEP
#define PKV_DEPTH_DEEP 5
#endif
#ifndef PKV_DEPTH_FP8
#define PKV_DEPTH_FP8 4
#endif
#ifndef PKV_DEPTH_FP8_DEEP
#define PKV_DEPTH_FP8_DEEP 8
#endif
constexpr int kDepth = PKV_DEPTH;                 // bf16 cache: 12 loads per block
constexpr int kDepthDeep = PKV_DEPTH_DEEP;        // (vmcnt counts at most 63 loads)
constexpr int kDepthFp8 = PKV_DEPTH_FP8;          // 8-bit cache: 6 loads per block
constexpr int kDepthFp8Deep = PKV_DEPTH_FP8_DEEP;

// K/V tiles are read exactly once per decode call: stream them with the
// non-temporal hint so they do not displace reusable lines.  On MI355X this
// lifts a 4 KiB-tile gather from about 6.1 to about 6.85 TB/s.
template <typename T>
__device__ __forceinline__ T stream_load(const T* p) { return __builtin_nontemporal_load(p); }

// ---------------------------------------------------------------------------
// kv_append
// ---------------------------------------------------------------------------
// Slot of token i: given, or the last position of row i of the tables (decode
// step).  -1 when the row or the slot is invalid (the token is skipped).
__device__ __forceinline__ int append_slot(const AppendParams& p, int i) {
  const int B = p.block_size;
  int slot;
  if (p.slots) {
    slot = p.slots[i];
  } else {
    const int len = p.lens[i];
    if (len < 1 || len > p.max_blocks * B) return -1;
    const int b = p.tables[static_cast<size_t>(i) * p.max_blocks + (len - 1) / B];
    if (b < 0 || static_cast<int64_t>(b) * B >= p.num_slots) return -1;
    slot = b * B + (len - 1) % B;
  }
  if (slot < 0 || static_cast<int64_t>(slot) >= p.num_slots) return -1;
  return slot;
}

// Offset of value column e of token slot o in a (block, KV head) V tile
// [B/4][d/4][4][4].
__device__ __forceinline__ size_t v_index(int e, int o, int d) {
  return (static_cast<size_t>(o >> 2) * d + e) * 4 + (o & 3);
}

// One wave writes token o of a (block, KV head) tile: kt / vt point at the
// tile's K and V (layouts [d/x][B][x] and [B/4][d/4][4][4]), ks / vs at the
// token's d values.
template <typename T>
__device__ __forceinline__ void write_token(T* kt, T* vt, const T* ks, const T* vs, int d, int B, int o) {
  constexpr int x = 16 / sizeof(T);
  for (int ch = threadIdx.x; ch < d / x; ch += 64)
    *reinterpret_cast<u32x4*>(kt + (static_cast<size_t>(ch) * B + o) * x) =
        *reinterpret_cast<const u32x4*>(ks + ch * x);
  for (int e = threadIdx.x; e < d; e += 64) vt[v_index(e, o, d)] = vs[e];
}

// Wide form, for 64 / (d / x) heads per wave: one wave takes token i of a
// group of consecutive KV heads.  For K, lane l moves 16-byte chunk
// l % (d / x) of head l / (d / x) of the group; for V, value k * 64 + l of
// the group's rows in step k, so each V store covers 64 consecutive columns
// of one head, as in kv_append_kernel.  The k_new / v_new reads are issued
// before the slot lookup, which they do not depend on.  The same bytes as
// write_token.
template <typename T>
__global__ __launch_bounds__(64) void kv_append_wide_kernel(AppendParams p) {
  constexpr int x = 16 / sizeof(T);
  const int i = blockIdx.x;
  const int d = p.head_dim;
  const int Hkv = p.num_kv_heads;
  const int cpr = d / x;                               // chunks per row, divides 64
  const int h0 = blockIdx.y * (64 / cpr);
  const int l = threadIdx.x;
  const int hk = h0 + l / cpr;
  const int c = l % cpr;
  const size_t row0 = static_cast<size_t>(i) * Hkv;
  const T* ksrc = static_cast<const T*>(p.k_new);
  const T* vsrc = static_cast<const T*>(p.v_new);
  const u32x4 kw = *reinterpret_cast<const u32x4*>(ksrc + (row0 + (hk < Hkv ? hk : 0)) * d + c * x);
  T vals[x];
#pragma unroll
  for (int k = 0; k < x; ++k) {
    const int v = k * 64 + l;
    const int hv = h0 + v / d;
    vals[k] = vsrc[(row0 + (hv < Hkv ? hv : 0)) * d + v % d];
  }
  const int B = p.block_size;
  const int slot = append_slot(p, i);
  if (slot < 0) return;
  const int b = slot / B;
  const int o = slot - b * B;
  const size_t blk = static_cast<size_t>(b) * Hkv;
  if (hk < Hkv)
    *reinterpret_cast<u32x4*>(static_cast<T*>(p.k_cache) + (blk + hk) * d * B + (static_cast<size_t>(c) * B + o) * x) = kw;
#pragma unroll
  for (int k = 0; k < x; ++k) {
    const int v = k * 64 + l;
    const int hv = h0 + v / d;
    if (hv < Hkv) static_cast<T*>(p.v_cache)[(blk + hv) * d * B + v_index(v % d, o, d)] = vals[k];
  }
}

template <typename T>
__global__ __launch_bounds__(64) void kv_append_kernel(AppendParams p) {
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int B = p.block_size;
  const int slot = append_slot(p, i);
  if (slot < 0) return;
  const int d = p.head_dim;
  const int b = slot / B;
  const int o = slot - b * B;
  const T* ks = static_cast<const T*>(p.k_new) + (static_cast<size_t>(i) * p.num_kv_heads + h) * d;
  const T* vs = static_cast<const T*>(p.v_new) + (static_cast<size_t>(i) * p.num_kv_heads + h) * d;
  const size_t tile = (static_cast<size_t>(b) * p.num_kv_heads + h) * static_cast<size_t>(d) * B;
  write_token<T>(static_cast<T*>(p.k_cache) + tile, static_cast<T*>(p.v_cache) + tile, ks, vs, d, B, o);
}

// 8-bit cache: one wave quantises one (token, KV head) row of K and of V.
// scale = amax / 448 (the largest E4M3 magnitude), code = E4M3 nearest to
// value / scale (hardware conversion, round to nearest even); a row of zeros
// gets scale 0 and codes 0.  B = 16; K codes [d/16][B][16]; V codes
// [d/64][B/4][16][4][4] (column 64a + 4c + b of slot 4u + w at [a][u][c][b][w]).
__device__ __forceinline__ uint8_t e4m3_code(float v, float scale) {
  const float y = scale > 0.f ? v / scale : 0.f;
  return static_cast<uint8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0u, false) & 0xFFu);
}

// 8-bit form of write_token: row = block * num_kv_heads + head; quantises
// the token's K and V rows and writes their codes and scales.
__device__ __forceinline__ void write_token_fp8(uint8_t* k_cache, uint8_t* v_cache, float* k_scale, float* v_scale,
                                                size_t row, const __bf16* ks, const __bf16* vs, int d, int o) {
  float ka = 0.f, va = 0.f;
  for (int e = threadIdx.x; e < d; e += 64) {
    ka = fmaxf(ka, fabsf(static_cast<float>(ks[e])));
    va = fmaxf(va, fabsf(static_cast<float>(vs[e])));
  }
  const float kscale = wave_max(ka) / 448.f;
  const float vscale = wave_max(va) / 448.f;
  uint8_t* kd = k_cache + row * kBlock * d;
  uint8_t* vd = v_cache + row * kBlock * d;
  for (int e = threadIdx.x; e < d; e += 64) {
    kd[(e >> 4) * (kBlock * 16) + o * 16 + (e & 15)] = e4m3_code(static_cast<float>(ks[e]), kscale);
    vd[(e >> 6) * 1024 + (o >> 2) * 256 + ((e & 63) >> 2) * 16 + (e & 3) * 4 + (o & 3)] =
        e4m3_code(static_cast<float>(vs[e]), vscale);
  }
  if (threadIdx.x == 0) {
    k_scale[row * kBlock + o] = kscale;
    v_scale[row * kBlock + o] = vscale;
  }
}

__global__ __launch_bounds__(64) void kv_append_fp8_kernel(AppendParams p) {
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int slot = append_slot(p, i);
  if (slot < 0) return;
  const int d = p.head_dim;
  const int b = slot / kBlock;
  const int o = slot - b * kBlock;
  const __bf16* ks = static_cast<const __bf16*>(p.k_new) + (static_cast<size_t>(i) * p.num_kv_heads + h) * d;
  const __bf16* vs = static_cast<const __bf16*>(p.v_new) + (static_cast<size_t>(i) * p.num_kv_heads + h) * d;
  write_token_fp8(static_cast<uint8_t*>(p.k_cache), static_cast<uint8_t*>(p.v_cache), p.k_scale, p.v_scale,
                  static_cast<size_t>(b) * p.num_kv_heads + h, ks, vs, d, o);
}

// Wide 8-bit form for D = 64 or 128: one wave takes token i of a group of
// 512 / D consecutive KV heads, eight values per lane (value k * 64 + l of
// the group's rows in step k, so loads and code stores cover 64 consecutive
// columns of one head).  The k_new / v_new reads are issued before the slot
// lookup.  Same scales and codes as write_token_fp8: the per-row amax is a
// max, whichever lanes take part.
template <int D>
__global__ __launch_bounds__(64) void kv_append_fp8_wide_kernel(AppendParams p) {
  constexpr int G = 512 / D;          // heads per wave
  constexpr int kph = D / 64;         // values per lane and head
  const int i = blockIdx.x;
  const int Hkv = p.num_kv_heads;
  const int h0 = blockIdx.y * G;
  const int l = threadIdx.x;
  const size_t row0 = static_cast<size_t>(i) * Hkv;
  const __bf16* ks = static_cast<const __bf16*>(p.k_new);
  const __bf16* vs = static_cast<const __bf16*>(p.v_new);
  float kv[8], vv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int hv = h0 + k / kph;
    const size_t idx = (row0 + (hv < Hkv ? hv : 0)) * D + (k % kph) * 64 + l;
    kv[k] = static_cast<float>(ks[idx]);
    vv[k] = static_cast<float>(vs[idx]);
  }
  const int slot = append_slot(p, i);
  if (slot < 0) return;
  const int b = slot / kBlock;
  const int o = slot - b * kBlock;
  float ksc = 0.f, vsc = 0.f;         // lane hl < G keeps head hl's scales
#pragma unroll
  for (int hl = 0; hl < G; ++hl) {
    float ka = 0.f, va = 0.f;
#pragma unroll
    for (int j = 0; j < kph; ++j) {
      ka = fmaxf(ka, fabsf(kv[hl * kph + j]));
      va = fmaxf(va, fabsf(vv[hl * kph + j]));
    }
    const float kscale = wave_max(ka) / 448.f;
    const float vscale = wave_max(va) / 448.f;
    if (l == hl) { ksc = kscale; vsc = vscale; }
    const int hv = h0 + hl;
    if (hv >= Hkv) continue;
    const size_t row = static_cast<size_t>(b) * Hkv + hv;
    uint8_t* kd = static_cast<uint8_t*>(p.k_cache) + row * kBlock * D;
    uint8_t* vd = static_cast<uint8_t*>(p.v_cache) + row * kBlock * D;
#pragma unroll
    for (int j = 0; j < kph; ++j) {
      const int e = j * 64 + l;
      kd[(e >> 4) * (kBlock * 16) + o * 16 + (e & 15)] = e4m3_code(kv[hl * kph + j], kscale);
      vd[(e >> 6) * 1024 + (o >> 2) * 256 + ((e & 63) >> 2) * 16 + (e & 3) * 4 + (o & 3)] =
          e4m3_code(vv[hl * kph + j], vscale);
    }
  }
  if (l < G && h0 + l < Hkv) {
    const size_t row = static_cast<size_t>(b) * Hkv + h0 + l;
    p.k_scale[row * kBlock + o] = ksc;
    p.v_scale[row * kBlock + o] = vsc;
  }
}

// ---------------------------------------------------------------------------
// table_upload: block tables and lengths from the pinned staging buffer
// (host memory the GPU reads directly) to the device arrays, in one launch.
// ---------------------------------------------------------------------------
// With `vec` (both table pointers 16-byte aligned) the tables move as
// 16-byte chunks: a quarter of the reads across the host link.
__global__ __launch_bounds__(256) void table_upload_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ tab,
                                                           int64_t n_tab, int32_t* __restrict__ lens, int32_t n_len,
                                                           bool vec) {
  const int64_t n_vec = vec ? n_tab / 4 : 0;          // 16-byte chunks of the tables
  const int64_t tail0 = 4 * n_vec;                    // first value moved singly
  const int64_t total = n_vec + (n_tab - tail0) + n_len;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    if (i < n_vec) {
      reinterpret_cast<u32x4*>(tab)[i] = reinterpret_cast<const u32x4*>(src)[i];
    } else {
      const int64_t j = tail0 + (i - n_vec);
      const int32_t v = src[j];
      if (j < n_tab) tab[j] = v;
      else lens[j - n_tab] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// copy_blocks
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksParams p) {
  const int pair = blockIdx.x;
  const int layer = blockIdx.y;
  const int src = p.pairs[2 * pair];
  const int dst = p.pairs[2 * pair + 1];
  // z: 0 = K, 1 = V, 2 = K scales, 3 = V scales (8-bit pools)
  const int z = blockIdx.z;
  char* base = static_cast<char*>(z == 0 ? p.k[layer] : z == 1 ? p.v[layer] : z == 2 ? p.ks[layer] : p.vs[layer]);
  const int64_t bytes = z < 2 ? p.block_bytes : p.scale_bytes;
  const u32x4* s = reinterpret_cast<const u32x4*>(base + static_cast<int64_t>(src) * bytes);
  u32x4* d = reinterpret_cast<u32x4*>(base + static_cast<int64_t>(dst) * bytes);
  const int64_t n16 = bytes / 16;
  for (int64_t i = threadIdx.x; i < n16; i += 256) d[i] = s[i];
}

// ---------------------------------------------------------------------------
// decode: shared prologue
// ---------------------------------------------------------------------------
// A wave streams a run of up to `ppw` consecutive partitions of one
// (sequence, KV head, query-head group); the last run of a sequence may also
// take the partitions left over after whole runs.  At most kMaxWaveBlocks
// blocks (five id registers of 64 lanes).
constexpr int kMaxWaveBlocks = 320;

// Partitions are aligned to absolute positions (partition k holds tokens
// [k·P, (k+1)·P)); with a sliding window they are numbered from the first
// one that overlaps the window, and only the window's tokens count.
struct WaveTask {
  int s, kvh, h0, nh;           // sequence, KV head, first query head, heads here
  int n, P;                     // length, partitions of this sequence (in the window)
  int part0, part_end;          // partitions [part0, part_end) of this wave
  int t_lo, t_end;              // the wave's tokens: [t_lo, t_end)
  int blk_first, nblk;          // first logical block and block count
  int boundary0;                // wave-local block count that closes its first partition
  int id0, id1, id2, id3, id4;  // lane l of idC holds block blk_first + 64C + l
};

// First partition overlapping the window of a sequence of length n, and the
// number of partitions from there to the end.
__device__ __forceinline__ void window_partitions(const DecodeParams& p, int n, int& t0, int& pf, int& P) {
  t0 = p.window > 0 ? max(0, n - p.window) : 0;
  pf = t0 / p.partition;
  P = (n - 1) / p.partition - pf + 1;
}

template <typename T, int D>
__device__ __forceinline__ void write_nan_rows(const DecodeParams& p, int s, int h0, int nh) {
  T* out = static_cast<T*>(p.out) + (static_cast<size_t>(s) * p.Hq + h0) * D;
  for (int e = threadIdx.x; e < nh * D; e += 64) out[e] = static_cast<T>(NAN);
}

template <int D>
__device__ __forceinline__ void write_nan_partials(const DecodeParams& p, const WaveTask& w) {
  for (int part = w.part0; part < w.part_end; ++part)
    for (int h = 0; h < w.nh; ++h) {
      const size_t row = (static_cast<size_t>(w.s) * p.Hq + w.h0 + h) * p.pmax + part;
      for (int e = threadIdx.x; e < D; e += 64) p.part_acc[row * D + e] = NAN;
      if (threadIdx.x == 0) {
        p.part_ml[2 * row] = NAN;
        p.part_ml[2 * row + 1] = NAN;
      }
    }
}

// Decodes blockIdx into the wave's task, loads its block ids and validates
// lengths and table entries.  Returns false when the wave has nothing to do
// (after writing NaN results for an invalid sequence).
// Without a window a task's first block does not depend on the length, so
// its block ids are requested together with the length: one round trip, not
// two, precedes the first block load.  The early ids are checked once the
// length is known.  issue_q(w) requests the queries once the task is known
// to be non-empty (a grid sized for the longest sequence holds many empty
// tasks in mixed batches), so they travel with the first block loads.
template <typename T, int D, typename IssueQ>
__device__ __forceinline__ bool setup_task(const DecodeParams& p, WaveTask& w, IssueQ&& issue_q) {
  const int lane = threadIdx.x;
  w.kvh = blockIdx.x % p.Hkv;
  const int cell = blockIdx.x / p.Hkv;
  // The wave's partitions: [part0, part_lim), clipped below to the device
  // length.
  int part0, part_lim;
  if (!decode_cell(p, cell, w.s, part0, part_lim)) return false;   // a sweep chunk the hint covers
  w.h0 = w.kvh * p.G + blockIdx.y * 16;
  w.nh = min(16, p.G - static_cast<int>(blockIdx.y) * 16);
  w.n = p.seq_lens[w.s];
  const int bpp = p.partition / kBlock;
  const bool early = p.window == 0;
  const int early_first = part0 * bpp;                         // = blk_first when there is no window
  const int early_lim = min((part_lim - part0) * bpp, p.max_blocks - early_first);   // blocks the run can hold
  int ids[5] = {0, 0, 0, 0, 0};
  {
    const int32_t* row = p.block_tables + static_cast<size_t>(w.s) * p.max_blocks + early_first;
#pragma unroll
    for (int c = 0; c < 5; ++c)
      if (early && 64 * c < early_lim && 64 * c + lane < early_lim) ids[c] = row[64 * c + lane];
  }
  if (w.n < 1 || w.n > p.max_seq_len) {
    if (part0 == 0) write_nan_rows<T, D>(p, w.s, w.h0, w.nh);   // exactly one wave per row starts at 0
    return false;
  }
  int t0, pf;
  window_partitions(p, w.n, t0, pf, w.P);
  w.part0 = part0;
  if (w.part0 >= w.P) return false;
  issue_q(w);
  w.part_end = min(w.P, part_lim);
  w.t_lo = max(t0, (pf + w.part0) * p.partition);
  w.t_end = min(w.n, (pf + w.part_end) * p.partition);
  w.blk_first = w.t_lo / kBlock;
  w.nblk = (w.t_end - w.blk_first * kBlock + kBlock - 1) / kBlock;
  w.boundary0 = (pf + w.part0 + 1) * (p.partition / kBlock) - w.blk_first;
  bool bad = w.blk_first + w.nblk > p.max_blocks || w.nblk > kMaxWaveBlocks;
  bool bad_lane = false;
  const int32_t* row = p.block_tables + static_cast<size_t>(w.s) * p.max_blocks + w.blk_first;
  auto fetch = [&](int c) {
    const int idx = 64 * c + lane;
    int b = 0;
    if (!bad && idx < w.nblk) b = early ? ids[c] : row[idx];
    const bool bl = static_cast<unsigned>(b) >= static_cast<unsigned>(p.num_blocks);
    bad_lane = bad_lane || bl;
    return bl ? 0 : b;
  };
  w.id0 = fetch(0);
  w.id1 = fetch(1);
  w.id2 = fetch(2);
  w.id3 = fetch(3);
  w.id4 = fetch(4);
  bad = bad || __any(bad_lane);
  if (bad) {
    if (w.P == 1) write_nan_rows<T, D>(p, w.s, w.h0, w.nh);
    else write_nan_partials<D>(p, w);
    return false;
  }
  return true;
}

// Physical id of a wave's i-th block (i wave-uniform) from the five id
// registers.
__device__ __forceinline__ int block_id(int id0, int id1, int id2, int id3, int id4, int i) {
  const int c = i >> 6;
  const int v = c == 0 ? id0 : c == 1 ? id1 : c == 2 ? id2 : c == 3 ? id3 : id4;
  return __builtin_amdgcn_readlane(v, i & 63);
}

// Fused append (p.k_new set).  Every wave whose partitions end at the
// sequence end (one per group of 16 query heads) holds the step's new token,
// position n - 1, in registers: lane l keeps 32-bit word l of its K row and
// of its V row (bf16 values; D / 2 words each), requested with the queries.
// Once the wave's last block (the one holding slot o = (n - 1) % 16) has been
// loaded, the token is substituted for slot o in the wave's copy of it, so the
// attention sees the token whatever the load returned for that slot.  After
// the wave's last load, head group 0 also writes the token into the pool,
// with the same bytes as the append kernels (no wait in the stream depends on
// these stores, and no load of this kernel depends on them either).
struct NewToken {
  uint32_t k, v;        // word `lane` of the token's K and V rows
};

template <int D>
__device__ __forceinline__ NewToken load_new_token(const DecodeParams& p, int s, int kvh) {
  NewToken t{0u, 0u};
  const size_t row = (static_cast<size_t>(s) * p.Hkv + kvh) * (D / 2);     // in 32-bit words
  if (threadIdx.x < D / 2) {
    t.k = static_cast<const uint32_t*>(p.k_new)[row + threadIdx.x];
    t.v = static_cast<const uint32_t*>(p.v_new)[row + threadIdx.x];
  }
  return t;
}

// Replaces 16-bit half `half` of w by the low 16 bits of x.
__device__ __forceinline__ uint32_t put_half(uint32_t w, uint32_t x, int half) {
  const int sh = 16 * half;
  return (w & ~(0xFFFFu << sh)) | ((x & 0xFFFFu) << sh);
}
// Replaces byte `b` of w by the low 8 bits of x.
__device__ __forceinline__ uint32_t put_byte(uint32_t w, uint32_t x, int b) {
  const int sh = 8 * b;
  return (w & ~(0xFFu << sh)) | ((x & 0xFFu) << sh);
}
__device__ __forceinline__ uint32_t lane_word(uint32_t x, int src) {
  return static_cast<uint32_t>(__shfl(static_cast<int>(x), src));
}

// bf16 cache: the token's value words go to slot o of the wave's registers of
// one block (lane layout of decode_partial_bf16: per 32-wide slice c of the
// head dimension, lane (c16, g4) holds words 16c + 4g4 .. +3 of token c16's K;
// per value tile t, token 4g4 + w of column 16t + c16 in half w % 2 of word
// w / 2).
template <int D>
__device__ __forceinline__ void patch_token_bf16(u32x4* k, u32x2* v, const NewToken& t, int o) {
  const int c16 = threadIdx.x & 15, g4 = threadIdx.x >> 4;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = lane_word(t.k, 16 * c + 4 * g4 + j);
      if (c16 == o) k[c][j] = w;
    }
  const int w_idx = (o & 3) >> 1, half = o & 1;
#pragma unroll
  for (int tt = 0; tt < D / 16; ++tt) {
    const uint32_t w = lane_word(t.v, 8 * tt + (c16 >> 1)) >> (16 * (c16 & 1));
    if (g4 == (o >> 2)) {
      if (w_idx == 0) v[tt].x = put_half(v[tt].x, w, half);
      else v[tt].y = put_half(v[tt].y, w, half);
    }
  }
}

// The token's pool bytes as kv_append_kernel writes them (K [d/8][B][8],
// V [B/4][d/4][4][4] in 16-bit values): lane l writes word l of each row.
template <int D>
__device__ __forceinline__ void store_token_bf16(const DecodeParams& p, size_t row, const NewToken& t, int o) {
  const int l = threadIdx.x;
  if (l >= D / 2) return;
  uint32_t* kt = static_cast<uint32_t*>(const_cast<void*>(p.k_cache)) + row * (kBlock * D / 2);
  uint16_t* vt = static_cast<uint16_t*>(const_cast<void*>(p.v_cache)) + row * (kBlock * D);
  kt[((l >> 2) * kBlock + o) * 4 + (l & 3)] = t.k;
  vt[v_index(2 * l, o, D)] = static_cast<uint16_t>(t.v & 0xFFFFu);
  vt[v_index(2 * l + 1, o, D)] = static_cast<uint16_t>(t.v >> 16);
}

// 8-bit cache: the token quantised as kv_append_fp8_kernel quantises it (per
// row: scale = amax / 448, codes by the hardware conversion); lane l holds
// the codes of values 2l and 2l + 1 (low 16 bits of kc / vc) and, for
// l < D / 4, the four codes of values 4l .. 4l + 3 (k4 / v4).
struct NewTokenFp8 {
  uint32_t kc, vc, k4, v4;
  float ks, vs;
};

template <int D>
__device__ __forceinline__ NewTokenFp8 quantize_token(const NewToken& t) {
  const int l = threadIdx.x;
  auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
  auto hi = [](uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); };
  float ka = 0.f, va = 0.f;
  if (l < D / 2) {
    ka = fmaxf(fabsf(lo(t.k)), fabsf(hi(t.k)));
    va = fmaxf(fabsf(lo(t.v)), fabsf(hi(t.v)));
  }
  NewTokenFp8 q;
  q.ks = wave_max(ka) / 448.f;
  q.vs = wave_max(va) / 448.f;
  q.kc = e4m3_code(lo(t.k), q.ks) | (static_cast<uint32_t>(e4m3_code(hi(t.k), q.ks)) << 8);
  q.vc = e4m3_code(lo(t.v), q.vs) | (static_cast<uint32_t>(e4m3_code(hi(t.v), q.vs)) << 8);
  q.k4 = (lane_word(q.kc, 2 * l) & 0xFFFFu) | (lane_word(q.kc, 2 * l + 1) << 16);
  q.v4 = (lane_word(q.vc, 2 * l) & 0xFFFFu) | (lane_word(q.vc, 2 * l + 1) << 16);
  return q;
}

// 8-bit cache: codes and scales of the token to slot o of the wave's
// registers of one block (lane (c16, g4): per 64-value segment c of K, word
// j = codes of values 16(4c + g4) + 4j .. +3 of token c16; per segment a of V,
// byte w of word b = column 64a + 4c16 + b of token 4g4 + w; the scales of
// tokens 4g4 .. 4g4 + 3).
template <int D>
__device__ __forceinline__ void patch_token_fp8(u32x4* k, u32x4* v, f32x4& ks, f32x4& vs, const NewTokenFp8& q,
                                                int o) {
  const int c16 = threadIdx.x & 15, g4 = threadIdx.x >> 4;
#pragma unroll
  for (int c = 0; c < D / 64; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = lane_word(q.k4, 4 * (4 * c + g4) + j);
      if (c16 == o) k[c][j] = w;
    }
  const int w = o & 3;
#pragma unroll
  for (int a = 0; a < D / 64; ++a) {
    const uint32_t codes = lane_word(q.v4, 16 * a + c16);     // columns 64a + 4c16 + b, b = 0..3
    if (g4 == (o >> 2)) {
      v[a].x = put_byte(v[a].x, codes, w);
      v[a].y = put_byte(v[a].y, codes >> 8, w);
      v[a].z = put_byte(v[a].z, codes >> 16, w);
      v[a].w = put_byte(v[a].w, codes >> 24, w);
    }
  }
  if (g4 == (o >> 2)) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j == w) {
        ks[j] = q.ks;
        vs[j] = q.vs;
      }
  }
}

// The 8-bit token's pool bytes as kv_append_fp8_kernel writes them.
template <int D>
__device__ __forceinline__ void store_token_fp8(const DecodeParams& p, size_t row, const NewTokenFp8& q, int o) {
  const int l = threadIdx.x;
  if (l < D / 2) {
    uint8_t* kd = static_cast<uint8_t*>(const_cast<void*>(p.k_cache)) + row * kBlock * D;
    uint8_t* vd = static_cast<uint8_t*>(const_cast<void*>(p.v_cache)) + row * kBlock * D;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 2 * l + h;
      kd[(e >> 4) * (kBlock * 16) + o * 16 + (e & 15)] = static_cast<uint8_t>(q.kc >> (8 * h));
      vd[(e >> 6) * 1024 + (o >> 2) * 256 + ((e & 63) >> 2) * 16 + (e & 3) * 4 + (o & 3)] =
          static_cast<uint8_t>(q.vc >> (8 * h));
    }
  }
  if (l == 0) {
    const_cast<float*>(p.k_scale)[row * kBlock + o] = q.ks;
    const_cast<float*>(p.v_scale)[row * kBlock + o] = q.vs;
  }
}

// ---------------------------------------------------------------------------
// decode_partial, bf16 queries (bf16 cache, or 8-bit E4M3 cache)
//
// Work unit: one 16-token block of one KV head.  With lane l = 16*g + c
// (g = l/16, c = l%16):
//   scores S^T = K · Q^T with v_mfma_f32_16x16x32_bf16 over 32-wide slices of
//   the head dimension: A = K tile (row = token c, k = 8 values of 16-byte
//   chunk g of the slice), B = Q^T (column = query head c, same k).
//   Lane l receives the scores of tokens 4g..4g+3 for head c.
//   out^T += V^T · P with v_mfma_f32_16x16x16_bf16 per 16 value columns:
//   A = V^T (row = a value column, k = tokens 4g..4g+3), B = P (the lane's
//   own four probabilities, head c).
// The token order inside k is the same on both operands, so only the max and
// sum reductions move data between lanes.  NBUF blocks are in flight per
// wave in rotating register sets: block i+NBUF is requested as soon as
// block i has been consumed.
//
// bf16 cache: the K chunk is read as it lies; V^T row c of tile t is value
// column 16t+c, whose tokens 4g..4g+3 are one 8-byte run of the V tile (the
// 16 lanes of a group read 128 contiguous bytes, the four groups a quarter
// tile apart); lane l accumulates value columns 16t+4g..16t+4g+3 of head c.
//
// 8-bit cache: each lane reads 16 bytes per 1 KiB of K (one token's 16
// codes; MFMA 2i+h takes head-dimension values 16(4i+g)+8h.. of the chunk,
// and Q is loaded in that order) and 16 bytes per 1 KiB of V (four value
// columns 64a+4c+b, b = 0..3, of the lane's four tokens).  Codes become bf16
// exactly (v_cvt_scalef32_pk_bf16_fp8, scale 1).  The per-token K scale
// multiplies the lane's scores; the per-token V scale multiplies its
// probabilities before they are rounded to bf16 for the PV product, so no
// value is rescaled.  Tile t = 4a+b holds value column 64a+4c+b in row c;
// lane l accumulates columns 64a+16g+4j+b (j = 0..3).
// ---------------------------------------------------------------------------

template <int D, bool kFp8>
struct BlockRegs;
template <int D>
struct BlockRegs<D, false> {
  u32x4 k[D / 32];
  u32x2 v[D / 16];
};
template <int D>
struct BlockRegs<D, true> {
  u32x4 k[D / 64];
  u32x4 v[D / 64];
  f32x4 ks;              // scales of the lane's tokens 4g..4g+3
  f32x4 vs;
};

// Four E4M3 codes (one 32-bit word) -> four bf16 values, exactly.  The packed
// result is used whole (as a 32-bit word) on purpose.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
  const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return u32x2{lo, hi};
}

// Value column of accumulator element j of tile t for lane group g4.
template <bool kFp8>
__device__ __forceinline__ int acc_column(int t, int j, int g4) {
  return kFp8 ? 64 * (t >> 2) + 16 * g4 + 4 * j + (t & 3) : 16 * t + 4 * g4 + j;
}

// (The 8-bit shallow variant is held to two waves per SIMD: its merge of
// staged partitions would otherwise take it past 256 registers.)
template <int D, int NBUF, bool kFp8>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kFp8 && NBUF == kDepthFp8 ? 2 : 1)))
void decode_partial_bf16(DecodeParams p) {
  constexpr int KC = D / 32;                   // QK MFMAs per block
  constexpr int NT = D / 16;                   // PV MFMAs (value tiles) per block
  constexpr int ELEM = kFp8 ? 1 : 2;           // cache bytes per value
  // Partials of the wave's finished partitions wait here until its load
  // stream ends: a global store in the middle of the stream would make every
  // later wait drain all loads in flight (stores and loads share vmcnt).
  extern __shared__ float staged[];
  const int lane = threadIdx.x;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;
  // Q^T operand of QK MFMA c: head c16, the head-dimension values that the
  // K operand's lane holds (see above).  Requested during the task set-up.
  bf16x8 qreg[KC];
  auto issue_q = [&](const WaveTask& wt) {
    const __bf16* q = static_cast<const __bf16*>(p.q) + (static_cast<size_t>(wt.s) * p.Hq + wt.h0 + c16) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int off = kFp8 ? 64 * (c >> 1) + 16 * g4 + 8 * (c & 1) : 32 * c + 8 * g4;
      u32x4 v = {0, 0, 0, 0};
      if (c16 < wt.nh) v = *reinterpret_cast<const u32x4*>(q + off);
      qreg[c] = __builtin_bit_cast(bf16x8, v);
    }
  };
  int s_, kvh, h0, nh, P, part0, part_end, t_lo, t_end, blk_first, nblk, boundary0, id0, id1, id2, id3, id4;
  int n_;
  bool new_token;              // this wave's last block receives the step's new token (fused append)
  NewToken tok{0u, 0u};
  {
    WaveTask w;
    if (!setup_task<__bf16, D>(p, w, issue_q)) return;
    new_token = p.k_new != nullptr && w.part_end == w.P;
    if (new_token) tok = load_new_token<D>(p, w.s, w.kvh);   // in flight with the queries
    n_ = w.n;
    s_ = w.s; kvh = w.kvh; h0 = w.h0; nh = w.nh; P = w.P; part0 = w.part0; part_end = w.part_end;
    t_lo = w.t_lo; t_end = w.t_end; blk_first = w.blk_first; nblk = w.nblk; boundary0 = w.boundary0;
    id0 = w.id0; id1 = w.id1; id2 = w.id2; id3 = w.id3; id4 = w.id4;
  }
  // 8-bit cache, runs of several partitions: the two waves of a SIMD swap
  // issue priority every 2^12 ticks of the 100 MHz real-time counter (41 us),
  // so each is favoured half the time and both end together; with plain
  // age order the older wave finishes first and the younger streams alone.
  // (Hardware wave slot parity from HW_ID tells the two apart.)
  const bool prio_swap = kFp8 && p.ppw > 1;
  const unsigned slot_bit = prio_swap ? (__builtin_amdgcn_s_getreg((31 << 11) | 4) & 1) : 0;

  const size_t tile_bytes = static_cast<size_t>(kBlock) * D * ELEM;  // one (block, head) tile
  const size_t blk_bytes = static_cast<size_t>(p.Hkv) * tile_bytes;
  const char* kc_b = static_cast<const char*>(p.k_cache) + kvh * tile_bytes;
  const char* vc_b = static_cast<const char*>(p.v_cache) + kvh * tile_bytes;
  // Block bases are wave-uniform; per-lane byte offsets are 32-bit.
  const uint32_t k_off = static_cast<uint32_t>(lane) * 16u;
  const uint32_t v_off = kFp8 ? static_cast<uint32_t>(lane) * 16u : static_cast<uint32_t>(D * g4 + c16) * 8u;

  auto load_block = [&](BlockRegs<D, kFp8>& r, int i) {
    const size_t b = static_cast<size_t>(block_id(id0, id1, id2, id3, id4, i));
    const u32x4* kp = reinterpret_cast<const u32x4*>(kc_b + b * blk_bytes + k_off);
    if constexpr (kFp8) {
      const u32x4* vp = reinterpret_cast<const u32x4*>(vc_b + b * blk_bytes + v_off);
#pragma unroll
      for (int c = 0; c < D / 64; ++c) r.k[c] = stream_load(kp + 64 * c);
#pragma unroll
      for (int a = 0; a < D / 64; ++a) r.v[a] = stream_load(vp + 64 * a);
      const size_t srow = (b * p.Hkv + kvh) * kBlock + 4 * g4;
      r.ks = stream_load(reinterpret_cast<const f32x4*>(p.k_scale + srow));
      r.vs = stream_load(reinterpret_cast<const f32x4*>(p.v_scale + srow));
    } else {
      const u32x2* vp = reinterpret_cast<const u32x2*>(vc_b + b * blk_bytes + v_off);
#pragma unroll
      for (int c = 0; c < KC; ++c) r.k[c] = stream_load(kp + 64 * c);
#pragma unroll
      for (int t = 0; t < NT; ++t) r.v[t] = stream_load(vp + 16 * t);
    }
  };

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const int bpp = p.partition / kBlock;        // blocks per partition
  int next_boundary = boundary0;               // block count that closes a partition
  int staged_parts = 0;
  // Staged partitions in LDS: accumulator rows [partition][head][D] (16-byte
  // aligned, so staging and copying out move 16 bytes per lane), then (m, l)
  // pairs [partition][head][2].
  const int n_stage = part_end - part0 - 1;
  float* staged_ml = staged + n_stage * nh * D;

  // Closes a partition that is not the wave's last: park (acc, m, l) in LDS
  // and restart the running statistics.
  auto stage_partition = [&]() {
    const float l_tot = sum_over_rows(l_run);
    if (c16 < nh) {
      float* dst = staged + (staged_parts * nh + c16) * D;
      if constexpr (kFp8) {
#pragma unroll
        for (int a = 0; a < D / 64; ++a)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<f32x4*>(dst + acc_column<true>(4 * a, j, g4)) =
                f32x4{acc[4 * a][j], acc[4 * a + 1][j], acc[4 * a + 2][j], acc[4 * a + 3][j]};
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(dst + acc_column<false>(t, 0, g4)) = acc[t];
      }
      if (g4 == 0) {
        staged_ml[2 * (staged_parts * nh + c16)] = m_run;
        staged_ml[2 * (staged_parts * nh + c16) + 1] = l_tot;
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
    ++staged_parts;
  };

  // kTail: the block may hold tokens past the sequence end (only the wave's
  // last block can).  Only the wave's first block can start before t_lo (a
  // sliding window's first token); that check is one scalar compare.
  auto compute_block = [&](const BlockRegs<D, kFp8>& r, int i, auto tail_tag) {
    constexpr bool kTail = decltype(tail_tag)::value;
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kFp8) {
#pragma unroll
      for (int c = 0; c < D / 64; ++c) {
        const u32x2 a0 = e4m3x4_to_bf16x4(r.k[c].x), a1 = e4m3x4_to_bf16x4(r.k[c].y);
        const u32x2 a2 = e4m3x4_to_bf16x4(r.k[c].z), a3 = e4m3x4_to_bf16x4(r.k[c].w);
        const u32x4 lo = {a0.x, a0.y, a1.x, a1.y};
        const u32x4 hi = {a2.x, a2.y, a3.x, a3.y};
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo), qreg[2 * c], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi), qreg[2 * c + 1], sc, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int c = 0; c < KC; ++c)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.k[c]), qreg[c], sc, 0, 0, 0);
    }
    const int tok0 = (blk_first + i) * kBlock + 4 * g4;           // token of x[0]
    const bool tail = (kTail && (blk_first + i + 1) * kBlock > t_end) || (blk_first + i) * kBlock < t_lo;
    auto outside = [&](int tok) { return tok >= t_end || tok < t_lo; };
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (kFp8) x[j] = sc[j] * (r.ks[j] * p.scale_log2);
      else x[j] = sc[j] * p.scale_log2;
    }
    if (tail) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (outside(tok0 + j)) x[j] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = max_over_rows(mx);
    const float m_new = fmaxf(m_run, mx);
    // Rescale only when some column's maximum grew (alpha is exactly 1
    // elsewhere); once the running maxima settle this is skipped.
    if (__any(m_new > m_run)) {
      const float alpha = exp2_fast(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] *= alpha;
      m_run = m_new;
    }
    bf16x4 pb;
    float ps = 0.f;
    if constexpr (kFp8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = exp2_fast(x[j] - m_run);
        const float vsj = (tail && outside(tok0 + j)) ? 0.f : r.vs[j];   // NaN-poisoned slots
        pb[j] = static_cast<__bf16>(e * vsj);
        ps += e;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const __bf16 e = static_cast<__bf16>(exp2_fast(x[j] - m_run));
        pb[j] = e;
        ps += static_cast<float>(e);
      }
    }
    l_run += ps;
    if constexpr (kFp8) {
      uint32_t mk = 0xFFFFFFFFu;                // byte k of a word = token 4g+k
      if (tail) {
        mk = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) mk |= (outside(tok0 + j) ? 0u : 0xFFu) << (8 * j);
      }
#pragma unroll
      for (int a = 0; a < D / 64; ++a) {
        const uint32_t w[4] = {r.v[a].x, r.v[a].y, r.v[a].z, r.v[a].w};
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[4 * a + b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              __builtin_bit_cast(bf16x4, e4m3x4_to_bf16x4(w[b] & mk)), pb, acc[4 * a + b], 0, 0, 0);
      }
    } else {
      uint32_t mk0 = 0xFFFFFFFFu, mk1 = 0xFFFFFFFFu;
      if (tail) {
        auto half = [&](int tok) -> uint32_t { return outside(tok) ? 0u : 0xFFFFu; };
        mk0 = half(tok0) | (half(tok0 + 1) << 16);
        mk1 = half(tok0 + 2) | (half(tok0 + 3) << 16);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x2 vv = {r.v[t].x & mk0, r.v[t].y & mk1};
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vv), pb, acc[t], 0, 0, 0);
      }
    }
    if (i + 1 == next_boundary && i + 1 < nblk) {
      stage_partition();
      next_boundary += bpp;
    }
  };

  // Steady state: every iteration consumes NBUF blocks and requests the next
  // NBUF, all unconditionally, so NBUF blocks stay in flight.  The drain loop
  // finishes the last blocks (and short runs).
  using NoTail = std::integral_constant<bool, false>;
  using MayTail = std::integral_constant<bool, true>;
  BlockRegs<D, kFp8> buf[NBUF];
  int i = 0;
  // Fused append: the token's slot in the last block, and (8-bit cache) its
  // codes, made once the drain loop reaches that block.
  const int tok_slot = (n_ - 1) % kBlock;
  NewTokenFp8 tok8{};
  auto patch_last = [&](BlockRegs<D, kFp8>& r) {
    if constexpr (kFp8) {
      tok8 = quantize_token<D>(tok);
      patch_token_fp8<D>(r.k, r.v, r.ks, r.vs, tok8, tok_slot);
    } else {
      patch_token_bf16<D>(r.k, r.v, tok, tok_slot);
    }
  };
  if (nblk >= 2 * NBUF) {
    // Issue order matters: the loop expects buf[0] to be the oldest load in
    // flight on entry (as it is on the back edge), otherwise the wait at the
    // loop head must drain everything.  The barriers keep this order.
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      load_block(buf[u], u);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (; i + 2 * NBUF <= nblk; i += NBUF) {
      if (prio_swap) {
        if ((static_cast<unsigned>(__builtin_amdgcn_s_memrealtime() >> 12) ^ slot_bit) & 1)
          __builtin_amdgcn_s_setprio(1);
        else
          __builtin_amdgcn_s_setprio(0);
      }
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        compute_block(buf[u], i + u, NoTail{});
        load_block(buf[u], i + u + NBUF);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < NBUF; ++u)
      if (u < nblk) load_block(buf[u], u);
  }
  // The last block is always consumed here (the steady loop stops at least
  // NBUF blocks before the end).
  for (; i < nblk; i += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      if (i + u < nblk) {
        if (new_token && i + u == nblk - 1) patch_last(buf[u]);
        compute_block(buf[u], i + u, MayTail{});
        if (i + u + NBUF < nblk) load_block(buf[u], i + u + NBUF);
      }
    }
  }
  // Every load has been consumed: the new token's pool write can go now.
  if (new_token && blockIdx.y == 0) {
    const size_t row = static_cast<size_t>(block_id(id0, id1, id2, id3, id4, nblk - 1)) * p.Hkv + kvh;
    if constexpr (kFp8) store_token_fp8<D>(p, row, tok8, tok_slot);
    else store_token_bf16<D>(p, row, tok, tok_slot);
  }

  // The stream has ended.  A single partition is the output.  Otherwise the
  // partitions go to the workspace in merge groups of kMergeGroup (see the
  // reduce kernels): a group the wave holds whole is merged here and written
  // once, at its first partition's slot, its sum negated to mark it; the
  // partitions of a group the wave holds in part are written one by one.
  // (LDS accesses of one wave complete in order: no barrier is needed.)
  const float l_tot = sum_over_rows(l_run);
  if (P == 1) {
    if (c16 >= nh) return;
    const float inv = 1.f / l_tot;
    __bf16* out = static_cast<__bf16*>(p.out) + (static_cast<size_t>(s_) * p.Hq + h0 + c16) * D;
    if constexpr (kFp8) {
#pragma unroll
      for (int a = 0; a < D / 64; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 o;
#pragma unroll
          for (int b = 0; b < 4; ++b) o[b] = static_cast<__bf16>(acc[4 * a + b][j] * inv);
          *reinterpret_cast<bf16x4*>(out + acc_column<true>(4 * a, j, g4)) = o;
        }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = static_cast<__bf16>(acc[t][j] * inv);
        *reinterpret_cast<bf16x4*>(out + acc_column<false>(t, 0, g4)) = o;
      }
    }
    return;
  }
  const size_t row0 = (static_cast<size_t>(s_) * p.Hq + h0) * p.pmax;    // + h * pmax + partition
  const int last = part_end - 1;                                          // in registers; the rest staged
  auto write_last = [&]() {
    if (c16 >= nh) return;
    const size_t row = row0 + static_cast<size_t>(c16) * p.pmax + last;
    float* pa = p.part_acc + row * D;
    if constexpr (kFp8) {
#pragma unroll
      for (int a = 0; a < D / 64; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(pa + acc_column<true>(4 * a, j, g4)) =
              f32x4{acc[4 * a][j], acc[4 * a + 1][j], acc[4 * a + 2][j], acc[4 * a + 3][j]};
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(pa + acc_column<false>(t, 0, g4)) = acc[t];
    }
    if (g4 == 0) {
      p.part_ml[2 * row] = m_run;
      p.part_ml[2 * row + 1] = l_tot;
    }
  };
  // Staged partitions [a, b) one by one; lane l moves 16-byte chunks l,
  // l + 64, ... of the nh accumulator rows.
  auto write_staged = [&](int a, int b) {
    for (int part = a; part < b; ++part) {
      const int sp = part - part0;
      for (int c = lane; c < nh * (D / 4); c += 64) {
        const int h = c / (D / 4), e = (c % (D / 4)) * 4;
        const f32x4 v = *reinterpret_cast<const f32x4*>(staged + (sp * nh + h) * D + e);
        *reinterpret_cast<f32x4*>(p.part_acc + (row0 + static_cast<size_t>(h) * p.pmax + part) * D + e) = v;
      }
      if (lane < nh) {
        const size_t row = row0 + static_cast<size_t>(lane) * p.pmax + part;
        p.part_ml[2 * row] = staged_ml[2 * (sp * nh + lane)];
        p.part_ml[2 * row + 1] = staged_ml[2 * (sp * nh + lane) + 1];
      }
    }
  };
  if (part_end - part0 == 1) {        // one partition (the work list's waves): nothing to merge
    write_last();
    return;
  }
  // Accumulator chunk q of the lane's head, as staged (four value columns).
  auto acc_chunk = [&](int q) -> f32x4 {
    if constexpr (kFp8) {
      const int a = q >> 2, j = q & 3;
      return f32x4{acc[4 * a][j], acc[4 * a + 1][j], acc[4 * a + 2][j], acc[4 * a + 3][j]};
    } else {
      return acc[q];
    }
  };
  auto chunk_column = [&](int q) { return kFp8 ? acc_column<true>(4 * (q >> 2), q & 3, g4) : acc_column<false>(q, 0, g4); };
  for (int g = part0 / kMergeGroup; g <= last / kMergeGroup; ++g) {
    const int g0 = g * kMergeGroup;
    if (g0 >= part0 && g0 + kMergeGroup <= part_end) {
      // The whole group: M = max m_i, w_i = 2^(m_i - M), L = sum l_i w_i and
      // A = sum acc_i w_i, each a chain of fused multiply-adds in partition order.
      if (c16 < nh) {
        float m_i[kMergeGroup], l_i[kMergeGroup];
        float M = -INFINITY;
#pragma unroll
        for (int u = 0; u < kMergeGroup; ++u) {
          const int sp = g0 + u - part0;
          m_i[u] = g0 + u == last ? m_run : staged_ml[2 * (sp * nh + c16)];
          l_i[u] = g0 + u == last ? l_tot : staged_ml[2 * (sp * nh + c16) + 1];
          M = fmaxf(M, m_i[u]);
        }
        float w[kMergeGroup];
        float L = 0.f;
#pragma unroll
        for (int u = 0; u < kMergeGroup; ++u) {
          w[u] = exp2_fast(m_i[u] - M);
          L = __builtin_fmaf(l_i[u], w[u], L);
        }
        const size_t row = row0 + static_cast<size_t>(c16) * p.pmax + g0;
#pragma unroll
        for (int q = 0; q < NT; ++q) {
          f32x4 A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < kMergeGroup; ++u) {
            const f32x4 v = g0 + u == last ? acc_chunk(q)
                                           : *reinterpret_cast<const f32x4*>(
                                                 staged + ((g0 + u - part0) * nh + c16) * D + chunk_column(q));
#pragma unroll
            for (int e = 0; e < 4; ++e) A[e] = __builtin_fmaf(v[e], w[u], A[e]);
          }
          *reinterpret_cast<f32x4*>(p.part_acc + row * D + chunk_column(q)) = A;
        }
        if (g4 == 0) {
          p.part_ml[2 * row] = M;
          p.part_ml[2 * row + 1] = -L;          // negative: a merged group
        }
      }
    } else {
      const int a = g0 > part0 ? g0 : part0;
      const int b = g0 + kMergeGroup < part_end ? g0 + kMergeGroup : part_end;
      write_staged(a, b < last ? b : last);
      if (b == part_end) write_last();
    }
  }
}

// ---------------------------------------------------------------------------
// decode_partial, fp32: v_mfma_f32_16x16x4_f32, one block per step.
//   QK: MFMA (c, j) uses k-slot g = element 16c + 4g + j of the head dim;
//   A = K (row = token c16), B = Q^T (column = head c16).
//   PV: MFMA j uses k-slot g = token 4g + j of the block; A = V^T (row =
//   value column), B = P.  Lane layouts of the results match the bf16 path.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void decode_partial_f32(DecodeParams p) {
  constexpr int KC = D / 16;
  constexpr int NT = D / 16;
  int s_, kvh, h0, nh, P, part0, t_lo, t_end, blk_first, nblk, id0, id1, id2, id3, id4;
  {
    WaveTask w;
    if (!setup_task<float, D>(p, w, [](const WaveTask&) {})) return;
    s_ = w.s; kvh = w.kvh; h0 = w.h0; nh = w.nh; P = w.P; part0 = w.part0;
    t_lo = w.t_lo; t_end = w.t_end; blk_first = w.blk_first; nblk = w.nblk;
    id0 = w.id0; id1 = w.id1; id2 = w.id2; id3 = w.id3; id4 = w.id4;
  }
  const int lane = threadIdx.x;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;

  f32x4 qreg[KC];
  {
    const float* q = static_cast<const float*>(p.q) + (static_cast<size_t>(s_) * p.Hq + h0 + c16) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (c16 < nh) v = *reinterpret_cast<const f32x4*>(q + 16 * c + 4 * g4);
      qreg[c] = v;
    }
  }
  const size_t tile = static_cast<size_t>(kBlock) * D;
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * tile;
  const float* kc = static_cast<const float*>(p.k_cache) + static_cast<size_t>(kvh) * tile;
  const float* vc = static_cast<const float*>(p.v_cache) + static_cast<size_t>(kvh) * tile;

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  for (int i = 0; i < nblk; ++i) {    // one partition per wave (ppw = 1)
    const int b = block_id(id0, id1, id2, id3, id4, i);
    const f32x4* kp = reinterpret_cast<const f32x4*>(kc + b * blk_stride) + lane;
    const f32x4* vp = reinterpret_cast<const f32x4*>(vc + b * blk_stride) + D * g4 + c16;   // [B/4][D/4][4][4]
    f32x4 kr[KC], vr[NT];
#pragma unroll
    for (int c = 0; c < KC; ++c) kr[c] = stream_load(kp + 64 * c);
#pragma unroll
    for (int t = 0; t < NT; ++t) vr[t] = stream_load(vp + 16 * t);
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) sc = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[c][j], qreg[c][j], sc, 0, 0, 0);
    const int tok0 = (blk_first + i) * kBlock + 4 * g4;
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = (tok0 + j < t_end && tok0 + j >= t_lo) ? sc[j] * p.scale_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = max_over_rows(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2_fast(m_run - m_new);
    m_run = m_new;
    float pr[4];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pr[j] = exp2_fast(x[j] - m_new);
      ps += pr[j];
    }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc[t] *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = (tok0 + j < t_end && tok0 + j >= t_lo) ? vr[t][j] : 0.f;
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, pr[j], acc[t], 0, 0, 0);
      }
    }
  }

  const float l_tot = sum_over_rows(l_run);
  if (c16 >= nh) return;
  const size_t head_row = static_cast<size_t>(s_) * p.Hq + h0 + c16;
  if (P == 1) {
    const float inv = 1.f / l_tot;
    float* out = static_cast<float*>(p.out) + head_row * D + 4 * g4;
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(out + 16 * t) = acc[t] * inv;
  } else {
    const size_t row = head_row * p.pmax + part0;
    float* pa = p.part_acc + row * D + 4 * g4;
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(pa + 16 * t) = acc[t];
    if (g4 == 0) {
      p.part_ml[2 * row] = m_run;
      p.part_ml[2 * row + 1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// decode_reduce: merges the P > 1 partitions of each (sequence, query head)
// row, always in one order of operations (so the result does not depend on
// which kernel, or which partial-kernel wave, merges what):
//   partitions in groups of kMergeGroup, g = [K g, K g + K) within [0, P):
//     M_g = max m_i,  w_i = 2^(m_i - M_g),
//     L_g = l_0 w_0 + l_1 w_1 + ...,  A_g = acc_0 w_0 + acc_1 w_1 + ...
//   then the groups:  M = max M_g,  W_g = 2^(M_g - M),
//     L = L_0 W_0 + L_1 W_1 + ...,  out = (A_0 W_0 + A_1 W_1 + ...) / L,
// every sum a chain of fused multiply-adds from 0 in index order.  A group
// the partial kernel merged itself sits at its first partition's slot with
// its sum negated (a partition's own sum is at least 1).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_max_256(float x, float* scratch) {
  x = wave_max(x);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  x = fmaxf(fmaxf(scratch[0], scratch[1]), fmaxf(scratch[2], scratch[3]));
  __syncthreads();
  return x;
}

__device__ __forceinline__ bool merged_group(const float* ml, int g0) { return ml[2 * g0 + 1] < 0.f; }

// M_g of group g (partitions [g0, min(g0 + K, P))).
__device__ __forceinline__ float group_max(const float* ml, int g0, int P) {
  if (merged_group(ml, g0)) return ml[2 * g0];
  float M = -INFINITY;
  for (int i = g0; i < g0 + kMergeGroup && i < P; ++i) M = fmaxf(M, ml[2 * i]);
  return M;
}

// One workgroup per row, for launches with more than kRowReduceMaxParts
// partitions: PH groups at a time are merged in parallel (thread (cg, ph):
// four value columns of group c0 + ph) into LDS, then the first CG threads
// fold them into the output columns in group order.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeParams p) {
  constexpr int CG = D / 4;        // float4 column groups
  constexpr int PH = 256 / CG;     // merge groups per round
  __shared__ f32x4 red[PH][CG];
  __shared__ float red_m[PH], red_l[PH];
  __shared__ float scratch[4];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int s = row / p.Hq;
  const int n = p.seq_lens[s];
  if (n < 1 || n > p.max_seq_len) return;
  int t0, pf, P;
  window_partitions(p, n, t0, pf, P);
  if (P <= 1) return;
  const float* ml = p.part_ml + static_cast<size_t>(row) * p.pmax * 2;
  const float* acc = p.part_acc + static_cast<size_t>(row) * p.pmax * D;
  const int NG = (P + kMergeGroup - 1) / kMergeGroup;
  const int cg = tid % CG;
  const int ph = tid / CG;
  // The thread's groups in the first two rounds: their (m, l) and first
  // accumulator chunk (all of a merged group) are requested together with
  // the maxima, so one round trip precedes the merge instead of three.
  constexpr int R = 2;                               // (the selects below assume 2)
  float pm[R], pl[R];
  f32x4 pa[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int g = r * PH + ph;
    const int g0 = (g < NG ? g : 0) * kMergeGroup;
    pm[r] = ml[2 * g0];
    pl[r] = ml[2 * g0 + 1];
    pa[r] = *reinterpret_cast<const f32x4*>(acc + static_cast<size_t>(g0) * D + 4 * cg);
  }
  float M = -INFINITY;
  for (int g = tid; g < NG; g += 256) M = fmaxf(M, group_max(ml, g * kMergeGroup, P));
  M = block_max_256(M, scratch);
  float L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < NG; c0 += PH) {
    const int g = c0 + ph;
    if (g < NG) {
      const int g0 = g * kMergeGroup;
      const int r = c0 / PH;
      float Mg, Lg;
      f32x4 Ag;
      const float plr = r == 0 ? pl[0] : pl[1];
      if (r < R && plr < 0.f) {                          // merged group, prefetched
        Mg = r == 0 ? pm[0] : pm[1];
        Lg = -plr;
        Ag = r == 0 ? pa[0] : pa[1];
      } else if (merged_group(ml, g0)) {
        Mg = ml[2 * g0];
        Lg = -ml[2 * g0 + 1];
        Ag = *reinterpret_cast<const f32x4*>(acc + static_cast<size_t>(g0) * D + 4 * cg);
      } else {
        Mg = group_max(ml, g0, P);
        Lg = 0.f;
        Ag = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int i = g0; i < g0 + kMergeGroup && i < P; ++i) {
          const float w = exp2_fast(ml[2 * i] - Mg);
          Lg = __builtin_fmaf(ml[2 * i + 1], w, Lg);
          const f32x4 a = *reinterpret_cast<const f32x4*>(acc + static_cast<size_t>(i) * D + 4 * cg);
#pragma unroll
          for (int e = 0; e < 4; ++e) Ag[e] = __builtin_fmaf(a[e], w, Ag[e]);
        }
      }
      red[ph][cg] = Ag;
      if (cg == 0) {
        red_m[ph] = Mg;
        red_l[ph] = Lg;
      }
    }
    __syncthreads();
    if (tid < CG) {
      for (int u = 0; u < PH && c0 + u < NG; ++u) {
        const float W = exp2_fast(red_m[u] - M);
        L = __builtin_fmaf(red_l[u], W, L);
        const f32x4 a = red[u][tid];
#pragma unroll
        for (int e = 0; e < 4; ++e) O[e] = __builtin_fmaf(a[e], W, O[e]);
      }
    }
    __syncthreads();
  }
  if (tid < CG) {
    T* out = static_cast<T*>(p.out) + static_cast<size_t>(row) * D + 4 * tid;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = static_cast<T>(O[e] / L);
  }
}

// The same merge for launches with few partitions (pmax <= kRowReduceMaxParts),
// one wave per (sequence, query head) row and four rows per workgroup: in a
// mixed batch most rows have one partition and exit after reading their
// length, and a quarter of the workgroups dispatch faster than one per row.
// Lane i < P reads partition i's (m, l); lane c merges value columns
// c * D/64 ... group by group.
constexpr int kRowReduceMaxParts = 32;

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_rows_kernel(DecodeParams p) {
  constexpr int CPL = D / 64;      // columns per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.S * p.Hq) return;
  const int s = row / p.Hq;
  const int n = p.seq_lens[s];
  if (n < 1 || n > p.max_seq_len) return;
  int t0, pf, P;
  window_partitions(p, n, t0, pf, P);
  if (P <= 1) return;
  const float* ml = p.part_ml + static_cast<size_t>(row) * p.pmax * 2;
  const float* acc = p.part_acc + static_cast<size_t>(row) * p.pmax * D + CPL * lane;
  // Lane i: partition i's m and l, and whether its group was merged (then
  // only the group's first slot was written).
  const int gi = lane - lane % kMergeGroup;
  const float m_i = lane < P ? ml[2 * lane] : -INFINITY;
  const float l_i = lane < P ? ml[2 * lane + 1] : 0.f;
  const float l_g = lane < P ? ml[2 * gi + 1] : 0.f;
  const bool live = lane < P && (l_g >= 0.f || lane == gi);
  const float M = wave_max(live ? m_i : -INFINITY);
  float L = 0.f;
  float o[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) o[j] = 0.f;
  for (int g0 = 0; g0 < P; g0 += kMergeGroup) {
    const int cnt = P - g0 < kMergeGroup ? P - g0 : kMergeGroup;
    float Mg, Lg = 0.f;
    float ag[CPL];
    if (__shfl(l_i, g0) < 0.f) {                   // merged by the partial kernel
      Mg = __shfl(m_i, g0);
      Lg = -__shfl(l_i, g0);
#pragma unroll
      for (int j = 0; j < CPL; ++j) ag[j] = acc[static_cast<size_t>(g0) * D + j];
    } else {
      float mu[kMergeGroup], lu[kMergeGroup], a[kMergeGroup][CPL];
      Mg = -INFINITY;
#pragma unroll
      for (int u = 0; u < kMergeGroup; ++u) {
        mu[u] = __shfl(m_i, g0 + u);
        lu[u] = __shfl(l_i, g0 + u);
        if (u < cnt) Mg = fmaxf(Mg, mu[u]);
#pragma unroll
        for (int j = 0; j < CPL; ++j) a[u][j] = u < cnt ? acc[static_cast<size_t>(g0 + u) * D + j] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < CPL; ++j) ag[j] = 0.f;
#pragma unroll
      for (int u = 0; u < kMergeGroup; ++u) {
        if (u < cnt) {
          const float w = exp2_fast(mu[u] - Mg);
          Lg = __builtin_fmaf(lu[u], w, Lg);
#pragma unroll
          for (int j = 0; j < CPL; ++j) ag[j] = __builtin_fmaf(a[u][j], w, ag[j]);
        }
      }
    }
    const float W = exp2_fast(Mg - M);
    L = __builtin_fmaf(Lg, W, L);
#pragma unroll
    for (int j = 0; j < CPL; ++j) o[j] = __builtin_fmaf(ag[j], W, o[j]);
  }
  T* out = static_cast<T*>(p.out) + static_cast<size_t>(row) * D + CPL * lane;
#pragma unroll
  for (int j = 0; j < CPL; ++j) out[j] = static_cast<T>(o[j] / L);
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t stream) {
  if (p.n_pairs <= 0 || p.n_layers <= 0) return hipSuccess;
  dim3 grid(p.n_pairs, p.n_layers, p.scale_bytes > 0 ? 4 : 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_table_upload(const int32_t* host_src, int32_t* dev_tables, int64_t n_tab, int32_t* dev_lens,
                               int32_t n_len, hipStream_t stream) {
  if (n_tab + n_len <= 0) return hipSuccess;
  const bool vec = (reinterpret_cast<uintptr_t>(host_src) & 15) == 0 && (reinterpret_cast<uintptr_t>(dev_tables) & 15) == 0;
  const int64_t total = (vec ? n_tab / 4 + n_tab % 4 : n_tab) + n_len;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 1024);
  hipLaunchKernelGGL(table_upload_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, host_src,
                     dev_tables, n_tab, dev_lens, n_len, vec);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream) {
  if (p.n <= 0) return hipSuccess;
  dim3 grid(p.n, p.num_kv_heads);
  const int cpr = p.elem_bytes > 1 ? p.head_dim * p.elem_bytes / 16 : 0;   // 16-byte chunks per row
  if (cpr > 0 && cpr <= 64 && 64 % cpr == 0) {         // several heads per wave
    const int hpw = 64 / cpr;
    dim3 g(p.n, (p.num_kv_heads + hpw - 1) / hpw);
    if (p.elem_bytes == 4)
      hipLaunchKernelGGL(kv_append_wide_kernel<uint32_t>, g, dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL(kv_append_wide_kernel<uint16_t>, g, dim3(64), 0, stream, p);
  } else if (p.elem_bytes == 1 && (p.head_dim == 64 || p.head_dim == 128)) {
    const int hpw = 512 / p.head_dim;
    dim3 g(p.n, (p.num_kv_heads + hpw - 1) / hpw);
    if (p.head_dim == 64)
      hipLaunchKernelGGL(kv_append_fp8_wide_kernel<64>, g, dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL(kv_append_fp8_wide_kernel<128>, g, dim3(64), 0, stream, p);
  } else if (p.elem_bytes == 1)
    hipLaunchKernelGGL(kv_append_fp8_kernel, grid, dim3(64), 0, stream, p);
  else if (p.elem_bytes == 4)
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

bool decode_shape_supported(int kind, int head_dim, int block_size) {
  if (block_size != kBlock) return false;
  if (kind == kDecodeF32 || kind == kDecodeBF16) return head_dim == 64 || head_dim == 128;
  if (kind == kDecodeFP8KV) return head_dim == 64 || head_dim == 128;
  return false;
}

// Resident waves of one decode variant on this device, and the LDS each of
// them may take for staged partials without lowering that residency.
struct Residency {
  int waves;
  int lds_per_wave;
};

template <int D, int NBUF, bool kFp8>
static Residency query_residency() {
  int dev = 0, cus = 0, per_cu = 0, lds = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
      lds <= 0)
    lds = 160 * 1024;                      // a gfx950 CU's LDS
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_partial_bf16<D, NBUF, kFp8>, 64, 0) !=
          hipSuccess || per_cu <= 0)
    per_cu = 8;
  return Residency{cus * per_cu, lds / per_cu};
}

template <int D, int NBUF, bool kFp8>
static const Residency& residency() {
  static const Residency r = query_residency<D, NBUF, kFp8>();
  return r;
}

static int env_int(const char* name) {
  const char* e = std::getenv(name);
  return e ? std::max(0, std::atoi(e)) : -1;
}

// Long runs pay only for batches of equal-length sequences (per the caller's
// length hint) with at least three rounds of work for `waves` resident waves;
// mixed lengths balance better with one partition per wave, and without the
// hint nothing is known.
static bool long_uniform(const DecodeParams& p, int waves) {
  return p.tasks_hint > 0 && p.uniform_hint && p.tasks_hint >= 3LL * waves;
}

// Largest run (in partitions) that fits the five id registers and the wave's
// LDS share for staged partials.
static int max_run(const DecodeParams& p, const Residency& r) {
  const int rows = std::min(16, p.G);
  const int lds_row = (p.d + 2) * static_cast<int>(sizeof(float));
  const int by_ids = kMaxWaveBlocks * kBlock / p.partition;
  return std::max(1, std::min(by_ids, 1 + r.lds_per_wave / (rows * lds_row)));
}

// Partitions per wave.  Each wave streams a run of consecutive partitions;
// for long uniform batches runs are made as long as possible while the grid
// still fills every resident wave slot once (one round: equal-length runs then
// finish together instead of leaving a partly filled last round), within
// max_run.  PKV_WAVE_PARTITIONS overrides the choice.
static int pick_partitions_per_wave(const DecodeParams& p, const Residency& r) {
  static const int forced = env_int("PKV_WAVE_PARTITIONS");
  // leave room for a short remainder to join the last run
  const int max_ppw = std::min(p.pmax, std::max(1, max_run(p, r) - 1));
  if (forced > 0) return std::min(forced, max_ppw);
  if (!long_uniform(p, r.waves)) return 1;
  return static_cast<int>(std::min<long long>(p.tasks_hint / r.waves, max_ppw));
}

// Runs of ppw partitions; partitions left over after whole runs join the last
// run when that run still fits (a short leftover run would otherwise wait for
// a free slot and finish last), else they form one more run.
static void set_runs(DecodeParams& p, const Residency& r) {
  p.ppw = pick_partitions_per_wave(p, r);
  const int whole = p.pmax / p.ppw;
  const int rest = p.pmax - whole * p.ppw;
  p.groups = (rest == 0 || (whole > 0 && p.ppw + rest <= max_run(p, r))) ? std::max(1, whole) : whole + 1;
}

// Longest run of a launch, in partitions.
static int longest_run(const DecodeParams& p) {
  return std::max(p.ppw, p.pmax - (p.groups - 1) * p.ppw);
}

// The host's work list (one partition per wave) replaces the plain grid of
// every (partition, sequence) cell up to max_seq_len: in a batch of mixed
// lengths most of those cells are empty, and each empty wave still holds a
// wave slot for a round trip to read its length.  Here the launcher fixes the
// run capacity (the last hinted cell of a sequence and the sweep cells may
// take several partitions) and the sweep chunks, and returns the grid's cell
// count.  PKV_DECODE_ORDER=0 keeps the plain grid.
static long long settle_order(DecodeParams& p, const Residency& r) {
  static const int forced = env_int("PKV_DECODE_ORDER");
  DecodeOrder& o = p.order;
  if (p.ppw != 1 || p.groups != p.pmax || forced == 0) o.active = 0;
  if (!o.active) return static_cast<long long>(p.groups) * p.S;
  o.run_cap = max_run(p, r);
  int covered = INT_MAX;                 // every sequence's partitions below this have a listed wave
  for (int s = 0; s < p.S; ++s) covered = std::min(covered, o.hinted[s] - 1 + o.run_cap);
  o.sweep_c0 = covered / o.run_cap;
  o.sweep_chunks = std::max(0, (p.pmax + o.run_cap - 1) / o.run_cap - o.sweep_c0);
  const long long cells = o.n_full + o.n_partial + static_cast<long long>(p.S) * o.sweep_chunks;
  if (cells * p.Hkv > 0x7fffffffLL) {    // beyond a grid dimension: the plain grid (checked by the caller)
    o.active = 0;
    return static_cast<long long>(p.groups) * p.S;
  }
  return cells;
}

// With `dry` the launch is only planned: the plan goes there and nothing
// runs on the device.
template <int D, int NBUF, bool kFp8>
static hipError_t launch_variant(DecodeParams p, hipStream_t stream, DecodeLaunchPlan* dry) {
  const Residency& r = residency<D, NBUF, kFp8>();
  set_runs(p, r);
  const long long cells = settle_order(p, r);
  dim3 grid(static_cast<unsigned>(cells * p.Hkv), (p.G + 15) / 16);
  const int longest = p.order.active ? p.order.run_cap : longest_run(p);
  const size_t shmem = static_cast<size_t>(longest - 1) * std::min(16, p.G) * (p.d + 2) * sizeof(float);
  if (dry) {
    *dry = DecodeLaunchPlan{p, cells, static_cast<int>(grid.y), NBUF, r.waves, kMaxWaveBlocks, shmem};
    return hipSuccess;
  }
  static const int trace = env_int("PKV_TRACE_SCHEDULE");   // print the first choice of each variant
  static std::atomic<bool> traced{false};
  if (trace > 0 && !traced.exchange(true))
    std::fprintf(stderr, "decode_partial<d=%d, depth=%d, fp8=%d>: %d resident waves, %d B LDS each; ppw=%d, "
                 "grid=%ux%u, %zu B LDS; work list %d (%d full, %d partial cells, run capacity %d, %d sweep "
                 "chunks)\n", D, NBUF, kFp8 ? 1 : 0, r.waves, r.lds_per_wave, p.ppw, grid.x, grid.y, shmem,
                 p.order.active, p.order.n_full, p.order.n_partial, p.order.run_cap, p.order.sweep_chunks);
  hipLaunchKernelGGL((decode_partial_bf16<D, NBUF, kFp8>), grid, dim3(64), shmem, stream, p);
  return hipGetLastError();
}

// bf16 cache with at least four partitions per deep wave slot, streamed in
// runs (not from the work list): the deep variant; else the shallow one.
// With the work list (one partition per wave, mixed lengths) two waves per
// SIMD hide each other's set-up: full_step 398 -> 388 us.
// PKV_DECODE_DEEP=0/1 forces the choice.
template <int D, bool kFp8>
static hipError_t launch_bf16q(const DecodeParams& p, hipStream_t stream, DecodeLaunchPlan* dry) {
  constexpr int kShallow = kFp8 ? kDepthFp8 : kDepth;
  constexpr int kDeep = kFp8 ? kDepthFp8Deep : kDepthDeep;
  static const int forced = env_int("PKV_DECODE_DEEP");
  const int deep_waves = residency<D, kDeep, kFp8>().waves;
  const bool listed = p.order.active && !long_uniform(p, deep_waves);   // would take the work list
  const bool deep = forced >= 0 ? forced > 0 : !kFp8 && !listed && p.tasks_hint >= 4LL * deep_waves;
  return deep ? launch_variant<D, kDeep, kFp8>(p, stream, dry) : launch_variant<D, kShallow, kFp8>(p, stream, dry);
}

static hipError_t launch_or_plan(const DecodeParams& p0, int kind, hipStream_t stream, DecodeLaunchPlan* dry) {
  DecodeParams p = p0;
  switch (kind) {
    case kDecodeBF16:
      if (p.d == 128) return launch_bf16q<128, false>(p, stream, dry);
      if (p.d == 64) return launch_bf16q<64, false>(p, stream, dry);
      return hipErrorInvalidValue;
    case kDecodeFP8KV:
      if (p.d == 128) return launch_bf16q<128, true>(p, stream, dry);
      if (p.d == 64) return launch_bf16q<64, true>(p, stream, dry);
      return hipErrorInvalidValue;
    case kDecodeF32: {
      p.ppw = 1;
      p.groups = p.pmax;
      p.order.active = 0;
      dim3 grid(static_cast<unsigned>(static_cast<long long>(p.pmax) * p.S * p.Hkv), (p.G + 15) / 16);
      if (dry) {
        if (p.d != 128 && p.d != 64) return hipErrorInvalidValue;
        *dry = DecodeLaunchPlan{p, static_cast<long long>(p.pmax) * p.S, static_cast<int>(grid.y), 1, 0,
                                kMaxWaveBlocks, 0};
        return hipSuccess;
      }
      if (p.d == 128) hipLaunchKernelGGL(decode_partial_f32<128>, grid, dim3(64), 0, stream, p);
      else if (p.d == 64) hipLaunchKernelGGL(decode_partial_f32<64>, grid, dim3(64), 0, stream, p);
      else return hipErrorInvalidValue;
      return hipGetLastError();
    }
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_partial(const DecodeParams& p, int kind, hipStream_t stream) {
  return launch_or_plan(p, kind, stream, nullptr);
}

hipError_t plan_decode_partial(const DecodeParams& p, int kind, DecodeLaunchPlan* plan) {
  return launch_or_plan(p, kind, nullptr, plan);
}

// The static decode workspace.  In host code `scratch` names a host-side
// stand-in, not device memory: only the address hipGetSymbolAddress returns
// (per device, with that device current) is handed to kernels.
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

hipError_t static_workspace(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode_reduce(const DecodeParams& p, int kind, hipStream_t stream) {
  if (p.pmax <= 1) return hipSuccess;
  if (p.pmax <= kRowReduceMaxParts) {
    const dim3 rgrid(static_cast<unsigned>((static_cast<long long>(p.S) * p.Hq + 3) / 4));
    const bool bf16_out = kind == kDecodeBF16 || kind == kDecodeFP8KV;
    if (p.d == 128) {
      if (bf16_out) hipLaunchKernelGGL((decode_reduce_rows_kernel<__bf16, 128>), rgrid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((decode_reduce_rows_kernel<float, 128>), rgrid, dim3(256), 0, stream, p);
    } else if (p.d == 64) {
      if (bf16_out) hipLaunchKernelGGL((decode_reduce_rows_kernel<__bf16, 64>), rgrid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((decode_reduce_rows_kernel<float, 64>), rgrid, dim3(256), 0, stream, p);
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  dim3 grid(static_cast<unsigned>(p.S * p.Hq));
  if (kind == kDecodeBF16 || kind == kDecodeFP8KV) {   // bf16 outputs
    if (p.d == 128) hipLaunchKernelGGL((decode_reduce_kernel<__bf16, 128>), grid, dim3(256), 0, stream, p);
    else if (p.d == 64) hipLaunchKernelGGL((decode_reduce_kernel<__bf16, 64>), grid, dim3(256), 0, stream, p);
    else return hipErrorInvalidValue;
  } else {
    if (p.d == 128) hipLaunchKernelGGL((decode_reduce_kernel<float, 128>), grid, dim3(256), 0, stream, p);
    else if (p.d == 64) hipLaunchKernelGGL((decode_reduce_kernel<float, 64>), grid, dim3(256), 0, stream, p);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
