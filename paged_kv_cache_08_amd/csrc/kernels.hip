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
//   K [block][kv_head][d/x][B][x]    V [block][kv_head][d][B]
// The K layout makes one 16-byte load per lane, 64 lanes wide, read 1 KiB of
// contiguous memory that is already in the MFMA A-operand order (lane l:
// token l%16, 16-byte chunk l/16 of the head dimension slice).  The V layout
// stores tokens fastest, so a lane's run of consecutive tokens for one value
// column is contiguous, which is the PV product's operand order.
//
// Scores are kept in base-2 units (score * scale * log2 e) so the softmax
// uses the hardware exp2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.hpp"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 16;   // tokens per block on the decode path

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the four lanes l, l^16, l^32, l^48 (one MFMA column).
__device__ __forceinline__ float max_over_rows(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float sum_over_rows(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// ---------------------------------------------------------------------------
// kv_append
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void kv_append_kernel(AppendParams p) {
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int slot = p.slots[i];
  if (slot < 0 || static_cast<int64_t>(slot) >= p.num_slots) return;
  constexpr int x = 16 / sizeof(T);
  const int B = p.block_size;
  const int d = p.head_dim;
  const int b = slot / B;
  const int o = slot - b * B;
  const T* ks = static_cast<const T*>(p.k_new) + (static_cast<size_t>(i) * p.num_kv_heads + h) * d;
  const T* vs = static_cast<const T*>(p.v_new) + (static_cast<size_t>(i) * p.num_kv_heads + h) * d;
  const size_t tile = (static_cast<size_t>(b) * p.num_kv_heads + h) * static_cast<size_t>(d) * B;
  T* kd = static_cast<T*>(p.k_cache) + tile;
  T* vd = static_cast<T*>(p.v_cache) + tile;
  for (int ch = threadIdx.x; ch < d / x; ch += 64)
    *reinterpret_cast<u32x4*>(kd + (static_cast<size_t>(ch) * B + o) * x) =
        *reinterpret_cast<const u32x4*>(ks + ch * x);
  for (int e = threadIdx.x; e < d; e += 64) vd[static_cast<size_t>(e) * B + o] = vs[e];
}

// ---------------------------------------------------------------------------
// copy_blocks
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksParams p) {
  const int pair = blockIdx.x;
  const int layer = blockIdx.y;
  const int src = p.pairs[2 * pair];
  const int dst = p.pairs[2 * pair + 1];
  char* base = static_cast<char*>(blockIdx.z ? p.v[layer] : p.k[layer]);
  const u32x4* s = reinterpret_cast<const u32x4*>(base + static_cast<int64_t>(src) * p.block_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(base + static_cast<int64_t>(dst) * p.block_bytes);
  const int64_t n16 = p.block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n16; i += 256) d[i] = s[i];
}

// ---------------------------------------------------------------------------
// decode: shared prologue
// ---------------------------------------------------------------------------
struct WaveTask {
  int s, kvh, part, h0, nh;     // sequence, KV head, partition, first q head, heads here
  int n, P;                     // length, partitions of this sequence
  int t_end;                    // one past the last token of this partition
  int blk_first, nblk;          // first logical block and block count
  int myblk;                    // lane l holds the id of block blk_first + l
  bool status_ok;
};

template <typename T, int D>
__device__ __forceinline__ void write_nan_rows(const DecodeParams& p, int s, int h0, int nh) {
  T* out = static_cast<T*>(p.out) + (static_cast<size_t>(s) * p.Hq + h0) * D;
  for (int e = threadIdx.x; e < nh * D; e += 64) out[e] = static_cast<T>(NAN);
}

template <int D>
__device__ __forceinline__ void write_nan_partials(const DecodeParams& p, const WaveTask& w) {
  for (int h = 0; h < w.nh; ++h) {
    const size_t row = (static_cast<size_t>(w.s) * p.Hq + w.h0 + h) * p.pmax + w.part;
    for (int e = threadIdx.x; e < D; e += 64) p.part_acc[row * D + e] = NAN;
    if (threadIdx.x == 0) {
      p.part_ml[2 * row] = NAN;
      p.part_ml[2 * row + 1] = NAN;
    }
  }
}

// Decodes blockIdx into the wave's task and validates lengths and table
// entries.  Returns false when the wave has nothing to do (it may have
// written NaN rows for an invalid sequence first).
template <typename T, int D>
__device__ __forceinline__ bool setup_task(const DecodeParams& p, WaveTask& w) {
  const int lane = threadIdx.x;
  w.kvh = blockIdx.x % p.Hkv;
  const int rest = blockIdx.x / p.Hkv;
  w.s = rest % p.S;
  w.part = rest / p.S;
  w.h0 = w.kvh * p.G + blockIdx.y * 16;
  w.nh = min(16, p.G - static_cast<int>(blockIdx.y) * 16);
  w.n = p.seq_lens[w.s];
  if (w.n < 1 || w.n > p.max_seq_len) {
    if (w.part == 0) write_nan_rows<T, D>(p, w.s, w.h0, w.nh);
    return false;
  }
  w.P = (w.n + p.partition - 1) / p.partition;
  if (w.part >= w.P) return false;
  const int t_begin = w.part * p.partition;
  w.t_end = min(w.n, t_begin + p.partition);
  w.blk_first = t_begin / kBlock;
  w.nblk = (w.t_end - t_begin + kBlock - 1) / kBlock;
  bool bad = w.blk_first + w.nblk > p.max_blocks;
  int b = 0;
  if (!bad && lane < w.nblk) b = p.block_tables[static_cast<size_t>(w.s) * p.max_blocks + w.blk_first + lane];
  const bool bad_lane = static_cast<unsigned>(b) >= static_cast<unsigned>(p.num_blocks);
  bad = bad || __any(bad_lane);
  w.myblk = bad_lane ? 0 : b;
  if (bad) {
    if (w.P == 1) write_nan_rows<T, D>(p, w.s, w.h0, w.nh);
    else write_nan_partials<D>(p, w);
    return false;
  }
  return true;
}

__device__ __forceinline__ int block_id(const WaveTask& w, int i) {
  return __builtin_amdgcn_readlane(w.myblk, i);
}

// ---------------------------------------------------------------------------
// decode_partial, bf16: v_mfma_f32_16x16x32_bf16
//
// Per pair of blocks (32 tokens), with lane l = 16*g + c (g = l/16,
// c = l%16):
//   S^T = K · Q^T: A = K tile (row = token c, k = 8 head-dim values of chunk
//   g), B = Q^T (column = head c, same k).  Result lane l holds the scores
//   of tokens 4g..4g+3 for head c.
//   out^T += V^T · P: A = V^T (row = value column c of the tile, k = the
//   lane's 8 tokens: 4g..4g+3 of the first block and of the second), B = P
//   (the lane's own 8 probabilities, same token order, head c).  Result lane
//   l holds value columns 16t+4g..16t+4g+3 of head c for tile t.
// The token order inside the k dimension is the same on both operands, so
// no data moves between lanes except the max / sum reductions.
// ---------------------------------------------------------------------------
template <int D>
struct PairRegs {
  u32x4 k0[D / 32], k1[D / 32];
  u32x2 v0[D / 16], v1[D / 16];
};

template <int D>
__global__ __launch_bounds__(64) void decode_partial_bf16(DecodeParams p) {
  constexpr int KC = D / 32;
  constexpr int NT = D / 16;
  WaveTask w;
  if (!setup_task<__bf16, D>(p, w)) return;
  const int lane = threadIdx.x;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;

  // Q^T operand: head c16, head-dim values 32c + 8g4 .. +7.
  bf16x8 qreg[KC];
  {
    const __bf16* q = static_cast<const __bf16*>(p.q) + (static_cast<size_t>(w.s) * p.Hq + w.h0 + c16) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4 v = {0, 0, 0, 0};
      if (c16 < w.nh) v = *reinterpret_cast<const u32x4*>(q + 32 * c + 8 * g4);
      qreg[c] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const size_t tile = static_cast<size_t>(kBlock) * D;               // elements per (block, head)
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * tile;
  const __bf16* kc = static_cast<const __bf16*>(p.k_cache) + static_cast<size_t>(w.kvh) * tile;
  const __bf16* vc = static_cast<const __bf16*>(p.v_cache) + static_cast<size_t>(w.kvh) * tile;
  const int npair = (w.nblk + 1) / 2;

  auto load_pair = [&](PairRegs<D>& r, int i) {
    const int b0 = block_id(w, 2 * i);
    const int b1 = (2 * i + 1 < w.nblk) ? block_id(w, 2 * i + 1) : b0;
    const u32x4* k0 = reinterpret_cast<const u32x4*>(kc + b0 * blk_stride) + lane;
    const u32x4* k1 = reinterpret_cast<const u32x4*>(kc + b1 * blk_stride) + lane;
    const u32x2* v0 = reinterpret_cast<const u32x2*>(vc + b0 * blk_stride) + c16 * 4 + g4;
    const u32x2* v1 = reinterpret_cast<const u32x2*>(vc + b1 * blk_stride) + c16 * 4 + g4;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      r.k0[c] = k0[64 * c];
      r.k1[c] = k1[64 * c];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      r.v0[t] = v0[64 * t];
      r.v1[t] = v1[64 * t];
    }
  };

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  auto compute_pair = [&](const PairRegs<D>& r, int i) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
    f32x4 s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.k0[c]), qreg[c], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.k1[c]), qreg[c], s1, 0, 0, 0);
    }
    const int tok0 = (w.blk_first + 2 * i) * kBlock + 4 * g4;     // token of x[0]
    const bool tail = (w.blk_first + 2 * i + 2) * kBlock > w.t_end;
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = s0[j] * p.scale_log2;
      x[4 + j] = s1[j] * p.scale_log2;
    }
    if (tail) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (tok0 + j >= w.t_end) x[j] = -INFINITY;
        if (tok0 + kBlock + j >= w.t_end) x[4 + j] = -INFINITY;
      }
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
    mx = max_over_rows(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2_fast(m_run - m_new);
    m_run = m_new;
    bf16x8 pb;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const __bf16 e = static_cast<__bf16>(exp2_fast(x[j] - m_new));
      pb[j] = e;
      ps += static_cast<float>(e);
    }
    l_run = l_run * alpha + ps;
    uint32_t mk0 = 0xFFFFFFFFu, mk1 = 0xFFFFFFFFu, mk2 = 0xFFFFFFFFu, mk3 = 0xFFFFFFFFu;
    if (tail) {
      auto half = [&](int tok) -> uint32_t { return tok < w.t_end ? 0xFFFFu : 0u; };
      mk0 = half(tok0) | (half(tok0 + 1) << 16);
      mk1 = half(tok0 + 2) | (half(tok0 + 3) << 16);
      mk2 = half(tok0 + kBlock) | (half(tok0 + kBlock + 1) << 16);
      mk3 = half(tok0 + kBlock + 2) | (half(tok0 + kBlock + 3) << 16);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc[t] *= alpha;
      const u32x4 vv = {r.v0[t].x & mk0, r.v0[t].y & mk1, r.v1[t].x & mk2, r.v1[t].y & mk3};
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pb, acc[t], 0, 0, 0);
    }
  };

  // Two register sets: the next pair's loads are in flight while the current
  // pair is computed.
  PairRegs<D> ra, rb;
  load_pair(ra, 0);
  for (int i = 0; i < npair; i += 2) {
    if (i + 1 < npair) load_pair(rb, i + 1);
    compute_pair(ra, i);
    if (i + 1 >= npair) break;
    if (i + 2 < npair) load_pair(ra, i + 2);
    compute_pair(rb, i + 1);
  }

  const float l_tot = sum_over_rows(l_run);
  if (c16 >= w.nh) return;
  const size_t head_row = static_cast<size_t>(w.s) * p.Hq + w.h0 + c16;
  if (w.P == 1) {
    const float inv = 1.f / l_tot;
    __bf16* out = static_cast<__bf16*>(p.out) + head_row * D + 4 * g4;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = static_cast<__bf16>(acc[t][j] * inv);
      *reinterpret_cast<bf16x4*>(out + 16 * t) = o;
    }
  } else {
    const size_t row = head_row * p.pmax + w.part;
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
  WaveTask w;
  if (!setup_task<float, D>(p, w)) return;
  const int lane = threadIdx.x;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;

  f32x4 qreg[KC];
  {
    const float* q = static_cast<const float*>(p.q) + (static_cast<size_t>(w.s) * p.Hq + w.h0 + c16) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (c16 < w.nh) v = *reinterpret_cast<const f32x4*>(q + 16 * c + 4 * g4);
      qreg[c] = v;
    }
  }
  const size_t tile = static_cast<size_t>(kBlock) * D;
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * tile;
  const float* kc = static_cast<const float*>(p.k_cache) + static_cast<size_t>(w.kvh) * tile;
  const float* vc = static_cast<const float*>(p.v_cache) + static_cast<size_t>(w.kvh) * tile;

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  for (int i = 0; i < w.nblk; ++i) {
    const int b = block_id(w, i);
    const f32x4* kp = reinterpret_cast<const f32x4*>(kc + b * blk_stride) + lane;
    const f32x4* vp = reinterpret_cast<const f32x4*>(vc + b * blk_stride) + c16 * 4 + g4;
    f32x4 kr[KC], vr[NT];
#pragma unroll
    for (int c = 0; c < KC; ++c) kr[c] = kp[64 * c];
#pragma unroll
    for (int t = 0; t < NT; ++t) vr[t] = vp[64 * t];
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) sc = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[c][j], qreg[c][j], sc, 0, 0, 0);
    const int tok0 = (w.blk_first + i) * kBlock + 4 * g4;
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = (tok0 + j < w.t_end) ? sc[j] * p.scale_log2 : -INFINITY;
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
        const float v = (tok0 + j < w.t_end) ? vr[t][j] : 0.f;
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, pr[j], acc[t], 0, 0, 0);
      }
    }
  }

  const float l_tot = sum_over_rows(l_run);
  if (c16 >= w.nh) return;
  const size_t head_row = static_cast<size_t>(w.s) * p.Hq + w.h0 + c16;
  if (w.P == 1) {
    const float inv = 1.f / l_tot;
    float* out = static_cast<float*>(p.out) + head_row * D + 4 * g4;
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(out + 16 * t) = acc[t] * inv;
  } else {
    const size_t row = head_row * p.pmax + w.part;
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
// decode_reduce: one wave per (sequence, query head) with more than one
// partition.  M = max_p m_p, L = sum_p l_p 2^(m_p - M),
// out = sum_p acc_p 2^(m_p - M) / L, rounded to the output type.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeParams p) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const int s = row / p.Hq;
  const int n = p.seq_lens[s];
  if (n < 1 || n > p.max_seq_len) return;
  const int P = (n + p.partition - 1) / p.partition;
  if (P <= 1) return;
  const float* ml = p.part_ml + static_cast<size_t>(row) * p.pmax * 2;
  const float* acc = p.part_acc + static_cast<size_t>(row) * p.pmax * D;
  float M = -INFINITY;
  for (int i = lane; i < P; i += 64) M = fmaxf(M, ml[2 * i]);
  M = wave_max(M);
  float L = 0.f;
  for (int i = lane; i < P; i += 64) L += ml[2 * i + 1] * exp2_fast(ml[2 * i] - M);
  L = wave_sum(L);
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int base = 0; base < P; base += 64) {
    const float wl = (base + lane < P) ? exp2_fast(ml[2 * (base + lane)] - M) : 0.f;
    const int cnt = min(64, P - base);
    for (int j = 0; j < cnt; ++j) {
      const float wj = lane_value(wl, j);
      const float* a = acc + static_cast<size_t>(base + j) * D + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] += wj * a[e];
    }
  }
  const float inv = 1.f / L;
  T* out = static_cast<T*>(p.out) + static_cast<size_t>(row) * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = static_cast<T>(o[e] * inv);
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t stream) {
  if (p.n_pairs <= 0 || p.n_layers <= 0) return hipSuccess;
  dim3 grid(p.n_pairs, p.n_layers, 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream) {
  if (p.n <= 0) return hipSuccess;
  dim3 grid(p.n, p.num_kv_heads);
  if (p.elem_bytes == 4)
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

bool decode_shape_supported(int dtype, int head_dim, int block_size) {
  return block_size == kBlock && (dtype == 0 || dtype == 1) && (head_dim == 64 || head_dim == 128);
}

hipError_t launch_decode_partial(const DecodeParams& p, int dtype, hipStream_t stream) {
  const long long gx = static_cast<long long>(p.pmax) * p.S * p.Hkv;
  dim3 grid(static_cast<unsigned>(gx), (p.G + 15) / 16);
  if (dtype == 1) {
    if (p.d == 128) hipLaunchKernelGGL(decode_partial_bf16<128>, grid, dim3(64), 0, stream, p);
    else if (p.d == 64) hipLaunchKernelGGL(decode_partial_bf16<64>, grid, dim3(64), 0, stream, p);
    else return hipErrorInvalidValue;
  } else {
    if (p.d == 128) hipLaunchKernelGGL(decode_partial_f32<128>, grid, dim3(64), 0, stream, p);
    else if (p.d == 64) hipLaunchKernelGGL(decode_partial_f32<64>, grid, dim3(64), 0, stream, p);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeParams& p, int dtype, hipStream_t stream) {
  if (p.pmax <= 1) return hipSuccess;
  dim3 grid(static_cast<unsigned>(p.S * p.Hq));
  if (dtype == 1) {
    if (p.d == 128) hipLaunchKernelGGL((decode_reduce_kernel<__bf16, 128>), grid, dim3(64), 0, stream, p);
    else if (p.d == 64) hipLaunchKernelGGL((decode_reduce_kernel<__bf16, 64>), grid, dim3(64), 0, stream, p);
    else return hipErrorInvalidValue;
  } else {
    if (p.d == 128) hipLaunchKernelGGL((decode_reduce_kernel<float, 128>), grid, dim3(64), 0, stream, p);
    else if (p.d == 64) hipLaunchKernelGGL((decode_reduce_kernel<float, 64>), grid, dim3(64), 0, stream, p);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
