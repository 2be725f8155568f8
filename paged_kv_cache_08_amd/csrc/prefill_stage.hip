// Dequantising copy of an 8-bit (E4M3) cache for the paged prefill kernel.
//
// «¿Cuánta memoria reservar para la caché KV?», "Reducir la precisión": an
// 8-bit cache stores codes and per-(token, KV head) scales; a value is its
// code times its scale.  The prefill kernel reads bf16 tiles, so for a
// prefill over an 8-bit cache every block a sequence holds is first written
// as bf16 (code × scale in fp32, rounded to nearest even) into a copy laid
// out as a bf16 pool: copy block s * nb + j holds block j of sequence s.
// Slots past a sequence's length become zeros; with a sliding window, blocks
// that lie wholly before the first query's window are skipped (the prefill
// reads neither them nor their table entries).  A block id outside the pool
// becomes -1 in the copy's table, so the prefill writes NaN rows wherever it
// would have read that block, as it does on a bf16 cache.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_util.hpp"
#include "prefill_stage.hpp"

namespace pkv {
namespace {

constexpr int kTok = 16;   // tokens per cache block

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Sixteen E4M3 codes (four words, bytes in order) to fp32 by the hardware
// conversion, which is exact.
__device__ __forceinline__ void decode16(const u32x4& w, float (&f)[16]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int word = static_cast<int>(w[k]);
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);   // bytes 0, 1
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);    // bytes 2, 3
    f[4 * k + 0] = lo[0];
    f[4 * k + 1] = lo[1];
    f[4 * k + 2] = hi[0];
    f[4 * k + 3] = hi[1];
  }
}

// One workgroup per (sequence s, block j, KV head g), 2·d threads: thread i
// < d converts K chunk i (16 head-dim values of one token), thread d + i V
// chunk i (four value columns of four tokens).
__global__ __launch_bounds__(256) void prefill_stage_kernel(PrefillStageParams p) {
  const int x = blockIdx.x;                        // s * nb + j: the copy block
  const int s = x / p.nb;
  const int j = x - s * p.nb;
  const int g = blockIdx.y;
  const int n = p.seq_lens[s];
  if (n < 1 || n > p.max_seq_len || j * kTok >= n) return;     // a block the prefill never reads
  if (p.window > 0) {            // nor one wholly before the first query's window (its entry stays unwritten)
    const int first = n - (p.query_start[s + 1] - p.query_start[s]);
    if ((j + 1) * kTok <= first - p.window + 1) return;
  }
  const int32_t b = p.block_tables[static_cast<size_t>(s) * p.max_blocks + j];
  const bool ok = b >= 0 && b < p.num_blocks;
  if (g == 0 && threadIdx.x == 0) p.tables_out[static_cast<size_t>(s) * p.max_blocks + j] = ok ? x : -1;
  if (!ok) return;
  const int t_end = min(kTok, n - j * kTok);       // written slots of the block
  const int d = p.d;
  const int tid = threadIdx.x;
  const size_t tile = static_cast<size_t>(kTok) * d;                     // values of one (block, head) tile
  const size_t src = (static_cast<size_t>(b) * p.Hkv + g) * tile;        // bytes (codes)
  const size_t dst = (static_cast<size_t>(x) * p.Hkv + g) * tile;        // bf16 elements
  const size_t srow = (static_cast<size_t>(b) * p.Hkv + g) * kTok;       // scales of the tile's slots
  float f[16];
  if (tid < d) {
    // K codes [d/16][B][16]: chunk tid = (c, t) holds head dims 16c .. 16c+15
    // of slot t; bf16 K [d/8][B][8]: chunks (2c, t) and (2c + 1, t).
    const int c = tid >> 4, t = tid & 15;
    decode16(*reinterpret_cast<const u32x4*>(p.k_cache + src + static_cast<size_t>(tid) * 16), f);
    const float sc = t < t_end ? p.k_scale[srow + t] : 0.f;
    bf16x8 lo, hi;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = static_cast<__bf16>(f[e] * sc);
      hi[e] = static_cast<__bf16>(f[8 + e] * sc);
    }
    if (t >= t_end) lo = hi = bf16x8{};                                 // free slots: zeros, whatever they hold
    __bf16* k = p.k_out + dst;
    *reinterpret_cast<bf16x8*>(k + (static_cast<size_t>(2 * c) * kTok + t) * 8) = lo;
    *reinterpret_cast<bf16x8*>(k + (static_cast<size_t>(2 * c + 1) * kTok + t) * 8) = hi;
  } else if (tid < 2 * d) {
    // V codes [d/64][B/4][16][4][4]: chunk i = (a, u, c) holds columns
    // 64a + 4c + b (b = 0..3) of slots 4u + w (w = 0..3), byte 4b + w.  The
    // bf16 V [B/4][d/4][4][4] keeps the same [b][w] order in its run
    // (u, 16a + c), so the chunk becomes one 32-byte run.
    const int i = tid - d;
    const int a = i >> 6, u = (i >> 4) & 3, c = i & 15;
    decode16(*reinterpret_cast<const u32x4*>(p.v_cache + src + static_cast<size_t>(i) * 16), f);
    float sc[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) sc[w] = 4 * u + w < t_end ? p.v_scale[srow + 4 * u + w] : 0.f;
    bf16x8 lo, hi;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = 4 * u + (e & 3) < t_end ? static_cast<__bf16>(f[e] * sc[e & 3]) : static_cast<__bf16>(0.f);
      hi[e] = 4 * u + (e & 3) < t_end ? static_cast<__bf16>(f[8 + e] * sc[e & 3]) : static_cast<__bf16>(0.f);
    }
    __bf16* v = p.v_out + dst + (static_cast<size_t>(u) * (d / 4) + 16 * a + c) * 16;
    *reinterpret_cast<bf16x8*>(v) = lo;
    *reinterpret_cast<bf16x8*>(v + 8) = hi;
  }
}

}  // namespace

size_t prefill_stage_bytes(int64_t S, int64_t Hkv, int64_t d, int64_t max_blocks, int64_t nb) {
  const size_t tables = align256(static_cast<size_t>(S) * max_blocks * sizeof(int32_t));
  const size_t copy = align256(static_cast<size_t>(S) * nb * Hkv * kTok * d * sizeof(uint16_t));
  return tables + 2 * copy;
}

void prefill_stage_layout(PrefillStageParams* p, void* workspace) {
  const size_t tables = align256(static_cast<size_t>(p->S) * p->max_blocks * sizeof(int32_t));
  const size_t copy = align256(static_cast<size_t>(p->S) * p->nb * p->Hkv * kTok * p->d * sizeof(uint16_t));
  char* w = static_cast<char*>(workspace);
  p->tables_out = reinterpret_cast<int32_t*>(w);
  p->k_out = reinterpret_cast<__bf16*>(w + tables);
  p->v_out = reinterpret_cast<__bf16*>(w + tables + copy);
}

hipError_t launch_prefill_stage(const PrefillStageParams& p, hipStream_t stream) {
  if (p.d != 64 && p.d != 128) return hipErrorInvalidValue;
  const int64_t blocks = static_cast<int64_t>(p.S) * p.nb;
  if (blocks < 1) return hipSuccess;
  if (blocks > 0x7fffffffLL || p.Hkv > 65535) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(p.Hkv));
  hipLaunchKernelGGL(prefill_stage_kernel, grid, dim3(2 * p.d), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
