// Read-bandwidth calibration: how fast can this GPU read the bytes a decode
// launch reads, with the attention arithmetic taken away?
//
// The decode partial kernel reads each sequence's KV cache as tiles of 16
// tokens of one KV head (4 KiB at d = 128 in bf16, 2 KiB in 8-bit codes or
// at d = 64 in bf16, 1 KiB in 8-bit codes at d = 64)
// scattered through the pool in block-table order.  This kernel reads the same kind of tiles from a buffer,
// in an order given by the caller (a seeded permutation for the gather, none
// for a contiguous stream), with non-temporal 16-byte loads and nothing else
// per byte than an xor, so its rate is the ceiling that access pattern allows
// on the device.  The xor of everything a lane read goes to a sink so that no
// load can be dropped, and a test can check it on the host.
#include "device_util.hpp"
#include "kernels.hpp"

namespace pkv {

namespace {

constexpr int kReadDepth = 8;                       // tiles in flight per wave

__device__ __forceinline__ int64_t tile_id(const int32_t* order, int64_t i) {
  return order ? static_cast<int64_t>(order[i]) : i;
}

// kTileVecs: 16-byte vectors per tile (256, 128 or 64 for 4, 2 or 1 KiB); lane l
// reads vectors l, l + 64, ... of each tile.
template <int kTileVecs>
__global__ __launch_bounds__(64) void read_tiles_kernel(const u32x4* __restrict__ base, int64_t base_tiles,
                                                        const int32_t* __restrict__ order, int64_t n_tiles,
                                                        int tiles_per_wave, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * tiles_per_wave;
  const int cnt = static_cast<int>(min<int64_t>(tiles_per_wave, n_tiles - first));
  u32x4 acc = {0u, 0u, 0u, 0u};
  int i = 0;
  for (; i + kReadDepth <= cnt; i += kReadDepth) {
    int64_t t[kReadDepth];
#pragma unroll
    for (int u = 0; u < kReadDepth; ++u) t[u] = tile_id(order, first + i + u);
    // An id outside the buffer reads tile 0 and is masked out of the xor, so
    // every load is issued unconditionally, one after the other.
    u32x4 v[kReadDepth][kTileVecs / 64];
    uint32_t keep[kReadDepth];
#pragma unroll
    for (int u = 0; u < kReadDepth; ++u) {
      const bool ok = t[u] >= 0 && t[u] < base_tiles;
      keep[u] = ok ? ~0u : 0u;
      const u32x4* src = base + (ok ? t[u] : 0) * kTileVecs + lane;
#pragma unroll
      for (int c = 0; c < kTileVecs / 64; ++c) v[u][c] = __builtin_nontemporal_load(src + 64 * c);
    }
    __builtin_amdgcn_sched_barrier(0);        // all loads leave before the first is consumed
#pragma unroll
    for (int u = 0; u < kReadDepth; ++u)
#pragma unroll
      for (int c = 0; c < kTileVecs / 64; ++c) acc ^= v[u][c] & keep[u];
  }
  for (; i < cnt; ++i) {
    const int64_t t = tile_id(order, first + i);
    if (t < 0 || t >= base_tiles) continue;
    const u32x4* src = base + t * kTileVecs + lane;
#pragma unroll
    for (int c = 0; c < kTileVecs / 64; ++c) acc ^= __builtin_nontemporal_load(src + 64 * c);
  }
  sink[static_cast<int64_t>(blockIdx.x) * 64 + lane] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

hipError_t launch_read_tiles(const void* base, int64_t base_tiles, int tile_bytes, const int32_t* order,
                             int64_t n_tiles, int tiles_per_wave, uint32_t* sink, hipStream_t stream) {
  const int64_t waves = (n_tiles + tiles_per_wave - 1) / tiles_per_wave;
  const dim3 grid(static_cast<unsigned>(waves));
  const u32x4* b = static_cast<const u32x4*>(base);
  if (tile_bytes == 4096)
    hipLaunchKernelGGL(read_tiles_kernel<256>, grid, dim3(64), 0, stream, b, base_tiles, order, n_tiles,
                       tiles_per_wave, sink);
  else if (tile_bytes == 2048)
    hipLaunchKernelGGL(read_tiles_kernel<128>, grid, dim3(64), 0, stream, b, base_tiles, order, n_tiles,
                       tiles_per_wave, sink);
  else if (tile_bytes == 1024)
    hipLaunchKernelGGL(read_tiles_kernel<64>, grid, dim3(64), 0, stream, b, base_tiles, order, n_tiles,
                       tiles_per_wave, sink);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
