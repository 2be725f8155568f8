// Host-side launchers of the HIP kernels (defined in kernels.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <hip/amd_detail/host_defines.h>

#include <cstddef>
#include <cstdint>

namespace pkv {

// Copy-on-write block copies for up to kCopyMaxLayers layers and
// kCopyMaxPairs pairs per launch (the caller chunks larger requests).
constexpr int kCopyMaxLayers = 32;
constexpr int kCopyMaxPairs = 64;

struct CopyBlocksParams {
  void* k[kCopyMaxLayers];
  void* v[kCopyMaxLayers];
  void* ks[kCopyMaxLayers];   // 8-bit pools: per-slot scales of K and V
  void* vs[kCopyMaxLayers];
  int32_t pairs[2 * kCopyMaxPairs];
  int32_t n_layers;
  int32_t n_pairs;
  int64_t block_bytes;   // bytes of one block (all heads) in one layer's K or V
  int64_t scale_bytes;   // bytes of one block's scales (0: no scale arrays)
};

struct AppendParams {
  const void* k_new;
  const void* v_new;
  const int32_t* slots;          // slot per token, or null: derive it from
  const int32_t* tables;         //   tables[i][(lens[i]-1) / B] (decode step)
  const int32_t* lens;
  int32_t max_blocks;
  void* k_cache;
  void* v_cache;
  int64_t num_slots;     // num_blocks * block_size
  int32_t n;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t elem_bytes;    // 4 (fp32) or 2 (bf16) of the pool; 1: 8-bit pool
  float* k_scale;        // 8-bit pool: per-slot scales [block][head][B]
  float* v_scale;
};

// Work list of a decode launch with one partition per wave, built on the
// host from the caller's length hint (P_h(s) = the hint's partition count of
// sequence s, at least 1).  The grid then holds only the cells the hint
// calls non-empty, largest first, instead of every (partition, sequence)
// cell up to max_seq_len; whatever the hint says, every partition the device
// lengths imply is still computed exactly once.  Partitions are numbered as
// the kernel numbers them (with a window, from the first one that overlaps
// it).  Ranks number the sequences by hinted partition count, most first;
// wave k takes:
//  - k < n_full: a partition before its sequence's last, group-major:
//    partition g of rank k - full_start[g] (full_start[g+1] - full_start[g]
//    ranks have more than g + 1 partitions);
//  - then, up to n_full + n_partial: each sequence's last partition, largest
//    first: partial[j] = rank | g << 9 (a sequence the hint calls empty lists
//    partition 0 here, last);
//  - then the sweep: for s = j % S and chunk c = sweep_c0 + j / S, the
//    partitions of [c * run_cap, (c + 1) * run_cap) from P_h(s) - 1 + run_cap
//    on, as one run; a chunk that the hint already covers exits before
//    touching memory.
// The wave of a sequence's last hinted partition (its partial entry, g =
// P_h(s) - 1) also takes the partitions up to g + run_cap - 1 that the
// device length holds (one run, staged as usual).  The launcher sets run_cap (a run's capacity) and
// the sweep chunks.
constexpr int kOrderMaxSeqs = 512;
constexpr int kOrderMaxGroups = 128;
struct DecodeOrder {
  int32_t active;
  int32_t n_full, n_partial;
  int32_t run_cap;
  int32_t sweep_c0, sweep_chunks;
  int32_t full_start[kOrderMaxGroups + 1];
  uint16_t rank_seq[kOrderMaxSeqs];     // sequence of each rank
  uint16_t partial[kOrderMaxSeqs];
  uint8_t hinted[kOrderMaxSeqs];        // P_h(s)
};

struct DecodeParams {
  const void* q;
  void* out;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const float* k_scale;  // 8-bit cache: per-slot scales [block][head][B]
  const float* v_scale;
  const void* k_new;     // fused append: the step's new token [S][Hkv][d] (bf16 for an
  const void* v_new;     //   8-bit cache), written at position seq_lens[s] - 1; or null
  float* part_ml;        // [S][Hq][Pmax][2]   (running max in log2 units, sum)
  float* part_acc;       // [S][Hq][Pmax][d]   unnormalised accumulators
  int32_t S, Hq, Hkv, G, d;
  int32_t num_blocks, max_blocks, max_seq_len;
  int32_t window;        // > 0: attend to the last `window` positions only
  int32_t partition, pmax;
  int32_t ppw;           // partitions streamed per wave (set by the launcher)
  int32_t groups;        // runs per (sequence, KV head, head group); the last takes the rest
  int64_t tasks_hint;    // exact (sequence, KV head, head group, partition) count, 0 = unknown
  int32_t uniform_hint;  // 1 if every sequence attends to about the same number of tokens
  float scale_log2;      // scale * log2(e): scores are kept in base-2 units
  DecodeOrder order;     // used by the partial kernel when order.active and ppw == 1
};

// Grid cell `cell` of a decode partial launch (blockIdx.x / Hkv): its
// sequence s and partitions [part0, part_lim) before the device length
// clips them (numbered from the window's first partition with a window).
// False for a sweep cell that the hint's cells already cover (the wave exits
// before touching memory).  Shared by the kernel and the host's launch plan.
__host__ __device__ inline bool decode_cell(const DecodeParams& p, int cell, int& s, int& part0, int& part_lim) {
  if (p.order.active) {
    const DecodeOrder& o = p.order;
    if (cell < o.n_full) {
      int g = 0;
      while (g < kOrderMaxGroups - 1 && o.full_start[g + 1] <= cell) ++g;
      s = o.rank_seq[cell - o.full_start[g]];
      part0 = g;
      part_lim = part0 + 1;
    } else if (cell < o.n_full + o.n_partial) {
      const int e = o.partial[cell - o.n_full];
      s = o.rank_seq[e & 511];
      part0 = e >> 9;
      part_lim = part0 + o.run_cap;                  // the sequence's last hinted partition
    } else {
      const int j = cell - o.n_full - o.n_partial;
      s = j % p.S;
      const int c = o.sweep_c0 + j / p.S;
      part0 = c * o.run_cap;
      const int from = o.hinted[s] - 1 + o.run_cap;
      if (from > part0) part0 = from;
      part_lim = (c + 1) * o.run_cap;
      if (part0 >= part_lim || part0 >= p.pmax) return false;
    }
  } else {
    s = cell % p.S;
    const int grp = cell / p.S;
    part0 = grp * p.ppw;
    part_lim = grp == p.groups - 1 ? p.pmax : part0 + p.ppw;     // the last run takes the rest
  }
  if (part_lim > p.pmax) part_lim = p.pmax;
  return true;
}

struct PrefillParams {
  const void* q;                 // [T][Hq][d] bf16, sequence s's rows from query_start[s]
  void* out;                     // [T][Hq][d] bf16
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;   // [S][max_blocks]
  const int32_t* seq_lens;       // [S] tokens in the cache, the chunk included
  const int32_t* query_start;    // [S + 1] prefix sums of the chunk lengths
  int32_t S, Hq, Hkv, G, d;
  int32_t num_blocks, max_blocks, max_seq_len, max_query_len;
  int32_t window;                // > 0: a query attends to its last `window` positions
  float scale_log2;
};

hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
bool prefill_shape_supported(int head_dim, int block_size);
// Copies n_tab table entries and n_len lengths from a device-visible pinned
// host buffer (tables first, lengths right after) into device arrays.
hipError_t launch_table_upload(const int32_t* host_src, int32_t* dev_tables, int64_t n_tab, int32_t* dev_lens,
                               int32_t n_len, hipStream_t stream);
hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream);
// Decode kernel families.  Returns hipErrorInvalidValue for shapes without a
// kernel (checked by the caller first).
enum DecodeKind : int {
  kDecodeF32 = 0,      // fp32 queries, fp32 cache
  kDecodeBF16 = 1,     // bf16 queries, bf16 cache
  kDecodeFP8KV = 2,    // bf16 queries, 8-bit E4M3 cache with per-slot scales
};
hipError_t launch_decode_partial(const DecodeParams& p, int kind, hipStream_t stream);
// A decode partial launch as launch_decode_partial would make it, without
// launching: the kernel variant, the grid and the parameters with the runs
// and the work list settled (plan->params; decode_cell() maps its cells).
struct DecodeLaunchPlan {
  DecodeParams params;
  long long cells;       // grid x = cells * Hkv
  int grid_y;            // query-head groups of 16
  int depth;             // blocks in flight per wave (the pipeline variant)
  int resident_waves;    // wave slots of that variant on the device
  int max_wave_blocks;   // most blocks one wave may stream
  size_t lds_bytes;      // dynamic LDS per wave for staged partials
};
hipError_t plan_decode_partial(const DecodeParams& p, int kind, DecodeLaunchPlan* plan);
hipError_t launch_decode_reduce(const DecodeParams& p, int kind, hipStream_t stream);
// The library's own decode workspace for callers that cannot allocate: a
// device array of kStaticWorkspaceBytes in the library's code object, one
// per device.  static_workspace() gives its address on the current device
// (looked up on the first call on each device).
constexpr size_t kStaticWorkspaceBytes = size_t(64) << 20;
hipError_t static_workspace(void** ptr);
bool decode_shape_supported(int kind, int head_dim, int block_size);
// Read-bandwidth calibration: wave w reads tiles order[w*tpw ...] (or
// w*tpw ... without an order) of tile_bytes (2048 or 4096) each and writes
// the xor of what each lane read to sink[w*64 + lane].
hipError_t launch_read_tiles(const void* base, int64_t base_tiles, int tile_bytes, const int32_t* order,
                             int64_t n_tiles, int tiles_per_wave, uint32_t* sink, hipStream_t stream);

}  // namespace pkv
