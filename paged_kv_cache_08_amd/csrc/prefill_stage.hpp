// Paged prefill over an 8-bit (E4M3) cache: the blocks the prefill may read
// are first dequantised into a bf16 copy in the caller's workspace, laid out
// as a bf16 pool, with tables of their own; the bf16 prefill kernel then runs
// on that copy.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace pkv {

struct PrefillStageParams {
  const uint8_t* k_cache;        // 8-bit pool, one layer: K codes [num_blocks][Hkv][d/16][B][16]
  const uint8_t* v_cache;        // V codes [num_blocks][Hkv][d/64][B/4][16][4][4]
  const float* k_scale;          // [num_blocks][Hkv][B]
  const float* v_scale;
  const int32_t* block_tables;   // [S][max_blocks]
  const int32_t* seq_lens;       // [S]
  const int32_t* query_start;    // [S + 1]: with a window, blocks before every query's window are skipped
  int32_t window;                // > 0: sliding window of the prefill
  int32_t S, Hkv, d;
  int32_t num_blocks, max_blocks, max_seq_len;
  int32_t nb;                    // copy blocks per sequence: ceil(max_seq_len / B)
  int32_t* tables_out;           // [S][max_blocks]: copy block s * nb + j, or -1 for a block id outside the pool
  __bf16* k_out;                 // [S * nb][Hkv][d/8][B][8]
  __bf16* v_out;                 // [S * nb][Hkv][B/4][d/4][4][4]
};

// Workspace bytes: the copy's tables, then its K and V blocks (each part
// 256-byte aligned).
size_t prefill_stage_bytes(int64_t S, int64_t Hkv, int64_t d, int64_t max_blocks, int64_t nb);
// Points the copy's arrays into a workspace of prefill_stage_bytes() bytes.
void prefill_stage_layout(PrefillStageParams* p, void* workspace);
hipError_t launch_prefill_stage(const PrefillStageParams& p, hipStream_t stream);

}  // namespace pkv
