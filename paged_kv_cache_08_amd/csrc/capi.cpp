// C ABI of the paged KV cache library (declared in include/pkv.h).
//
// Argument checking, allocator calls and kernel launches.  No C++ exception
// leaves this file: every entry point catches and returns a status.
#include "pkv.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <array>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <new>
#include <string>
#include <vector>

#include "block_pool.hpp"
#include "kernels.hpp"
#include "prefill_stage.hpp"

struct pkv_pool {
  pkv::BlockPool alloc;
  int32_t num_layers, num_kv_heads, head_dim, dtype;
  std::vector<void*> k_cache, v_cache;    // empty for an allocator-only pool
  std::vector<void*> k_scale, v_scale;    // 8-bit pools: per-slot scales
  // Pinned staging buffers for table uploads, a ring: upload u fills buffer
  // u % kStagingRing.  Uploads form groups of kUploadsPerEvent, and events
  // mark a group's end (one per run of uploads on one stream), so a stream
  // holds one event marker per group rather than one per upload: a marker
  // between an upload and the next kernel leaves the GPU idle for about
  // 4.5 us.  A buffer is refilled only after the events of the group that
  // last used it have completed.
  static constexpr int kStagingRing = 8;
  static constexpr int kUploadsPerEvent = 4;
  struct UploadGroup {
    hipEvent_t ev[kUploadsPerEvent] = {};
    int n_ev = 0;                 // events recorded for the group
    bool pending = false;
  };
  void* staging[kStagingRing] = {};
  size_t staging_bytes[kStagingRing] = {};
  UploadGroup groups[kStagingRing / kUploadsPerEvent];
  uint64_t uploads = 0;           // uploads launched so far
  hipStream_t last_stream = nullptr;

  pkv_pool(int32_t nb, int32_t bs, const int32_t* perm) : alloc(nb, bs, perm) {}
};

namespace {

thread_local std::string g_error;

int fail(int status, const std::string& msg) {
  g_error = msg;
  return status;
}

int from_alloc(pkv::Status st, const pkv_pool* pool) {
  if (st == pkv::Status::Ok) return PKV_OK;
  g_error = pool->alloc.error();
  return static_cast<int>(st);
}

int from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Bytes per cached value.
int elem_bytes(int32_t dtype) { return dtype == PKV_F32 ? 4 : dtype == PKV_BF16 ? 2 : 1; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename F>
int guarded(F&& f) {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return fail(PKV_ERR_INVALID, "host allocation failed");
  } catch (const std::exception& e) {
    return fail(PKV_ERR_INVALID, e.what());
  } catch (...) {
    return fail(PKV_ERR_INVALID, "unknown error");
  }
}

int32_t effective_partition(int32_t partition) { return partition == 0 ? 512 : partition; }

// Partitions a sequence of up to max_len tokens can touch: all of them, or
// with a window of W tokens at most floor((W - 2) / part) + 2 (the window may
// start just before a partition boundary).
int64_t partitions_bound(int32_t max_len, int32_t part, int32_t window) {
  int64_t pmax = (static_cast<int64_t>(max_len) + part - 1) / part;
  if (window > 0) pmax = std::min<int64_t>(pmax, (static_cast<int64_t>(window) + part - 2) / part + 1);
  return pmax;
}

size_t workspace_bytes(int64_t rows, int32_t head_dim) {
  const size_t ml_bytes = (static_cast<size_t>(rows) * 2 * sizeof(float) + 255) & ~size_t(255);
  return ml_bytes + static_cast<size_t>(rows) * head_dim * sizeof(float);
}

// Checks the decode arguments and fills the kernel parameter block.
int prepare_decode(const pkv_decode_args* a, pkv::DecodeParams* p, int* kind_out) {
  if (!a) return fail(PKV_ERR_INVALID, "decode: null args");
  if (a->dtype != PKV_F32 && a->dtype != PKV_BF16) return fail(PKV_ERR_INVALID, "decode: bad dtype");
  if (a->kv_dtype != a->dtype && !(a->kv_dtype == PKV_FP8_E4M3 && a->dtype == PKV_BF16))
    return fail(PKV_ERR_INVALID, "decode: kv_dtype must equal dtype, or be PKV_FP8_E4M3 with PKV_BF16 queries");
  const int kind = a->kv_dtype == PKV_FP8_E4M3 ? pkv::kDecodeFP8KV
                   : a->dtype == PKV_BF16    ? pkv::kDecodeBF16
                                             : pkv::kDecodeF32;
  if (a->num_seqs < 1 || a->num_kv_heads < 1 || a->num_q_heads < 1 || a->head_dim < 1 ||
      a->block_size < 1 || a->num_blocks < 1 || a->max_blocks < 1 || a->max_seq_len < 1)
    return fail(PKV_ERR_INVALID, "decode: sizes must be positive");
  if (a->num_q_heads % a->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "decode: num_q_heads must be a multiple of num_kv_heads");
  const int32_t part = effective_partition(a->partition);
  if (part < 32 || part > 1024 || part % 32 != 0)
    return fail(PKV_ERR_INVALID, "decode: partition must be a multiple of 32 in [32, 1024]");
  if (a->window < 0) return fail(PKV_ERR_INVALID, "decode: window must be >= 0");
  if (!pkv::decode_shape_supported(kind, a->head_dim, a->block_size))
    return fail(PKV_ERR_UNSUPPORTED, "decode: supported shapes are block_size 16, head_dim 64 or 128");
  if (!a->q || !a->out || !a->k_cache || !a->v_cache || !a->block_tables || !a->seq_lens)
    return fail(PKV_ERR_INVALID, "decode: null device pointer");
  if (!aligned16(a->q) || !aligned16(a->out) || !aligned16(a->k_cache) || !aligned16(a->v_cache))
    return fail(PKV_ERR_INVALID, "decode: q, out and caches must be 16-byte aligned");
  if (kind == pkv::kDecodeFP8KV &&
      (!a->k_scale || !a->v_scale || !aligned16(a->k_scale) || !aligned16(a->v_scale)))
    return fail(PKV_ERR_INVALID, "decode: an 8-bit cache needs 16-byte aligned k_scale and v_scale");
  const int64_t pmax = partitions_bound(a->max_seq_len, part, a->window);
  const int64_t gx = pmax * a->num_seqs * a->num_kv_heads;
  if (gx > 0x7fffffffLL || static_cast<int64_t>(a->num_seqs) * a->num_q_heads > 0x7fffffffLL)
    return fail(PKV_ERR_INVALID, "decode: grid too large");
  const int64_t rows = pmax > 1 ? static_cast<int64_t>(a->num_seqs) * a->num_q_heads * pmax : 0;
  const size_t need = rows > 0 ? workspace_bytes(rows, a->head_dim) : 0;
  if (need > 0 && (!a->workspace || a->workspace_bytes < need))
    return fail(PKV_ERR_INVALID, "decode: workspace missing or smaller than pkv_decode_workspace_bytes()");
  if (need > 0 && !aligned16(a->workspace))
    return fail(PKV_ERR_INVALID, "decode: workspace must be 16-byte aligned");
  if ((a->k_new == nullptr) != (a->v_new == nullptr))
    return fail(PKV_ERR_INVALID, "decode: k_new and v_new go together");
  if (a->k_new && (!aligned16(a->k_new) || !aligned16(a->v_new)))
    return fail(PKV_ERR_INVALID, "decode: k_new and v_new must be 16-byte aligned");
  p->q = a->q;
  p->out = a->out;
  p->k_cache = a->k_cache;
  p->v_cache = a->v_cache;
  p->block_tables = a->block_tables;
  p->seq_lens = a->seq_lens;
  p->k_scale = kind == pkv::kDecodeFP8KV ? a->k_scale : nullptr;
  p->v_scale = kind == pkv::kDecodeFP8KV ? a->v_scale : nullptr;
  p->k_new = a->k_new;
  p->v_new = a->v_new;
  p->S = a->num_seqs;
  p->Hq = a->num_q_heads;
  p->Hkv = a->num_kv_heads;
  p->G = a->num_q_heads / a->num_kv_heads;
  p->d = a->head_dim;
  p->num_blocks = a->num_blocks;
  p->max_blocks = a->max_blocks;
  p->max_seq_len = a->max_seq_len;
  p->window = a->window;
  p->partition = part;
  p->pmax = static_cast<int32_t>(pmax);
  p->ppw = 1;
  p->tasks_hint = 0;
  p->uniform_hint = 0;
  if (a->host_seq_lens) {
    // exact partition count from the host copy of the lengths
    // Uniform: every sequence attends to within 1/8 of the longest one's
    // tokens (equal static runs then carry equal work).
    int64_t sum = 0, lo = INT64_MAX, hi = 0;
    for (int32_t i = 0; i < a->num_seqs; ++i) {
      const int32_t n = a->host_seq_lens[i];
      if (n < 1 || n > a->max_seq_len) continue;
      const int32_t t0 = a->window > 0 ? std::max(0, n - a->window) : 0;
      sum += (n - 1) / part - t0 / part + 1;
      lo = std::min<int64_t>(lo, n - t0);
      hi = std::max<int64_t>(hi, n - t0);
    }
    const int64_t hg = (p->G + 15) / 16;
    p->tasks_hint = sum * a->num_kv_heads * hg;
    p->uniform_hint = sum > 0 && lo * 8 >= hi * 7;
  }
  p->scale_log2 = a->scale * 1.4426950408889634f;
  if (need > 0) {
    const size_t ml_bytes = (static_cast<size_t>(rows) * 2 * sizeof(float) + 255) & ~size_t(255);
    p->part_ml = static_cast<float*>(a->workspace);
    p->part_acc = reinterpret_cast<float*>(static_cast<char*>(a->workspace) + ml_bytes);
  } else {
    p->part_ml = nullptr;
    p->part_acc = nullptr;
  }
  *kind_out = kind;
  return PKV_OK;
}

// The partial kernel's work list (DecodeOrder) from the host length hint,
// for up to kOrderMaxSeqs sequences and kOrderMaxGroups partitions.
// Partitions are counted as the kernel counts them: with a window, from the
// first one that overlaps it.  Lengths outside [1, max_seq_len] count as 0;
// such a sequence lists partition 0.  Every partition of a sequence but its
// last is listed as full (all hold a whole partition, except the first one of
// a window), group-major, sequences with more partitions first; then each
// sequence's last partition, largest first: the launch's last waves are
// short ones.
void build_order(const pkv_decode_args* a, pkv::DecodeParams* p) {
  pkv::DecodeOrder& o = p->order;
  o.active = 0;
  if (!a->host_seq_lens || p->S > pkv::kOrderMaxSeqs || p->pmax > pkv::kOrderMaxGroups) return;
  const int S = p->S, part = p->partition;
  std::array<int32_t, pkv::kOrderMaxSeqs> parts{}, last{}, rank_seq{};   // partitions, tokens in the last one
  for (int i = 0; i < S; ++i) {
    const int32_t v = a->host_seq_lens[i];
    if (v >= 1 && v <= a->max_seq_len) {
      const int32_t t0 = a->window > 0 ? std::max(0, v - a->window) : 0;
      const int32_t pf = t0 / part;
      parts[i] = (v - 1) / part - pf + 1;
      last[i] = v - std::max(t0, (pf + parts[i] - 1) * part);
    }
    o.hinted[i] = static_cast<uint8_t>(std::max(1, parts[i]));
    rank_seq[i] = i;
  }
  std::stable_sort(rank_seq.begin(), rank_seq.begin() + S,
                   [&](int x, int y) { return parts[x] > parts[y] || (parts[x] == parts[y] && last[x] > last[y]); });
  std::array<int32_t, pkv::kOrderMaxGroups> full{};              // per group: ranks with a full partition there
  std::array<int32_t, pkv::kOrderMaxSeqs> partial_rank{};
  for (int r = 0; r < S; ++r) {
    const int sq = rank_seq[r];
    for (int g = 0; g + 1 < parts[sq]; ++g) ++full[g];
    partial_rank[r] = r;
    o.rank_seq[r] = static_cast<uint16_t>(sq);
  }
  std::stable_sort(partial_rank.begin(), partial_rank.begin() + S,
                   [&](int x, int y) { return last[rank_seq[x]] > last[rank_seq[y]]; });
  for (int j = 0; j < S; ++j) {
    const int r = partial_rank[j];
    o.partial[j] = static_cast<uint16_t>(r | (o.hinted[rank_seq[r]] - 1) << 9);
  }
  o.full_start[0] = 0;
  for (int g = 0; g < p->pmax; ++g) o.full_start[g + 1] = o.full_start[g] + full[g];
  o.n_full = o.full_start[p->pmax];
  o.n_partial = S;
  o.active = 1;
}

// Largest batch, in (sequence, KV head) rows, whose new tokens the partial
// kernel writes itself (PKV_FUSED_APPEND_MAX_ROWS overrides it).  The
// appending waves hold the token in registers from their set-up on, use it in
// place of the token's slot when their last block arrives, and write it to
// the pool after their last load, so neither a wait nor a load depends on
// those writes.
constexpr int64_t kFusedAppendMaxRows = 1024;

int64_t fused_append_max_rows() {
  static const int64_t v = [] {
    const char* e = std::getenv("PKV_FUSED_APPEND_MAX_ROWS");
    return e ? std::max<int64_t>(0, std::atoll(e)) : kFusedAppendMaxRows;
  }();
  return v;
}

// The partial kernel writes the new tokens (k_new) itself for bf16 and 8-bit
// caches up to fused_append_max_rows() rows; otherwise the append kernel
// (the pkv_kv_append_last path) runs first and the partial kernel only reads.
// The fp32 cache always takes the append kernel.
bool fuses_append(const pkv::DecodeParams& p, int kind) {
  return p.k_new && kind != pkv::kDecodeF32 && static_cast<int64_t>(p.S) * p.Hkv <= fused_append_max_rows();
}

int run_partial(const pkv_decode_args* a, pkv::DecodeParams& p, int kind, hipStream_t st) {
  if (p.k_new && !fuses_append(p, kind)) {
    if (static_cast<int64_t>(a->max_blocks) * a->block_size > 0x7fffffffLL)
      return fail(PKV_ERR_INVALID, "decode: max_blocks too large");
    pkv::AppendParams ap{};
    ap.k_new = a->k_new;
    ap.v_new = a->v_new;
    ap.slots = nullptr;
    ap.tables = a->block_tables;
    ap.lens = a->seq_lens;
    ap.max_blocks = a->max_blocks;
    ap.k_cache = a->k_cache;
    ap.v_cache = a->v_cache;
    ap.num_slots = static_cast<int64_t>(a->num_blocks) * a->block_size;
    ap.n = a->num_seqs;
    ap.num_kv_heads = a->num_kv_heads;
    ap.head_dim = a->head_dim;
    ap.block_size = a->block_size;
    ap.elem_bytes = kind == pkv::kDecodeF32 ? 4 : kind == pkv::kDecodeBF16 ? 2 : 1;
    ap.k_scale = a->k_scale;
    ap.v_scale = a->v_scale;
    const int rc = from_hip(pkv::launch_kv_append(ap, st), "decode: append");
    if (rc) return rc;
    p.k_new = nullptr;
    p.v_new = nullptr;
  }
  return from_hip(pkv::launch_decode_partial(p, kind, st), "decode_partial");
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID: return "PKV_ERR_INVALID";
    case PKV_ERR_NO_BLOCKS: return "PKV_ERR_NO_BLOCKS";
    case PKV_ERR_BAD_SEQ: return "PKV_ERR_BAD_SEQ";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    default: return "PKV_ERR_UNKNOWN";
  }
}

const char* pkv_last_error(void) { return g_error.c_str(); }

int pkv_version(void) { return 300; }

int pkv_pool_create(const pkv_pool_desc* d, pkv_pool** out) {
  return guarded([&]() -> int {
    if (!d || !out) return fail(PKV_ERR_INVALID, "pool_create: null argument");
    *out = nullptr;
    if (d->num_layers < 1 || d->num_kv_heads < 1 || d->head_dim < 1 || d->block_size < 1 ||
        d->num_blocks < 1)
      return fail(PKV_ERR_INVALID, "pool_create: sizes must be positive");
    if (d->dtype != PKV_F32 && d->dtype != PKV_BF16 && d->dtype != PKV_FP8_E4M3)
      return fail(PKV_ERR_INVALID, "pool_create: bad dtype");
    if ((d->head_dim * elem_bytes(d->dtype)) % 16 != 0)
      return fail(PKV_ERR_INVALID, "pool_create: head_dim must be a multiple of 16 bytes");
    const bool fp8 = d->dtype == PKV_FP8_E4M3;
    if (fp8 && (d->head_dim % 64 != 0 || d->block_size != 16))
      return fail(PKV_ERR_INVALID, "pool_create: an 8-bit pool needs head_dim % 64 == 0 and block_size 16");
    if (fp8 && d->k_cache && (!d->k_scale || !d->v_scale))
      return fail(PKV_ERR_INVALID, "pool_create: an 8-bit pool needs k_scale and v_scale arrays");
    if (static_cast<int64_t>(d->num_blocks) * d->block_size > 0x7fffffffLL)
      return fail(PKV_ERR_INVALID, "pool_create: num_blocks * block_size must fit in int32 slots");
    if ((d->k_cache == nullptr) != (d->v_cache == nullptr))
      return fail(PKV_ERR_INVALID, "pool_create: give both k_cache and v_cache, or neither");
    if (d->k_cache && (d->block_size % 4 != 0 || d->head_dim % 4 != 0))
      return fail(PKV_ERR_INVALID, "pool_create: device pools need block_size and head_dim multiples of 4");
    if (d->init_perm) {
      std::vector<char> seen(d->num_blocks, 0);
      for (int32_t i = 0; i < d->num_blocks; ++i) {
        const int32_t b = d->init_perm[i];
        if (b < 0 || b >= d->num_blocks || seen[b])
          return fail(PKV_ERR_INVALID, "pool_create: init_perm is not a permutation");
        seen[b] = 1;
      }
    }
    auto* pool = new pkv_pool(d->num_blocks, d->block_size, d->init_perm);
    pool->num_layers = d->num_layers;
    pool->num_kv_heads = d->num_kv_heads;
    pool->head_dim = d->head_dim;
    pool->dtype = d->dtype;
    if (d->k_cache) {
      for (int32_t l = 0; l < d->num_layers; ++l) {
        if (!d->k_cache[l] || !d->v_cache[l] || !aligned16(d->k_cache[l]) || !aligned16(d->v_cache[l])) {
          delete pool;
          return fail(PKV_ERR_INVALID, "pool_create: layer caches must be non-null and 16-byte aligned");
        }
        pool->k_cache.push_back(d->k_cache[l]);
        pool->v_cache.push_back(d->v_cache[l]);
        if (fp8) {
          if (!d->k_scale[l] || !d->v_scale[l] || !aligned16(d->k_scale[l]) || !aligned16(d->v_scale[l])) {
            delete pool;
            return fail(PKV_ERR_INVALID, "pool_create: layer scale arrays must be non-null and 16-byte aligned");
          }
          pool->k_scale.push_back(d->k_scale[l]);
          pool->v_scale.push_back(d->v_scale[l]);
        }
      }
    }
    *out = pool;
    return PKV_OK;
  });
}

int pkv_pool_destroy(pkv_pool* pool) {
  if (!pool) return PKV_OK;
  int st = PKV_OK;
  // The last uploads of an unfinished group have no event yet (and their
  // stream may be gone): wait for the device instead.
  if (pool->uploads % pkv_pool::kUploadsPerEvent != 0)
    st = from_hip(hipDeviceSynchronize(), "pool_destroy");
  for (auto& g : pool->groups) {
    for (int e = 0; e < g.n_ev; ++e)
      if (g.pending && st == PKV_OK) st = from_hip(hipEventSynchronize(g.ev[e]), "pool_destroy");
    for (hipEvent_t ev : g.ev)
      if (ev) (void)hipEventDestroy(ev);
  }
  for (void* buf : pool->staging)
    if (buf) (void)hipHostFree(buf);
  delete pool;
  return st;
}

int pkv_seq_create(pkv_pool* pool, int64_t* id) {
  if (!pool || !id) return fail(PKV_ERR_INVALID, "seq_create: null argument");
  return guarded([&] { return from_alloc(pool->alloc.create(id), pool); });
}

int pkv_seq_fork(pkv_pool* pool, int64_t parent, int64_t* child) {
  if (!pool || !child) return fail(PKV_ERR_INVALID, "seq_fork: null argument");
  return guarded([&] { return from_alloc(pool->alloc.fork(parent, child), pool); });
}

int pkv_seq_free(pkv_pool* pool, int64_t id) {
  if (!pool) return fail(PKV_ERR_INVALID, "seq_free: null pool");
  return guarded([&] { return from_alloc(pool->alloc.release(id), pool); });
}

int pkv_seq_release_before(pkv_pool* pool, int64_t id, int32_t pos, int32_t* n_released) {
  if (!pool) return fail(PKV_ERR_INVALID, "seq_release_before: null pool");
  int32_t dummy = 0;
  return guarded([&] { return from_alloc(pool->alloc.release_before(id, pos, n_released ? n_released : &dummy), pool); });
}

int pkv_prefix_register(pkv_pool* pool, int64_t id, const int32_t* tokens, int32_t n_tokens, uint64_t ns,
                        int32_t* n_added) {
  if (!pool) return fail(PKV_ERR_INVALID, "prefix_register: null pool");
  int32_t dummy = 0;
  return guarded([&] {
    return from_alloc(pool->alloc.prefix_register(id, tokens, n_tokens, ns, n_added ? n_added : &dummy), pool);
  });
}

int pkv_prefix_match(pkv_pool* pool, const int32_t* tokens, int32_t n_tokens, uint64_t ns, int64_t* seq_id,
                     int32_t* n_matched) {
  if (!pool || !seq_id) return fail(PKV_ERR_INVALID, "prefix_match: null argument");
  int32_t dummy = 0;
  return guarded([&] {
    return from_alloc(pool->alloc.prefix_match(tokens, n_tokens, ns, seq_id, n_matched ? n_matched : &dummy), pool);
  });
}

int pkv_prefix_evict(pkv_pool* pool, int32_t max_blocks, int32_t* n_freed) {
  if (!pool) return fail(PKV_ERR_INVALID, "prefix_evict: null pool");
  int32_t dummy = 0;
  return guarded([&] { return from_alloc(pool->alloc.prefix_evict(max_blocks, n_freed ? n_freed : &dummy), pool); });
}

int pkv_prefix_clear(pkv_pool* pool, int32_t* n_dropped) {
  if (!pool) return fail(PKV_ERR_INVALID, "prefix_clear: null pool");
  int32_t dummy = 0;
  return guarded([&] { return from_alloc(pool->alloc.prefix_clear(n_dropped ? n_dropped : &dummy), pool); });
}

int pkv_prefix_snapshot(const pkv_pool* pool, int64_t* n_entries, int64_t* entry_out, uint64_t* ns_out,
                        int64_t* parent_out, int32_t* block_out, int64_t* last_use_out, int32_t* tokens_out) {
  if (!pool || !n_entries) return fail(PKV_ERR_INVALID, "prefix_snapshot: null size pointer");
  const auto& pc = pool->alloc.prefix_entries();
  *n_entries = static_cast<int64_t>(pc.size());
  const int32_t B = pool->alloc.block_size();
  int64_t i = 0;
  for (const auto& kv : pc) {
    if (entry_out) entry_out[i] = kv.first;
    if (ns_out) ns_out[i] = kv.second.key.ns;
    if (parent_out) parent_out[i] = kv.second.key.parent;
    if (block_out) block_out[i] = kv.second.block;
    if (last_use_out) last_use_out[i] = kv.second.last_use;
    if (tokens_out) std::copy(kv.second.key.tokens.begin(), kv.second.key.tokens.end(), tokens_out + i * B);
    ++i;
  }
  return PKV_OK;
}

int pkv_seq_extend(pkv_pool* pool, int64_t id, int32_t ntok, int32_t* slots, int32_t* cow,
                   int32_t* n_cow) {
  if (!pool || !n_cow || !cow || (ntok > 0 && !slots)) return fail(PKV_ERR_INVALID, "seq_extend: null argument");
  return guarded([&] { return from_alloc(pool->alloc.extend(id, ntok, slots, cow, n_cow), pool); });
}

int pkv_append_slots(pkv_pool* pool, const int64_t* ids, int32_t n, int32_t* slots, int32_t* cow,
                     int32_t* n_cow) {
  if (!pool || !n_cow || (n > 0 && (!ids || !slots || !cow)))
    return fail(PKV_ERR_INVALID, "append_slots: null argument");
  return guarded([&] { return from_alloc(pool->alloc.append(ids, n, slots, cow, n_cow), pool); });
}

int pkv_seq_length(const pkv_pool* pool, int64_t id, int32_t* len) {
  if (!pool || !len) return fail(PKV_ERR_INVALID, "seq_length: null argument");
  const pkv::Sequence* s = pool->alloc.find(id);
  if (!s) return fail(PKV_ERR_BAD_SEQ, "seq_length: unknown sequence id " + std::to_string(id));
  *len = s->len;
  return PKV_OK;
}

int pkv_seq_table(const pkv_pool* pool, int64_t id, int32_t* table, int32_t cap, int32_t* nblocks) {
  if (!pool || !nblocks || (cap > 0 && !table)) return fail(PKV_ERR_INVALID, "seq_table: null argument");
  const pkv::Sequence* s = pool->alloc.find(id);
  if (!s) return fail(PKV_ERR_BAD_SEQ, "seq_table: unknown sequence id " + std::to_string(id));
  const int32_t nb = static_cast<int32_t>(s->table.size());
  *nblocks = nb;
  std::copy_n(s->table.begin(), std::min(std::max(cap, 0), nb), table);
  return PKV_OK;
}

int pkv_sync_tables(pkv_pool* pool, const int64_t* ids, int32_t n, int32_t* dev_tables,
                    int32_t max_blocks, int32_t* dev_lens, int32_t* host_lens_out, void* stream) {
  return guarded([&]() -> int {
    if (!pool || n < 0 || max_blocks < 1) return fail(PKV_ERR_INVALID, "sync_tables: bad argument");
    if (n == 0) return PKV_OK;
    if (!ids || !dev_tables || !dev_lens) return fail(PKV_ERR_INVALID, "sync_tables: null pointer");
    std::vector<const pkv::Sequence*> seqs(n);
    for (int32_t i = 0; i < n; ++i) {
      seqs[i] = pool->alloc.find(ids[i]);
      if (!seqs[i]) return fail(PKV_ERR_BAD_SEQ, "sync_tables: unknown sequence id " + std::to_string(ids[i]));
      if (static_cast<int32_t>(seqs[i]->table.size()) > max_blocks)
        return fail(PKV_ERR_INVALID, "sync_tables: sequence " + std::to_string(ids[i]) +
                                         " holds more than max_blocks blocks");
    }
    const size_t table_bytes = static_cast<size_t>(n) * max_blocks * sizeof(int32_t);
    const size_t need = table_bytes + static_cast<size_t>(n) * sizeof(int32_t);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint64_t u = pool->uploads;
    const int k = static_cast<int>(u % pkv_pool::kStagingRing);
    const int pos = static_cast<int>(u % pkv_pool::kUploadsPerEvent);
    auto& grp = pool->groups[(u / pkv_pool::kUploadsPerEvent) % (pkv_pool::kStagingRing / pkv_pool::kUploadsPerEvent)];
    int rc;
    if (pos == 0 && grp.pending) {     // the group that last used these buffers
      for (int e = 0; e < grp.n_ev; ++e) {
        rc = from_hip(hipEventSynchronize(grp.ev[e]), "sync_tables: wait for an earlier upload");
        if (rc) return rc;
      }
      grp.pending = false;
      grp.n_ev = 0;
    }
    // Pinning host memory takes milliseconds: the first call sizes the whole
    // ring (no buffer is in use yet); later a buffer grows when its turn comes.
    const size_t cap = std::max(need, static_cast<size_t>(1) << 20);
    for (int b = (u == 0 ? 0 : k); b < (u == 0 ? pkv_pool::kStagingRing : k + 1); ++b) {
      if (pool->staging_bytes[b] >= need) continue;
      if (pool->staging[b]) (void)hipHostFree(pool->staging[b]);
      pool->staging[b] = nullptr;
      pool->staging_bytes[b] = 0;
      rc = from_hip(hipHostMalloc(&pool->staging[b], cap, hipHostMallocDefault), "sync_tables: pinned staging");
      if (rc) return rc;
      pool->staging_bytes[b] = cap;
    }
    int32_t* tab = static_cast<int32_t*>(pool->staging[k]);
    int32_t* lens = tab + static_cast<size_t>(n) * max_blocks;
    for (int32_t i = 0; i < n; ++i) {
      int32_t* row = tab + static_cast<size_t>(i) * max_blocks;
      const auto& t = seqs[i]->table;
      std::copy(t.begin(), t.end(), row);
      std::fill(row + t.size(), row + max_blocks, -1);
      lens[i] = seqs[i]->len;
      if (host_lens_out) host_lens_out[i] = seqs[i]->len;
    }
    rc = from_hip(pkv::launch_table_upload(tab, dev_tables, static_cast<int64_t>(n) * max_blocks, dev_lens, n, st),
                  "sync_tables: upload");
    if (rc) return rc;
    const hipStream_t prev = pool->last_stream;
    pool->uploads = u + 1;
    pool->last_stream = st;
    // The events only tell the host when uploads have finished reading their
    // staging buffers; no device write has to reach the host.  So they record
    // without the system-scope fence (a cache write-back and invalidation).
    auto mark = [&](hipStream_t s) -> int {
      hipEvent_t& ev = grp.ev[grp.n_ev];
      int r = PKV_OK;
      if (!ev) r = from_hip(hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence),
                            "sync_tables: event");
      if (!r) r = from_hip(hipEventRecord(ev, s), "sync_tables: record");
      if (r) {                          // no event: make sure the buffers are free before returning
        (void)hipDeviceSynchronize();
        return r;
      }
      ++grp.n_ev;
      grp.pending = true;
      return PKV_OK;
    };
    if (pos > 0 && st != prev) {        // the group's uploads on the previous stream end here
      rc = mark(prev);
      if (rc) return rc;
    }
    if (pos == pkv_pool::kUploadsPerEvent - 1) return mark(st);
    return PKV_OK;
  });
}

int pkv_copy_blocks(pkv_pool* pool, const int32_t* pairs, int32_t n_pairs, void* stream) {
  if (!pool || n_pairs < 0 || (n_pairs > 0 && !pairs)) return fail(PKV_ERR_INVALID, "copy_blocks: bad argument");
  if (n_pairs == 0) return PKV_OK;
  if (pool->k_cache.empty()) return fail(PKV_ERR_INVALID, "copy_blocks: pool has no device caches");
  const int32_t nb = pool->alloc.num_blocks();
  for (int32_t i = 0; i < 2 * n_pairs; ++i)
    if (pairs[i] < 0 || pairs[i] >= nb) return fail(PKV_ERR_INVALID, "copy_blocks: block id out of range");
  const int64_t block_bytes = static_cast<int64_t>(pool->num_kv_heads) * pool->head_dim *
                              pool->alloc.block_size() * elem_bytes(pool->dtype);
  for (int32_t l0 = 0; l0 < pool->num_layers; l0 += pkv::kCopyMaxLayers) {
    for (int32_t p0 = 0; p0 < n_pairs; p0 += pkv::kCopyMaxPairs) {
      pkv::CopyBlocksParams p{};
      p.n_layers = std::min(pkv::kCopyMaxLayers, pool->num_layers - l0);
      p.n_pairs = std::min(pkv::kCopyMaxPairs, n_pairs - p0);
      p.block_bytes = block_bytes;
      const bool scaled = !pool->k_scale.empty();
      p.scale_bytes = scaled ? static_cast<int64_t>(pool->num_kv_heads) * pool->alloc.block_size() * 4 : 0;
      for (int32_t l = 0; l < p.n_layers; ++l) {
        p.k[l] = pool->k_cache[l0 + l];
        p.v[l] = pool->v_cache[l0 + l];
        if (scaled) {
          p.ks[l] = pool->k_scale[l0 + l];
          p.vs[l] = pool->v_scale[l0 + l];
        }
      }
      std::memcpy(p.pairs, pairs + 2 * p0, sizeof(int32_t) * 2 * p.n_pairs);
      const int rc = from_hip(pkv::launch_copy_blocks(p, static_cast<hipStream_t>(stream)), "copy_blocks");
      if (rc) return rc;
    }
  }
  return PKV_OK;
}

int pkv_kv_append(pkv_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                  const int32_t* dev_slots, int32_t n, void* stream) {
  if (!pool || n < 0) return fail(PKV_ERR_INVALID, "kv_append: bad argument");
  if (n == 0) return PKV_OK;
  if (pool->k_cache.empty()) return fail(PKV_ERR_INVALID, "kv_append: pool has no device caches");
  if (layer < 0 || layer >= pool->num_layers) return fail(PKV_ERR_INVALID, "kv_append: layer out of range");
  if (!k_new || !v_new || !dev_slots) return fail(PKV_ERR_INVALID, "kv_append: null pointer");
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(PKV_ERR_INVALID, "kv_append: inputs must be 16-byte aligned");
  pkv::AppendParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.slots = dev_slots;
  p.tables = nullptr;
  p.lens = nullptr;
  p.max_blocks = 0;
  p.k_cache = pool->k_cache[layer];
  p.v_cache = pool->v_cache[layer];
  p.num_slots = static_cast<int64_t>(pool->alloc.num_blocks()) * pool->alloc.block_size();
  p.n = n;
  p.num_kv_heads = pool->num_kv_heads;
  p.head_dim = pool->head_dim;
  p.block_size = pool->alloc.block_size();
  p.elem_bytes = elem_bytes(pool->dtype);
  if (!pool->k_scale.empty()) {
    p.k_scale = static_cast<float*>(pool->k_scale[layer]);
    p.v_scale = static_cast<float*>(pool->v_scale[layer]);
  }
  return from_hip(pkv::launch_kv_append(p, static_cast<hipStream_t>(stream)), "kv_append");
}

int pkv_kv_append_last(pkv_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                       const int32_t* dev_tables, int32_t max_blocks, const int32_t* dev_lens, int32_t n,
                       void* stream) {
  if (!pool || n < 0 || max_blocks < 1) return fail(PKV_ERR_INVALID, "kv_append_last: bad argument");
  if (n == 0) return PKV_OK;
  if (pool->k_cache.empty()) return fail(PKV_ERR_INVALID, "kv_append_last: pool has no device caches");
  if (layer < 0 || layer >= pool->num_layers) return fail(PKV_ERR_INVALID, "kv_append_last: layer out of range");
  if (!k_new || !v_new || !dev_tables || !dev_lens) return fail(PKV_ERR_INVALID, "kv_append_last: null pointer");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_ERR_INVALID, "kv_append_last: inputs must be 16-byte aligned");
  if (static_cast<int64_t>(max_blocks) * pool->alloc.block_size() > 0x7fffffffLL)
    return fail(PKV_ERR_INVALID, "kv_append_last: max_blocks too large");
  pkv::AppendParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.slots = nullptr;
  p.tables = dev_tables;
  p.lens = dev_lens;
  p.max_blocks = max_blocks;
  p.k_cache = pool->k_cache[layer];
  p.v_cache = pool->v_cache[layer];
  p.num_slots = static_cast<int64_t>(pool->alloc.num_blocks()) * pool->alloc.block_size();
  p.n = n;
  p.num_kv_heads = pool->num_kv_heads;
  p.head_dim = pool->head_dim;
  p.block_size = pool->alloc.block_size();
  p.elem_bytes = elem_bytes(pool->dtype);
  if (!pool->k_scale.empty()) {
    p.k_scale = static_cast<float*>(pool->k_scale[layer]);
    p.v_scale = static_cast<float*>(pool->v_scale[layer]);
  }
  return from_hip(pkv::launch_kv_append(p, static_cast<hipStream_t>(stream)), "kv_append_last");
}

int pkv_pool_stats(const pkv_pool* pool, pkv_stats* out) {
  if (!pool || !out) return fail(PKV_ERR_INVALID, "pool_stats: null argument");
  const auto& a = pool->alloc;
  pkv_stats s{};
  s.num_blocks = a.num_blocks();
  s.free_blocks = static_cast<int64_t>(a.free_stack().size());
  s.used_blocks = s.num_blocks - s.free_blocks;
  s.num_seqs = static_cast<int64_t>(a.sequences().size());
  for (int32_t r : a.refcounts()) s.sum_ref += r;
  for (const auto& kv : a.sequences()) {
    s.sum_len += kv.second.len;
    s.tail_waste += static_cast<int64_t>(kv.second.table.size()) * a.block_size() - kv.second.len;
  }
  *out = s;
  return PKV_OK;
}

int pkv_pool_snapshot(const pkv_pool* pool, int32_t* free_out, int32_t* ref_out, int64_t* ids_out,
                      int32_t* lens_out, int64_t* table_off_out, int32_t* tables_out, int64_t* n_free,
                      int64_t* n_seqs, int64_t* n_entries, int64_t* next_id) {
  return guarded([&]() -> int {
    if (!pool || !n_free || !n_seqs || !n_entries || !next_id)
      return fail(PKV_ERR_INVALID, "pool_snapshot: null size pointer");
    const auto& a = pool->alloc;
    std::vector<int64_t> ids;
    ids.reserve(a.sequences().size());
    int64_t entries = 0;
    for (const auto& kv : a.sequences()) {
      ids.push_back(kv.first);
      entries += static_cast<int64_t>(kv.second.table.size());
    }
    std::sort(ids.begin(), ids.end());
    *n_free = static_cast<int64_t>(a.free_stack().size());
    *n_seqs = static_cast<int64_t>(ids.size());
    *n_entries = entries;
    *next_id = a.next_id();
    if (free_out) std::copy(a.free_stack().begin(), a.free_stack().end(), free_out);
    if (ref_out) std::copy(a.refcounts().begin(), a.refcounts().end(), ref_out);
    int64_t off = 0;
    for (size_t i = 0; i < ids.size(); ++i) {
      const pkv::Sequence* s = a.find(ids[i]);
      if (ids_out) ids_out[i] = ids[i];
      if (lens_out) lens_out[i] = s->len;
      if (table_off_out) table_off_out[i] = off;
      if (tables_out) std::copy(s->table.begin(), s->table.end(), tables_out + off);
      off += static_cast<int64_t>(s->table.size());
    }
    if (table_off_out) table_off_out[ids.size()] = off;
    return PKV_OK;
  });
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_seq_len, int32_t partition) {
  const int32_t part = effective_partition(partition);
  if (num_seqs < 1 || num_q_heads < 1 || head_dim < 1 || max_seq_len < 1 || part < 1) return 0;
  const int64_t pmax = partitions_bound(max_seq_len, part, 0);
  if (pmax <= 1) return 0;
  return workspace_bytes(static_cast<int64_t>(num_seqs) * num_q_heads * pmax, head_dim);
}

int pkv_paged_decode_partial(const pkv_decode_args* a, void* stream) {
  pkv::DecodeParams p{};
  int kind = 0;
  const int rc = prepare_decode(a, &p, &kind);
  if (rc) return rc;
  build_order(a, &p);
  return run_partial(a, p, kind, static_cast<hipStream_t>(stream));
}

int pkv_paged_decode_reduce(const pkv_decode_args* a, void* stream) {
  pkv::DecodeParams p{};
  int kind = 0;
  const int rc = prepare_decode(a, &p, &kind);
  if (rc) return rc;
  return from_hip(pkv::launch_decode_reduce(p, kind, static_cast<hipStream_t>(stream)), "decode_reduce");
}

int pkv_paged_attention_decode(const pkv_decode_args* a, void* stream) {
  pkv::DecodeParams p{};
  int kind = 0;
  int rc = prepare_decode(a, &p, &kind);
  if (rc) return rc;
  build_order(a, &p);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = run_partial(a, p, kind, st);
  if (rc) return rc;
  return from_hip(pkv::launch_decode_reduce(p, kind, st), "decode_reduce");
}

int pkv_paged_attention_decode_static(const pkv_decode_args* a, void* stream) {
  if (!a) return fail(PKV_ERR_INVALID, "decode_static: null args");
  // Check the arguments as the decode call does, with a stand-in workspace
  // of any size, to learn the workspace this call needs.
  pkv_decode_args b = *a;
  b.workspace = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  b.workspace_bytes = SIZE_MAX;
  pkv::DecodeParams p{};
  int kind = 0;
  const int rc = prepare_decode(&b, &p, &kind);
  if (rc) return rc;
  const size_t need = p.pmax > 1 ? workspace_bytes(static_cast<int64_t>(p.S) * p.Hq * p.pmax, p.d) : 0;
  if (need > pkv::kStaticWorkspaceBytes)
    return fail(PKV_ERR_INVALID, "decode_static: the call needs " + std::to_string(need) +
                                     " bytes of workspace, more than the library's " +
                                     std::to_string(pkv::kStaticWorkspaceBytes));
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (need > 0) {
    const int hrc = from_hip(pkv::static_workspace(&b.workspace), "decode_static: workspace address");
    if (hrc) return hrc;
    b.workspace_bytes = pkv::kStaticWorkspaceBytes;
  }
  return pkv_paged_attention_decode(&b, stream);
}

int pkv_decode_fuses_append(const pkv_decode_args* a) {
  pkv::DecodeParams p{};
  int kind = 0;
  const int rc = prepare_decode(a, &p, &kind);
  if (rc) return rc;
  return fuses_append(p, kind) ? 1 : 0;
}

int pkv_decode_plan(const pkv_decode_args* a, pkv_decode_plan_info* info, int32_t* cells, int64_t cap) {
  if (!info) return fail(PKV_ERR_INVALID, "decode_plan: null info");
  if (cap < 0 || (cap > 0 && !cells)) return fail(PKV_ERR_INVALID, "decode_plan: bad cells buffer");
  pkv::DecodeParams p{};
  int kind = 0;
  const int rc = prepare_decode(a, &p, &kind);
  if (rc) return rc;
  build_order(a, &p);
  pkv::DecodeLaunchPlan plan{};
  const int prc = from_hip(pkv::plan_decode_partial(p, kind, &plan), "decode_plan");
  if (prc) return prc;
  const pkv::DecodeParams& q = plan.params;
  info->cells = plan.cells;
  info->listed_cells = q.order.active ? q.order.n_full + q.order.n_partial : 0;
  info->head_groups = plan.grid_y;
  info->pipeline_depth = plan.depth;
  info->resident_waves = plan.resident_waves;
  info->partitions_per_wave = q.ppw;
  info->work_list = q.order.active;
  info->run_cap = q.order.active ? q.order.run_cap : 0;
  info->max_wave_blocks = plan.max_wave_blocks;
  info->fused_append = fuses_append(p, kind) ? 1 : 0;
  info->partitions_bound = q.pmax;
  info->lds_bytes = static_cast<int32_t>(plan.lds_bytes);
  const int64_t n = std::min<int64_t>(cap, plan.cells);
  for (int64_t c = 0; c < n; ++c) {
    int s = 0, part0 = 0, part_lim = 0;
    if (!pkv::decode_cell(q, static_cast<int>(c), s, part0, part_lim)) part0 = part_lim = q.pmax;
    cells[3 * c] = s;
    cells[3 * c + 1] = part0;
    cells[3 * c + 2] = part_lim;
  }
  return PKV_OK;
}

size_t pkv_prefill_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t max_blocks, int32_t max_seq_len, int32_t dtype) {
  if (dtype != PKV_FP8_E4M3 || num_seqs < 1 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 ||
      max_blocks < 1 || max_seq_len < 1)
    return 0;
  const int64_t nb = (static_cast<int64_t>(max_seq_len) + block_size - 1) / block_size;
  return pkv::prefill_stage_bytes(num_seqs, num_kv_heads, head_dim, max_blocks, nb);
}

int pkv_paged_prefill(const pkv_prefill_args* a, void* stream) {
  if (!a) return fail(PKV_ERR_INVALID, "prefill: null args");
  if (a->dtype != PKV_BF16 && a->dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_UNSUPPORTED, "prefill: bf16 or 8-bit (E4M3) caches only");
  if (a->num_seqs < 1 || a->num_kv_heads < 1 || a->num_q_heads < 1 || a->head_dim < 1 || a->block_size < 1 ||
      a->num_blocks < 1 || a->max_blocks < 1 || a->max_seq_len < 1 || a->max_query_len < 0)
    return fail(PKV_ERR_INVALID, "prefill: sizes must be positive");
  if (a->num_q_heads % a->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "prefill: num_q_heads must be a multiple of num_kv_heads");
  if (a->window < 0) return fail(PKV_ERR_INVALID, "prefill: window must be >= 0");
  if (!(a->scale > 0.f) || !(a->scale < INFINITY))
    return fail(PKV_ERR_INVALID, "prefill: scale must be positive and finite");
  if (!pkv::prefill_shape_supported(a->head_dim, a->block_size))
    return fail(PKV_ERR_UNSUPPORTED, "prefill: supported shapes are block_size 16, head_dim 64 or 128");
  if (!a->q || !a->out || !a->k_cache || !a->v_cache || !a->block_tables || !a->seq_lens || !a->query_start)
    return fail(PKV_ERR_INVALID, "prefill: null device pointer");
  if (!aligned16(a->q) || !aligned16(a->out) || !aligned16(a->k_cache) || !aligned16(a->v_cache))
    return fail(PKV_ERR_INVALID, "prefill: q, out and caches must be 16-byte aligned");
  const int64_t G = a->num_q_heads / a->num_kv_heads;
  const int64_t tiles = (static_cast<int64_t>(a->max_query_len) * G + 63) / 64;   // >= the real count
  if (tiles > 65535 || static_cast<int64_t>(a->num_seqs) * a->num_kv_heads > 0x7fffffffLL)
    return fail(PKV_ERR_INVALID, "prefill: grid too large");
  const bool fp8 = a->dtype == PKV_FP8_E4M3;
  const int64_t nb = (static_cast<int64_t>(a->max_seq_len) + a->block_size - 1) / a->block_size;
  if (fp8) {
    if (!a->k_scale || !a->v_scale) return fail(PKV_ERR_INVALID, "prefill: an 8-bit cache needs its scales");
    const size_t need = pkv::prefill_stage_bytes(a->num_seqs, a->num_kv_heads, a->head_dim, a->max_blocks, nb);
    if (!a->workspace || a->workspace_bytes < need)
      return fail(PKV_ERR_INVALID, "prefill: an 8-bit cache needs a workspace of pkv_prefill_workspace_bytes() (" +
                                       std::to_string(need) + " bytes)");
    if (reinterpret_cast<uintptr_t>(a->workspace) % 256 != 0)
      return fail(PKV_ERR_INVALID, "prefill: workspace must be 256-byte aligned");
    if (static_cast<int64_t>(a->num_seqs) * nb > 0x7fffffffLL)
      return fail(PKV_ERR_INVALID, "prefill: too many blocks for the 8-bit copy");
  }
  if (a->max_query_len == 0) return PKV_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  pkv::PrefillParams p{};
  p.q = a->q;
  p.out = a->out;
  p.k_cache = a->k_cache;
  p.v_cache = a->v_cache;
  p.block_tables = a->block_tables;
  p.seq_lens = a->seq_lens;
  p.query_start = a->query_start;
  p.S = a->num_seqs;
  p.Hq = a->num_q_heads;
  p.Hkv = a->num_kv_heads;
  p.G = static_cast<int32_t>(G);
  p.d = a->head_dim;
  p.num_blocks = a->num_blocks;
  p.max_blocks = a->max_blocks;
  p.max_seq_len = a->max_seq_len;
  p.max_query_len = a->max_query_len;
  p.window = a->window;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  if (fp8) {                        // attend over a bf16 copy of the blocks the sequences hold
    pkv::PrefillStageParams sp{};
    sp.k_cache = static_cast<const uint8_t*>(a->k_cache);
    sp.v_cache = static_cast<const uint8_t*>(a->v_cache);
    sp.k_scale = a->k_scale;
    sp.v_scale = a->v_scale;
    sp.block_tables = a->block_tables;
    sp.seq_lens = a->seq_lens;
    sp.query_start = a->query_start;
    sp.window = a->window;
    sp.S = a->num_seqs;
    sp.Hkv = a->num_kv_heads;
    sp.d = a->head_dim;
    sp.num_blocks = a->num_blocks;
    sp.max_blocks = a->max_blocks;
    sp.max_seq_len = a->max_seq_len;
    sp.nb = static_cast<int32_t>(nb);
    pkv::prefill_stage_layout(&sp, a->workspace);
    const int rc = from_hip(pkv::launch_prefill_stage(sp, st), "prefill: 8-bit copy");
    if (rc) return rc;
    p.k_cache = sp.k_out;
    p.v_cache = sp.v_out;
    p.block_tables = sp.tables_out;
    p.num_blocks = static_cast<int32_t>(static_cast<int64_t>(a->num_seqs) * nb);
  }
  return from_hip(pkv::launch_prefill(p, st), "prefill");
}

int pkv_read_tiles(const void* base, int64_t base_bytes, int32_t tile_bytes, const int32_t* order, int64_t n_tiles,
                   int32_t tiles_per_wave, uint32_t* sink, void* stream) {
  if (tile_bytes != 1024 && tile_bytes != 2048 && tile_bytes != 4096)
    return fail(PKV_ERR_INVALID, "read_tiles: tile_bytes must be 1024, 2048 or 4096");
  if (!base || !sink || base_bytes < tile_bytes || n_tiles < 1 || tiles_per_wave < 1)
    return fail(PKV_ERR_INVALID, "read_tiles: bad argument");
  if (!aligned16(base)) return fail(PKV_ERR_INVALID, "read_tiles: base must be 16-byte aligned");
  const int64_t base_tiles = base_bytes / tile_bytes;
  if (!order && n_tiles > base_tiles) return fail(PKV_ERR_INVALID, "read_tiles: n_tiles exceeds the buffer");
  if ((n_tiles + tiles_per_wave - 1) / tiles_per_wave > 0x7fffffffLL)
    return fail(PKV_ERR_INVALID, "read_tiles: grid too large");
  return from_hip(pkv::launch_read_tiles(base, base_tiles, tile_bytes, order, n_tiles, tiles_per_wave, sink,
                                         static_cast<hipStream_t>(stream)),
                  "read_tiles");
}

}  // extern "C"
