/*
 * pkv — paged KV cache and paged decode attention for AMD MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Every function returns an int
 * status (PKV_OK = 0, negative on failure); no C++ exception crosses this
 * boundary.  pkv_last_error() gives a thread-local message for the last
 * failure on the calling thread.
 *
 * Sources of the operations (page titles; sections as printed on them):
 *  - «¿Cómo gestiona Paged Attention la caché KV…?», "PagedAttention divide
 *    el estado KV en bloques de tamaño fijo": blocks come from one shared
 *    pool as tokens arrive; a block table maps logical token order to
 *    physical blocks; the indirection moves data without changing meaning.
 *    "Los bloques liberados regresan…": finished requests return unshared
 *    blocks to the pool at once.  "La gestión de bloques…": the runtime keeps
 *    block tables, reference counts and attention kernels for paged layouts.
 *  - «PagedAttention e vLLM», "Approfondimento tecnico": fixed-size pages
 *    holding keys and values of a fixed number of tokens; one block table per
 *    sequence; identical prefixes share pages by copy-on-write.
 *  - «Paged Attention optimiza el uso de memoria»: 16-token pages allocated
 *    on demand; copy-on-write copies only the diverging page.
 *  - «Servicio…presupuesto de memoria» §6: exact attention = scaled
 *    query-key scores, softmax, weighted values, computable blockwise with
 *    running normalisation statistics.  §8: release must not free pages in
 *    use; no request may see another's private continuation.
 *  - «¿Cuánta memoria reservar para la caché KV?», "Emplear las cabezas KV":
 *    grouped-query attention, several query heads per KV head.  The same
 *    page, on quantising the cache, and «Servicio…presupuesto de memoria» §4:
 *    a lower-precision KV cache is a separate choice that changes the
 *    numerics (here: the 8-bit PKV_FP8_E4M3 pool).
 *
 * Ownership: all device memory (per-layer K/V pools, q, out, block tables,
 * sequence lengths, slot mappings, workspace) belongs to the caller; the
 * library keeps raw pointers and never frees them.  Host allocator state is
 * owned by the opaque pkv_pool.  Device work is enqueued on the caller's HIP
 * stream (a hipStream_t passed as void*, NULL = the null stream); no call
 * waits for the device except where stated.  A pkv_pool is not thread-safe:
 * the caller serialises calls on one pool.
 *
 * Pool byte layout of one layer (B = block_size tokens, a multiple of 4;
 * x = 16 / element size, i.e. 4 for fp32 and 8 for bf16; d must be a
 * multiple of x):
 *   K: [num_blocks][num_kv_heads][d / x][B][x]
 *   V: [num_blocks][num_kv_heads][B / 4][d / 4][4][4]: value column j of
 *      token offset o sits at [o / 4][j / 4][j % 4][o % 4] (each run of four
 *      values holds one column of four consecutive tokens)
 * Slot number s names block s / B, token offset s % B.  One block id
 * addresses the same token range in every layer's pool.
 *
 * 8-bit pools (PKV_FP8_E4M3; B = 16, d a multiple of 64): OCP E4M3 codes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; S.1111.111 = NaN;
 * largest magnitude 448) plus one fp32 scale per (slot, KV head) for K and
 * one for V.  The value of a code c in slot s is E4M3(c) * scale[s].
 *   K codes: [num_blocks][num_kv_heads][d / 16][B][16]   (x = 16)
 *   V codes: [num_blocks][num_kv_heads][d / 64][B / 4][16][4][4]: value
 *            column j = 64a + 4c + b of token offset o = 4u + w sits at
 *            [a][u][c][b][w] (each 16 bytes hold four columns of four
 *            consecutive tokens, the decode kernel's operand order).
 *   K and V scales: fp32 [num_blocks][num_kv_heads][B].
 * Appends quantise each (token, KV head) row of d values on its own:
 * scale = amax / 448 in fp32 (amax = largest |value|), code = the E4M3
 * value nearest to value / scale (fp32 quotient; ties to the even code); an
 * all-zero row gets scale 0 and codes 0.  Tokens, queries and outputs of an
 * 8-bit pool are bf16.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PKV_OK               0
#define PKV_ERR_INVALID     -1  /* bad argument or shape                      */
#define PKV_ERR_NO_BLOCKS   -2  /* pool exhausted; nothing was changed        */
#define PKV_ERR_BAD_SEQ     -3  /* unknown or already freed sequence id       */
#define PKV_ERR_HIP         -4  /* a HIP runtime call failed                  */
#define PKV_ERR_UNSUPPORTED -5  /* valid, but no kernel for this shape        */

/* ---- element types ----------------------------------------------------- */
#define PKV_F32      0
#define PKV_BF16     1
#define PKV_FP8_E4M3 2   /* KV pools only: 8-bit codes + per-slot scales */

/* Name of a status code (static string). */
const char* pkv_status_string(int status);
/* Message describing the last failure on this thread ("" if none). */
const char* pkv_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int pkv_version(void);

/* ---- pool and allocator ------------------------------------------------ */
typedef struct pkv_pool pkv_pool;

typedef struct pkv_pool_desc {
  int32_t num_layers;      /* >= 1                                          */
  int32_t num_kv_heads;    /* Hkv >= 1                                      */
  int32_t head_dim;        /* d, multiple of 16 bytes / element size        */
  int32_t block_size;      /* B tokens per block (16 for the attention      */
                           /*   kernels; a multiple of 4 with caches)       */
  int32_t num_blocks;      /* pool capacity in blocks, >= 1                 */
  int32_t dtype;           /* PKV_F32, PKV_BF16 or PKV_FP8_E4M3             */
  void* const* k_cache;    /* [num_layers] device pointers, or NULL for an  */
  void* const* v_cache;    /*   allocator-only pool (no device calls)       */
  const int32_t* init_perm;/* optional host [num_blocks] permutation: the   */
                           /*   free list hands out init_perm[0], [1], ...  */
  void* const* k_scale;    /* PKV_FP8_E4M3 with caches: [num_layers] device */
  void* const* v_scale;    /*   pointers to fp32 [num_blocks][Hkv][B]       */
                           /*   scale arrays; ignored for other dtypes      */
} pkv_pool_desc;

/* Create a pool.  The descriptor's arrays are copied.  Free list starts with
 * every block (in init_perm order, or 0, 1, 2, ...); reference counts 0.    */
int pkv_pool_create(const pkv_pool_desc* desc, pkv_pool** out);
/* Destroy a pool (waits for its last table upload to finish).  NULL is ok. */
int pkv_pool_destroy(pkv_pool* pool);

/* New empty sequence.  Ids start at 0, increase by one, are never reused. */
int pkv_seq_create(pkv_pool* pool, int64_t* seq_id);
/* New sequence sharing every block of `parent` (each block's reference count
 * +1), with the parent's length.                                            */
int pkv_seq_fork(pkv_pool* pool, int64_t parent, int64_t* child);
/* Release a sequence (finished or cancelled): walk its table in logical
 * order, decrement each block's count and push blocks that reach 0 onto the
 * free list (blocks the prefix cache or other sequences hold stay).        */
int pkv_seq_free(pkv_pool* pool, int64_t seq_id);

/* Sliding window: give back every block of a sequence that holds only
 * positions < pos (block i with (i + 1) * B <= pos), walking its table in
 * logical order; a block's count drops by one and it returns to the free
 * list at zero.  Released entries read -1 in tables (a table stays indexed
 * by position); they are never read again by appends or by a decode whose
 * window starts at or after pos.  0 <= pos <= length, else
 * PKV_ERR_INVALID.  *n_released (may be NULL) gets the number of blocks
 * released by this call.                                                   */
int pkv_seq_release_before(pkv_pool* pool, int64_t seq_id, int32_t pos, int32_t* n_released);

/* ---- prefix cache ------------------------------------------------------
 * «Servicio…presupuesto de memoria» §8: a cache key names every input that
 * shapes the KV state (the namespace `ns` stands for model version and
 * configuration); reused pages never expose or let anyone change another
 * request's private continuation; eviction drops references without freeing
 * pages still in use.  «PagedAttention e vLLM»: a shared system prompt is
 * processed once.  Only full blocks are cached.  An entry is keyed exactly
 * by (ns, parent entry, the block's B token ids) and holds one reference to
 * its block.  "Use" is a logical clock advanced by each register or match. */

/* Enter the full blocks of a sequence, walked from position 0, under the
 * token ids tokens[0 .. n_tokens) (n_tokens >= its length, else
 * PKV_ERR_INVALID): a known key is touched (an entry naming another block
 * of the same content is kept), an unknown one becomes an entry for the
 * sequence's block (one more reference).  Stops at a released block.
 * *n_added (may be NULL) gets the number of new entries.                  */
int pkv_prefix_register(pkv_pool* pool, int64_t seq_id, const int32_t* tokens, int32_t n_tokens, uint64_t ns,
                        int32_t* n_added);
/* New sequence made of the longest cached chain matching the leading full
 * blocks of tokens[0 .. n_tokens): one more reference per block (as a
 * fork), length = matched tokens (*n_matched, a multiple of B, may be 0).
 * Its next token starts a fresh block, so cached blocks are never written. */
int pkv_prefix_match(pkv_pool* pool, const int32_t* tokens, int32_t n_tokens, uint64_t ns, int64_t* seq_id,
                     int32_t* n_matched);
/* Free up to max_blocks blocks: repeatedly drop the least recently used
 * entry that has no child entry and whose block only the cache holds
 * (deeper entries first on equal use); the block returns to the free list.
 * Blocks still used by a sequence are never freed.  *n_freed may be NULL. */
int pkv_prefix_evict(pkv_pool* pool, int32_t max_blocks, int32_t* n_freed);
/* Drop every entry (deepest first), e.g. after a model or configuration
 * change; blocks only the cache held return to the free list.             */
int pkv_prefix_clear(pkv_pool* pool, int32_t* n_dropped);
/* Cache entries by index: first call with NULL arrays for *n_entries, then
 * with arrays of that size (tokens_out: [n_entries][B]).  Host only.       */
int pkv_prefix_snapshot(const pkv_pool* pool, int64_t* n_entries, int64_t* entry_out, uint64_t* ns_out,
                        int64_t* parent_out, int32_t* block_out, int64_t* last_use_out, int32_t* tokens_out);

/* Reserve `ntok` >= 0 consecutive slots for one sequence (bulk prefill).
 * slots_out: host int32[ntok].  cow_pairs_out: host int32[2] receiving at
 * most one (src, dst) block pair; *n_cow gets the count (0 or 1).
 * All-or-nothing: PKV_ERR_NO_BLOCKS leaves the pool unchanged.             */
int pkv_seq_extend(pkv_pool* pool, int64_t seq_id, int32_t ntok, int32_t* slots_out,
                   int32_t* cow_pairs_out, int32_t* n_cow);

/* Reserve one slot for each of `n` distinct ids, in array order (the decode
 * step).  For the token at position pos = current length:
 *   pos % B == 0            -> pop a free block, count 1, append to table;
 *   else, last block count>1 -> pop a free block (count 1), the shared block
 *                              loses one reference, (old, new) is recorded
 *                              and replaces the table's last entry;
 *   slot = table[pos / B] * B + pos % B; length += 1.
 * slots_out: host int32[n].  cow_pairs_out: host int32[2 * n] receiving
 * (src, dst) pairs in order; *n_cow their count.  Recorded pairs must be
 * copied (pkv_copy_blocks) before the new tokens are written.  Duplicate ids
 * are PKV_ERR_INVALID.  All-or-nothing.                                    */
int pkv_append_slots(pkv_pool* pool, const int64_t* ids, int32_t n, int32_t* slots_out,
                     int32_t* cow_pairs_out, int32_t* n_cow);

/* Current length of a sequence. */
int pkv_seq_length(const pkv_pool* pool, int64_t seq_id, int32_t* len);
/* Host copy of a sequence's block table: writes min(cap, nblocks) entries to
 * table_out and the table length to *nblocks.                              */
int pkv_seq_table(const pkv_pool* pool, int64_t seq_id, int32_t* table_out, int32_t cap,
                  int32_t* nblocks);

/* Upload the block tables and lengths of `n` sequences to caller-owned
 * device arrays: dev_block_tables int32[n][max_blocks] (row i = ids[i],
 * unused entries -1) and dev_seq_lens int32[n].  Asynchronous on `stream`
 * by one small kernel that reads a pinned staging buffer owned by the pool.
 * The pool keeps a ring of eight such buffers and marks the end of every
 * fourth upload with an event, so a call waits (on the host) only at the
 * start of a group of four, for the group that used the same buffers eight
 * uploads earlier; calls may use different streams.  pkv_pool_destroy waits
 * for the device when uploads are in flight.  If
 * host_seq_lens_out is not NULL it also receives the lengths (host int32[n]),
 * e.g. to pass as pkv_decode_args.host_seq_lens.  PKV_ERR_INVALID if a
 * sequence holds more than max_blocks blocks.                              */
int pkv_sync_tables(pkv_pool* pool, const int64_t* ids, int32_t n, int32_t* dev_block_tables,
                    int32_t max_blocks, int32_t* dev_seq_lens, int32_t* host_seq_lens_out,
                    void* stream);

/* Copy-on-write copy: for each host pair (src, dst) in pairs[2 * n_pairs],
 * block dst := block src in K and V of every layer (all heads, all slots;
 * with the scales too in an 8-bit pool).  Runs one kernel on `stream`.     */
int pkv_copy_blocks(pkv_pool* pool, const int32_t* pairs, int32_t n_pairs, void* stream);

/* Write new tokens of one layer: token i's K and V (device, contiguous
 * [n][num_kv_heads][head_dim] in the pool dtype, bf16 for an 8-bit pool,
 * which quantises them as stated above) go to slot dev_slot_mapping[i]
 * (device int32[n]).  Slots outside the pool are skipped.  Runs one kernel
 * on `stream`.                                                             */
int pkv_kv_append(pkv_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                  const int32_t* dev_slot_mapping, int32_t n, void* stream);

/* The decode-step form of kv_append: token i's K and V go to the last
 * position (length - 1) of row i of tables uploaded by pkv_sync_tables,
 * i.e. to slot dev_block_tables[i][(len-1) / B] * B + (len-1) % B with
 * len = dev_seq_lens[i].  Rows with len < 1, len > max_blocks * B or a block
 * id outside the pool are skipped.  Runs one kernel on `stream`.           */
int pkv_kv_append_last(pkv_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                       const int32_t* dev_block_tables, int32_t max_blocks,
                       const int32_t* dev_seq_lens, int32_t n, void* stream);

typedef struct pkv_stats {
  int64_t num_blocks, free_blocks, used_blocks;
  int64_t num_seqs, sum_len, sum_ref, tail_waste;
} pkv_stats;
int pkv_pool_stats(const pkv_pool* pool, pkv_stats* out);

/* Allocator state for exact comparison.  First call with NULL arrays to get
 * the sizes (*n_free, *n_seqs, *n_entries = total table entries), then with
 * arrays of those sizes: free_out[n_free] (stack, bottom to top),
 * ref_out[num_blocks], ids_out[n_seqs] (ascending), lens_out[n_seqs],
 * table_off_out[n_seqs + 1] (row i = tables_out[off[i] .. off[i+1])),
 * tables_out[n_entries], *next_id.  Host only.                             */
int pkv_pool_snapshot(const pkv_pool* pool, int32_t* free_out, int32_t* ref_out,
                      int64_t* ids_out, int32_t* lens_out, int64_t* table_off_out,
                      int32_t* tables_out, int64_t* n_free, int64_t* n_seqs,
                      int64_t* n_entries, int64_t* next_id);

/* ---- paged decode attention --------------------------------------------
 * For each sequence s (length n = seq_lens[s]) and query head h, with
 * G = Hq / Hkv and KV head g = h / G:
 *   out[s][h] = sum_t softmax_t(scale * q[s][h] . K_s[t]) V_s[t],
 *   K_s[t] = K[block_tables[s][t / B]][g][token t % B], same for V,
 * accumulated in fp32, rounded to the q/out dtype (nearest even).  With
 * window W > 0 the sum runs over t = max(0, n - W) .. n - 1 only (sliding
 * window, «¿Cuánta memoria reservar para la caché KV?», "Adaptar…"); blocks
 * before the window are not read and may have been released.
 * Tokens are split into partitions of `partition` tokens (split-K); a
 * sequence with more than one partition writes fp32 partial results
 * (running max, running sum, unnormalised accumulator) to the workspace and
 * a reduce kernel merges them.  Sequences with n < 1, n > max_seq_len or a
 * block id outside [0, num_blocks) get NaN rows (the kernels read nothing
 * outside the pool).  Supported: block_size 16, head_dim 64 or 128, any
 * Hq multiple of Hkv; bf16 queries may read an 8-bit (PKV_FP8_E4M3) cache,
 * whose values are code * scale as stated above.                           */
typedef struct pkv_decode_args {
  const void* q;              /* device [S][Hq][d], dtype                   */
  void* out;                  /* device [S][Hq][d], dtype                   */
  void* k_cache;              /* device, one layer, layout above; written   */
  void* v_cache;              /*   only by the fused append (k_new)         */
  const int32_t* block_tables;/* device [S][max_blocks]                     */
  const int32_t* seq_lens;    /* device [S]                                 */
  void* workspace;            /* device, >= pkv_decode_workspace_bytes(...) */
  size_t workspace_bytes;
  int32_t num_seqs;           /* S >= 1                                     */
  int32_t num_q_heads;        /* Hq                                         */
  int32_t num_kv_heads;       /* Hkv, divides Hq                            */
  int32_t head_dim;           /* d                                          */
  int32_t block_size;         /* B                                          */
  int32_t num_blocks;         /* pool capacity (bounds check)               */
  int32_t max_blocks;         /* row stride of block_tables                 */
  int32_t max_seq_len;        /* upper bound of seq_lens (sizes the grid)   */
  int32_t partition;          /* tokens per split-K partition, multiple of  */
                              /*   32; 0 = 512                              */
  int32_t dtype;              /* PKV_F32 or PKV_BF16: q and out             */
  float scale;                /* score scale, e.g. 1/sqrt(d)                */
  const int32_t* host_seq_lens; /* optional host copy of seq_lens [S], read */
                              /*   only to plan the launch (which waves,    */
                              /*   how many partitions each); NULL =        */
                              /*   unknown.  Results do not depend on it,   */
                              /*   even when it is wrong or stale.          */
  float* k_scale;             /* 8-bit cache: device scales of this layer,  */
  float* v_scale;             /*   fp32 [num_blocks][Hkv][B]; else unused   */
  int32_t kv_dtype;           /* cache type: equal to dtype, or             */
                              /*   PKV_FP8_E4M3 with dtype PKV_BF16         */
  int32_t window;             /* > 0: attend to the last `window` positions */
                              /*   only; 0 = full attention                 */
  const void* k_new;          /* optional fused append: device [S][Hkv][d], */
  const void* v_new;          /*   16-byte aligned, in the cache dtype (bf16 */
                              /*   for an 8-bit cache); see below; NULL =   */
                              /*   none (both or neither)                   */
} pkv_decode_args;

/* Fused append (k_new, v_new set): row s of k_new / v_new is token
 * seq_lens[s] - 1 of sequence s.  The partial kernel writes it into the pool
 * exactly as pkv_kv_append_last with the same tables would (same bytes; an
 * 8-bit cache quantises it the same way), and the attention sees it: every
 * wave that reads the sequence's last block substitutes the token for its
 * slot in the registers holding that block, and the wave of the first 16
 * query heads writes it to the pool after its last load (no load depends on
 * that write).  With more than 1024 (sequence, KV head) rows, or an fp32
 * cache, the call runs the append kernel first instead (the writes inside
 * the partial kernel's read stream then cost more than that kernel).  Rows
 * the decode cannot read (a length outside [1, max_seq_len], or a block id
 * outside the pool among the last wave's blocks) may or may not receive the
 * token; their outputs are NaN.  The block that receives the token must not
 * be shared (copy it first, as for any append).  pkv_paged_decode_reduce
 * ignores these fields.                                                    */

/* Workspace bytes the decode call needs (0 when one partition suffices);
 * enough for any window, which needs at most as much.                     */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_seq_len, int32_t partition);
/* Partial kernel followed, when max_seq_len exceeds one partition, by the
 * reduce kernel; both on `stream`.  The call only launches kernels (no
 * allocation, copy, memset or synchronisation), all reading their inputs
 * through the pointers in `args`, so it can be captured in a HIP graph and
 * replayed: each replay reads the buffers' contents at that time.  The
 * launch plan (from host_seq_lens, when given) is fixed at capture; the
 * results never depend on it.                                              */
int pkv_paged_attention_decode(const pkv_decode_args* args, void* stream);
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that must not allocate, harnesses that forbid it):
 * pkv_paged_attention_decode with the library's own workspace instead of
 * args->workspace (ignored, as is workspace_bytes).  That workspace is a
 * device array of 64 MiB (67,108,864 bytes) inside the library, one per
 * device, held until the process ends; its address is looked up on the
 * first call on each device, and no call allocates anything.  A call whose
 * pkv_decode_workspace_bytes() exceeds 64 MiB fails with PKV_ERR_INVALID
 * before any device work.  Every call on one device uses the same array:
 * calls that overlap on a device (other streams, other threads) race on it,
 * so the caller serialises them.  The workspace needs no clearing (every
 * partial result is written before the reduce reads it).  Under graph
 * capture, make one call on the device outside the capture first (the
 * address lookup).  Other arguments, errors and results are those of
 * pkv_paged_attention_decode.                                              */
int pkv_paged_attention_decode_static(const pkv_decode_args* args, void* stream);
/* The partial kernel alone (single-partition sequences are finished here). */
int pkv_paged_decode_partial(const pkv_decode_args* args, void* stream);
/* The reduce kernel alone (no-op when one partition suffices). */
int pkv_paged_decode_reduce(const pkv_decode_args* args, void* stream);
/* 1 if a decode call with these arguments writes the new tokens in the
 * partial kernel (k_new set, a bf16 or 8-bit cache and at most 1024
 * (sequence, KV head) rows), 0 if it would run the append kernel first or
 * has no k_new; a negative status for invalid arguments (as the decode
 * call).  Reads nothing on the device.                                    */
int pkv_decode_fuses_append(const pkv_decode_args* args);

/* The partial kernel's launch as a decode call with these arguments would
 * make it, planned on the host; nothing runs and nothing on the device is
 * read.  The grid is cells x num_kv_heads waves by head_groups; cell c's
 * waves read sequence s and its partitions [first, end) (numbered from the
 * first partition that overlaps the window, clipped on the device to the
 * partitions the device length has), so that every partition a sequence
 * has is read by exactly one cell and exactly one cell per sequence starts
 * at partition 0, whatever the host lengths say.  The order of cells is the
 * launch order.  (The split into partitions merged by running statistics is
 * «Servicio…presupuesto de memoria» §6's blockwise attention; which wave
 * takes which partitions is this library's own scheduling.)
 *   info   out: the plan (below).
 *   cells  out, optional: 3 int32 per cell, (s, first, end), for the first
 *          min(cap, info->cells) cells; first == end == partitions_bound for
 *          a cell whose waves exit at once (a sweep range the host lengths
 *          already cover).
 * Returns PKV_OK or the decode call's status for invalid arguments.        */
typedef struct pkv_decode_plan_info {
  int64_t cells;
  int64_t listed_cells;         /* work list: the cells it names (the rest sweep partitions past
                                   the host lengths, in case the device lengths are longer) */
  int32_t head_groups;          /* grid y: query heads of a KV head, 16 per wave */
  int32_t pipeline_depth;       /* blocks in flight per wave in the chosen kernel */
  int32_t resident_waves;       /* wave slots of that kernel on the device (0: not queried) */
  int32_t partitions_per_wave;  /* plain grid: partitions per run; 1 with the work list */
  int32_t work_list;            /* 1 if cells follow the host lengths' work list */
  int32_t run_cap;              /* work list: most partitions one cell may take */
  int32_t max_wave_blocks;      /* most blocks one wave streams */
  int32_t fused_append;         /* 1 if the partial kernel writes k_new / v_new */
  int32_t partitions_bound;     /* partitions of max_seq_len (of the window, with one) */
  int32_t lds_bytes;            /* dynamic LDS per wave */
} pkv_decode_plan_info;
int pkv_decode_plan(const pkv_decode_args* args, pkv_decode_plan_info* info, int32_t* cells, int64_t cap);

/* ---- paged prefill attention -------------------------------------------
 * Chunked prefill («Servicio…presupuesto de memoria» §6: exact attention,
 * blockwise with running statistics; §2/§4: prefill work has another shape
 * than decode): sequence s holds n = seq_lens[s] tokens in the cache, the
 * last m = query_start[s+1] - query_start[s] of which are new and already
 * written (pkv_seq_extend + pkv_kv_append).  Query row query_start[s] + i
 * sits at position p = n - m + i; for query head h (KV head g = h / G):
 *   out[row][h] = sum_t softmax_t(scale * q[row][h] . K_s[t]) V_s[t],
 * t over 0 .. p (the last `window` of those when window > 0), K_s / V_s
 * gathered through block_tables as for decode.  fp32 accumulation, bf16
 * output (nearest even).  Sequences with m > n, n > max_seq_len or a needed
 * block id outside the pool get NaN rows; m = 0 is allowed (no rows).
 * Supported: bf16 q/out, block_size 16, head_dim 64 or 128; a bf16 cache,
 * or an 8-bit (PKV_FP8_E4M3) cache with its scales and a workspace of
 * pkv_prefill_workspace_bytes() bytes («¿Cuánta memoria reservar para la
 * caché KV?», "Reducir la precisión").  For the 8-bit cache the call first
 * writes every block the sequences hold as bf16 (code × scale in fp32,
 * rounded to nearest even) into the workspace, laid out as a bf16 pool
 * with tables of its own, and attends over that copy: the same kernel and
 * the same results as a bf16 cache holding those rounded values.  The
 * workspace is scratch, overwritten by each call (calls sharing it must not
 * overlap); it needs no clearing.                                          */
typedef struct pkv_prefill_args {
  const void* q;              /* device [T][Hq][d] bf16, T = query_start[S] */
  void* out;                  /* device [T][Hq][d] bf16                     */
  const void* k_cache;        /* device, one layer, pool layout             */
  const void* v_cache;
  const int32_t* block_tables;/* device [S][max_blocks]                     */
  const int32_t* seq_lens;    /* device [S]: tokens cached, chunk included  */
  const int32_t* query_start; /* device [S + 1]: prefix sums of chunk sizes */
  int32_t num_seqs;           /* S >= 1                                     */
  int32_t num_q_heads;        /* Hq                                         */
  int32_t num_kv_heads;       /* Hkv, divides Hq                            */
  int32_t head_dim;           /* d                                          */
  int32_t block_size;         /* B                                          */
  int32_t num_blocks;         /* pool capacity (bounds check)               */
  int32_t max_blocks;         /* row stride of block_tables                 */
  int32_t max_seq_len;        /* upper bound of seq_lens                    */
  int32_t max_query_len;      /* upper bound of the chunk sizes (grid)      */
  int32_t dtype;              /* PKV_BF16                                   */
  float scale;                /* score scale, e.g. 1/sqrt(d); positive and  */
                              /*   finite (else PKV_ERR_INVALID)            */
  int32_t window;             /* > 0: sliding window; 0 = causal, full      */
  /* 8-bit cache only (dtype PKV_FP8_E4M3; ignored for bf16):                */
  const float* k_scale;       /* device per-slot K scales [num_blocks][Hkv][B] */
  const float* v_scale;       /* device per-slot V scales, same shape        */
  void* workspace;            /* device, 256-byte aligned                    */
  size_t workspace_bytes;     /* >= pkv_prefill_workspace_bytes(...)         */
} pkv_prefill_args;
/* Workspace bytes pkv_paged_prefill needs: 0 for a bf16 cache; for an 8-bit
 * cache the bf16 copy (num_seqs · ceil(max_seq_len / block_size) blocks of
 * K and V) and its tables (num_seqs · max_blocks int32).  0 for sizes the
 * call would reject.                                                       */
size_t pkv_prefill_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks, int32_t max_seq_len,
                                   int32_t dtype);

/* One kernel on `stream`; no workspace.                                    */
int pkv_paged_prefill(const pkv_prefill_args* args, void* stream);

/* ---- read-bandwidth calibration ----------------------------------------
 * A measurement aid, not part of attention («Servicio…presupuesto de
 * memoria» §2: an IO-aware attention kernel is about the memory traffic it
 * causes, so a decode rate is set against what memory delivers for the same
 * access pattern).  Reads n_tiles tiles of tile_bytes bytes, 4096 (one KV
 * head's 16 tokens at d = 128, bf16), 2048 (the same in 8-bit codes, or at
 * d = 64 in bf16) or 1024 (8-bit codes at d = 64); else PKV_ERR_INVALID,
 * from the device buffer `base` (base_bytes long, 16-byte
 * aligned): wave w reads tile order[w * tpw + i] for i < tiles_per_wave
 * (tile w * tpw + i when order is NULL), each as 16-byte non-temporal
 * loads, lane l taking the vectors l, l + 64, ... of the tile.  sink (device uint32[ceil(n_tiles / tpw) * 64])
 * receives, per wave and lane, the xor of every 32-bit word the lane read.
 * order (device int32[n_tiles]) may hold any ids; ids outside the buffer
 * read nothing.  Without order, n_tiles * tile_bytes must fit in
 * base_bytes (else PKV_ERR_INVALID).  One kernel on `stream`.             */
int pkv_read_tiles(const void* base, int64_t base_bytes, int32_t tile_bytes, const int32_t* order,
                   int64_t n_tiles, int32_t tiles_per_wave, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
