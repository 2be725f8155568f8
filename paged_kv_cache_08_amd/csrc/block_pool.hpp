// Host-side block allocator of the paged KV cache (no HIP dependency).
//
// «¿Cómo gestiona Paged Attention la caché KV…?», "PagedAttention divide el
// estado KV en bloques de tamaño fijo": fixed-size blocks come from one
// shared pool as a request's tokens arrive, and a per-request table maps
// logical order onto them.  "Los bloques liberados regresan…": a finished
// request's unshared blocks go back to the pool at once.  «PagedAttention e
// vLLM», "Approfondimento tecnico", and «Paged Attention optimiza el uso de
// memoria» (copy-on-write paragraph): identical prefixes point at the same
// pages; a writer copies only the page it would change.  «Servicio…
// presupuesto de memoria» §8: release drops references without freeing
// pages still in use.
//
// Choices where the pages leave freedom (any free block is a correct pick):
// the free list is a stack (initial order handed out first, freed blocks
// reused first); ids count up from 0; a batch is served in array order; a
// release walks the table in logical order; every mutating call is
// all-or-nothing, checked before anything changes.
//
// Sliding window («¿Cuánta memoria reservar para la caché KV?», "Adaptar…":
// a windowed layer keeps a bounded history; «¿Cómo gestiona…?»: a window
// changes how much state a sequence keeps, paging how it is allocated):
// release_before gives back the blocks that hold only positions before the
// window and marks their table entries kHole, so tables stay indexed by
// position.
//
// Prefix cache («Servicio…presupuesto de memoria» §8: the key identifies every
// input that shapes the state, model version and configuration included; no
// request may see or change another's continuation; eviction drops
// references without freeing pages in use.  «PagedAttention e vLLM»: a shared
// system prompt is processed once): only full blocks are cached; an entry is
// keyed exactly by (namespace, parent entry, the block's token ids) and holds
// one reference to its block.  A match builds a new sequence from the longest
// cached chain (a block per matched full block, one more reference each);
// eviction drops the least recently used leaf entry whose block only the
// cache holds (deeper entries first on equal use), one at a time.  Use is a
// logical clock advanced once per register or match call.
#pragma once

#include <cstdint>
#include <map>
#include <string>
#include <unordered_map>
#include <vector>

namespace pkv {

enum class Status : int { Ok = 0, Invalid = -1, NoBlocks = -2, BadSeq = -3 };

constexpr int32_t kHole = -1;   // table entry of a block given back by release_before

struct Sequence {
  int32_t len = 0;
  std::vector<int32_t> table;
};

struct PrefixKey {
  uint64_t ns = 0;
  int64_t parent = -1;                 // entry index of the previous block, -1 at position 0
  std::vector<int32_t> tokens;         // the block's token ids
  bool operator==(const PrefixKey& o) const { return ns == o.ns && parent == o.parent && tokens == o.tokens; }
};

struct PrefixKeyHash {
  size_t operator()(const PrefixKey& k) const;
};

struct PrefixEntry {
  PrefixKey key;
  int32_t block = 0;
  int64_t last_use = 0;
  int32_t depth = 0;                   // block index in the chain
  int32_t children = 0;                // entries whose parent this is
};

class BlockPool {
 public:
  BlockPool(int32_t num_blocks, int32_t block_size, const int32_t* init_perm);

  int32_t num_blocks() const { return num_blocks_; }
  int32_t block_size() const { return block_; }

  Status create(int64_t* id);
  Status fork(int64_t parent, int64_t* child);
  Status release(int64_t id);
  // Gives back the blocks holding only positions < pos (0 <= pos <= length),
  // in logical order; their entries become kHole.
  Status release_before(int64_t id, int32_t pos, int32_t* n_released);
  // k slots for one sequence; at most one copy-on-write pair.
  Status extend(int64_t id, int32_t k, int32_t* slots, int32_t* cow, int32_t* n_cow);
  // one slot per id, in order.
  Status append(const int64_t* ids, int32_t n, int32_t* slots, int32_t* cow, int32_t* n_cow);

  // Prefix cache.
  Status prefix_register(int64_t id, const int32_t* tokens, int32_t n_tokens, uint64_t ns, int32_t* added);
  Status prefix_match(const int32_t* tokens, int32_t n_tokens, uint64_t ns, int64_t* id, int32_t* matched);
  Status prefix_evict(int32_t k, int32_t* freed);
  Status prefix_clear(int32_t* dropped);
  const std::map<int64_t, PrefixEntry>& prefix_entries() const { return pc_; }

  const Sequence* find(int64_t id) const;
  const std::vector<int32_t>& free_stack() const { return free_; }
  const std::vector<int32_t>& refcounts() const { return ref_; }
  const std::unordered_map<int64_t, Sequence>& sequences() const { return seqs_; }
  int64_t next_id() const { return next_id_; }
  const std::string& error() const { return err_; }

 private:
  // Takes the next block for `seq`'s token at its current length, copying a
  // shared partial block when needed; returns the slot.  Callers have
  // already checked that enough free blocks exist.
  int32_t take_slot(Sequence& seq, int32_t* cow, int32_t* n_cow);
  int32_t pop_free();
  void drop_entry(int64_t e);

  int32_t num_blocks_;
  int32_t block_;
  std::vector<int32_t> free_;    // stack: back() is the next block handed out
  std::vector<int32_t> ref_;
  std::unordered_map<int64_t, Sequence> seqs_;
  int64_t next_id_ = 0;
  std::unordered_map<PrefixKey, int64_t, PrefixKeyHash> pc_index_;
  std::map<int64_t, PrefixEntry> pc_;  // by entry index
  int64_t pc_next_ = 0;
  int64_t pc_clock_ = 0;
  std::string err_;
};

}  // namespace pkv
