// Host-side block allocator (see block_pool.hpp for the sources and choices).
#include "block_pool.hpp"

#include <algorithm>
#include <unordered_set>

namespace pkv {

BlockPool::BlockPool(int32_t num_blocks, int32_t block_size, const int32_t* init_perm)
    : num_blocks_(num_blocks), block_(block_size), ref_(num_blocks, 0) {
  free_.resize(num_blocks);
  // The stack's top (back) is handed out first, so store the order reversed.
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = init_perm ? init_perm[i] : i;
    free_[num_blocks - 1 - i] = b;
  }
}

Status BlockPool::create(int64_t* id) {
  const int64_t sid = next_id_++;
  seqs_.emplace(sid, Sequence{});
  *id = sid;
  return Status::Ok;
}

Status BlockPool::fork(int64_t parent, int64_t* child) {
  auto it = seqs_.find(parent);
  if (it == seqs_.end()) {
    err_ = "fork: unknown sequence id " + std::to_string(parent);
    return Status::BadSeq;
  }
  Sequence copy = it->second;
  for (int32_t b : copy.table)
    if (b != kHole) ref_[b] += 1;
  const int64_t sid = next_id_++;
  seqs_.emplace(sid, std::move(copy));
  *child = sid;
  return Status::Ok;
}

Status BlockPool::release(int64_t id) {
  auto it = seqs_.find(id);
  if (it == seqs_.end()) {
    err_ = "free: unknown sequence id " + std::to_string(id);
    return Status::BadSeq;
  }
  for (int32_t b : it->second.table) {
    if (b != kHole && --ref_[b] == 0) free_.push_back(b);
  }
  seqs_.erase(it);
  return Status::Ok;
}

Status BlockPool::release_before(int64_t id, int32_t pos, int32_t* n_released) {
  *n_released = 0;
  auto it = seqs_.find(id);
  if (it == seqs_.end()) {
    err_ = "release_before: unknown sequence id " + std::to_string(id);
    return Status::BadSeq;
  }
  Sequence& seq = it->second;
  if (pos < 0 || pos > seq.len) {
    err_ = "release_before: position " + std::to_string(pos) + " outside [0, " + std::to_string(seq.len) + "]";
    return Status::Invalid;
  }
  // block i holds positions [i*B, (i+1)*B): wholly before pos iff i < pos / B
  for (int32_t i = 0; i < pos / block_; ++i) {
    int32_t& b = seq.table[i];
    if (b == kHole) continue;
    if (--ref_[b] == 0) free_.push_back(b);
    b = kHole;
    *n_released += 1;
  }
  return Status::Ok;
}

int32_t BlockPool::pop_free() {
  const int32_t b = free_.back();
  free_.pop_back();
  return b;
}

int32_t BlockPool::take_slot(Sequence& seq, int32_t* cow, int32_t* n_cow) {
  const int32_t pos = seq.len;
  const int32_t off = pos % block_;
  if (off == 0) {
    const int32_t b = pop_free();
    ref_[b] = 1;
    seq.table.push_back(b);
  } else {
    const int32_t shared = seq.table.back();
    if (ref_[shared] > 1) {
      const int32_t b = pop_free();
      ref_[shared] -= 1;
      ref_[b] = 1;
      cow[2 * *n_cow] = shared;
      cow[2 * *n_cow + 1] = b;
      *n_cow += 1;
      seq.table.back() = b;
    }
  }
  seq.len = pos + 1;
  return seq.table[pos / block_] * block_ + off;
}

Status BlockPool::extend(int64_t id, int32_t k, int32_t* slots, int32_t* cow, int32_t* n_cow) {
  *n_cow = 0;
  if (k < 0) {
    err_ = "extend: negative token count";
    return Status::Invalid;
  }
  auto it = seqs_.find(id);
  if (it == seqs_.end()) {
    err_ = "extend: unknown sequence id " + std::to_string(id);
    return Status::BadSeq;
  }
  Sequence& seq = it->second;
  if (static_cast<int64_t>(seq.len) + k > INT32_MAX / 2) {
    err_ = "extend: sequence length overflow";
    return Status::Invalid;
  }
  // Blocks needed: one per block boundary crossed, plus one copy if the
  // first token lands in a shared partial block.
  int64_t need = 0;
  const int32_t first = seq.len;
  if (k > 0) {
    if (first % block_ != 0 && ref_[seq.table.back()] > 1) need += 1;
    const int32_t last = first + k - 1;
    // positions p in [first, last] with p % B == 0
    need += last / block_ - (first + block_ - 1) / block_ + 1;
  }
  if (need > static_cast<int64_t>(free_.size())) {
    err_ = "extend: pool exhausted (need " + std::to_string(need) + " blocks, " +
           std::to_string(free_.size()) + " free)";
    return Status::NoBlocks;
  }
  for (int32_t i = 0; i < k; ++i) slots[i] = take_slot(seq, cow, n_cow);
  return Status::Ok;
}

Status BlockPool::append(const int64_t* ids, int32_t n, int32_t* slots, int32_t* cow,
                         int32_t* n_cow) {
  *n_cow = 0;
  if (n < 0) {
    err_ = "append: negative batch size";
    return Status::Invalid;
  }
  std::unordered_set<int64_t> seen;
  seen.reserve(static_cast<size_t>(n) * 2);
  std::vector<Sequence*> seq(n);
  for (int32_t i = 0; i < n; ++i) {
    if (!seen.insert(ids[i]).second) {
      err_ = "append: duplicate id " + std::to_string(ids[i]) + " in batch";
      return Status::Invalid;
    }
    auto it = seqs_.find(ids[i]);
    if (it == seqs_.end()) {
      err_ = "append: unknown sequence id " + std::to_string(ids[i]);
      return Status::BadSeq;
    }
    seq[i] = &it->second;
  }
  // Dry run over reference counts: the batch's copy-on-write decisions can
  // depend on earlier entries of the same batch (two sharers of one block).
  std::unordered_map<int32_t, int32_t> dec;
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    const Sequence& s = *seq[i];
    if (s.len % block_ == 0) {
      need += 1;
    } else {
      const int32_t b = s.table.back();
      auto d = dec.find(b);
      const int32_t r = ref_[b] - (d == dec.end() ? 0 : d->second);
      if (r > 1) {
        need += 1;
        dec[b] += 1;
      }
    }
  }
  if (need > static_cast<int64_t>(free_.size())) {
    err_ = "append: pool exhausted (need " + std::to_string(need) + " blocks, " +
           std::to_string(free_.size()) + " free)";
    return Status::NoBlocks;
  }
  for (int32_t i = 0; i < n; ++i) slots[i] = take_slot(*seq[i], cow, n_cow);
  return Status::Ok;
}

size_t PrefixKeyHash::operator()(const PrefixKey& k) const {
  // FNV-1a over the key's words (only a bucket choice: keys compare exactly)
  uint64_t h = 1469598103934665603ull;
  auto mix = [&h](uint64_t w) {
    for (int i = 0; i < 8; ++i) {
      h ^= (w >> (8 * i)) & 0xFFu;
      h *= 1099511628211ull;
    }
  };
  mix(k.ns);
  mix(static_cast<uint64_t>(k.parent));
  for (int32_t t : k.tokens) mix(static_cast<uint32_t>(t));
  return static_cast<size_t>(h);
}

Status BlockPool::prefix_register(int64_t id, const int32_t* tokens, int32_t n_tokens, uint64_t ns,
                                  int32_t* added) {
  *added = 0;
  auto it = seqs_.find(id);
  if (it == seqs_.end()) {
    err_ = "prefix_register: unknown sequence id " + std::to_string(id);
    return Status::BadSeq;
  }
  Sequence& seq = it->second;
  if (n_tokens < seq.len || (n_tokens > 0 && !tokens)) {
    err_ = "prefix_register: fewer token ids than the sequence holds";
    return Status::Invalid;
  }
  pc_clock_ += 1;
  int64_t parent = -1;
  for (int32_t i = 0; i < seq.len / block_; ++i) {
    const int32_t b = seq.table[i];
    if (b == kHole) break;
    PrefixKey key{ns, parent, std::vector<int32_t>(tokens + static_cast<size_t>(i) * block_,
                                                   tokens + static_cast<size_t>(i + 1) * block_)};
    auto f = pc_index_.find(key);
    int64_t e;
    if (f == pc_index_.end()) {
      e = pc_next_++;
      PrefixEntry ent;
      ent.key = key;
      ent.block = b;
      ent.last_use = pc_clock_;
      ent.depth = i;
      pc_index_.emplace(std::move(key), e);
      pc_.emplace(e, std::move(ent));
      if (parent >= 0) pc_[parent].children += 1;
      ref_[b] += 1;
      *added += 1;
    } else {
      e = f->second;
      pc_[e].last_use = pc_clock_;
    }
    parent = e;
  }
  return Status::Ok;
}

Status BlockPool::prefix_match(const int32_t* tokens, int32_t n_tokens, uint64_t ns, int64_t* id,
                               int32_t* matched) {
  *matched = 0;
  if (n_tokens < 0 || (n_tokens > 0 && !tokens)) {
    err_ = "prefix_match: bad token array";
    return Status::Invalid;
  }
  pc_clock_ += 1;
  Sequence seq;
  int64_t parent = -1;
  std::vector<int64_t> chain;
  for (int32_t i = 0; i < n_tokens / block_; ++i) {
    PrefixKey key{ns, parent, std::vector<int32_t>(tokens + static_cast<size_t>(i) * block_,
                                                   tokens + static_cast<size_t>(i + 1) * block_)};
    auto f = pc_index_.find(key);
    if (f == pc_index_.end()) break;
    chain.push_back(f->second);
    parent = f->second;
  }
  for (int64_t e : chain) {
    PrefixEntry& ent = pc_[e];
    ent.last_use = pc_clock_;
    ref_[ent.block] += 1;
    seq.table.push_back(ent.block);
  }
  seq.len = static_cast<int32_t>(chain.size()) * block_;
  const int64_t sid = next_id_++;
  *matched = seq.len;
  seqs_.emplace(sid, std::move(seq));
  *id = sid;
  return Status::Ok;
}

void BlockPool::drop_entry(int64_t e) {
  auto it = pc_.find(e);
  const PrefixEntry& ent = it->second;
  if (ent.key.parent >= 0) pc_[ent.key.parent].children -= 1;
  if (--ref_[ent.block] == 0) free_.push_back(ent.block);
  pc_index_.erase(ent.key);
  pc_.erase(it);
}

Status BlockPool::prefix_evict(int32_t k, int32_t* freed) {
  *freed = 0;
  if (k < 0) {
    err_ = "prefix_evict: negative count";
    return Status::Invalid;
  }
  while (*freed < k) {
    // least recently used leaf held only by the cache; deeper first, then lower index
    int64_t best = -1;
    for (const auto& kv : pc_) {
      const PrefixEntry& ent = kv.second;
      if (ent.children != 0 || ref_[ent.block] != 1) continue;
      if (best < 0) {
        best = kv.first;
        continue;
      }
      const PrefixEntry& b = pc_[best];
      if (ent.last_use < b.last_use || (ent.last_use == b.last_use && ent.depth > b.depth)) best = kv.first;
    }
    if (best < 0) break;
    drop_entry(best);
    *freed += 1;
  }
  return Status::Ok;
}

Status BlockPool::prefix_clear(int32_t* dropped) {
  *dropped = 0;
  std::vector<std::pair<int32_t, int64_t>> order;       // (-depth, entry): children first
  order.reserve(pc_.size());
  for (const auto& kv : pc_) order.emplace_back(-kv.second.depth, kv.first);
  std::sort(order.begin(), order.end());
  for (const auto& o : order) {
    drop_entry(o.second);
    *dropped += 1;
  }
  return Status::Ok;
}

const Sequence* BlockPool::find(int64_t id) const {
  auto it = seqs_.find(id);
  return it == seqs_.end() ? nullptr : &it->second;
}

}  // namespace pkv
