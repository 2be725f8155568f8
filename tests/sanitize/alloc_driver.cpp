// Drives the library's host allocator (block_pool.cpp, no device code) from a
// line script on stdin, so that a test can run it built with AddressSanitizer
// and UndefinedBehaviorSanitizer and compare every step with the oracle.
//
// Input, one operation per line:
//   init N B P [perm_0 .. perm_{N-1}]      (P = 1 if a permutation follows)
//   create | fork PARENT | free ID | extend ID K | append N ID...
//   release ID POS | register ID NS N TOK... | match NS N TOK...
//   evict K | clear
// Output, one JSON object per operation (not for init): its status, its
// result, and the allocator's whole state (free stack, reference counts,
// sequences by id, next id, prefix-cache entries by index).
#include <cstdint>
#include <iostream>
#include <memory>
#include <sstream>
#include <string>
#include <vector>
#include <algorithm>

#include "block_pool.hpp"

using pkv::BlockPool;
using pkv::Status;

namespace {

template <typename T>
std::string list(const T* v, size_t n) {
  std::string s = "[";
  for (size_t i = 0; i < n; ++i) s += (i ? "," : "") + std::to_string(v[i]);
  return s + "]";
}

std::string pairs(const int32_t* cow, int32_t n) {
  std::string s = "[";
  for (int32_t i = 0; i < n; ++i) s += (i ? ",[" : "[") + std::to_string(cow[2 * i]) + "," + std::to_string(cow[2 * i + 1]) + "]";
  return s + "]";
}

std::string state(const BlockPool& p) {
  std::string s = "\"free\":" + list(p.free_stack().data(), p.free_stack().size());
  s += ",\"ref\":" + list(p.refcounts().data(), p.refcounts().size());
  std::vector<int64_t> ids;
  for (const auto& kv : p.sequences()) ids.push_back(kv.first);
  std::sort(ids.begin(), ids.end());
  s += ",\"seqs\":[";
  for (size_t i = 0; i < ids.size(); ++i) {
    const pkv::Sequence* q = p.find(ids[i]);
    s += (i ? ",[" : "[") + std::to_string(ids[i]) + "," + std::to_string(q->len) + "," +
         list(q->table.data(), q->table.size()) + "]";
  }
  s += "],\"next\":" + std::to_string(p.next_id()) + ",\"pc\":[";
  bool first = true;
  for (const auto& kv : p.prefix_entries()) {
    const pkv::PrefixEntry& e = kv.second;
    s += (first ? "[" : ",[") + std::to_string(kv.first) + "," + std::to_string(e.key.ns) + "," +
         std::to_string(e.key.parent) + "," + list(e.key.tokens.data(), e.key.tokens.size()) + "," +
         std::to_string(e.block) + "," + std::to_string(e.last_use) + "]";
    first = false;
  }
  return s + "]";
}

}  // namespace

int main() {
  std::unique_ptr<BlockPool> pool;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string op;
    if (!(in >> op)) continue;
    if (op == "init") {
      int32_t n = 0, b = 0, has = 0;
      in >> n >> b >> has;
      std::vector<int32_t> perm(has ? n : 0);
      for (auto& x : perm) in >> x;
      pool = std::make_unique<BlockPool>(n, b, has ? perm.data() : nullptr);
      continue;
    }
    if (!pool) return 2;
    Status st = Status::Invalid;
    std::string res = "null";
    if (op == "create") {
      int64_t id = -1;
      st = pool->create(&id);
      res = std::to_string(id);
    } else if (op == "fork") {
      int64_t parent = 0, child = -1;
      in >> parent;
      st = pool->fork(parent, &child);
      res = std::to_string(child);
    } else if (op == "free") {
      int64_t id = 0;
      in >> id;
      st = pool->release(id);
    } else if (op == "extend") {
      int64_t id = 0;
      int32_t k = 0, n_cow = 0;
      in >> id >> k;
      std::vector<int32_t> slots(std::max(k, 0)), cow(2);
      st = pool->extend(id, k, slots.data(), cow.data(), &n_cow);
      res = "[" + list(slots.data(), slots.size()) + "," + pairs(cow.data(), n_cow) + "]";
    } else if (op == "append") {
      int32_t n = 0, n_cow = 0;
      in >> n;
      std::vector<int64_t> ids(n);
      for (auto& x : ids) in >> x;
      std::vector<int32_t> slots(n), cow(2 * n);
      st = pool->append(ids.data(), n, slots.data(), cow.data(), &n_cow);
      res = "[" + list(slots.data(), slots.size()) + "," + pairs(cow.data(), n_cow) + "]";
    } else if (op == "release") {
      int64_t id = 0;
      int32_t pos = 0, released = 0;
      in >> id >> pos;
      st = pool->release_before(id, pos, &released);
      res = std::to_string(released);
    } else if (op == "register" || op == "match") {
      int64_t id = 0;
      uint64_t ns = 0;
      int32_t n = 0;
      if (op == "register") in >> id;
      in >> ns >> n;
      std::vector<int32_t> toks(n);
      for (auto& x : toks) in >> x;
      if (op == "register") {
        int32_t added = 0;
        st = pool->prefix_register(id, toks.data(), n, ns, &added);
        res = std::to_string(added);
      } else {
        int64_t sid = -1;
        int32_t matched = 0;
        st = pool->prefix_match(toks.data(), n, ns, &sid, &matched);
        res = "[" + std::to_string(sid) + "," + std::to_string(matched) + "]";
      }
    } else if (op == "evict") {
      int32_t k = 0, freed = 0;
      in >> k;
      st = pool->prefix_evict(k, &freed);
      res = std::to_string(freed);
    } else if (op == "clear") {
      int32_t dropped = 0;
      st = pool->prefix_clear(&dropped);
      res = std::to_string(dropped);
    } else {
      return 2;
    }
    std::cout << "{\"st\":" << static_cast<int>(st) << ",\"res\":" << (st == Status::Ok ? res : "null") << ","
              << state(*pool) << "}\n";
  }
  return 0;
}
