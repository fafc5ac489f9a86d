// Host-side slot pool and radix tree (C++17). See include/radix_attn.h for the
// contract; this header is internal to the library.
#pragma once

#include <cstdint>
#include <set>
#include <string>
#include <unordered_map>
#include <vector>

#include "radix_attn.h"

namespace radix {

void set_error(const std::string &msg);

// FIFO free list over slots 0..n-1 (page 4 §4: one pool for cache and running
// requests). Allocation takes from the head, release appends at the tail.
class SlotPool {
 public:
  explicit SlotPool(int64_t n);
  int64_t num_slots() const { return n_; }
  int64_t num_free() const { return count_; }
  bool alloc(int64_t k, int32_t *out);                 // false if fewer than k free
  radix_status release(const int32_t *s, int64_t k);  // validates all first
  void snapshot(int32_t *out) const;

 private:
  int64_t n_;
  std::vector<int32_t> ring_;
  int64_t head_ = 0, count_ = 0;
  std::vector<uint8_t> state_;  // 0 = in use, 1 = free, 2 = pending in a release
};

struct Node {
  std::vector<int32_t> key;    // tokens on the edge into this node
  std::vector<int32_t> value;  // their slots
  std::unordered_map<int32_t, int32_t> children;  // first token -> node index
  int32_t parent = -1;
  int64_t lock = 0;
  int64_t tick = 0;
  int64_t depth = 0;  // tokens from the root to the end of this node
  bool alive = false;
};

class RadixTree;

// Orders eviction candidates: smaller tick first, then the lexicographically
// smaller root-to-node token path, then the node index.
struct LruLess {
  const RadixTree *tree;
  bool operator()(int32_t a, int32_t b) const;
};

class RadixTree {
 public:
  explicit RadixTree(SlotPool *pool);
  ~RadixTree();

  int64_t peek(const int32_t *tok, int64_t n) const;
  int64_t match(const int32_t *tok, int64_t n, int32_t *out_slots, int32_t *last);
  int64_t insert(const int32_t *tok, const int32_t *slots, int64_t n);
  radix_status lock(int32_t node);
  radix_status unlock(int32_t node);
  radix_status alloc(int64_t n, int32_t *out);
  int64_t evict(int64_t need);
  radix_tree_stats stats() const;
  bool valid(int32_t node) const;
  const Node &node(int32_t i) const { return nodes_[i]; }
  SlotPool *pool() { return pool_; }
  void path_of(int32_t node, std::vector<int32_t> &out) const;

 private:
  friend struct LruLess;
  int32_t new_node();
  int64_t walk(const int32_t *tok, int64_t n, int32_t *out_slots, int32_t *last);
  int32_t split(int32_t c, int64_t k);
  bool is_candidate(int32_t i) const;
  void set_tick(int32_t i, int64_t t);
  void fix_depths(int32_t i);

  SlotPool *pool_;
  std::vector<Node> nodes_;
  std::vector<int32_t> free_nodes_;
  std::set<int32_t, LruLess> candidates_;
  int64_t tick_ = 0;
  int64_t evictable_ = 0;
  int64_t cached_ = 0;
  int64_t num_nodes_ = 0;
  int64_t evicted_total_ = 0;
};

}  // namespace radix
