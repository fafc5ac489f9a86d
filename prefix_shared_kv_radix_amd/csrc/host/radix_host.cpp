// Host-side slot pool, radix tree, scheduler, decode plan and the C ABI for them.
//
// Method: page "49 · RadixAttention, eviction và cache churn" — §2 (edges hold
// token runs and their K/V; token-by-token lookup; split where requests
// diverge; finished requests stay, outputs included), §4 (one pool for cache
// and running requests; reference-count pinning; unpinned leaves go first,
// least recently used first; childless parents become leaves), §5
// (longest-cached-prefix-first). The readings taken where the pages are
// silent (FIFO free list, one clock tick per match/insert, whole-node
// eviction with ties broken by token path, all-or-nothing allocation) are
// the same ones the oracle takes.
//
// Unlike the oracle, the tree keeps its eviction candidates (unpinned leaves)
// in an ordered set updated incrementally and tracks the evictable token
// count, so allocation under pressure costs O(log nodes) per evicted node.
#include "radix_host.hpp"

#include <algorithm>
#include <atomic>
#include <cstring>
#include <new>

namespace radix {

static thread_local std::string g_last_error;
void set_error(const std::string &msg) { g_last_error = msg; }

// ------------------------------------------------------------------ SlotPool
SlotPool::SlotPool(int64_t n) : n_(n), ring_(n > 0 ? n : 1), count_(n), state_(n, 1) {
  for (int64_t i = 0; i < n; ++i) ring_[i] = static_cast<int32_t>(i);
}

bool SlotPool::alloc(int64_t k, int32_t *out) {
  if (k < 0 || k > count_) return false;
  for (int64_t i = 0; i < k; ++i) {
    int32_t s = ring_[head_];
    head_ = (head_ + 1) % n_;
    state_[s] = 0;
    out[i] = s;
  }
  count_ -= k;
  return true;
}

radix_status SlotPool::release(const int32_t *s, int64_t k) {
  if (k < 0) {
    set_error("negative slot count");
    return RADIX_E_INVAL;
  }
  int64_t i = 0;
  for (; i < k; ++i) {
    int32_t x = s[i];
    if (x < 0 || x >= n_ || state_[x] != 0) break;
    state_[x] = 2;
  }
  if (i < k) {
    int32_t bad = s[i];
    for (int64_t j = 0; j < i; ++j) state_[s[j]] = 0;
    set_error("bad free of slot " + std::to_string(bad));
    return RADIX_E_INVAL;
  }
  for (i = 0; i < k; ++i) {
    state_[s[i]] = 1;
    ring_[(head_ + count_) % n_] = s[i];
    ++count_;
  }
  return RADIX_OK;
}

void SlotPool::snapshot(int32_t *out) const {
  for (int64_t i = 0; i < count_; ++i) out[i] = ring_[(head_ + i) % n_];
}

// ------------------------------------------------------------------ RadixTree
void RadixTree::path_of(int32_t i, std::vector<int32_t> &out) const {
  std::vector<int32_t> chain;
  for (int32_t x = i; x > 0; x = nodes_[x].parent) chain.push_back(x);
  out.clear();
  for (auto it = chain.rbegin(); it != chain.rend(); ++it) {
    const auto &k = nodes_[*it].key;
    out.insert(out.end(), k.begin(), k.end());
  }
}

bool LruLess::operator()(int32_t a, int32_t b) const {
  const Node &x = tree->nodes_[a], &y = tree->nodes_[b];
  if (x.tick != y.tick) return x.tick < y.tick;
  if (a == b) return false;
  std::vector<int32_t> pa, pb;
  tree->path_of(a, pa);
  tree->path_of(b, pb);
  if (pa != pb) return std::lexicographical_compare(pa.begin(), pa.end(), pb.begin(), pb.end());
  return a < b;
}

RadixTree::RadixTree(SlotPool *pool) : pool_(pool), candidates_(LruLess{this}) {
  nodes_.emplace_back();
  nodes_[0].alive = true;
}

RadixTree::~RadixTree() {
  for (size_t i = 1; i < nodes_.size(); ++i)
    if (nodes_[i].alive && !nodes_[i].value.empty())
      pool_->release(nodes_[i].value.data(), static_cast<int64_t>(nodes_[i].value.size()));
}

bool RadixTree::valid(int32_t i) const {
  return i >= 0 && static_cast<size_t>(i) < nodes_.size() && nodes_[i].alive;
}

int32_t RadixTree::new_node() {
  int32_t i;
  if (!free_nodes_.empty()) {
    i = free_nodes_.back();
    free_nodes_.pop_back();
    nodes_[i] = Node();
  } else {
    i = static_cast<int32_t>(nodes_.size());
    nodes_.emplace_back();
  }
  nodes_[i].alive = true;
  ++num_nodes_;
  return i;
}

bool RadixTree::is_candidate(int32_t i) const {
  const Node &n = nodes_[i];
  return i != 0 && n.alive && n.children.empty() && n.lock == 0;
}

void RadixTree::set_tick(int32_t i, int64_t t) {
  if (nodes_[i].tick == t) return;
  bool in = is_candidate(i);
  if (in) candidates_.erase(i);
  nodes_[i].tick = t;
  if (in) candidates_.insert(i);
}

int32_t RadixTree::split(int32_t c, int64_t k) {
  int32_t u = new_node();
  Node &C = nodes_[c];
  Node &U = nodes_[u];
  U.key.assign(C.key.begin(), C.key.begin() + k);
  U.value.assign(C.value.begin(), C.value.begin() + k);
  U.parent = C.parent;
  U.lock = C.lock;
  U.tick = tick_;
  U.depth = nodes_[C.parent].depth + k;
  nodes_[C.parent].children[U.key[0]] = u;
  C.key.erase(C.key.begin(), C.key.begin() + k);
  C.value.erase(C.value.begin(), C.value.begin() + k);
  C.parent = u;
  U.children[C.key[0]] = c;
  // c's candidacy, tick and path are unchanged; the upper node has a child.
  return u;
}

int64_t RadixTree::walk(const int32_t *tok, int64_t n, int32_t *out_slots, int32_t *last) {
  int32_t node = 0;
  int64_t i = 0;
  while (i < n) {
    auto it = nodes_[node].children.find(tok[i]);
    if (it == nodes_[node].children.end()) break;
    int32_t c = it->second;
    const auto &key = nodes_[c].key;
    int64_t klen = static_cast<int64_t>(key.size());
    int64_t lim = std::min(klen, n - i);
    int64_t k = 0;
    while (k < lim && key[k] == tok[i + k]) ++k;
    if (k < klen) c = split(c, k);
    set_tick(c, tick_);
    if (out_slots)
      std::memcpy(out_slots + i, nodes_[c].value.data(), sizeof(int32_t) * static_cast<size_t>(k));
    i += k;
    node = c;
  }
  if (last) *last = node;
  return i;
}

int64_t RadixTree::peek(const int32_t *tok, int64_t n) const {
  int32_t node = 0;
  int64_t i = 0;
  while (i < n) {
    auto it = nodes_[node].children.find(tok[i]);
    if (it == nodes_[node].children.end()) break;
    int32_t c = it->second;
    const auto &key = nodes_[c].key;
    int64_t klen = static_cast<int64_t>(key.size());
    int64_t lim = std::min(klen, n - i);
    int64_t k = 0;
    while (k < lim && key[k] == tok[i + k]) ++k;
    i += k;
    if (k < klen) break;
    node = c;
  }
  return i;
}

int64_t RadixTree::match(const int32_t *tok, int64_t n, int32_t *out_slots, int32_t *last) {
  ++tick_;
  return walk(tok, n, out_slots, last);
}

int64_t RadixTree::insert(const int32_t *tok, const int32_t *slots, int64_t n) {
  ++tick_;
  int32_t node = 0;
  int64_t i = walk(tok, n, nullptr, &node);
  if (i < n) {
    bool parent_was_candidate = is_candidate(node);
    if (parent_was_candidate) candidates_.erase(node);
    int32_t leaf = new_node();
    Node &L = nodes_[leaf];
    L.key.assign(tok + i, tok + n);
    L.value.assign(slots + i, slots + n);
    L.parent = node;
    L.lock = 0;
    L.tick = tick_;
    L.depth = nodes_[node].depth + (n - i);
    nodes_[node].children[tok[i]] = leaf;
    candidates_.insert(leaf);
    evictable_ += n - i;
    cached_ += n - i;
  }
  return i;
}

radix_status RadixTree::lock(int32_t i) {
  if (!valid(i)) {
    set_error("lock of an invalid node handle");
    return RADIX_E_INVAL;
  }
  for (int32_t x = i; x > 0; x = nodes_[x].parent) {
    Node &n = nodes_[x];
    if (n.lock == 0) {
      if (is_candidate(x)) candidates_.erase(x);
      evictable_ -= static_cast<int64_t>(n.key.size());
    }
    ++n.lock;
  }
  return RADIX_OK;
}

radix_status RadixTree::unlock(int32_t i) {
  if (!valid(i)) {
    set_error("unlock of an invalid node handle");
    return RADIX_E_INVAL;
  }
  for (int32_t x = i; x > 0; x = nodes_[x].parent)
    if (nodes_[x].lock <= 0) {
      set_error("unlock of an unpinned node");
      return RADIX_E_INVAL;
    }
  for (int32_t x = i; x > 0; x = nodes_[x].parent) {
    Node &n = nodes_[x];
    --n.lock;
    if (n.lock == 0) {
      evictable_ += static_cast<int64_t>(n.key.size());
      if (is_candidate(x)) candidates_.insert(x);
    }
  }
  return RADIX_OK;
}

int64_t RadixTree::evict(int64_t need) {
  int64_t freed = 0;
  while (freed < need && !candidates_.empty()) {
    int32_t v = *candidates_.begin();
    candidates_.erase(candidates_.begin());
    Node &n = nodes_[v];
    int64_t len = static_cast<int64_t>(n.value.size());
    pool_->release(n.value.data(), len);
    freed += len;
    evicted_total_ += len;
    evictable_ -= len;
    cached_ -= len;
    int32_t p = n.parent;
    nodes_[p].children.erase(n.key[0]);
    n = Node();
    free_nodes_.push_back(v);
    --num_nodes_;
    if (is_candidate(p)) candidates_.insert(p);
  }
  return freed;
}

radix_status RadixTree::alloc(int64_t n, int32_t *out) {
  if (n < 0) {
    set_error("negative allocation");
    return RADIX_E_INVAL;
  }
  if (pool_->num_free() >= n) {
    pool_->alloc(n, out);
    return RADIX_OK;
  }
  if (pool_->num_free() + evictable_ < n) {
    set_error("pool exhausted: " + std::to_string(pool_->num_free()) + " free + " +
              std::to_string(evictable_) + " evictable < " + std::to_string(n));
    return RADIX_E_NOMEM;
  }
  evict(n - pool_->num_free());
  pool_->alloc(n, out);
  return RADIX_OK;
}

radix_tree_stats RadixTree::stats() const {
  radix_tree_stats s;
  s.cached_tokens = cached_;
  s.evictable_tokens = evictable_;
  s.num_nodes = num_nodes_;
  s.evicted_tokens_total = evicted_total_;
  s.tick = tick_;
  // a pin covers every ancestor, so an unpinned node has no pinned descendant: every
  // cached token is either on a pinned node or evictable
  s.pinned_tokens = cached_ - evictable_;
  return s;
}

}  // namespace radix

// ====================================================================== C ABI
using radix::RadixTree;
using radix::set_error;
using radix::SlotPool;

// A pool is freed when its creator has destroyed it and no tree built on it is left:
// the creator's handle and every tree each hold one reference, so a tree destroyed
// after its pool (as a garbage collector may order them) still returns its cached slots
// into live memory.
struct radix_kv_pool {
  SlotPool p;
  std::atomic<int64_t> refs{1};
  explicit radix_kv_pool(int64_t n) : p(n) {}
};
static void pool_unref(radix_kv_pool *pool) {
  if (pool->refs.fetch_sub(1, std::memory_order_acq_rel) == 1) delete pool;
}
struct radix_tree {
  radix_kv_pool *owner;
  RadixTree t;
  explicit radix_tree(radix_kv_pool *p) : owner(p), t(&p->p) {}
};

#define RADIX_REQUIRE(cond, msg)  \
  do {                            \
    if (!(cond)) {                \
      set_error(msg);             \
      return RADIX_E_INVAL;       \
    }                             \
  } while (0)

extern "C" {

const char *radix_last_error(void) { return radix::g_last_error.c_str(); }
const char *radix_version(void) { return "radix_attn 0.1 (gfx950)"; }

radix_status radix_kv_pool_create(int64_t num_slots, radix_kv_pool **out) {
  RADIX_REQUIRE(out, "null output pointer");
  RADIX_REQUIRE(num_slots >= 0 && num_slots <= INT32_MAX, "pool size out of range");
  try {
    *out = new radix_kv_pool(num_slots);
  } catch (const std::bad_alloc &) {
    set_error("host allocation failed");
    return RADIX_E_NOMEM;
  }
  return RADIX_OK;
}

void radix_kv_pool_destroy(radix_kv_pool *pool) {
  if (pool) pool_unref(pool);
}

radix_status radix_kv_pool_alloc(radix_kv_pool *pool, int64_t n, int32_t *out_slots) {
  RADIX_REQUIRE(pool && (n == 0 || out_slots) && n >= 0, "bad arguments");
  if (!pool->p.alloc(n, out_slots)) {
    set_error("pool exhausted");
    return RADIX_E_NOMEM;
  }
  return RADIX_OK;
}

radix_status radix_kv_pool_free(radix_kv_pool *pool, const int32_t *slots, int64_t n) {
  RADIX_REQUIRE(pool && (n == 0 || slots) && n >= 0, "bad arguments");
  return pool->p.release(slots, n);
}

int64_t radix_kv_pool_num_free(const radix_kv_pool *pool) { return pool ? pool->p.num_free() : -1; }
int64_t radix_kv_pool_num_slots(const radix_kv_pool *pool) { return pool ? pool->p.num_slots() : -1; }

radix_status radix_kv_pool_free_list(const radix_kv_pool *pool, int32_t *out, int64_t cap,
                                     int64_t *n) {
  RADIX_REQUIRE(pool && n, "bad arguments");
  *n = pool->p.num_free();
  RADIX_REQUIRE(cap >= *n && (*n == 0 || out), "free-list capacity too small");
  pool->p.snapshot(out);
  return RADIX_OK;
}

radix_status radix_tree_create(radix_kv_pool *pool, radix_tree **out) {
  RADIX_REQUIRE(pool && out, "bad arguments");
  try {
    *out = new radix_tree(pool);
    pool->refs.fetch_add(1, std::memory_order_relaxed);
  } catch (const std::bad_alloc &) {
    set_error("host allocation failed");
    return RADIX_E_NOMEM;
  }
  return RADIX_OK;
}

void radix_tree_destroy(radix_tree *tree) {
  if (!tree) return;
  radix_kv_pool *owner = tree->owner;
  delete tree;   // gives the cached slots back to the owner's pool
  pool_unref(owner);
}

radix_status radix_tree_peek(const radix_tree *tree, const int32_t *tok, int64_t n,
                             int64_t *matched) {
  RADIX_REQUIRE(tree && matched && n >= 0 && (n == 0 || tok), "bad arguments");
  *matched = tree->t.peek(tok, n);
  return RADIX_OK;
}

radix_status radix_tree_match(radix_tree *tree, const int32_t *tok, int64_t n, int64_t *matched,
                              int32_t *out_slots, radix_node *last) {
  RADIX_REQUIRE(tree && matched && n >= 0 && (n == 0 || tok), "bad arguments");
  int32_t node = 0;
  *matched = tree->t.match(tok, n, out_slots, &node);
  if (last) *last = node;
  return RADIX_OK;
}

radix_status radix_tree_lock(radix_tree *tree, radix_node node) {
  RADIX_REQUIRE(tree && node >= 0 && node <= INT32_MAX, "bad arguments");
  return tree->t.lock(static_cast<int32_t>(node));
}

radix_status radix_tree_unlock(radix_tree *tree, radix_node node) {
  RADIX_REQUIRE(tree && node >= 0 && node <= INT32_MAX, "bad arguments");
  return tree->t.unlock(static_cast<int32_t>(node));
}

radix_status radix_tree_alloc(radix_tree *tree, int64_t n, int32_t *out_slots) {
  RADIX_REQUIRE(tree && n >= 0 && (n == 0 || out_slots), "bad arguments");
  return tree->t.alloc(n, out_slots);
}

radix_status radix_tree_insert(radix_tree *tree, const int32_t *tok, const int32_t *slots,
                               int64_t n, int64_t *already_cached) {
  RADIX_REQUIRE(tree && n >= 0 && (n == 0 || (tok && slots)), "bad arguments");
  int64_t c = tree->t.insert(tok, slots, n);
  if (already_cached) *already_cached = c;
  return RADIX_OK;
}

radix_status radix_tree_evict(radix_tree *tree, int64_t n_tokens, int64_t *freed) {
  RADIX_REQUIRE(tree && n_tokens >= 0, "bad arguments");
  int64_t f = tree->t.evict(n_tokens);
  if (freed) *freed = f;
  return RADIX_OK;
}

radix_status radix_tree_stats_get(const radix_tree *tree, radix_tree_stats *out) {
  RADIX_REQUIRE(tree && out, "bad arguments");
  *out = tree->t.stats();
  return RADIX_OK;
}

radix_status radix_sched_order(const radix_tree *tree, const int32_t *const *tok,
                               const int64_t *len, int64_t n, int32_t policy,
                               int64_t *out_order) {
  RADIX_REQUIRE(tree && n >= 0 && (n == 0 || (tok && len && out_order)), "bad arguments");
  RADIX_REQUIRE(policy == 0 || policy == 1, "unknown scheduling policy");
  std::vector<int64_t> order(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) order[i] = i;
  if (policy == 1) {
    std::vector<int64_t> m(static_cast<size_t>(n));
    for (int64_t i = 0; i < n; ++i) {
      RADIX_REQUIRE(len[i] >= 0 && (len[i] == 0 || tok[i]), "bad request tokens");
      m[i] = tree->t.peek(tok[i], len[i]);
    }
    std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return m[a] > m[b]; });
  }
  std::copy(order.begin(), order.end(), out_order);
  return RADIX_OK;
}

radix_status radix_route(const radix_tree *const *trees, int32_t n_workers, const int64_t *loads,
                         const int32_t *tok, int64_t n, int32_t policy, int64_t balance_abs,
                         double balance_rel, int64_t *rr_counter, int32_t *out_worker,
                         int64_t *out_matched) {
  RADIX_REQUIRE(trees && n_workers > 0 && loads && out_worker && n >= 0 && (n == 0 || tok),
                "bad arguments");
  RADIX_REQUIRE(policy >= 0 && policy <= 2, "unknown routing policy");
  RADIX_REQUIRE(policy != 0 || rr_counter, "round robin needs its counter");
  for (int32_t i = 0; i < n_workers; ++i) RADIX_REQUIRE(trees[i], "missing worker tree");
  int32_t pick = 0;
  auto least_loaded = [&]() {
    int32_t best = 0;
    for (int32_t i = 1; i < n_workers; ++i)
      if (loads[i] < loads[best]) best = i;
    return best;
  };
  if (policy == 0) {
    pick = static_cast<int32_t>(*rr_counter % n_workers);
    ++*rr_counter;
  } else if (policy == 2) {
    pick = least_loaded();
  } else {
    int64_t lo = loads[0], hi = loads[0];
    for (int32_t i = 1; i < n_workers; ++i) {
      lo = std::min(lo, loads[i]);
      hi = std::max(hi, loads[i]);
    }
    if (hi - lo > balance_abs && static_cast<double>(hi) > balance_rel * static_cast<double>(lo)) {
      pick = least_loaded();
    } else {
      int64_t best_m = -1;
      for (int32_t i = 0; i < n_workers; ++i) {
        const int64_t m = trees[i]->t.peek(tok, n);
        if (m > best_m || (m == best_m && loads[i] < loads[pick])) {
          best_m = m;
          pick = i;
        }
      }
    }
  }
  *out_worker = pick;
  if (out_matched) *out_matched = trees[pick]->t.peek(tok, n);
  return RADIX_OK;
}

radix_status radix_req_admit(radix_tree *tree, const int32_t *tok, int64_t n, int32_t *out_row,
                             int64_t *prefix_len, radix_node *node) {
  RADIX_REQUIRE(tree && prefix_len && node && n >= 0 && (n == 0 || (tok && out_row)),
                "bad arguments");
  int32_t last = 0;
  int64_t m = tree->t.match(tok, n, out_row, &last);
  *prefix_len = m;
  tree->t.lock(last);
  radix_status st = tree->t.alloc(n - m, out_row + m);
  if (st != RADIX_OK) {
    tree->t.unlock(last);
    return st;
  }
  *node = last;
  return RADIX_OK;
}

radix_status radix_req_finish(radix_tree *tree, const int32_t *tok, const int32_t *row, int64_t n,
                              int64_t prefix_len, radix_node node, int64_t *already_cached) {
  RADIX_REQUIRE(tree && n >= 0 && (n == 0 || (tok && row)), "bad arguments");
  RADIX_REQUIRE(prefix_len >= 0 && prefix_len <= n, "prefix length out of range");
  RADIX_REQUIRE(node >= 0 && node <= INT32_MAX && tree->t.valid(static_cast<int32_t>(node)),
                "invalid node handle");
  int64_t c = tree->t.insert(tok, row, n);
  if (c > prefix_len) {
    radix_status st = tree->t.pool()->release(row + prefix_len, c - prefix_len);
    if (st != RADIX_OK) return st;
  }
  if (already_cached) *already_cached = c;
  return tree->t.unlock(static_cast<int32_t>(node));
}

radix_status radix_req_admit_batch(radix_tree *tree, const int32_t *tok, const int64_t *tok_off,
                                   int64_t n, int64_t max_batch, int32_t *rows,
                                   int64_t row_stride, int64_t *prefix_len, radix_node *nodes,
                                   int64_t *admitted) {
  RADIX_REQUIRE(tree && admitted && n >= 0 && max_batch >= 0 && row_stride >= 0, "bad arguments");
  RADIX_REQUIRE(n == 0 || (tok_off && tok && rows && prefix_len && nodes), "bad arguments");
  for (int64_t i = 0; i < n; ++i)
    RADIX_REQUIRE(tok_off[i + 1] >= tok_off[i] && tok_off[i + 1] - tok_off[i] <= row_stride,
                  "request longer than row_stride");
  int64_t k = 0;
  for (int64_t i = 0; i < n && k < max_batch; ++i) {
    const int64_t len = tok_off[i + 1] - tok_off[i];
    int64_t m = 0;
    radix_node node = 0;
    radix_status st = radix_req_admit(tree, tok + tok_off[i], len, rows + k * row_stride, &m, &node);
    if (st == RADIX_E_NOMEM) break;
    if (st != RADIX_OK) {
      *admitted = k;
      return st;
    }
    prefix_len[k] = m;
    nodes[k] = node;
    ++k;
  }
  *admitted = k;
  return RADIX_OK;
}

radix_status radix_req_finish_batch(radix_tree *tree, const int32_t *tok, const int64_t *tok_off,
                                    const int32_t *rows, int64_t row_stride,
                                    const int64_t *prefix_len, const radix_node *nodes, int64_t n,
                                    int64_t *already_cached) {
  RADIX_REQUIRE(tree && n >= 0, "bad arguments");
  RADIX_REQUIRE(n == 0 || (tok && tok_off && rows && prefix_len && nodes), "bad arguments");
  for (int64_t i = 0; i < n; ++i) {
    const int64_t len = tok_off[i + 1] - tok_off[i];
    RADIX_REQUIRE(len >= 0 && len <= row_stride, "request longer than row_stride");
    int64_t c = 0;
    radix_status st = radix_req_finish(tree, tok + tok_off[i], rows + i * row_stride, len,
                                       prefix_len[i], nodes[i], &c);
    if (st != RADIX_OK) return st;
    if (already_cached) already_cached[i] = c;
  }
  return RADIX_OK;
}

radix_status radix_tree_decode_plan(const radix_tree *tree, const radix_node *nodes,
                                    int32_t batch, int32_t min_members, int32_t split_keys,
                                    int32_t cap_seg, int32_t cap_mem, int32_t cap_items,
                                    int32_t *seg_row, int32_t *seg_start, int32_t *seg_end,
                                    int32_t *seg_member_off, int32_t *seg_members,
                                    int32_t *seg_member_slot, int32_t *seg_split_off,
                                    int32_t *seg_member_part, int32_t *seg_items,
                                    int32_t *req_num_shared,
                                    int32_t *req_num_parts, int32_t *req_private_start,
                                    int32_t *req_order, int32_t *num_segments,
                                    int32_t *num_member_entries, int32_t *max_members,
                                    int32_t *max_shared, int32_t *num_seg_items,
                                    int32_t *max_parts, int32_t *max_seg_splits) {
  RADIX_REQUIRE(tree && batch >= 0 && (batch == 0 || nodes) && min_members >= 2,
                "bad arguments");
  RADIX_REQUIRE(num_segments && num_member_entries && max_members && max_shared &&
                    num_seg_items && max_parts && max_seg_splits,
                "null output pointer");
  RADIX_REQUIRE(batch == 0 || (req_num_shared && req_num_parts && req_private_start && req_order),
                "null output pointer");
  // key chunks of a segment of len tokens
  auto chunks_of = [split_keys](int64_t len) -> int32_t {
    if (split_keys <= 0 || len <= split_keys) return 1;
    return static_cast<int32_t>((len + split_keys - 1) / split_keys);
  };
  const RadixTree &t = tree->t;
  // paths (root first) and the number of running requests on each node
  std::vector<std::vector<int32_t>> paths(static_cast<size_t>(batch));
  std::unordered_map<int32_t, int32_t> count;
  for (int32_t b = 0; b < batch; ++b) {
    RADIX_REQUIRE(nodes[b] >= 0 && nodes[b] <= INT32_MAX &&
                      t.valid(static_cast<int32_t>(nodes[b])),
                  "invalid node handle in plan");
    for (int32_t x = static_cast<int32_t>(nodes[b]); x > 0; x = t.node(x).parent)
      paths[b].push_back(x);
    std::reverse(paths[b].begin(), paths[b].end());
    for (int32_t x : paths[b]) ++count[x];
  }
  // a segment = a maximal chain of path nodes with the same (>= min_members) count;
  // member sets nest along a path, so equal counts mean equal member sets
  struct Member {
    int32_t b, rank, part;
  };
  struct Seg {
    int32_t row, start, end, chunks;
    std::vector<Member> members;
  };
  std::vector<Seg> segs;
  std::unordered_map<int32_t, int32_t> seg_of_head;
  int32_t total_mem = 0, maxsh = 0, maxparts = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const auto &p = paths[b];
    int32_t rank = 0, parts = 0;
    int64_t start = 0, priv = 0;
    size_t i = 0;
    while (i < p.size() && count[p[i]] >= min_members) {
      int32_t head = p[i];
      int32_t c = count[head];
      size_t j = i;
      while (j + 1 < p.size() && count[p[j + 1]] == c) ++j;
      int64_t end = t.node(p[j]).depth;
      auto it = seg_of_head.find(head);
      int32_t sid;
      if (it == seg_of_head.end()) {
        sid = static_cast<int32_t>(segs.size());
        seg_of_head[head] = sid;
        segs.push_back(Seg{b, static_cast<int32_t>(start), static_cast<int32_t>(end),
                           chunks_of(end - start), {}});
      } else {
        sid = it->second;
      }
      segs[sid].members.push_back(Member{b, rank, parts});
      parts += segs[sid].chunks;
      ++rank;
      ++total_mem;
      start = end;
      priv = end;
      i = j + 1;
    }
    req_num_shared[b] = rank;
    req_num_parts[b] = parts;
    req_private_start[b] = static_cast<int32_t>(priv);
    maxsh = std::max(maxsh, rank);
    maxparts = std::max(maxparts, parts);
  }
  // Launch order: segments whose key chunks are longest first (longest work first), so
  // their blocks start at once instead of behind many short ones; ties keep creation
  // order. Every array below follows this order.
  auto chunk_len = [](const Seg &g) {
    const int32_t len = g.end - g.start;
    return ((len + g.chunks - 1) / g.chunks + 63) / 64 * 64;
  };
  std::stable_sort(segs.begin(), segs.end(),
                   [&](const Seg &x, const Seg &y) { return chunk_len(x) > chunk_len(y); });
  // requests grouped by their root-most shared segment (in the order above), then the
  // requests without any, in batch order
  {
    int32_t k = 0;
    std::vector<uint8_t> placed(static_cast<size_t>(batch), 0);
    for (const auto &sg : segs)
      for (const auto &m : sg.members)
        if (m.rank == 0 && !placed[m.b]) {
          placed[m.b] = 1;
          req_order[k++] = m.b;
        }
    for (int32_t b = 0; b < batch; ++b)
      if (!placed[b]) req_order[k++] = b;
  }
  *num_segments = static_cast<int32_t>(segs.size());
  *num_member_entries = total_mem;
  *max_shared = maxsh;
  *max_parts = maxparts;
  int32_t maxm = 0, items = 0, maxchunks = 0;
  for (const auto &s : segs) {
    maxm = std::max(maxm, static_cast<int32_t>(s.members.size()));
    items += s.chunks;
    maxchunks = std::max(maxchunks, s.chunks);
  }
  *max_members = maxm;
  *num_seg_items = items;
  *max_seg_splits = maxchunks;
  RADIX_REQUIRE(static_cast<int32_t>(segs.size()) <= cap_seg && total_mem <= cap_mem &&
                    items <= cap_items,
                "decode plan capacity too small");
  RADIX_REQUIRE(segs.empty() || (seg_row && seg_start && seg_end && seg_member_off &&
                                 seg_members && seg_member_slot && seg_split_off &&
                                 seg_member_part && seg_items),
                "null output pointer");
  int32_t off = 0, chunk_off = 0;
  for (size_t s = 0; s < segs.size(); ++s) {
    seg_row[s] = segs[s].row;
    seg_start[s] = segs[s].start;
    seg_end[s] = segs[s].end;
    seg_member_off[s] = off;
    seg_split_off[s] = chunk_off;
    // chunk k covers [start + k*clen, min(end, start + (k+1)*clen)), clen = the
    // segment's length over its chunk count rounded up to 64 keys (one key tile);
    // trailing chunks may be empty
    const int32_t len = segs[s].end - segs[s].start, pieces = segs[s].chunks;
    const int32_t clen = ((len + pieces - 1) / pieces + 63) / 64 * 64;
    for (int32_t k = 0; k < pieces; ++k) {
      int32_t *r = seg_items + static_cast<int64_t>(chunk_off + k) * 8;
      const int64_t lo = std::min<int64_t>(segs[s].end, segs[s].start + static_cast<int64_t>(k) * clen);
      r[0] = static_cast<int32_t>(lo);
      r[1] = static_cast<int32_t>(std::min<int64_t>(segs[s].end, lo + clen));
      r[2] = off;
      r[3] = static_cast<int32_t>(segs[s].members.size());
      r[4] = segs[s].row;
      r[5] = static_cast<int32_t>(s);
      r[6] = k;
      r[7] = 0;
    }
    chunk_off += segs[s].chunks;
    for (auto &m : segs[s].members) {
      seg_members[off] = m.b;
      seg_member_slot[off] = m.rank;
      seg_member_part[off] = m.part;
      ++off;
    }
  }
  if (seg_member_off) seg_member_off[segs.size()] = off;
  if (seg_split_off) seg_split_off[segs.size()] = chunk_off;
  return RADIX_OK;
}

}  // extern "C"
