// Host prefix cache for the dual-pool KV cache (include/prefix_tree.h).
//
// A radix tree over token ids, token-granular. Each node holds one edge of
// the path (a run of positions) with, per position, the ring that still holds
// its SWA KV (or none), and, per page index the run touches, a Full page id.
// This is the node content the pages prescribe for a prefix tree under
// sliding-window layers ([YLY] "KVCache系统重构：让缓存真正省下来": a Full
// segment index plus an SWA segment map per node, evicted independently; the
// match cut to the window-safe length; SWA eviction tied to the request's
// lifecycle so SWA occupancy stays at window scale).
//
// Bookkeeping that keeps every operation proportional to what it touches:
//   - a registry per ring maps each position it holds to the node holding it,
//     so moving a ring's window (one decode step) or releasing a ring costs
//     the positions dropped, not a tree walk; node splits re-point the
//     registry entries of the positions that move;
//   - a reference count per page id: a node that starts inside a page shares
//     that page index with its parent, and right after a split the two halves
//     share the same page id.
// One source ring per position. A ring handed over to the tree (stable until
// the tree evicts it) takes a position from a live ring (whose window moves
// on); otherwise the existing source is kept.
#include <algorithm>
#include <cstdint>
#include <map>
#include <memory>
#include <queue>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "../../include/prefix_tree.h"
#include "status.hpp"

namespace {

struct Node {
  Node* parent = nullptr;
  int64_t start = 0;                  // first position of the run
  std::vector<int32_t> tokens;        // positions [start, end())
  std::vector<int32_t> pages;         // page indices [start / ps, ceil(end() / ps))
  std::vector<int32_t> swa;           // source ring per position, -1 = none
  std::unordered_map<int32_t, std::unique_ptr<Node>> children;   // keyed by first token
  int64_t last_use = 0;
  int64_t serial = 0;                 // creation order, breaks LRU ties
  int32_t lock = 0;
  int64_t end() const { return start + static_cast<int64_t>(tokens.size()); }
};

struct Ring {
  bool owned = false;                 // handed over to the tree
  int64_t last_use = 0;
  std::map<int64_t, Node*> held;      // position -> node holding it
};

}  // namespace

struct ha_prefix_tree {
  int32_t window = 0;
  int32_t ps = 0;
  Node root;
  std::unordered_map<int32_t, Ring> rings;
  std::unordered_map<int32_t, int32_t> page_refs;
  int64_t clock = 0;
  int64_t serial = 0;
  int64_t nodes = 0;
};

namespace {

using Tree = ha_prefix_tree;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Follows tokens [0, n) from the root without changing anything. Returns the
// common prefix length m; path gets the nodes holding [0, m) in order (the
// last one possibly only up to m).
int64_t walk(const Tree& t, const int32_t* tokens, int64_t n, std::vector<Node*>* path) {
  const Node* node = &t.root;
  int64_t pos = 0;
  while (pos < n) {
    auto it = node->children.find(tokens[pos]);
    if (it == node->children.end()) break;
    Node* c = it->second.get();
    const int64_t len = static_cast<int64_t>(c->tokens.size());
    int64_t k = 0;
    while (k < len && pos + k < n && c->tokens[k] == tokens[pos + k]) ++k;
    path->push_back(c);
    pos += k;
    if (k < len) break;
    node = c;
  }
  return pos;
}

// Splits c at position at (c->start < at < c->end()): a new node takes
// [c->start, at) and becomes c's parent. Returns the new node.
Node* split(Tree& t, Node* c, int64_t at) {
  const int64_t ps = t.ps;
  const int64_t k = at - c->start;
  auto p = std::make_unique<Node>();
  p->parent = c->parent;
  p->start = c->start;
  p->tokens.assign(c->tokens.begin(), c->tokens.begin() + k);
  p->swa.assign(c->swa.begin(), c->swa.begin() + k);
  const int64_t first = c->start / ps;
  const int64_t p_last = ceil_div(at, ps);        // p's page indices [first, p_last)
  const int64_t c_first = at / ps;                // c's page indices [c_first, ...)
  p->pages.assign(c->pages.begin(), c->pages.begin() + (p_last - first));
  c->pages.erase(c->pages.begin(), c->pages.begin() + (c_first - first));
  if (p_last > c_first) ++t.page_refs[p->pages.back()];   // the page index both halves touch
  c->tokens.erase(c->tokens.begin(), c->tokens.begin() + k);
  c->swa.erase(c->swa.begin(), c->swa.begin() + k);
  c->start = at;
  p->last_use = c->last_use;
  p->lock = c->lock;
  p->serial = ++t.serial;
  for (int64_t i = 0; i < k; ++i)
    if (p->swa[i] >= 0) t.rings[p->swa[i]].held[p->start + i] = p.get();
  Node* parent = c->parent;
  const int32_t key = p->tokens[0];
  std::unique_ptr<Node> owned_c = std::move(parent->children[key]);
  c->parent = p.get();
  p->children[c->tokens[0]] = std::move(owned_c);
  Node* raw = p.get();
  parent->children[key] = std::move(p);
  ++t.nodes;
  return raw;
}

// The node of path holding position pos (path covers [0, m), pos < m).
struct Cursor {
  const std::vector<Node*>& path;
  size_t i = 0;
  Node* at(int64_t pos) {
    while (pos >= path[i]->end()) ++i;
    return path[i];
  }
};

void drop_position(Node* node, int64_t pos) {
  node->swa[pos - node->start] = -1;
}

// Keeps only positions >= new_len - W of ring r.
void advance(Tree& t, Ring& r, int64_t new_len) {
  const int64_t lo = new_len - t.window;
  auto it = r.held.begin();
  while (it != r.held.end() && it->first < lo) {
    drop_position(it->second, it->first);
    it = r.held.erase(it);
  }
}

ha_status check_tokens(const int32_t* tokens, int64_t n) {
  if (n < 0) return ha::set_error(HA_ERR_RANGE, "token count %lld is negative", static_cast<long long>(n));
  if (n > 0 && !tokens) return ha::set_error(HA_ERR_NULL, "tokens is NULL");
  return HA_OK;
}

}  // namespace

extern "C" {

ha_status ha_tree_create(int32_t window, int32_t page_size, ha_prefix_tree** out_tree) {
  if (!out_tree) return ha::set_error(HA_ERR_NULL, "out_tree is NULL");
  if (window < 1 || page_size < 1)
    return ha::set_error(HA_ERR_RANGE, "window (%d) and page_size (%d) must be >= 1", window, page_size);
  auto* t = new ha_prefix_tree();
  t->window = window;
  t->ps = page_size;
  *out_tree = t;
  return ha::clear_error();
}

void ha_tree_destroy(ha_prefix_tree* tree) { delete tree; }

ha_status ha_tree_insert(ha_prefix_tree* tree, const int32_t* tokens, int64_t n, const int32_t* pages,
                         int32_t ring_id, int64_t ring_len, int32_t transfer_ring, uint8_t* page_kept,
                         int32_t* ring_kept) {
  if (!tree) return ha::set_error(HA_ERR_NULL, "tree is NULL");
  if (ha_status st = check_tokens(tokens, n); st != HA_OK) return st;
  if (n > 0 && !pages) return ha::set_error(HA_ERR_NULL, "pages is NULL");
  if (ring_id < -1 || ring_len < 0)
    return ha::set_error(HA_ERR_RANGE, "ring id %d / ring length %lld out of range", ring_id,
                         static_cast<long long>(ring_len));
  Tree& t = *tree;
  const int64_t ps = t.ps;
  const int64_t np = ceil_div(n, ps);
  for (int64_t i = 0; i < np; ++i)
    if (pages[i] < 0) return ha::set_error(HA_ERR_RANGE, "page id %d at index %lld is negative", pages[i],
                                           static_cast<long long>(i));
  if (ring_id >= 0) {
    auto it = t.rings.find(ring_id);
    if (it != t.rings.end() && it->second.owned)
      return ha::set_error(HA_ERR_RANGE, "ring %d already belongs to the tree", ring_id);
  }
  std::vector<Node*> path;
  const int64_t m = walk(t, tokens, n, &path);
  // the caller's pages for the new positions [m, n) must be new to the tree
  for (int64_t i = m / ps; i < np && m < n; ++i)
    if (t.page_refs.count(pages[i]))
      return ha::set_error(HA_ERR_RANGE,
                           "page %d (index %lld) already holds cached positions; a page that holds new "
                           "positions must be the request's own (copy a borrowed page before writing)",
                           pages[i], static_cast<long long>(i));

  const int64_t now = ++t.clock;
  Node* tail = &t.root;
  if (!path.empty()) {
    if (m < path.back()->end()) path.back() = split(t, path.back(), m);
    tail = path.back();
  }
  for (Node* x : path) x->last_use = now;
  if (m < n) {
    auto leaf = std::make_unique<Node>();
    leaf->parent = tail;
    leaf->start = m;
    leaf->tokens.assign(tokens + m, tokens + n);
    leaf->swa.assign(n - m, -1);
    leaf->pages.assign(pages + m / ps, pages + np);
    for (int32_t pg : leaf->pages) ++t.page_refs[pg];
    leaf->last_use = now;
    leaf->serial = ++t.serial;
    path.push_back(leaf.get());
    tail->children[tokens[m]] = std::move(leaf);
    ++t.nodes;
  }
  bool kept = false;
  if (ring_id >= 0) {
    Ring& r = t.rings[ring_id];
    r.owned = transfer_ring != 0;
    r.last_use = now;
    advance(t, r, ring_len);
    Cursor cur{path};
    for (int64_t p = std::max<int64_t>(0, ring_len - t.window); p < std::min(ring_len, n); ++p) {
      Node* x = cur.at(p);
      int32_t& src = x->swa[p - x->start];
      if (src == ring_id) continue;
      if (src >= 0) {
        Ring& old = t.rings[src];
        if (old.owned || !r.owned) continue;        // keep the existing source
        old.held.erase(p);
      }
      src = ring_id;
      r.held[p] = x;
    }
    kept = !r.held.empty();
    if (!kept) t.rings.erase(ring_id);
  }
  if (page_kept)
    for (int64_t i = 0; i < np; ++i) page_kept[i] = t.page_refs.count(pages[i]) ? 1 : 0;
  if (ring_kept) *ring_kept = kept ? 1 : 0;
  return ha::clear_error();
}

ha_status ha_tree_match(ha_prefix_tree* tree, const int32_t* tokens, int64_t n, int64_t* out_matched,
                        uint8_t* swa_valid, int32_t* swa_ring, int32_t* pages) {
  if (!tree || !out_matched) return ha::set_error(HA_ERR_NULL, "tree or out_matched is NULL");
  if (ha_status st = check_tokens(tokens, n); st != HA_OK) return st;
  if (n > 0 && !swa_valid) return ha::set_error(HA_ERR_NULL, "swa_valid is NULL");
  Tree& t = *tree;
  const int64_t ps = t.ps;
  std::vector<Node*> path;
  const int64_t m = walk(t, tokens, n, &path);
  const int64_t now = ++t.clock;
  for (Node* x : path) x->last_use = now;
  Cursor cur{path};
  for (int64_t p = 0; p < n; ++p) {
    int32_t src = -1;
    if (p < m) {
      Node* x = cur.at(p);
      src = x->swa[p - x->start];
      if (src >= 0) t.rings[src].last_use = now;
    }
    swa_valid[p] = src >= 0 ? 1 : 0;
    if (swa_ring) swa_ring[p] = src;
  }
  if (pages) {
    Cursor pc{path};
    const int64_t np = ceil_div(n, ps);
    for (int64_t i = 0; i < np; ++i) {
      if (i * ps >= m) {
        pages[i] = -1;
        continue;
      }
      const int64_t last = std::min(m, (i + 1) * ps) - 1;
      Node* x = pc.at(last);
      pages[i] = x->pages[i - x->start / ps];
    }
  }
  *out_matched = m;
  return ha::clear_error();
}

ha_status ha_tree_lock(ha_prefix_tree* tree, const int32_t* tokens, int64_t n, int32_t delta) {
  if (!tree) return ha::set_error(HA_ERR_NULL, "tree is NULL");
  if (ha_status st = check_tokens(tokens, n); st != HA_OK) return st;
  if (delta != 1 && delta != -1) return ha::set_error(HA_ERR_RANGE, "delta must be +1 or -1 (got %d)", delta);
  Tree& t = *tree;
  std::vector<Node*> path;
  const int64_t m = walk(t, tokens, n, &path);
  if (m < n)
    return ha::set_error(HA_ERR_RANGE, "only %lld of %lld positions are cached", static_cast<long long>(m),
                         static_cast<long long>(n));
  if (!path.empty() && n < path.back()->end()) {
    if (delta < 0) return ha::set_error(HA_ERR_RANGE, "no lock ends at position %lld", static_cast<long long>(n));
    path.back() = split(t, path.back(), n);
  }
  if (delta < 0)
    for (Node* x : path)
      if (x->lock <= 0) return ha::set_error(HA_ERR_RANGE, "unlock of a node that is not locked");
  for (Node* x : path) x->lock += delta;
  return ha::clear_error();
}

ha_status ha_tree_ring_advance(ha_prefix_tree* tree, int32_t ring_id, int64_t new_len) {
  if (!tree) return ha::set_error(HA_ERR_NULL, "tree is NULL");
  if (new_len < 0) return ha::set_error(HA_ERR_RANGE, "ring length is negative");
  auto it = tree->rings.find(ring_id);
  if (it == tree->rings.end()) return ha::clear_error();
  if (it->second.owned) return ha::set_error(HA_ERR_RANGE, "ring %d belongs to the tree", ring_id);
  advance(*tree, it->second, new_len);
  if (it->second.held.empty()) tree->rings.erase(it);
  return ha::clear_error();
}

ha_status ha_tree_ring_release(ha_prefix_tree* tree, int32_t ring_id) {
  if (!tree) return ha::set_error(HA_ERR_NULL, "tree is NULL");
  auto it = tree->rings.find(ring_id);
  if (it == tree->rings.end()) return ha::clear_error();
  if (it->second.owned) return ha::set_error(HA_ERR_RANGE, "ring %d belongs to the tree", ring_id);
  for (auto& [pos, node] : it->second.held) drop_position(node, pos);
  tree->rings.erase(it);
  return ha::clear_error();
}

ha_status ha_tree_evict_full(ha_prefix_tree* tree, int64_t want_pages, int32_t* freed_pages, int64_t page_cap,
                             int64_t* out_pages, int32_t* freed_rings, int64_t ring_cap, int64_t* out_rings) {
  if (!tree || !out_pages || !out_rings) return ha::set_error(HA_ERR_NULL, "tree or an output count is NULL");
  if (want_pages < 0 || page_cap < 0 || ring_cap < 0) return ha::set_error(HA_ERR_RANGE, "negative size");
  if ((page_cap > 0 && !freed_pages) || (ring_cap > 0 && !freed_rings))
    return ha::set_error(HA_ERR_NULL, "output array is NULL");
  Tree& t = *tree;
  using Key = std::tuple<int64_t, int64_t, Node*>;
  std::priority_queue<Key, std::vector<Key>, std::greater<Key>> heap;
  auto evictable = [](const Node* x) { return x->children.empty() && x->lock == 0; };
  std::vector<Node*> stack;
  for (auto& kv : t.root.children) stack.push_back(kv.second.get());
  while (!stack.empty()) {
    Node* x = stack.back();
    stack.pop_back();
    if (evictable(x)) heap.emplace(x->last_use, x->serial, x);
    for (auto& kv : x->children) stack.push_back(kv.second.get());
  }
  int64_t np = 0, nr = 0;
  while (np < want_pages && !heap.empty()) {
    Node* x = std::get<2>(heap.top());
    heap.pop();
    // what evicting x frees
    int64_t pages_freed = 0;
    for (int32_t pg : x->pages) pages_freed += t.page_refs[pg] == 1;
    std::unordered_map<int32_t, int64_t> lost;
    for (int32_t src : x->swa)
      if (src >= 0) ++lost[src];
    int64_t rings_freed = 0;
    for (auto& [rid, cnt] : lost) {
      const Ring& r = t.rings[rid];
      rings_freed += r.owned && static_cast<int64_t>(r.held.size()) == cnt;
    }
    if (np + pages_freed > page_cap || nr + rings_freed > ring_cap) break;
    for (int32_t pg : x->pages) {
      auto it = t.page_refs.find(pg);
      if (--it->second == 0) {
        freed_pages[np++] = pg;
        t.page_refs.erase(it);
      }
    }
    for (int64_t i = 0; i < static_cast<int64_t>(x->swa.size()); ++i) {
      const int32_t src = x->swa[i];
      if (src < 0) continue;
      auto rit = t.rings.find(src);
      rit->second.held.erase(x->start + i);
      if (rit->second.held.empty()) {
        if (rit->second.owned) freed_rings[nr++] = src;
        t.rings.erase(rit);
      }
    }
    Node* parent = x->parent;
    parent->children.erase(x->tokens[0]);   // destroys x
    --t.nodes;
    if (parent != &t.root && evictable(parent)) heap.emplace(parent->last_use, parent->serial, parent);
  }
  *out_pages = np;
  *out_rings = nr;
  return ha::clear_error();
}

ha_status ha_tree_evict_swa(ha_prefix_tree* tree, int64_t want_rings, int32_t* freed_rings, int64_t ring_cap,
                            int64_t* out_rings) {
  if (!tree || !out_rings) return ha::set_error(HA_ERR_NULL, "tree or out_rings is NULL");
  if (want_rings < 0 || ring_cap < 0) return ha::set_error(HA_ERR_RANGE, "negative size");
  if (ring_cap > 0 && !freed_rings) return ha::set_error(HA_ERR_NULL, "freed_rings is NULL");
  Tree& t = *tree;
  std::vector<std::pair<int64_t, int32_t>> order;
  for (auto& [rid, r] : t.rings)
    if (r.owned) order.emplace_back(r.last_use, rid);
  std::sort(order.begin(), order.end());
  int64_t nr = 0;
  for (auto& [use, rid] : order) {
    if (nr >= want_rings || nr >= ring_cap) break;
    auto it = t.rings.find(rid);
    for (auto& [pos, node] : it->second.held) drop_position(node, pos);
    t.rings.erase(it);
    freed_rings[nr++] = rid;
  }
  *out_rings = nr;
  return ha::clear_error();
}

ha_status ha_tree_stats(const ha_prefix_tree* tree, int64_t out[6]) {
  if (!tree || !out) return ha::set_error(HA_ERR_NULL, "tree or out is NULL");
  int64_t positions = 0, owned = 0, live = 0, most = 0;
  for (auto& [rid, r] : tree->rings) {
    const int64_t h = static_cast<int64_t>(r.held.size());
    positions += h;
    owned += r.owned;
    live += !r.owned && h > 0;
    most = std::max(most, h);
  }
  out[0] = tree->nodes;
  out[1] = static_cast<int64_t>(tree->page_refs.size());
  out[2] = positions;
  out[3] = owned;
  out[4] = live;
  out[5] = most;
  return ha::clear_error();
}

}  // extern "C"
