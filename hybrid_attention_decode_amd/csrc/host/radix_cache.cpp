// Hybrid prefix cache: radix tree over token ids with KV pages on every node
// and GDN state slots (checkpoints) on the nodes where a state was saved.
//
// Hybrid prefix caching (24-ai.news TokenSpeed article, optimisation list;
// zubnet.ai TokenSpeed article, second paragraph): the host-side logical
// cache keeps KV pages and saved recurrent states of past requests, and
// shares both without ever writing them (a writer copies a shared page
// first; a state slot is read by index and never overwritten).  A hybrid
// model can resume a request only where both the KV and the recurrent state
// of the prefix exist, so a match ends at the deepest node of the query's
// path that holds a slot.
//
// Node layout: a node covers the token depths [start, end) of its edge and
// holds the physical pages of the page indices [start / P, ceil(end / P)).
// A page straddling the boundary between a node and its child is held by
// both; the child's copy holds the parent's rows too (a sequence writes all
// of its tokens), and a match takes each page from the deepest node on its
// path that covers it.  The cache owns one page reference per (node, page)
// and one slot reference per checkpoint, through the public page-table and
// slot-pool calls.
#include <algorithm>
#include <cstdint>
#include <map>
#include <new>
#include <vector>

#include "had.h"
#include "status.h"

using had::fail;

struct had_radix {
  had_kvpt* kv = nullptr;
  had_slots* slots = nullptr;
  int32_t P = 0;
  struct Node {
    bool live = false;
    int32_t parent = -1;
    int32_t start = 0, end = 0;       // token depths of the edge
    std::vector<int32_t> toks;        // edge tokens
    std::vector<int32_t> pages;       // pages of indices [start / P, ceil(end / P))
    int32_t slot = -1;                // state after token end - 1, or -1
    int32_t lock = 0;                 // matches in use through this node
    uint64_t tick = 0;                // last use (LRU)
    std::map<int32_t, int32_t> kids;  // first edge token -> child
  };
  std::vector<Node> nodes;  // nodes[0] is the root (depth 0, no pages)
  std::vector<int32_t> free_ids;
  uint64_t clock = 0;
  int64_t queried = 0, matched = 0;

  int32_t first_page(int32_t depth) const { return depth / P; }
  int32_t end_page(int32_t depth) const { return (depth + P - 1) / P; }

  int32_t new_node() {
    int32_t id;
    if (!free_ids.empty()) {
      id = free_ids.back();
      free_ids.pop_back();
      nodes[id] = Node();
    } else {
      id = static_cast<int32_t>(nodes.size());
      nodes.emplace_back();
    }
    nodes[id].live = true;
    return id;
  }

  // Walk the query from the root along whole edges; stops before an edge
  // that the query leaves or ends inside.  path: the nodes passed.
  void walk(const int32_t* tokens, int32_t n, std::vector<int32_t>& path, int32_t& depth) const {
    int32_t cur = 0;
    depth = 0;
    while (depth < n) {
      auto it = nodes[cur].kids.find(tokens[depth]);
      if (it == nodes[cur].kids.end()) break;
      const Node& c = nodes[it->second];
      const int32_t len = c.end - c.start;
      if (depth + len > n || !std::equal(c.toks.begin(), c.toks.end(), tokens + depth)) break;
      depth += len;
      cur = it->second;
      path.push_back(cur);
    }
  }

  void release_node(Node& x) {
    for (int32_t p : x.pages) had_kvpt_page_release(kv, p);
    x.pages.clear();
    if (x.slot >= 0) had_slots_release(slots, x.slot);
    x.slot = -1;
  }
};

namespace {

int check_tokens(const int32_t* tokens, int32_t n, const char* who) {
  if (n < 0 || (n > 0 && !tokens)) return fail(HAD_ERR_INVALID_ARG, "%s: bad token array (n=%d)", who, n);
  return HAD_OK;
}

}  // namespace

extern "C" {

int had_radix_create(had_kvpt* kv, had_slots* slots, had_radix** out) {
  if (!kv || !slots || !out) return fail(HAD_ERR_INVALID_ARG, "radix_create: NULL argument");
  int32_t np = 0, ps = 0;
  int st = had_kvpt_info(kv, &np, &ps);
  if (st != HAD_OK) return st;
  had_radix* r = new (std::nothrow) had_radix;
  if (!r) return fail(HAD_ERR_INVALID_ARG, "radix_create: out of host memory");
  r->kv = kv;
  r->slots = slots;
  r->P = ps;
  r->nodes.resize(1);
  r->nodes[0].live = true;
  *out = r;
  return had::ok();
}

int had_radix_destroy(had_radix* r) {
  if (!r) return had::ok();
  for (auto& x : r->nodes)
    if (x.live) r->release_node(x);
  delete r;
  return had::ok();
}

int had_radix_match(had_radix* r, const int32_t* tokens, int32_t n, int32_t* matched, int32_t* slot,
                    int32_t* pages, int32_t max_pages, int32_t* lock) {
  if (!r || !matched || !slot || !lock || max_pages < 0 || (max_pages > 0 && !pages))
    return fail(HAD_ERR_INVALID_ARG, "radix_match: NULL or bad argument");
  int st = check_tokens(tokens, n, "radix_match");
  if (st != HAD_OK) return st;
  std::vector<int32_t> path;
  int32_t depth = 0;
  r->walk(tokens, n, path, depth);
  // deepest node of the path that holds a checkpoint
  int32_t best = -1;
  for (int32_t i = static_cast<int32_t>(path.size()) - 1; i >= 0; --i)
    if (r->nodes[path[i]].slot >= 0) {
      best = i;
      break;
    }
  const int32_t len = best >= 0 ? r->nodes[path[best]].end : 0;
  const int32_t need = r->end_page(len);
  if (need > max_pages) return fail(HAD_ERR_CAPACITY, "radix_match: %d pages do not fit max_pages %d", need, max_pages);
  for (int32_t i = 0; i < need; ++i) pages[i] = -1;
  for (int32_t i = best; i >= 0; --i) {  // deepest node first
    const had_radix::Node& x = r->nodes[path[i]];
    const int32_t p0 = r->first_page(x.start);
    for (int32_t k = 0; k < static_cast<int32_t>(x.pages.size()); ++k)
      if (p0 + k < need && pages[p0 + k] < 0) pages[p0 + k] = x.pages[k];
  }
  const uint64_t now = ++r->clock;
  for (int32_t id : path) r->nodes[id].tick = now;
  if (best >= 0)
    for (int32_t id = path[best]; id > 0; id = r->nodes[id].parent) ++r->nodes[id].lock;
  r->queried += n;
  r->matched += len;
  *matched = len;
  *slot = best >= 0 ? r->nodes[path[best]].slot : -1;
  *lock = best >= 0 ? path[best] : -1;
  return had::ok();
}

int had_radix_unlock(had_radix* r, int32_t lock) {
  if (!r) return fail(HAD_ERR_INVALID_ARG, "radix_unlock: NULL handle");
  if (lock == -1) return had::ok();
  if (lock <= 0 || lock >= static_cast<int32_t>(r->nodes.size()) || !r->nodes[lock].live || r->nodes[lock].lock <= 0)
    return fail(HAD_ERR_INVALID_ARG, "radix_unlock: %d is not a held lock", lock);
  for (int32_t id = lock; id > 0; id = r->nodes[id].parent) --r->nodes[id].lock;
  return had::ok();
}

int had_radix_insert(had_radix* r, const int32_t* tokens, int32_t n, const int32_t* pages, int32_t slot,
                     int32_t* new_tokens) {
  if (!r) return fail(HAD_ERR_INVALID_ARG, "radix_insert: NULL handle");
  int st = check_tokens(tokens, n, "radix_insert");
  if (st != HAD_OK) return st;
  if (n > 0 && !pages) return fail(HAD_ERR_INVALID_ARG, "radix_insert: pages is NULL");
  // 1. find where the tokens leave the tree (no change yet)
  std::vector<int32_t> path;
  int32_t depth = 0;
  r->walk(tokens, n, path, depth);
  int32_t cur = path.empty() ? 0 : path.back();
  int32_t split_child = -1, m = 0;
  if (depth < n) {
    auto it = r->nodes[cur].kids.find(tokens[depth]);
    if (it != r->nodes[cur].kids.end()) {  // the tokens leave (or end) inside this edge
      split_child = it->second;
      const had_radix::Node& c = r->nodes[split_child];
      while (m < c.end - c.start && depth + m < n && c.toks[m] == tokens[depth + m]) ++m;
    }
  }
  const int32_t at = depth + m;  // depth of the node the slot or the new leaf hangs from
  const bool leaf = at < n;
  const bool attach = !leaf && slot >= 0 && at > 0 &&
                      (split_child >= 0 || r->nodes[cur].slot < 0);  // a split node starts without a slot
  // 2. take the new references (all or nothing)
  std::vector<int32_t> taken;
  if (leaf) {
    for (int32_t k = r->first_page(at); k < r->end_page(n); ++k) {
      st = had_kvpt_page_retain(r->kv, pages[k]);
      if (st != HAD_OK) {
        for (int32_t p : taken) had_kvpt_page_release(r->kv, p);
        return st;
      }
      taken.push_back(pages[k]);
    }
  }
  if ((leaf || attach) && slot >= 0) {
    st = had_slots_retain(r->slots, slot);
    if (st != HAD_OK) {
      for (int32_t p : taken) had_kvpt_page_release(r->kv, p);
      return st;
    }
  }
  // 3. split the edge the tokens leave, then hang the rest
  if (split_child >= 0 && m > 0) {
    const int32_t mid = r->new_node();  // may move r->nodes: no references held across
    had_radix::Node& c = r->nodes[split_child];
    had_radix::Node& x = r->nodes[mid];
    x.parent = c.parent;
    x.start = c.start;
    x.end = c.start + m;
    x.toks.assign(c.toks.begin(), c.toks.begin() + m);
    x.lock = c.lock;
    x.tick = c.tick;
    const int32_t keep = r->end_page(x.end) - r->first_page(x.start);
    x.pages.assign(c.pages.begin(), c.pages.begin() + keep);
    for (int32_t p : x.pages) had_kvpt_page_retain(r->kv, p);
    const int32_t drop = r->first_page(x.end) - r->first_page(c.start);
    for (int32_t k = 0; k < drop; ++k) had_kvpt_page_release(r->kv, c.pages[k]);
    c.pages.erase(c.pages.begin(), c.pages.begin() + drop);
    c.toks.erase(c.toks.begin(), c.toks.begin() + m);
    c.start = x.end;
    c.parent = mid;
    x.kids[c.toks[0]] = split_child;
    r->nodes[x.parent].kids[x.toks[0]] = mid;
    cur = mid;
    path.push_back(mid);
  }
  const uint64_t now = ++r->clock;
  for (int32_t id : path) r->nodes[id].tick = now;
  if (leaf) {
    const int32_t id = r->new_node();
    had_radix::Node& y = r->nodes[id];
    y.parent = cur;
    y.start = at;
    y.end = n;
    y.toks.assign(tokens + at, tokens + n);
    y.pages = taken;
    y.slot = slot;
    y.tick = now;
    r->nodes[cur].kids[tokens[at]] = id;
  } else if (attach) {
    r->nodes[cur].slot = slot;
  }
  if (new_tokens) *new_tokens = n - at;
  return had::ok();
}

int had_radix_evict(had_radix* r, int32_t min_free_pages, int32_t min_free_slots, int32_t* n_evicted) {
  if (!r) return fail(HAD_ERR_INVALID_ARG, "radix_evict: NULL handle");
  int32_t count = 0;
  for (;;) {
    int32_t pf = 0, pu = 0, sf = 0, su = 0;
    had_kvpt_stats(r->kv, &pf, &pu);
    had_slots_stats(r->slots, &sf, &su);
    const bool short_pages = pf < min_free_pages, short_slots = sf < min_free_slots;
    if (!short_pages && !short_slots) break;
    // least recently used unlocked leaf
    int32_t victim = -1;
    for (int32_t id = 1; id < static_cast<int32_t>(r->nodes.size()); ++id) {
      const had_radix::Node& x = r->nodes[id];
      if (x.live && x.kids.empty() && x.lock == 0 && (victim < 0 || x.tick < r->nodes[victim].tick)) victim = id;
    }
    if (victim >= 0) {
      had_radix::Node& x = r->nodes[victim];
      r->release_node(x);
      r->nodes[x.parent].kids.erase(x.toks[0]);
      x.live = false;
      x.kids.clear();
      r->free_ids.push_back(victim);
      ++count;
      continue;
    }
    if (!short_slots) break;
    // no leaf left to take: drop the least recently used unlocked inner checkpoint
    for (int32_t id = 1; id < static_cast<int32_t>(r->nodes.size()); ++id) {
      const had_radix::Node& x = r->nodes[id];
      if (x.live && x.slot >= 0 && x.lock == 0 && (victim < 0 || x.tick < r->nodes[victim].tick)) victim = id;
    }
    if (victim < 0) break;
    had_slots_release(r->slots, r->nodes[victim].slot);
    r->nodes[victim].slot = -1;
    ++count;
  }
  if (n_evicted) *n_evicted = count;
  return had::ok();
}

int had_radix_stats(const had_radix* r, int32_t* n_nodes, int64_t* cached_tokens, int32_t* n_checkpoints,
                    int64_t* queried_tokens, int64_t* matched_tokens) {
  if (!r || !n_nodes || !cached_tokens || !n_checkpoints || !queried_tokens || !matched_tokens)
    return fail(HAD_ERR_INVALID_ARG, "radix_stats: NULL argument");
  int32_t nn = 0, nc = 0;
  int64_t toks = 0;
  for (size_t id = 1; id < r->nodes.size(); ++id) {
    const had_radix::Node& x = r->nodes[id];
    if (!x.live) continue;
    ++nn;
    toks += x.end - x.start;
    nc += x.slot >= 0;
  }
  *n_nodes = nn;
  *cached_tokens = toks;
  *n_checkpoints = nc;
  *queried_tokens = r->queried;
  *matched_tokens = r->matched;
  return had::ok();
}

}  // extern "C"
