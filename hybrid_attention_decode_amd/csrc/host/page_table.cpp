// Host-side logical KV cache: page table with reference-counted pages,
// prefix forking, copy-on-write of a shared partially filled last page, and
// the reference-counted state-slot pool of the linear-attention layers.
//
// The engine keeps its logical cache in C++ and the physical tensors in
// Python (24-ai.news TokenSpeed article, optimisation list, hybrid prefix
// caching); cached checkpoints are reused without mutation through
// copy-on-write and reached by index (zubnet.ai TokenSpeed article, second
// paragraph).  The allocation policy is fixed so that results can be
// compared bit for bit: free list popped from its end, freed ids pushed to
// its end, lowest unused sequence id.
#include <cstdint>
#include <new>
#include <vector>

#include "had.h"
#include "status.h"

using had::fail;

struct had_kvpt {
  int32_t num_pages = 0, page_size = 0, max_seqs = 0, max_pages = 0;
  std::vector<int32_t> free_list;   // back() is the next page handed out
  std::vector<int32_t> ref;         // per physical page
  struct Seq {
    bool live = false;
    int32_t len = 0;
    std::vector<int32_t> pages;
  };
  std::vector<Seq> seqs;

  int32_t pages_for(int64_t n) const { return static_cast<int32_t>((n + page_size - 1) / page_size); }
  Seq* get(int32_t s) {
    if (s < 0 || s >= max_seqs || !seqs[s].live) return nullptr;
    return &seqs[s];
  }
  const Seq* get(int32_t s) const {
    if (s < 0 || s >= max_seqs || !seqs[s].live) return nullptr;
    return &seqs[s];
  }
  int32_t new_id() const {
    for (int32_t s = 0; s < max_seqs; ++s)
      if (!seqs[s].live) return s;
    return -1;
  }
  void drop_last_page(Seq& q) {
    int32_t p = q.pages.back();
    q.pages.pop_back();
    if (--ref[p] == 0) free_list.push_back(p);
  }
};

struct had_slots {
  int32_t n = 0;
  std::vector<int32_t> free_list;
  std::vector<int32_t> ref;
  bool held(int32_t s) const { return s >= 0 && s < n && ref[s] > 0; }
};

namespace {

// Checks that `order` holds each id of [0, n) exactly once.
bool is_permutation(const int32_t* order, int32_t n) {
  std::vector<char> seen(n, 0);
  for (int32_t i = 0; i < n; ++i) {
    int32_t v = order[i];
    if (v < 0 || v >= n || seen[v]) return false;
    seen[v] = 1;
  }
  return true;
}

}  // namespace

extern "C" {

int had_kvpt_create(int32_t num_pages, int32_t page_size, int32_t max_seqs,
                    int32_t max_pages_per_seq, const int32_t* free_order, had_kvpt** out) {
  if (!out) return fail(HAD_ERR_INVALID_ARG, "kvpt_create: out is NULL");
  if (num_pages <= 0 || page_size <= 0 || max_seqs <= 0 || max_pages_per_seq <= 0)
    return fail(HAD_ERR_INVALID_ARG, "kvpt_create: sizes must be positive (num_pages=%d page_size=%d max_seqs=%d max_pages=%d)",
                num_pages, page_size, max_seqs, max_pages_per_seq);
  if (free_order && !is_permutation(free_order, num_pages))
    return fail(HAD_ERR_INVALID_ARG, "kvpt_create: free_order is not a permutation of [0, %d)", num_pages);
  had_kvpt* h = new (std::nothrow) had_kvpt;
  if (!h) return fail(HAD_ERR_INVALID_ARG, "kvpt_create: out of host memory");
  h->num_pages = num_pages;
  h->page_size = page_size;
  h->max_seqs = max_seqs;
  h->max_pages = max_pages_per_seq;
  h->free_list.resize(num_pages);
  for (int32_t i = 0; i < num_pages; ++i) h->free_list[i] = free_order ? free_order[i] : i;
  h->ref.assign(num_pages, 0);
  h->seqs.resize(max_seqs);
  *out = h;
  return had::ok();
}

int had_kvpt_destroy(had_kvpt* h) {
  delete h;
  return had::ok();
}

int had_kvpt_seq_create(had_kvpt* h, int32_t* seq) {
  if (!h || !seq) return fail(HAD_ERR_INVALID_ARG, "seq_create: NULL argument");
  int32_t s = h->new_id();
  if (s < 0) return fail(HAD_ERR_CAPACITY, "seq_create: all %d sequence ids are live", h->max_seqs);
  h->seqs[s].live = true;
  h->seqs[s].len = 0;
  h->seqs[s].pages.clear();
  *seq = s;
  return had::ok();
}

int had_kvpt_seq_fork(had_kvpt* h, int32_t src, int32_t prefix_len, int32_t* seq) {
  if (!h || !seq) return fail(HAD_ERR_INVALID_ARG, "seq_fork: NULL argument");
  had_kvpt::Seq* s = h->get(src);
  if (!s) return fail(HAD_ERR_BAD_SEQ, "seq_fork: sequence %d is not live", src);
  if (prefix_len < 0 || prefix_len > s->len)
    return fail(HAD_ERR_RANGE, "seq_fork: prefix_len %d outside [0, %d]", prefix_len, s->len);
  int32_t id = h->new_id();
  if (id < 0) return fail(HAD_ERR_CAPACITY, "seq_fork: all %d sequence ids are live", h->max_seqs);
  int32_t n = h->pages_for(prefix_len);
  had_kvpt::Seq& d = h->seqs[id];
  d.pages.assign(s->pages.begin(), s->pages.begin() + n);
  for (int32_t p : d.pages) ++h->ref[p];
  d.len = prefix_len;
  d.live = true;
  *seq = id;
  return had::ok();
}

int had_kvpt_seq_create_from(had_kvpt* h, const int32_t* pages, int32_t n_pages, int32_t len, int32_t* seq) {
  if (!h || !seq || (n_pages > 0 && !pages)) return fail(HAD_ERR_INVALID_ARG, "seq_create_from: NULL argument");
  if (len < 0 || n_pages != h->pages_for(len))
    return fail(HAD_ERR_RANGE, "seq_create_from: %d pages do not cover exactly %d tokens", n_pages, len);
  if (n_pages > h->max_pages)
    return fail(HAD_ERR_CAPACITY, "seq_create_from: %d pages > max_pages_per_seq %d", n_pages, h->max_pages);
  for (int32_t i = 0; i < n_pages; ++i)
    if (pages[i] < 0 || pages[i] >= h->num_pages || h->ref[pages[i]] == 0)
      return fail(HAD_ERR_INVALID_ARG, "seq_create_from: page %d is not a held page", pages[i]);
  const int32_t id = h->new_id();
  if (id < 0) return fail(HAD_ERR_CAPACITY, "seq_create_from: all %d sequence ids are live", h->max_seqs);
  had_kvpt::Seq& d = h->seqs[id];
  d.pages.assign(pages, pages + n_pages);
  for (int32_t p : d.pages) ++h->ref[p];
  d.len = len;
  d.live = true;
  *seq = id;
  return had::ok();
}

int had_kvpt_page_retain(had_kvpt* h, int32_t page) {
  if (!h) return fail(HAD_ERR_INVALID_ARG, "page_retain: NULL handle");
  if (page < 0 || page >= h->num_pages || h->ref[page] == 0)
    return fail(HAD_ERR_INVALID_ARG, "page_retain: page %d is not held", page);
  ++h->ref[page];
  return had::ok();
}

int had_kvpt_page_release(had_kvpt* h, int32_t page) {
  if (!h) return fail(HAD_ERR_INVALID_ARG, "page_release: NULL handle");
  if (page < 0 || page >= h->num_pages || h->ref[page] == 0)
    return fail(HAD_ERR_INVALID_ARG, "page_release: page %d is not held", page);
  if (--h->ref[page] == 0) h->free_list.push_back(page);
  return had::ok();
}

int had_kvpt_reserve(had_kvpt* h, int32_t seq, int32_t n_tokens, int32_t* cow, int32_t* n_cow) {
  if (!h || !cow || !n_cow) return fail(HAD_ERR_INVALID_ARG, "reserve: NULL argument");
  had_kvpt::Seq* s = h->get(seq);
  if (!s) return fail(HAD_ERR_BAD_SEQ, "reserve: sequence %d is not live", seq);
  if (n_tokens < 0) return fail(HAD_ERR_INVALID_ARG, "reserve: n_tokens %d < 0", n_tokens);
  *n_cow = 0;
  if (n_tokens == 0) return had::ok();
  const int64_t new_len = static_cast<int64_t>(s->len) + n_tokens;
  if (new_len > static_cast<int64_t>(h->max_pages) * h->page_size)
    return fail(HAD_ERR_CAPACITY, "reserve: length %lld exceeds max_pages_per_seq=%d", (long long)new_len, h->max_pages);
  const bool need_cow = (s->len % h->page_size) != 0 && h->ref[s->pages.back()] > 1;
  const int32_t need = h->pages_for(new_len) - static_cast<int32_t>(s->pages.size());
  if (static_cast<int64_t>(need) + (need_cow ? 1 : 0) > static_cast<int64_t>(h->free_list.size()))
    return fail(HAD_ERR_OUT_OF_PAGES, "reserve: need %d pages, %zu free", need + (need_cow ? 1 : 0), h->free_list.size());
  if (need_cow) {
    const int32_t src = s->pages.back();
    const int32_t dst = h->free_list.back();
    h->free_list.pop_back();
    --h->ref[src];
    h->ref[dst] = 1;
    s->pages.back() = dst;
    cow[0] = src;
    cow[1] = dst;
    cow[2] = s->len % h->page_size;
    *n_cow = 1;
  }
  for (int32_t i = 0; i < need; ++i) {
    const int32_t p = h->free_list.back();
    h->free_list.pop_back();
    h->ref[p] = 1;
    s->pages.push_back(p);
  }
  s->len = static_cast<int32_t>(new_len);
  return had::ok();
}

int had_kvpt_truncate(had_kvpt* h, int32_t seq, int32_t new_len) {
  if (!h) return fail(HAD_ERR_INVALID_ARG, "truncate: NULL handle");
  had_kvpt::Seq* s = h->get(seq);
  if (!s) return fail(HAD_ERR_BAD_SEQ, "truncate: sequence %d is not live", seq);
  if (new_len < 0 || new_len > s->len)
    return fail(HAD_ERR_RANGE, "truncate: new_len %d outside [0, %d]", new_len, s->len);
  const size_t keep = static_cast<size_t>(h->pages_for(new_len));
  while (s->pages.size() > keep) h->drop_last_page(*s);
  s->len = new_len;
  return had::ok();
}

int had_kvpt_seq_free(had_kvpt* h, int32_t seq) {
  if (!h) return fail(HAD_ERR_INVALID_ARG, "seq_free: NULL handle");
  had_kvpt::Seq* s = h->get(seq);
  if (!s) return fail(HAD_ERR_BAD_SEQ, "seq_free: sequence %d is not live", seq);
  while (!s->pages.empty()) h->drop_last_page(*s);
  s->len = 0;
  s->live = false;
  return had::ok();
}

int had_kvpt_seq_len(const had_kvpt* h, int32_t seq, int32_t* len) {
  if (!h || !len) return fail(HAD_ERR_INVALID_ARG, "seq_len: NULL argument");
  const had_kvpt::Seq* s = h->get(seq);
  if (!s) return fail(HAD_ERR_BAD_SEQ, "seq_len: sequence %d is not live", seq);
  *len = s->len;
  return had::ok();
}

int had_kvpt_export(const had_kvpt* h, const int32_t* seqs, int32_t n, int32_t* page_table,
                    int32_t max_pages, int32_t* seq_lens) {
  if (!h || (n > 0 && (!seqs || !page_table || !seq_lens)) || n < 0 || max_pages <= 0)
    return fail(HAD_ERR_INVALID_ARG, "export: bad argument (n=%d max_pages=%d)", n, max_pages);
  for (int32_t i = 0; i < n; ++i) {  // validate everything before writing
    const had_kvpt::Seq* s = h->get(seqs[i]);
    if (!s) return fail(HAD_ERR_BAD_SEQ, "export: sequence %d is not live", seqs[i]);
    if (static_cast<int32_t>(s->pages.size()) > max_pages)
      return fail(HAD_ERR_INVALID_ARG, "export: sequence %d holds %zu pages > max_pages %d", seqs[i], s->pages.size(), max_pages);
  }
  for (int32_t i = 0; i < n; ++i) {
    const had_kvpt::Seq* s = h->get(seqs[i]);
    int32_t* row = page_table + static_cast<int64_t>(i) * max_pages;
    const int32_t np = static_cast<int32_t>(s->pages.size());
    for (int32_t j = 0; j < max_pages; ++j) row[j] = j < np ? s->pages[j] : -1;
    seq_lens[i] = s->len;
  }
  return had::ok();
}

int had_kvpt_info(const had_kvpt* h, int32_t* num_pages, int32_t* page_size) {
  if (!h || !num_pages || !page_size) return fail(HAD_ERR_INVALID_ARG, "kvpt_info: NULL argument");
  *num_pages = h->num_pages;
  *page_size = h->page_size;
  return had::ok();
}

int had_kvpt_stats(const had_kvpt* h, int32_t* n_free, int32_t* n_used) {
  if (!h || !n_free || !n_used) return fail(HAD_ERR_INVALID_ARG, "stats: NULL argument");
  *n_free = static_cast<int32_t>(h->free_list.size());
  int32_t used = 0;
  for (int32_t r : h->ref) used += r > 0;
  *n_used = used;
  return had::ok();
}

// ---------------------------------------------------------------- slots ---

int had_slots_create(int32_t n_slots, const int32_t* free_order, had_slots** out) {
  if (!out || n_slots <= 0) return fail(HAD_ERR_INVALID_ARG, "slots_create: bad argument (n_slots=%d)", n_slots);
  if (free_order && !is_permutation(free_order, n_slots))
    return fail(HAD_ERR_INVALID_ARG, "slots_create: free_order is not a permutation of [0, %d)", n_slots);
  had_slots* h = new (std::nothrow) had_slots;
  if (!h) return fail(HAD_ERR_INVALID_ARG, "slots_create: out of host memory");
  h->n = n_slots;
  h->free_list.resize(n_slots);
  for (int32_t i = 0; i < n_slots; ++i) h->free_list[i] = free_order ? free_order[i] : i;
  h->ref.assign(n_slots, 0);
  *out = h;
  return had::ok();
}

int had_slots_destroy(had_slots* h) {
  delete h;
  return had::ok();
}

int had_slots_acquire(had_slots* h, int32_t* slot) {
  if (!h || !slot) return fail(HAD_ERR_INVALID_ARG, "slots_acquire: NULL argument");
  if (h->free_list.empty()) return fail(HAD_ERR_OUT_OF_SLOTS, "slots_acquire: all %d slots held", h->n);
  const int32_t s = h->free_list.back();
  h->free_list.pop_back();
  h->ref[s] = 1;
  *slot = s;
  return had::ok();
}

int had_slots_retain(had_slots* h, int32_t slot) {
  if (!h) return fail(HAD_ERR_INVALID_ARG, "slots_retain: NULL handle");
  if (!h->held(slot)) return fail(HAD_ERR_BAD_SLOT, "slots_retain: slot %d is not held", slot);
  ++h->ref[slot];
  return had::ok();
}

int had_slots_release(had_slots* h, int32_t slot) {
  if (!h) return fail(HAD_ERR_INVALID_ARG, "slots_release: NULL handle");
  if (!h->held(slot)) return fail(HAD_ERR_BAD_SLOT, "slots_release: slot %d is not held", slot);
  if (--h->ref[slot] == 0) h->free_list.push_back(slot);
  return had::ok();
}

int had_slots_stats(const had_slots* h, int32_t* n_free, int32_t* n_used) {
  if (!h || !n_free || !n_used) return fail(HAD_ERR_INVALID_ARG, "slots_stats: NULL argument");
  *n_free = static_cast<int32_t>(h->free_list.size());
  int32_t used = 0;
  for (int32_t r : h->ref) used += r > 0;
  *n_used = used;
  return had::ok();
}

int had_gdn_check_slots(int32_t n_seqs, int32_t T, int32_t n_slots, const int32_t* in_idx, const int32_t* out_idx,
                        int32_t allow_in_place) {
  if (n_seqs < 0 || T < 1 || n_slots < 1 || (n_seqs > 0 && (!in_idx || !out_idx)))
    return fail(HAD_ERR_INVALID_ARG, "gdn_check_slots: bad argument (n_seqs=%d T=%d n_slots=%d)", n_seqs, T, n_slots);
  std::vector<int32_t> writer(n_slots, -1);  // sequence that writes each slot
  for (int32_t s = 0; s < n_seqs; ++s) {
    if (in_idx[s] < -1 || in_idx[s] >= n_slots)
      return fail(HAD_ERR_BAD_SLOT, "gdn_check_slots: in_idx[%d] = %d outside [-1, %d)", s, in_idx[s], n_slots);
    for (int32_t t = 0; t < T; ++t) {
      const int32_t o = out_idx[static_cast<int64_t>(s) * T + t];
      if (o < 0 || o >= n_slots)
        return fail(HAD_ERR_BAD_SLOT, "gdn_check_slots: out_idx[%d][%d] = %d outside [0, %d)", s, t, o, n_slots);
      if (writer[o] >= 0) return fail(HAD_ERR_BAD_SLOT, "gdn_check_slots: slot %d is written twice", o);
      writer[o] = s;
      if (o == in_idx[s] && !allow_in_place)
        return fail(HAD_ERR_BAD_SLOT, "gdn_check_slots: sequence %d reads and writes slot %d", s, o);
    }
  }
  for (int32_t s = 0; s < n_seqs; ++s) {
    const int32_t i = in_idx[s];
    if (i >= 0 && writer[i] >= 0 && writer[i] != s)
      return fail(HAD_ERR_BAD_SLOT, "gdn_check_slots: slot %d is read by sequence %d and written by sequence %d", i, s,
                  writer[i]);
  }
  return had::ok();
}

int had_spec_rollback(had_kvpt* kv, had_slots* slots, int32_t seq, int32_t T, int32_t accepted,
                      int32_t in_slot, const int32_t* out_slots, int32_t* current_slot) {
  if (!kv || !slots || !current_slot || (T > 0 && !out_slots) || T < 0)
    return fail(HAD_ERR_INVALID_ARG, "spec_rollback: bad argument");
  if (accepted < 0 || accepted > T)
    return fail(HAD_ERR_INVALID_ARG, "spec_rollback: accepted %d outside [0, %d]", accepted, T);
  had_kvpt::Seq* s = kv->get(seq);
  if (!s) return fail(HAD_ERR_BAD_SEQ, "spec_rollback: sequence %d is not live", seq);
  if (s->len < T) return fail(HAD_ERR_RANGE, "spec_rollback: length %d < T %d", s->len, T);
  for (int32_t i = 0; i < T; ++i)
    for (int32_t j = 0; j < i; ++j)
      if (out_slots[i] == out_slots[j])
        return fail(HAD_ERR_INVALID_ARG, "spec_rollback: out slot %d repeated", out_slots[i]);
  for (int32_t i = 0; i < T; ++i)
    if (!slots->held(out_slots[i]) || out_slots[i] == in_slot)
      return fail(HAD_ERR_BAD_SLOT, "spec_rollback: out slot %d not held or equal to in_slot", out_slots[i]);
  if (accepted > 0 && in_slot >= 0 && !slots->held(in_slot))
    return fail(HAD_ERR_BAD_SLOT, "spec_rollback: in slot %d is not held", in_slot);
  const int32_t new_len = s->len - T + accepted;
  const size_t keep = static_cast<size_t>(kv->pages_for(new_len));
  while (s->pages.size() > keep) kv->drop_last_page(*s);
  s->len = new_len;
  const int32_t cur = accepted == 0 ? in_slot : out_slots[accepted - 1];
  for (int32_t t = 0; t < T; ++t) {
    if (t == accepted - 1) continue;
    const int32_t x = out_slots[t];
    if (--slots->ref[x] == 0) slots->free_list.push_back(x);
  }
  if (accepted > 0 && in_slot >= 0 && --slots->ref[in_slot] == 0) slots->free_list.push_back(in_slot);
  *current_slot = cur;
  return had::ok();
}

}  // extern "C"
