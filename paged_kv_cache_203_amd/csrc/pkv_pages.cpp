// Host page allocator for the paged KV pools: reference-counted pages, sequences that share pages
// after a fork, copy-on-write when a sequence grows into a page it shares, and a prefix cache (a
// radix tree whose edges are whole pages of token ids) that lets a new sequence start on the
// pages of a cached prefix.  Host memory and host logic only; it produces the page tables and
// lengths the attention calls take, and the page copies a copy-on-write needs
// (pkv_copy_pages runs them on the device).
//
//  * Pages: a free set (the lowest free id is always taken first, so allocation is deterministic)
//    and a reference count per page: one per sequence that lists it, one if the prefix cache holds
//    it.  A page returns to the free set when its count reaches zero.
//  * Sequences: a page list and a token count.  Growing by n tokens first replaces a shared,
//    partly filled last page by a fresh copy (the slots past the length would be written, and
//    another holder reads the page), then takes new pages for the rest.  Pages are only ever
//    shared whole or up to a sequence's length, so a shared page is never written.
//  * Prefix cache: node = (parent node, the page_size token ids of one page) -> page.  Inserting a
//    sequence's first full pages adds missing nodes (the cache takes a reference); a lookup walks
//    the tree page by page, comparing token ids exactly.  Eviction removes least recently used
//    leaves whose page nobody else holds.
// Pages: CacheIR page, "Current Capabilities" (shared page allocator accounting across forked
// request sessions); TorchInferno page, "Runtime Scaffolds" (runtime.paged page-table-shaped
// allocation; runtime.prefix radix prefix tree; runtime.prefix_cache prefix lookup).
#include <cstdint>
#include <map>
#include <set>
#include <string>
#include <vector>

#include "../../include/pkv.h"

namespace {

struct Node {
  int32_t parent;                 // -1: child of the root
  std::vector<int32_t> tokens;    // page_size token ids
  int32_t page;
  uint64_t last_use;
  int32_t children = 0;
};

struct Seq {
  std::vector<int32_t> pages;
  int64_t length = 0;
  bool live = false;
};

thread_local std::string g_page_error;

int err(int code, const char* msg) {
  g_page_error = msg;
  return code;
}

}  // namespace

struct pkv_page_allocator {
  int32_t num_pages = 0, page_size = 0;
  std::vector<int32_t> refs;
  std::set<int32_t> free_pages;
  std::vector<Seq> seqs;
  std::vector<int32_t> free_seq_ids;
  std::vector<Node> nodes;                          // index = node id; page < 0: removed
  std::map<std::pair<int32_t, std::vector<int32_t>>, int32_t> index;   // (parent, tokens) -> node
  uint64_t clock = 0;

  int32_t take_page() {
    const int32_t p = *free_pages.begin();
    free_pages.erase(free_pages.begin());
    refs[p] = 1;
    return p;
  }
  void drop(int32_t p) {
    if (--refs[p] == 0) free_pages.insert(p);
  }
  Seq* seq(int32_t id) {
    if (id < 0 || id >= int32_t(seqs.size()) || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
  int32_t new_seq() {
    int32_t id;
    if (!free_seq_ids.empty()) {
      id = free_seq_ids.back();
      free_seq_ids.pop_back();
    } else {
      id = int32_t(seqs.size());
      seqs.emplace_back();
    }
    seqs[id] = Seq{};
    seqs[id].live = true;
    return id;
  }
};

extern "C" {

const char* pkv_pages_last_error(void) { return g_page_error.c_str(); }

pkv_page_allocator* pkv_pages_create(int32_t num_pages, int32_t page_size) {
  if (num_pages <= 0 || page_size <= 0) {
    err(PKV_EINVAL, "num_pages and page_size must be > 0");
    return nullptr;
  }
  auto* a = new pkv_page_allocator;
  a->num_pages = num_pages;
  a->page_size = page_size;
  a->refs.assign(num_pages, 0);
  for (int32_t p = 0; p < num_pages; ++p) a->free_pages.insert(a->free_pages.end(), p);
  return a;
}

void pkv_pages_destroy(pkv_page_allocator* a) { delete a; }

int32_t pkv_pages_free_count(const pkv_page_allocator* a) {
  return a ? int32_t(a->free_pages.size()) : -1;
}

int32_t pkv_pages_refcount(const pkv_page_allocator* a, int32_t page) {
  if (!a || page < 0 || page >= a->num_pages) return -1;
  return a->refs[page];
}

int pkv_pages_seq_create(pkv_page_allocator* a, int32_t* seq_out) {
  if (!a || !seq_out) return err(PKV_EINVAL, "allocator and seq_out must be non-NULL");
  *seq_out = a->new_seq();
  return PKV_OK;
}

int pkv_pages_seq_fork(pkv_page_allocator* a, int32_t src, int32_t* seq_out) {
  if (!a || !seq_out) return err(PKV_EINVAL, "allocator and seq_out must be non-NULL");
  if (!a->seq(src)) return err(PKV_EINVAL, "no such sequence");
  const int32_t id = a->new_seq();
  Seq& s = a->seqs[src];   // after new_seq: the vector may have grown
  a->seqs[id].pages = s.pages;
  a->seqs[id].length = s.length;
  for (int32_t p : s.pages) ++a->refs[p];
  *seq_out = id;
  return PKV_OK;
}

int pkv_pages_seq_release(pkv_page_allocator* a, int32_t seq) {
  if (!a) return err(PKV_EINVAL, "allocator must be non-NULL");
  Seq* s = a->seq(seq);
  if (!s) return err(PKV_EINVAL, "no such sequence");
  for (int32_t p : s->pages) a->drop(p);
  *s = Seq{};
  a->free_seq_ids.push_back(seq);
  return PKV_OK;
}

int pkv_pages_seq_reserve(pkv_page_allocator* a, int32_t seq, int32_t n_tokens,
                          int32_t* copies_out, int32_t max_copies, int32_t* n_copies) {
  if (!a || !n_copies) return err(PKV_EINVAL, "allocator and n_copies must be non-NULL");
  Seq* s = a->seq(seq);
  if (!s) return err(PKV_EINVAL, "no such sequence");
  if (n_tokens < 0) return err(PKV_EINVAL, "n_tokens must be >= 0");
  const int64_t PS = a->page_size;
  const int64_t new_len = s->length + n_tokens;
  if (new_len > int64_t(INT32_MAX)) return err(PKV_EINVAL, "sequence length overflows int32");
  const int64_t have = int64_t(s->pages.size());
  const int64_t need = (new_len + PS - 1) / PS;
  const bool cow = n_tokens > 0 && s->length % PS != 0 && a->refs[s->pages.back()] > 1;
  const int64_t take = (need - have) + (cow ? 1 : 0);
  if (cow && (!copies_out || max_copies < 1))
    return err(PKV_EWORKSPACE, "a copy-on-write is needed: copies_out must hold one pair");
  if (take > int64_t(a->free_pages.size())) return err(PKV_EWORKSPACE, "out of free pages");
  *n_copies = 0;
  if (cow) {   // the shared, partly filled last page is replaced by a private copy
    const int32_t old = s->pages.back();
    const int32_t fresh = a->take_page();
    a->drop(old);
    s->pages.back() = fresh;
    copies_out[0] = old;
    copies_out[1] = fresh;
    *n_copies = 1;
  }
  for (int64_t i = have; i < need; ++i) s->pages.push_back(a->take_page());
  s->length = new_len;
  return PKV_OK;
}

int pkv_pages_seq_length(const pkv_page_allocator* a, int32_t seq, int32_t* len_out) {
  if (!a || !len_out) return err(PKV_EINVAL, "allocator and len_out must be non-NULL");
  auto* self = const_cast<pkv_page_allocator*>(a);
  Seq* s = self->seq(seq);
  if (!s) return err(PKV_EINVAL, "no such sequence");
  *len_out = int32_t(s->length);
  return PKV_OK;
}

int pkv_pages_seq_table(const pkv_page_allocator* a, int32_t seq, int32_t* row,
                        int32_t max_pages, int32_t* n_pages) {
  if (!a || !row || !n_pages) return err(PKV_EINVAL, "allocator, row and n_pages must be non-NULL");
  auto* self = const_cast<pkv_page_allocator*>(a);
  Seq* s = self->seq(seq);
  if (!s) return err(PKV_EINVAL, "no such sequence");
  *n_pages = int32_t(s->pages.size());
  if (int64_t(s->pages.size()) > max_pages)
    return err(PKV_EWORKSPACE, "the sequence has more pages than the row holds");
  for (int32_t i = 0; i < max_pages; ++i)
    row[i] = i < int32_t(s->pages.size()) ? s->pages[i] : -1;
  return PKV_OK;
}

int pkv_pages_prefix_insert(pkv_page_allocator* a, int32_t seq, const int32_t* tokens,
                            int32_t n_tokens) {
  if (!a || (!tokens && n_tokens > 0)) return err(PKV_EINVAL, "allocator and tokens must be non-NULL");
  Seq* s = a->seq(seq);
  if (!s) return err(PKV_EINVAL, "no such sequence");
  if (n_tokens < 0 || n_tokens > s->length)
    return err(PKV_EINVAL, "n_tokens must be in [0, the sequence's length]");
  const int32_t PS = a->page_size;
  int32_t parent = -1;
  ++a->clock;
  for (int32_t i = 0; i < n_tokens / PS; ++i) {
    std::vector<int32_t> key(tokens + int64_t(i) * PS, tokens + int64_t(i + 1) * PS);
    auto it = a->index.find({parent, key});
    int32_t node;
    if (it == a->index.end()) {
      node = int32_t(a->nodes.size());
      a->nodes.push_back(Node{parent, key, s->pages[i], a->clock});
      if (parent >= 0) ++a->nodes[parent].children;
      a->index.emplace(std::make_pair(parent, std::move(key)), node);
      ++a->refs[s->pages[i]];   // the cache holds the page
    } else {
      node = it->second;
      a->nodes[node].last_use = a->clock;
    }
    parent = node;
  }
  return PKV_OK;
}

int pkv_pages_seq_create_with_prefix(pkv_page_allocator* a, const int32_t* tokens,
                                     int32_t n_tokens, int32_t* seq_out,
                                     int32_t* matched_tokens) {
  if (!a || !seq_out || !matched_tokens || (!tokens && n_tokens > 0))
    return err(PKV_EINVAL, "allocator, tokens, seq_out and matched_tokens must be non-NULL");
  if (n_tokens < 0) return err(PKV_EINVAL, "n_tokens must be >= 0");
  const int32_t PS = a->page_size;
  const int32_t id = a->new_seq();
  Seq& s = a->seqs[id];
  int32_t parent = -1;
  ++a->clock;
  for (int32_t i = 0; i < n_tokens / PS; ++i) {
    std::vector<int32_t> key(tokens + int64_t(i) * PS, tokens + int64_t(i + 1) * PS);
    auto it = a->index.find({parent, key});
    if (it == a->index.end()) break;
    const int32_t node = it->second;
    a->nodes[node].last_use = a->clock;
    s.pages.push_back(a->nodes[node].page);
    ++a->refs[a->nodes[node].page];
    parent = node;
  }
  s.length = int64_t(s.pages.size()) * PS;
  *seq_out = id;
  *matched_tokens = int32_t(s.length);
  return PKV_OK;
}

int pkv_pages_prefix_evict(pkv_page_allocator* a, int32_t max_pages, int32_t* evicted) {
  if (!a || !evicted) return err(PKV_EINVAL, "allocator and evicted must be non-NULL");
  *evicted = 0;
  while (*evicted < max_pages) {
    int32_t best = -1;
    for (int32_t n = 0; n < int32_t(a->nodes.size()); ++n) {
      const Node& x = a->nodes[n];
      if (x.page < 0 || x.children != 0 || a->refs[x.page] != 1) continue;
      if (best < 0 || x.last_use < a->nodes[best].last_use) best = n;
    }
    if (best < 0) break;
    Node& x = a->nodes[best];
    a->index.erase({x.parent, x.tokens});
    if (x.parent >= 0) --a->nodes[x.parent].children;
    a->drop(x.page);
    x.page = -1;
    ++*evicted;
  }
  return PKV_OK;
}

}  // extern "C"
