// Host-side manager of the paged, position-free KV pool (lazyattn_cache.h):
// block free list, cached documents with reference counts, least-recently-used
// eviction of unreferenced documents, and block-table rows in the kernels'
// (block id | frame start << 16) format.
//
// Paging and the free list follow ai-engineering.academy, "KV Cache, Flash
// Attention & Otimização de Inferência" (sections "PagedAttention" and
// "Exercícios" 3); the cache keys under comparison follow gist.science,
// "Resumo Técnico: LazyAttention" ("Declaração do Problema", "Metodologia").
#include "lazyattn_cache.h"

#include <stddef.h>

#include <list>
#include <map>
#include <new>
#include <set>
#include <vector>

namespace {

constexpr int kBlockTokens = 16;
constexpr int kMaxBlocks = 65536;
constexpr int kMaxFrameStart = 65535;

typedef std::vector<int32_t> Key;

struct Entry {
  std::vector<int32_t> blocks;
  int refs = 0;
  bool evictable = false;
  std::list<const Key *>::iterator lru;  // valid while evictable
};

struct Request {
  std::vector<const Key *> docs;   // one per document occurrence
  std::vector<int32_t> prompt;     // the prompt's blocks
};

}  // namespace

struct lazyattn_cache {
  int num_blocks = 0;
  int mode = 0;
  std::vector<int32_t> free_list;          // a stack: the next block is at the back
  std::map<Key, Entry> docs;
  std::list<const Key *> lru;              // unreferenced documents, oldest first
  std::map<int32_t, Request> requests;
  int32_t next_request = 0;
  int64_t n_requests = 0, doc_hits = 0, doc_misses = 0, tok_hits = 0, tok_misses = 0, evicted = 0;
  int64_t doc_blocks = 0, prompt_blocks = 0;

  Key key_of(const int32_t *ids, int i, int pos) const {
    if (mode == LAZYATTN_CACHE_AGNOSTIC) return Key{ids[i]};
    if (mode == LAZYATTN_CACHE_AWARE) return Key{ids[i], pos};
    return Key(ids, ids + i + 1);  // prefix: the document sequence up to i
  }

  void take(Entry &e) {
    if (e.evictable) {
      lru.erase(e.lru);
      e.evictable = false;
    }
    ++e.refs;
  }

  void drop(const Key *k) {
    Entry &e = docs.at(*k);
    if (--e.refs == 0) {
      e.lru = lru.insert(lru.end(), k);
      e.evictable = true;
    }
  }

  // Evict unreferenced documents, oldest first, until n blocks are free.
  // The caller has checked that enough blocks can be freed.
  void make_room(int n) {
    while ((int)free_list.size() < n) {
      const Key *k = lru.front();
      lru.pop_front();
      Entry &e = docs.at(*k);
      for (auto it = e.blocks.rbegin(); it != e.blocks.rend(); ++it) free_list.push_back(*it);
      doc_blocks -= (int64_t)e.blocks.size();
      docs.erase(*k);
      ++evicted;
    }
  }

  std::vector<int32_t> alloc(int n) {
    std::vector<int32_t> b((size_t)n);
    for (int i = 0; i < n; ++i) {
      b[(size_t)i] = free_list.back();
      free_list.pop_back();
    }
    return b;
  }
};

extern "C" {

lazyattn_cache *lazyattn_cache_create(int num_blocks, int mode) {
  if (num_blocks < 1 || num_blocks > kMaxBlocks) return nullptr;
  if (mode != LAZYATTN_CACHE_AGNOSTIC && mode != LAZYATTN_CACHE_AWARE && mode != LAZYATTN_CACHE_PREFIX)
    return nullptr;
  lazyattn_cache *c = new (std::nothrow) lazyattn_cache;
  if (!c) return nullptr;
  c->num_blocks = num_blocks;
  c->mode = mode;
  c->free_list.reserve((size_t)num_blocks);
  for (int b = num_blocks - 1; b >= 0; --b) c->free_list.push_back(b);  // block 0 is handed out first
  return c;
}

void lazyattn_cache_destroy(lazyattn_cache *c) { delete c; }

int lazyattn_cache_acquire(lazyattn_cache *c, const int32_t *doc_ids, const int32_t *doc_lens, int n_docs,
                           int prompt_len, uint32_t *table_row, int max_blocks, uint8_t *miss,
                           int32_t *request_id) {
  if (!c || n_docs < 0 || prompt_len < 0 || max_blocks < 0 || !request_id) return LAZYATTN_CACHE_ERR_ARG;
  if (n_docs > 0 && (!doc_ids || !doc_lens || !miss)) return LAZYATTN_CACHE_ERR_ARG;
  // frame starts, keys and sizes
  std::vector<Key> keys((size_t)n_docs);
  std::vector<int> pos((size_t)n_docs);
  long long p = 0, words = 0;
  for (int i = 0; i < n_docs; ++i) {
    if (doc_lens[i] <= 0 || doc_lens[i] % kBlockTokens) return LAZYATTN_CACHE_ERR_ARG;
    if (p > kMaxFrameStart) return LAZYATTN_CACHE_ERR_POSITION;
    pos[(size_t)i] = (int)p;
    keys[(size_t)i] = c->key_of(doc_ids, i, (int)p);
    p += doc_lens[i];
    words += doc_lens[i] / kBlockTokens;
  }
  const int prompt_nb = (prompt_len + kBlockTokens - 1) / kBlockTokens;
  if (prompt_len > 0 && p > kMaxFrameStart) return LAZYATTN_CACHE_ERR_POSITION;
  if (p + prompt_len > kMaxFrameStart + 1) return LAZYATTN_CACHE_ERR_POSITION;  // last position < 65536
  words += prompt_nb;
  if (!table_row && words > 0) return LAZYATTN_CACHE_ERR_ARG;
  if (words > max_blocks) return LAZYATTN_CACHE_ERR_NOSPACE;

  // dry run: blocks to allocate (a key missing twice in one request is
  // allocated once) against free blocks plus those of unreferenced documents
  // this request does not hit.  A document must keep its length: a key
  // cached (or named earlier in this request) with another block count is
  // rejected, since the row would get the cached blocks, not doc_lens[i].
  std::set<Key> hit_keys;
  std::map<Key, int> new_keys;
  long long need = prompt_nb;
  for (int i = 0; i < n_docs; ++i) {
    const Key &k = keys[(size_t)i];
    const int nb = doc_lens[i] / kBlockTokens;
    auto it = c->docs.find(k);
    if (it != c->docs.end()) {
      if (it->second.blocks.size() != (size_t)nb) return LAZYATTN_CACHE_ERR_ARG;
      hit_keys.insert(k);
    } else {
      auto ins = new_keys.emplace(k, nb);
      if (ins.second) need += nb;
      else if (ins.first->second != nb) return LAZYATTN_CACHE_ERR_ARG;
    }
  }
  long long avail = (long long)c->free_list.size();
  for (const Key *k : c->lru)
    if (!hit_keys.count(*k)) avail += (long long)c->docs.at(*k).blocks.size();
  if (need > avail) return LAZYATTN_CACHE_ERR_NOSPACE;

  // references on every document already cached, then the misses in order
  Request req;
  req.docs.resize((size_t)n_docs);
  for (int i = 0; i < n_docs; ++i) {
    auto it = c->docs.find(keys[(size_t)i]);
    if (it != c->docs.end()) {
      c->take(it->second);
      req.docs[(size_t)i] = &it->first;
      miss[i] = 0;
    } else {
      req.docs[(size_t)i] = nullptr;
    }
  }
  for (int i = 0; i < n_docs; ++i) {
    if (req.docs[(size_t)i]) continue;
    auto it = c->docs.find(keys[(size_t)i]);
    if (it != c->docs.end()) {  // a repeat of a document this request already placed
      c->take(it->second);
      req.docs[(size_t)i] = &it->first;
      miss[i] = 0;
      continue;
    }
    const int nb = doc_lens[i] / kBlockTokens;
    c->make_room(nb);
    Entry e;
    e.blocks = c->alloc(nb);
    e.refs = 1;
    c->doc_blocks += nb;
    auto ins = c->docs.emplace(keys[(size_t)i], std::move(e)).first;
    req.docs[(size_t)i] = &ins->first;
    miss[i] = 1;
  }
  c->make_room(prompt_nb);
  req.prompt = c->alloc(prompt_nb);
  c->prompt_blocks += prompt_nb;

  // the table row, in logical order
  int w = 0;
  for (int i = 0; i < n_docs; ++i) {
    const Entry &e = c->docs.at(*req.docs[(size_t)i]);
    for (size_t j = 0; j < e.blocks.size(); ++j)
      table_row[w++] = (uint32_t)e.blocks[j] | ((uint32_t)pos[(size_t)i] << 16);
    if (miss[i]) {
      ++c->doc_misses;
      c->tok_misses += doc_lens[i];
    } else {
      ++c->doc_hits;
      c->tok_hits += doc_lens[i];
    }
  }
  for (int32_t b : req.prompt) table_row[w++] = (uint32_t)b | ((uint32_t)p << 16);
  ++c->n_requests;
  const int32_t id = c->next_request++;
  c->requests.emplace(id, std::move(req));
  *request_id = id;
  return w;
}

int lazyattn_cache_release(lazyattn_cache *c, int32_t request_id) {
  if (!c) return LAZYATTN_CACHE_ERR_ARG;
  auto it = c->requests.find(request_id);
  if (it == c->requests.end()) return LAZYATTN_CACHE_ERR_ARG;
  for (const Key *k : it->second.docs) c->drop(k);
  const std::vector<int32_t> &pb = it->second.prompt;
  for (auto b = pb.rbegin(); b != pb.rend(); ++b) c->free_list.push_back(*b);
  c->prompt_blocks -= (int64_t)pb.size();
  c->requests.erase(it);
  return LAZYATTN_CACHE_OK;
}

int lazyattn_cache_stats(const lazyattn_cache *c, int64_t *out, int n) {
  if (!c || !out || n < 0) return LAZYATTN_CACHE_ERR_ARG;
  const int64_t v[10] = {c->n_requests, c->doc_hits,      c->doc_misses,        c->tok_hits,
                         c->tok_misses, c->evicted,       (int64_t)c->free_list.size(),
                         c->doc_blocks, c->prompt_blocks, (int64_t)c->docs.size()};
  const int m = n < 10 ? n : 10;
  for (int i = 0; i < m; ++i) out[i] = v[i];
  return m;
}

}  // extern "C"
