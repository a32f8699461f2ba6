/*
 * lazyattn_cache.h -- host-side manager of the paged, position-free KV pool:
 * the step before the attention kernels, which turns "this request reads
 * documents d0, d1, ... then a prompt" into a block-table row.
 *
 * Sources (the pages):
 *  - ai-engineering.academy, "KV Cache, Flash Attention & Otimização de
 *    Inferência", section "PagedAttention": the KV cache lives in 16-token
 *    blocks and a page table maps logical positions to physical blocks;
 *    "Exercícios" 3: a free list of blocks, to which a finished sequence's
 *    blocks return.
 *  - gist.science, "Resumo Técnico: LazyAttention", "Declaração do Problema"
 *    and "Metodologia": a position-aware cache can reuse a document only at
 *    the position it was encoded for (or by storing another, re-encoded copy);
 *    a position-agnostic cache stores each document once, by content, and one
 *    physical copy serves any position (zero-copy reuse).  "Resultados
 *    Experimentais" reports hit rates under a KV memory budget.
 *
 * This is host code: plain C++ on the CPU, no device memory and no HIP calls.
 * It owns only its bookkeeping; the K/V pool itself is the caller's device
 * memory, [num_blocks][num_kv_heads][16][head_dim] per layer, and every layer's
 * pool shares the block ids this manager hands out.
 *
 * Documents are the unit of reuse: a document id plus its length in tokens (a
 * whole number of 16-token blocks).  A request places its documents one after
 * another from position 0, then its prompt; each block's table word is
 * (block id | frame start position << 16), the format lazyattn_decode and
 * lazyattn_prefill read.  A document's frame starts at its placement position;
 * the prompt's frame at the prompt's first position.
 *
 * Cache keys (the policy under comparison, `mode`):
 *  LAZYATTN_CACHE_AGNOSTIC  key = document id.  Any placement reuses the one
 *                           stored copy (the LazyAttention cache).
 *  LAZYATTN_CACHE_AWARE     key = (document id, placement position).  A copy
 *                           serves only the position it was encoded for; the
 *                           same document at another position is a miss and
 *                           gets a copy of its own.
 *  LAZYATTN_CACHE_PREFIX    key = the request's whole document sequence up to
 *                           and including this document.  A document hits only
 *                           when everything before it in the request matches a
 *                           cached prefix.
 *
 * Eviction (not specified by the pages; this manager's reading): when a
 * request needs more blocks than are free, cached documents that no live
 * request references are evicted in least-recently-used order.  A document
 * referenced by a live request is never evicted.  Prompt blocks belong to
 * their request and return to the free list when it is released.
 *
 * Threading: a manager is not internally synchronised; one thread at a time.
 * Errors: negative status, state unchanged (an acquire that cannot fit rolls
 * back everything it took).
 */
#ifndef LAZYATTN_CACHE_H
#define LAZYATTN_CACHE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LAZYATTN_CACHE_AGNOSTIC = 0, LAZYATTN_CACHE_AWARE = 1, LAZYATTN_CACHE_PREFIX = 2 };

enum {
  LAZYATTN_CACHE_OK = 0,
  LAZYATTN_CACHE_ERR_ARG = -1,      /* NULL pointer, bad size or mode, unknown request, or a
                                       document named with another length than it is cached
                                       (or named earlier in the same request) with */
  LAZYATTN_CACHE_ERR_NOSPACE = -2,  /* not enough free + evictable blocks, or the table row is too short */
  LAZYATTN_CACHE_ERR_POSITION = -3  /* a frame start would not fit the 16-bit offset field */
};

typedef struct lazyattn_cache lazyattn_cache;

/* A manager for a pool of num_blocks blocks (1..65536), all free.  NULL on a
 * bad argument or allocation failure. */
lazyattn_cache *lazyattn_cache_create(int num_blocks, int mode);
void lazyattn_cache_destroy(lazyattn_cache *c);

/*
 * Place one request: documents doc_ids[i] of doc_lens[i] tokens (i < n_docs;
 * lengths > 0 and multiples of 16), then a prompt of prompt_len >= 0 tokens.
 * Outputs (caller-owned host arrays):
 *   table_row[max_blocks]  the request's table words, blocks in logical order
 *                          (documents, then the prompt); entries past the
 *                          returned count are left untouched
 *   miss[n_docs]           1 where the document's blocks were newly allocated
 *                          (the caller must write their K/V, encoded in the
 *                          document's own frame), 0 where they were reused
 *   request_id             handle for lazyattn_cache_release
 * Returns the number of table words written (>= 0) or a negative status;
 * on a negative status nothing is placed and no output is written.  A
 * document's length is part of its identity: naming a cached document (or
 * one named earlier in the same request) with another length is
 * LAZYATTN_CACHE_ERR_ARG.
 * The request holds a reference on each of its documents until released.
 */
int lazyattn_cache_acquire(lazyattn_cache *c, const int32_t *doc_ids, const int32_t *doc_lens, int n_docs,
                           int prompt_len, uint32_t *table_row, int max_blocks, uint8_t *miss,
                           int32_t *request_id);

/* Drop a request's references (its documents stay cached, now evictable) and
 * free its prompt blocks. */
int lazyattn_cache_release(lazyattn_cache *c, int32_t request_id);

/*
 * Counters since creation, into out[n] (n <= 10):
 *   0 requests  1 document hits  2 document misses  3 tokens hit  4 tokens missed
 *   5 documents evicted  6 free blocks  7 blocks held by cached documents
 *   8 blocks held by prompts  9 cached documents
 * Returns the number written.
 */
int lazyattn_cache_stats(const lazyattn_cache *c, int64_t *out, int n);

#ifdef __cplusplus
}
#endif

#endif /* LAZYATTN_CACHE_H */
