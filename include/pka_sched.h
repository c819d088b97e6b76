/*
 * pka_sched.h - host-side producer of the paged attention calls' metadata.
 *
 * The steps just before the attention path: a page allocator over the KV pool,
 * a prefix cache that lets a new request reuse the pool pages of an earlier
 * request's identical prefix, and a batch builder that splits prompts into chunks
 * and emits, for one prefill or one decode call, the arrays pka_store_kv,
 * pka_paged_attn_prefill and pka_paged_attn_decode(_store) take: page_table,
 * seq_lens, prefix_lens, extend_lens, cu_extend and out_loc (include/pka.h).
 *
 * What the pages fix, and where:
 *  - The pool is one store every request allocates from; its smallest allocation
 *    unit is a page of page_size tokens (default 1) ["Mini-SGLang deployment guide"
 *    (dpshk.com), section 6.2 "Page Size"; "miniSGLang intro blog" (0539edu.com),
 *    section 1.2, KV cache module: a pool and a manager].
 *  - The cache manager is either a radix tree that shares prefixes across requests
 *    or a naive one that shares nothing [deployment guide, section 6.5 "Radix
 *    Cache"].
 *  - Long prompts are prefilled in chunks; the tokens one forward pass may extend
 *    are capped (max-prefill-length, 8192 by default) [deployment guide, section 6.1
 *    "Chunked Prefill"; intro blog, section 1.2].
 *
 * Readings of what the pages leave open (the pages give no algorithm):
 *  - Prefixes are shared in whole pages only. A new request reuses the longest
 *    cached prefix of its prompt made of whole pages, but never its last prompt
 *    token (at least one token is computed, as its output is needed).
 *  - Eviction is least-recently-used over leaf pages (a cached page no cached page
 *    extends) that no live request holds, one page at a time, and only when the
 *    free list is empty. A page's last use is the latest match or insertion that
 *    covered it; each admission and each finish is one tick of the clock.
 *  - A request's pages join the cache when it finishes: the whole pages of every
 *    token whose K/V is in the pool. Pages whose content is already cached (another
 *    request got there first) and the last partial page go back to the free list.
 *  - A prefill batch serves requests first-come first-served: those part-way
 *    through their prompt first, then new ones, each with the largest chunk that
 *    fits the token budget and the free pages; a request that gets no page waits.
 *
 * Threading: a scheduler object is not thread-safe; one thread drives it.
 * Memory: every array argument is a host pointer owned by the caller; the
 * scheduler owns only its internal state (freed by pka_sched_destroy).
 * Errors: negative status codes of include/pka.h, plus PKA_E_STATE,
 * PKA_E_CAPACITY and PKA_E_NOMEM below. A call that fails with any code but
 * PKA_E_NOMEM changes nothing.
 */
#ifndef PKA_SCHED_H
#define PKA_SCHED_H

#include <stdint.h>

#include "pka.h"

#ifdef __cplusplus
extern "C" {
#endif

#define PKA_E_STATE (-6)    /* unknown request id, duplicate id, or wrong request state */
#define PKA_E_CAPACITY (-7) /* an output array or a page-table row is too small */
#define PKA_E_NOMEM (-8)    /* host memory ran out; the scheduler must be destroyed */

#define PKA_CACHE_NAIVE 0 /* no prefix sharing */
#define PKA_CACHE_RADIX 1 /* radix-tree prefix sharing */

typedef struct pka_sched pka_sched; /* opaque */

/* Output of one batch call. The caller sets the four capacities and the array
 * pointers (host memory); the call fills the arrays and the four counts.
 *   req_ids      [max_batch]               request id of row b
 *   page_table   [max_batch * table_width] page ids, row b = request b; entries past
 *                                          ceil(seq_lens[b] / page_size) are not written
 *                                          (no attention call reads them)
 *   seq_lens, prefix_lens, extend_lens  [max_batch]
 *   cu_extend    [max_batch + 1]           exclusive prefix sums of extend_lens
 *   out_loc      [max_tokens]              slot of every new token, rows in order
 * A decode batch has extend_lens = 1 and prefix_lens = seq_lens - 1 for every row. */
typedef struct pka_batch {
  int32_t max_batch;
  int32_t table_width;
  int32_t max_tokens;
  int32_t reserved;
  int64_t* req_ids;
  int32_t* page_table;
  int32_t* seq_lens;
  int32_t* prefix_lens;
  int32_t* extend_lens;
  int32_t* cu_extend;
  int32_t* out_loc;
  int32_t batch;       /* rows written */
  int32_t num_tokens;  /* new tokens (sum of extend_lens) */
  int32_t max_extend;  /* largest extend_lens entry (0 if batch == 0) */
  int32_t max_seq_len; /* largest seq_lens entry (0 if batch == 0) */
} pka_batch;

typedef struct pka_sched_stats {
  int64_t free_pages;     /* on the free list */
  int64_t cached_pages;   /* held by the prefix cache */
  int64_t locked_pages;   /* cached pages a live request holds (not evictable) */
  int64_t private_pages;  /* held by live requests outside the cache */
  int64_t evicted_pages;  /* evicted since creation */
  int32_t waiting;        /* requests not yet admitted */
  int32_t prefilling;     /* admitted, prompt not complete */
  int32_t running;        /* prompt complete (decoding) */
  int32_t reserved;
} pka_sched_stats;

/* Create a scheduler over a pool of num_pages pages of page_size tokens.
 *   cache_policy        PKA_CACHE_NAIVE or PKA_CACHE_RADIX
 *   max_prefill_tokens  token budget of one prefill batch (the chunk size), >= 1
 * Returns PKA_OK and *out, or PKA_E_SHAPE / PKA_E_NULLPTR. */
int pka_sched_create(int32_t page_size, int64_t num_pages, int32_t cache_policy,
                     int32_t max_prefill_tokens, pka_sched** out);

/* Destroy a scheduler (NULL is a no-op). */
void pka_sched_destroy(pka_sched* s);

/* Queue a new request with its prompt tokens[0 .. n-1] (n >= 1; the tokens are
 * copied). PKA_E_STATE if req_id is already live. */
int pka_sched_add_request(pka_sched* s, int64_t req_id, const int32_t* tokens, int32_t n);

/* Build the next prefill batch (chunked prefill over cached prefixes). New requests
 * are admitted here: matched against the cache and their matched pages locked. Each
 * row's new tokens are counted as stored; the caller runs pka_store_kv and
 * pka_paged_attn_prefill with the arrays. The batch holds at most max_batch rows and
 * min(max_prefill_tokens, max_tokens) new tokens; batch == 0 when nothing fits.
 * PKA_E_CAPACITY if a queued prompt needs more than table_width pages (nothing
 * changes). */
int pka_sched_prefill_batch(pka_sched* s, pka_batch* out);

/* Give a running request (prompt complete) its next input token, i.e. the token
 * sampled from its last output. PKA_E_STATE if the request is not running or already
 * has a pending token. */
int pka_sched_push_token(pka_sched* s, int64_t req_id, int32_t token);

/* pka_sched_push_token for n requests at once (one call per decode step): request
 * req_ids[i] gets tokens[i]. All or nothing: PKA_E_STATE (and no change) if any id is
 * unknown, not running, already pending or listed twice. */
int pka_sched_push_tokens(pka_sched* s, const int64_t* req_ids, const int32_t* tokens,
                          int32_t n);

/* Build the next decode batch: every running request with a pending token, in the
 * order their prompts completed, each getting the slot of its new token (a new page
 * when it starts one). A request that gets no page, or finds the batch full
 * (max_batch rows or max_tokens tokens), waits for a later batch.
 * PKA_E_CAPACITY if a row would pass table_width (nothing changes). */
int pka_sched_decode_batch(pka_sched* s, pka_batch* out);

/* Retire a request in any state: its whole pages join the prefix cache (radix
 * policy) and its other pages return to the free list. A batch counts its rows' new
 * tokens as stored when it is built, so finish a request only after the store of the
 * last batch that extended it has run (or been ordered before any later use of the
 * pool on the same stream); otherwise the cache would hold pages never written. */
int pka_sched_finish(pka_sched* s, int64_t req_id);

/* Current page-table row of a live request: pages[0 .. *n_pages - 1] hold its
 * tokens 0 .. cached-1 (and the pages of any in-flight chunk); *cached is the number
 * of its tokens whose K/V the scheduler counts as stored. cap = capacity of pages. */
int pka_sched_request_pages(const pka_sched* s, int64_t req_id, int32_t* pages, int32_t cap,
                            int32_t* n_pages, int32_t* cached);

/* Counters of pages and requests. */
int pka_sched_get_stats(const pka_sched* s, pka_sched_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* PKA_SCHED_H */
