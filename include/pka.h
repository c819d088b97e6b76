/*
 * pka.h - paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels. Three operations form one serving step
 * of a paged KV cache:
 *
 *   pka_store_kv            new K/V rows -> their slots in the K/V pools
 *   pka_paged_attn_prefill  causal extend (chunked) prefill on top of a cached prefix
 *   pka_paged_attn_decode   batched GQA decode, split over the key axis, then merged
 *                           (small calls: one launch, merged on chip)
 *
 * and pka_paged_attn_decode_store, a decode step's store and decode in one launch.
 *
 * The pages this follows describe a pool shared by all requests whose
 * allocation unit is a page of page_size tokens (default 1) ["Mini-SGLang
 * deployment guide" (dpshk.com), section 6.2 "Page Size" and section 6.5 "Radix
 * Cache"]; attention that reads the pool's history together with the freshly
 * computed K/V, finding each request's tokens through a page table and position
 * metadata ["miniSGLang intro blog" (0539edu.com), section 1.3 "forward
 * computation"]; prefill and decode served by different kernels, with chunked
 * prefill extending a cached prefix [deployment guide, sections 6.1 and 6.3;
 * "Mini-SGLang: Efficient Inference Engine in a Nutshell", section on integrated
 * high-performance kernels].
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every call
 * ---------------------------------------------------------------------------
 * Data types. bf16 tensors are passed as `void*` (16-bit bf16 bit patterns);
 *   index arrays are int32; the softmax scale is a float.
 * Memory. Every pointer argument is a device pointer to contiguous row-major
 *   memory owned by the caller. The library allocates and frees nothing. bf16
 *   tensors and workspaces start on a 16-byte boundary and int32 arrays on a 4-byte
 *   one (every hipMalloc or torch allocation does); a call given a pointer that
 *   does not returns PKA_E_UNSUPPORTED.
 * Pools. k_pool and v_pool are each [num_pages * page_size, Hkv, D] bf16: slot-major,
 *   one slot holds one token's K (or V) for all Hkv kv heads, and page p owns
 *   slots p*page_size .. p*page_size + page_size - 1.
 * Page table. page_table[b * page_table_stride + n] is the page holding logical
 *   tokens n*P .. n*P+P-1 of request b. Token j of request b therefore lives in
 *   slot page_table[b*stride + j/P]*P + j%P. Entries past ceil(L_b/P) are never read.
 * GQA. q head h reads kv head h / (Hq / Hkv) (contiguous groups).
 * Streams. `stream` is a hipStream_t (NULL = the default stream). Every call only
 *   enqueues work: it never waits for the device and never copies device data to
 *   the host, so a sequence of calls can be captured into a HIP graph.
 * Order. Attention reads the new tokens' K/V from the pools, so store the step's
 *   new tokens with pka_store_kv first, on the same stream.
 * Errors. Host-side arguments (pointers, sizes, geometry) are checked before
 *   anything is enqueued; on error the call returns a negative status and enqueues
 *   nothing. A failed launch returns PKA_E_HIP. Device-resident metadata (page ids,
 *   slots, lengths) is not read by the host. A page id or slot outside the pool, or
 *   a page-table index past the row, is never dereferenced: store_kv skips such a
 *   row, attention reads a slot inside the pool instead, so the affected results are
 *   unspecified but no out-of-bounds access occurs.
 * Aliasing. out must not overlap q, the pools or the workspace; new K/V must not
 *   overlap the pools. Requests may share read-only prefix pages, but the slots the
 *   step writes must belong to one request only and must be pairwise distinct.
 */
#ifndef PKA_H
#define PKA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define PKA_OK 0
#define PKA_E_NULLPTR (-1)     /* a required pointer is NULL */
#define PKA_E_SHAPE (-2)       /* a size or geometry value is invalid */
#define PKA_E_UNSUPPORTED (-3) /* valid, but not supported by these kernels */
#define PKA_E_WORKSPACE (-4)   /* workspace missing or smaller than required */
#define PKA_E_HIP (-5)         /* the HIP runtime reported an error */
/* (-6 .. -8 are the scheduler's, in pka_sched.h) */
#define PKA_E_SCRATCH (-9)     /* the call needs more than the static scratch holds */

/* Pool and head geometry, shared by all calls.
 *   num_q_heads  Hq >= 1, a multiple of num_kv_heads
 *   num_kv_heads Hkv >= 1
 *   head_dim     D; attention supports D == 128, store_kv any D with D % 8 == 0
 *   page_size    P >= 1 tokens per page
 *   num_pages    pages in each pool; the pools hold num_pages * P slots      */
typedef struct pka_geom {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int64_t num_pages;
} pka_geom;

/* Library version: major * 10000 + minor * 100 + patch. */
int pka_version(void);

/* Human-readable text for a status code (static storage; never NULL). */
const char* pka_status_string(int status);

/*
 * pka_store_kv - write the step's new K/V rows into their pool slots.
 *
 * The new keys and values of a step join the pool's history before attention
 * reads them [miniSGLang intro blog, section 1.3]; a slot is one token of one
 * page [deployment guide, section 6.2].
 *
 *   k_new, v_new  [num_tokens, Hkv, D] bf16 (device)
 *   out_loc       [num_tokens] int32 slot ids (device); slot out_loc[t] receives
 *                 row t. Slots must be pairwise distinct; a slot outside
 *                 [0, num_pages*P) is skipped.
 *   k_pool, v_pool  the pools (device), updated in place
 * The copy is bit-exact. num_tokens == 0 is a no-op returning PKA_OK.
 */
int pka_store_kv(const pka_geom* geom, const void* k_new, const void* v_new,
                 const int32_t* out_loc, int32_t num_tokens, void* k_pool, void* v_pool,
                 void* stream);

/*
 * pka_paged_attn_decode - one new token per request attends to all its keys.
 *
 * Batched decode over the paged pool [deployment guide, sections 6.2-6.4]. For
 * request b, q head h and kv head g = h / (Hq/Hkv):
 *   out[b,h,:] = softmax_j(scale * q[b,h,:] . K_b[j,g,:]) . V_b[j,g,:], j < L_b,
 * where K_b[j] is the pool row of token j of request b. L_b = seq_lens[b] counts
 * the new token, whose K/V must already be stored.
 *
 *   q             [batch, Hq, D] bf16 (device)
 *   page_table    [batch, page_table_stride] int32 page ids (device)
 *   seq_lens      [batch] int32, 1 <= L_b <= max_seq_len (device)
 *   max_seq_len   host-known upper bound of seq_lens; sets the number of wavefronts
 *                 that share the keys (keys past it are not attended)
 *   scale         softmax scale (usually 1/sqrt(D))
 *   out           [batch, Hq, D] bf16 (device)
 *   workspace     device scratch of at least
 *                 pka_decode_workspace_bytes(geom, batch, max_seq_len) bytes (may be
 *                 NULL when that size is 0). Contents on entry are ignored. Calls
 *                 that run concurrently must not share a workspace.
 * Supported: D == 128, Hq/Hkv <= 16, batch <= 4096 and
 * batch * Hkv * ceil(max_seq_len / 64) < 2^31 (else PKA_E_UNSUPPORTED).
 * batch == 0 is a no-op. When ceil(max_seq_len / 64) <= 8 and
 * batch * Hkv * ceil(max_seq_len / 64) <= 2048 the call is one launch that merges a
 * pair's key blocks on chip (the workspace is then not used); otherwise the keys of
 * the batch are split between persistent wavefronts and a second launch merges them.
 */
int pka_paged_attn_decode(const pka_geom* geom, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* page_table,
                          int32_t page_table_stride, const int32_t* seq_lens, int32_t batch,
                          int32_t max_seq_len, float scale, void* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes pka_paged_attn_decode needs for this geometry and plan. */
size_t pka_decode_workspace_bytes(const pka_geom* geom, int32_t batch, int32_t max_seq_len);

/*
 * pka_paged_attn_decode_store - the decode step's store and decode in one launch.
 *
 * The same result as pka_store_kv(k_new, v_new, out_loc, batch) followed by
 * pka_paged_attn_decode on the same stream, for a decode step whose one new token per
 * request has just been given a slot [deployment guide, sections 6.2-6.4]: the new
 * token's K/V rows are written to the pools and attended in the same pass.
 *
 *   k_new, v_new  [batch, Hkv, D] bf16 (device): request b's new token's rows
 *   out_loc       [batch] int32 (device): slot of request b's new token. A slot outside
 *                 [0, num_pages*P) is skipped, as in pka_store_kv.
 *   k_pool, v_pool  the pools (device), read and updated in place
 *   other arguments, workspace size and support as in pka_paged_attn_decode.
 * Every key, including key L_b - 1, is read from the pools: the wavefront that reads
 * request b's last key block first writes the new rows to slot out_loc[b] and then
 * issues that block's loads, which see its own stores, so where the page table maps
 * key L_b - 1 to slot out_loc[b] (the usual decode step) the new rows are what it
 * attends to. The slots in out_loc must be pairwise distinct and must not be read as
 * another request's keys in the same call (new tokens' slots are private to their
 * request); then the result equals the two calls' bit for bit in the pools and within
 * rounding order in out. The store of request b is made by the wavefront that reads its
 * last key block, so it needs L_b >= 1 (as decode does).
 */
int pka_paged_attn_decode_store(const pka_geom* geom, const void* q, const void* k_new,
                                const void* v_new, const int32_t* out_loc, void* k_pool,
                                void* v_pool, const int32_t* page_table,
                                int32_t page_table_stride, const int32_t* seq_lens,
                                int32_t batch, int32_t max_seq_len, float scale, void* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * pka_paged_attn_decode_store_noalloc - pka_paged_attn_decode_store without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 *
 * The same launch and result as pka_paged_attn_decode_store (pools bit for bit, out
 * identical); the split partials go to a static device array of the library instead
 * of a caller workspace. Every argument is as in pka_paged_attn_decode_store.
 *   Limit: the call's workspace need (pka_decode_workspace_bytes for the same geometry,
 *          batch and max_seq_len) must be at most 16 MiB, else PKA_E_SCRATCH and nothing
 *          is enqueued (e.g. Hq/Hkv = 16 at 1024 split wavefronts needs 16.9 MB).
 *   Device: the array's address is looked up on the first call on a device (make that
 *          call outside graph capture); the current device must be the stream's device
 *          (else PKA_E_HIP). Each device holds its own copy until the process ends.
 *   Sharing: every call on a device uses the same array, whose contents it overwrites
 *          (they are never read before being written), so calls that overlap on one
 *          device race; serialise them (one stream, or events between streams).
 * The call allocates and frees nothing.
 */
int pka_paged_attn_decode_store_noalloc(const pka_geom* geom, const void* q, const void* k_new,
                                        const void* v_new, const int32_t* out_loc, void* k_pool,
                                        void* v_pool, const int32_t* page_table,
                                        int32_t page_table_stride, const int32_t* seq_lens,
                                        int32_t batch, int32_t max_seq_len, float scale,
                                        void* out, void* stream);

/*
 * pka_paged_attn_prefill - causal extend prefill on top of a cached prefix.
 *
 * Chunked prefill [deployment guide, section 6.1] over a prefix reused from the
 * radix cache [deployment guide, section 6.5]. Request b has p_b = prefix_lens[b]
 * cached tokens and e_b = extend_lens[b] new tokens; L_b = seq_lens[b] = p_b + e_b.
 * New token i of request b (q row cu_extend[b] + i) sits at absolute position
 * p_b + i and attends to keys 0 .. p_b + i of its request (causal, aligned to the
 * end of the sequence). All L_b keys, including the new ones, are read from the
 * pools, so the new tokens must be stored first.
 *
 *   q             [num_tokens, Hq, D] bf16 (device); requests packed in batch order
 *   page_table    [batch, page_table_stride] int32 page ids (device)
 *   seq_lens, prefix_lens, extend_lens  [batch] int32 (device)
 *   cu_extend     [batch + 1] int32 exclusive prefix sums of extend_lens (device)
 *   num_tokens    host-known sum of extend_lens
 *   max_extend    host-known upper bound of extend_lens
 *   max_seq_len   host-known upper bound of seq_lens
 *   out           [num_tokens, Hq, D] bf16 (device)
 *   workspace     device scratch of at least
 *                 pka_prefill_workspace_bytes(geom, batch, num_tokens, max_extend) bytes
 *                 (may be NULL when that size is 0); it holds the dispatch order of the
 *                 launch's work items, written by the launch itself
 * Supported: D == 128. Requests with e_b == 0 produce no rows. batch == 0 or
 * num_tokens == 0 is a no-op. max_extend sets how many 256-row q tiles each request
 * gets: output rows of new tokens past max_extend may be left unwritten.
 */
int pka_paged_attn_prefill(const pka_geom* geom, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* page_table,
                           int32_t page_table_stride, const int32_t* seq_lens,
                           const int32_t* prefix_lens, const int32_t* extend_lens,
                           const int32_t* cu_extend, int32_t batch, int32_t num_tokens,
                           int32_t max_extend, int32_t max_seq_len, float scale, void* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes pka_paged_attn_prefill needs: 16 bytes per (request, 256-row q
 * tile) item when batch > 1 (the launch orders its work heaviest first there and
 * keeps each item's request lengths beside it), else 0. Contents on entry are
 * ignored; calls that run concurrently must not share it. */
size_t pka_prefill_workspace_bytes(const pka_geom* geom, int32_t batch, int32_t num_tokens,
                                   int32_t max_extend);

#ifdef __cplusplus
}
#endif

#endif /* PKA_H */
