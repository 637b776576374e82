/*
 * paged_block_manager.h -- C ABI of the host-side KV block manager that
 * produces the block tables and slot mappings the paged-KV calls of
 * paged_attn.h consume.  Plain C++ on the CPU; no GPU work.
 *
 * Sources (web pages, by title):
 *   [NOTES01] "vLLM 学习笔记 01：一个请求在 vLLM 里的一生" -- section 1.4
 *             (each request counts computed and total tokens; the scheduler
 *             asks the KV cache manager for slots and preempts when blocks run
 *             out), 1.5 (16-token blocks, one block table per request, free
 *             blocks in a doubly linked queue taken and returned in constant
 *             time, a request takes one more block when it grows and returns
 *             all of them when it ends), 2.2 (prefix caching: every full block
 *             is keyed by a hash of the previous block's hash and its own
 *             tokens, plus extra keys when needed; a new request reuses its
 *             longest cached prefix; a block returned to the free queue keeps
 *             its content and hash until it is taken for new content; shared
 *             blocks are reference counted; partly filled blocks are never
 *             cached).
 *
 * Model.  A manager owns block ids [0, num_blocks) of one KV pool.  A request
 * (a caller-chosen int64 id) has known tokens (its prompt, then the tokens
 * appended as they are generated), a block table, and `computed`, the number
 * of leading tokens that have slots (allocated for a step).  Policies where
 * the pages leave the choice open:
 *   - new blocks come from the head of the free queue; released blocks go to
 *     its tail, a request's blocks in reverse table order (its last block
 *     first), so cached prefixes, which later blocks' hashes chain on, are
 *     reused last;
 *   - a cached prefix is matched only when a request has no block yet (at its
 *     first allocation) and covers at most (known tokens - 1) / 16 full
 *     blocks, so at least one token is always computed;
 *   - a block becomes a cache entry when a step's allocation fills it (its
 *     16 tokens are known); if an entry for the same content exists, the
 *     new block stays out of the cache;
 *   - the hash is FNV-1a (64-bit) over the parent hash, the request's salt
 *     (e.g. an adapter id; the pages' extra keys) and the 16 tokens, all
 *     little-endian; a match also compares the stored parent hash, salt and
 *     tokens, so only a 64-bit collision of the parent chain can alias.
 *
 * Return values: PAGED_BM_OK, or a PAGED_BM_E* code with a message from
 * paged_bm_last_error() (thread-local).  A manager is not thread-safe: calls
 * on one manager must not overlap.  All pointers are host pointers owned by
 * the caller.
 */
#ifndef PAGED_BLOCK_MANAGER_H
#define PAGED_BLOCK_MANAGER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PAGED_BM_OK = 0,
  PAGED_BM_EINVAL = 1,  /* null pointer, bad count, unknown or duplicate request id */
  PAGED_BM_ENOSPACE = 4 /* not enough free blocks: nothing was changed (the caller preempts) */
};

typedef struct paged_bm paged_bm;

/* A manager of num_blocks 16-token blocks, all free; prefix caching on when
 * enable_prefix_caching != 0.  Returns NULL for num_blocks outside
 * [1, 2^31 / 16). */
paged_bm* paged_bm_create(int64_t num_blocks, int32_t enable_prefix_caching);
void paged_bm_destroy(paged_bm* bm);

/* Registers request `req` with its n >= 1 known tokens (the prompt) and a
 * salt mixed into its blocks' cache keys.  No block is taken yet. */
int paged_bm_add_request(paged_bm* bm, int64_t req, const int32_t* tokens, int32_t n,
                         int64_t salt);

/* Appends n >= 0 known tokens (generated ones) to request `req`. */
int paged_bm_append_tokens(paged_bm* bm, int64_t req, const int32_t* tokens, int32_t n);

/* *num_cached = the tokens of `req` whose K/V the next allocation will not
 * compute: the cached prefix it would match (a multiple of 16) while it has no
 * block, else its computed count.  Read only; valid until the next call that
 * allocates or releases blocks. */
int paged_bm_num_cached_tokens(const paged_bm* bm, int64_t req, int32_t* num_cached);

/* Slots for the next num_new tokens of `req` ([NOTES01] 1.4, allocate_slots):
 * at its first allocation it first takes its cached prefix (reference
 * counts +1, leaving the free queue if they were free), then takes
 * ceil((computed + num_new) / 16) - (table length) blocks from the free
 * queue's head (dropping their cache entries), writes the num_new slots
 * (block * 16 + position) of positions computed .. computed + num_new - 1
 * to slots (may be NULL), advances computed and caches the blocks that are
 * now full.  computed + num_new must not exceed the known tokens.  Returns
 * PAGED_BM_ENOSPACE, changing nothing, when the free queue is too short. */
int paged_bm_allocate_slots(paged_bm* bm, int64_t req, int32_t num_new, int32_t* slots);

/* Ends `req`: each of its blocks, last first, loses one reference and
 * joins the free queue's tail at zero (content and cache entry kept). */
int paged_bm_free_request(paged_bm* bm, int64_t req);

/* The first min(max_entries, table length) entries of `req`'s block table;
 * *num_entries = the table length. */
int paged_bm_block_table(const paged_bm* bm, int64_t req, int32_t* table, int32_t max_entries,
                         int32_t* num_entries);

/* Metadata of one step over num_seqs requests in packing order, each having
 * just been given num_new[s] slots: block_tables [num_seqs, width] (rows
 * padded with -1), cu_seqlens_q [num_seqs + 1], seq_lens [num_seqs] (the
 * computed count, L) and slot_mapping [sum num_new] (slots of positions
 * L - num_new .. L - 1, in packing order): exactly the inputs of
 * paged_kv_write and paged_attention.  PAGED_BM_EINVAL if a table is wider
 * than width or num_new[s] exceeds L. */
int paged_bm_step_metadata(const paged_bm* bm, const int64_t* reqs, const int32_t* num_new,
                           int32_t num_seqs, int32_t width, int32_t* block_tables,
                           int32_t* cu_seqlens_q, int32_t* seq_lens, int32_t* slot_mapping);

/* Counters for callers and tests. */
int64_t paged_bm_num_free_blocks(const paged_bm* bm);
int64_t paged_bm_num_cached_blocks(const paged_bm* bm); /* cache entries (free or in use) */
int32_t paged_bm_ref_count(const paged_bm* bm, int64_t block); /* -1 for a bad id */
/* The free queue from head to tail: the first min(max_ids, length) ids;
 * returns the length. */
int64_t paged_bm_free_queue(const paged_bm* bm, int32_t* ids, int64_t max_ids);

const char* paged_bm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_BLOCK_MANAGER_H */
