/*
 * paged_attn.h -- C ABI of the paged-KV hot path for AMD Instinct MI355X
 * (gfx950): the KV block write and paged attention over a packed, unpadded
 * batch that mixes prefill, chunked-prefill and decode segments.
 *
 * Sources (web pages, by title):
 *   [NOTES01] "vLLM 学习笔记 01：一个请求在 vLLM 里的一生" -- section 1.4
 *             (computed vs. total tokens of a request), 1.5 (paged KV cache:
 *             16-token blocks, a per-request block table, physically scattered
 *             blocks), 1.6 (forward pass over an unpadded batch: segment
 *             bounds, the slot mapping and the block tables are handed to the
 *             attention operator), 2.1 (chunked prefill), 2.2 (prefix caching:
 *             full blocks shared by several requests).
 *   [INSIDE]  Chinese translation of "Inside vLLM: Anatomy of a
 *             High-Throughput LLM Inference System", engine-constructor part:
 *             block bytes = 2 * block_size * kv_heads * head_size * dtype_bytes.
 *
 * Conventions shared by every entry point
 *   - Tensors are bf16 (2-byte) unless stated; index arrays are int32.
 *   - The KV pool ("kv_cache") is [num_blocks, 2, 16, num_kv_heads, head_dim]
 *     bf16, contiguous: axis 1 index 0 = keys, 1 = values.  A block is
 *     paged_kv_block_bytes(16, Hkv, D, 2) bytes.
 *   - A slot is block * 16 + position; -1 means "no slot".
 *   - Device pointers are owned by the caller and must stay valid until the
 *     work enqueued on `stream` has finished.  Calls never synchronise the
 *     device, never read device memory on the host and never allocate.
 *   - Supported: head_dim 64 or 128; num_q_heads = G * num_kv_heads with
 *     1 <= G <= 16.
 *   - Return value: PAGED_OK, or a PAGED_E* code with a message available from
 *     paged_last_error() (thread-local, valid until the next failing call on
 *     the same thread).  Metadata that breaks the preconditions below is never
 *     a reason to touch memory outside the buffers: kernels skip such
 *     segments, slots and blocks and record it in the workspace status word
 *     (see paged_attention_device_status); paged_validate reports it exactly.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PAGED_OK = 0,
  PAGED_EINVAL = 1,       /* null pointer, negative count, bad shape, workspace too small */
  PAGED_EUNSUPPORTED = 2, /* head_dim or group size outside what is built */
  PAGED_EHIP = 3          /* a HIP runtime call or launch failed */
};

/* Bytes of one KV block for one layer: K and V of block_size slots for every
 * KV head ([INSIDE], block size formula).  Pure function; returns 0 when any
 * argument is not positive. */
size_t paged_kv_block_bytes(int32_t block_size, int32_t num_kv_heads,
                            int32_t head_dim, int32_t dtype_bytes);

/* KV block write ([NOTES01] section 1.6, slot mapping).
 *
 * For each token t in [0, num_tokens) with s = slot_mapping[t] != -1:
 *   kv_cache[s / 16, 0, s % 16, :, :] = k[t]   and
 *   kv_cache[s / 16, 1, s % 16, :, :] = v[t]   (bit copy).
 * k, v: bf16 rows of num_kv_heads * head_dim contiguous elements, token t at
 * element offset t * k_token_stride (v_token_stride).  Slots must be unique
 * within one call and in [0, num_blocks * 16); slots outside that range are
 * skipped (no write) and flagged by paged_validate.  Repeated slots give an
 * unspecified one of the rows.  kv_cache is updated in place; k, v and
 * slot_mapping are read only.  Enqueued on `stream`. */
int paged_kv_write(const void* k, const void* v, const int32_t* slot_mapping,
                   void* kv_cache, int32_t num_tokens, int32_t num_kv_heads,
                   int32_t head_dim, int64_t num_blocks, int64_t k_token_stride,
                   int64_t v_token_stride, hipStream_t stream);

/* Workspace bytes paged_attention needs for these shape bounds.
 * max_blocks_per_seq bounds every seq_len as max_blocks_per_seq * 16;
 * num_tokens bounds every segment's new tokens.  num_kv_heads is needed
 * because the decode partition size is chosen from the number of
 * (segment, partition, KV head) work items, and the partials the workspace
 * holds scale with the number of partitions.  The result depends on these
 * arguments and on the calling thread's paged_attention_set_partition_tokens
 * setting only (0 by default); a call made on the same thread with the same
 * arguments and setting is satisfied by it.  Returns 0 for negative sizes. */
size_t paged_attention_workspace_size(int32_t num_seqs, int32_t num_tokens,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_blocks_per_seq);

/* Paged attention over a packed batch ([NOTES01] sections 1.4-1.6, 2.1, 2.2).
 *
 * Segment s owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1]) of q and of
 * out: n = cu_seqlens_q[s+1] - cu_seqlens_q[s] new tokens of a sequence of
 * L = seq_lens[s] tokens whose K/V (all L of them, the new ones included,
 * written beforehand with paged_kv_write) sit in the blocks
 * block_tables[s, 0 .. ceil(L/16) - 1].  Query row i of the segment (absolute
 * position L - n + i) attends to keys 0 .. L - n + i of its own sequence only;
 * query head h uses KV head h / (num_q_heads / num_kv_heads).
 *   out[row, h, :] = sum_j softmax_j(scale * q[row, h, :] . K[j, h/G, :]) V[j, h/G, :]
 * computed with fp32 accumulation and rounded to bf16 (nearest even).
 *
 * q, out: [num_tokens, num_q_heads, head_dim] bf16, row r at element offset
 * r * q_token_stride (q) and r * num_q_heads * head_dim (out).  block_tables:
 * int32 [num_seqs, max_blocks_per_seq] row-major; entries past ceil(L/16) are
 * never read.  cu_seqlens_q: int32 [num_seqs + 1], non-decreasing from 0 to
 * at most num_tokens.  seq_lens: int32 [num_seqs] with n <= L <=
 * max_blocks_per_seq * 16.  PAGED_EINVAL when num_tokens / 32 + num_seqs
 * reaches 2^20 (about 33 M tokens in one call).  Segments with n = 0 are skipped; rows of out that
 * belong to no segment are left untouched.  The K/V pool is read only at
 * (block, position) pairs below each L.  out must not alias q or kv_cache.
 *
 * workspace: device memory of at least paged_attention_workspace_size(...)
 * bytes, owned by the caller; its contents need no initialisation and are
 * scratch between calls (the first 256 bytes hold the status word read by
 * paged_attention_device_status).  Two calls that share a workspace must be
 * ordered on one stream.  Enqueued on `stream`; no host synchronisation, no
 * device-to-host copy, so the call can be captured in a HIP graph. */
int paged_attention(const void* q, const void* kv_cache,
                    const int32_t* block_tables, const int32_t* cu_seqlens_q,
                    const int32_t* seq_lens, float scale, void* out,
                    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                    int32_t max_blocks_per_seq, int64_t q_token_stride,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* paged_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, result and kernels as
 * paged_attention minus the workspace: its scratch (work lists, decode
 * partials, the status word) is an array of PAGED_NOALLOC_SCRATCH_BYTES
 * bytes that the library holds on every GPU it runs on until the process
 * ends.  The call allocates nothing (no hipMalloc, no hipFree, no allocating
 * library routine); on its first call on a device it looks up that device's
 * array (hipGetSymbolAddress), with the device current.
 * Limits and errors: PAGED_EINVAL, with no work enqueued, when
 * paged_attention_workspace_size(num_seqs, num_tokens, num_q_heads,
 * num_kv_heads, head_dim, max_blocks_per_seq) on the calling thread exceeds
 * PAGED_NOALLOC_SCRATCH_BYTES (use paged_attention with a workspace then);
 * otherwise as paged_attention.  Every call on one GPU uses the same array
 * and leaves its contents behind (the plan kernel rewrites what must start
 * at zero, so nothing needs clearing): two calls that overlap on one GPU --
 * on different streams, or from threads that do not order their streams --
 * race and give undefined results.  Order them on one stream.  The status
 * word of skipped metadata is not exposed; paged_validate checks metadata. */
#define PAGED_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int paged_attention_noalloc(const void* q, const void* kv_cache,
                            const int32_t* block_tables, const int32_t* cu_seqlens_q,
                            const int32_t* seq_lens, float scale, void* out,
                            int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                            int32_t max_blocks_per_seq, int64_t q_token_stride,
                            hipStream_t stream);

/* Metadata of a steady-state decode step, on the device ([NOTES01] sections
 * 1.4 and 1.6): every one of the num_seqs segments gains one new token at
 * position L = seq_lens[s] (its current length).  In place on `stream`:
 *   seq_lens[s]      = L + 1
 *   cu_seqlens_q[s]  = s, cu_seqlens_q[num_seqs] = num_seqs
 *   slot_mapping[s]  = block_tables[s][L / 16] * 16 + L % 16, or -1 when
 *                      L / 16 >= max_blocks_per_seq or that entry is outside
 *                      [0, num_blocks) (paged_kv_write then skips the token
 *                      and paged_attention flags the block).
 * The caller keeps each table holding the blocks of the positions to come
 * (a block manager allocates them ahead).  With it, a decode step --
 * paged_decode_advance, paged_kv_write, paged_attention -- reads no host
 * metadata and can be captured once in a HIP graph and replayed.  All
 * pointers are device pointers: seq_lens, cu_seqlens_q ([num_seqs + 1]) and
 * slot_mapping ([num_seqs]) are written; block_tables is read.  No
 * allocation, no synchronisation. */
int paged_decode_advance(int32_t* seq_lens, int32_t* cu_seqlens_q, int32_t* slot_mapping,
                         const int32_t* block_tables, int32_t num_seqs,
                         int32_t max_blocks_per_seq, int64_t num_blocks, hipStream_t stream);

/* Debug check of the metadata preconditions of paged_kv_write and
 * paged_attention.  Synchronises `stream`, copies the index arrays to the
 * host and returns PAGED_OK or PAGED_EINVAL with the first violation in
 * paged_last_error().  Pass slot_mapping = NULL to skip the slot checks, or
 * block_tables = NULL to skip the attention checks.  Never on a timed path. */
int paged_validate(const int32_t* slot_mapping, int32_t num_new_tokens,
                   const int32_t* block_tables, const int32_t* cu_seqlens_q,
                   const int32_t* seq_lens, int32_t num_seqs, int32_t num_tokens,
                   int64_t num_blocks, int32_t max_blocks_per_seq,
                   hipStream_t stream);

/* Reads the status word the last paged_attention call on this workspace left
 * (synchronises `stream`): 0, or a bit set of PAGED_STATUS_* for metadata the
 * kernels skipped. */
enum {
  PAGED_STATUS_BAD_SEGMENT = 1, /* cu_seqlens_q / seq_lens out of range: segment skipped */
  PAGED_STATUS_BAD_BLOCK = 2    /* a block id outside the pool: its keys were left out */
};
int paged_attention_device_status(const void* workspace, uint32_t* status,
                                  hipStream_t stream);

/* Tokens per decode partition: 0 = automatic (the default), otherwise a
 * multiple of 32 in [32, 2048].  A tuning knob for measurements; it changes
 * only the split of long decode contexts, not the result beyond rounding.
 * It applies to the later paged_attention and paged_attention_workspace_size
 * calls of the calling thread only (other threads keep their own setting; a
 * smaller partition needs a larger workspace, so size the workspace after
 * setting it).  Returns PAGED_EINVAL for other values. */
int paged_attention_set_partition_tokens(int32_t tokens);

/* Most members of a shared-prefix group ("vLLM 学习笔记 01", section 2.2:
 * requests with a common cached prefix hold the same blocks).  Single-token
 * decode segments whose leading full partitions list the same block ids are
 * grouped, wherever they sit among the call's first 1024 segments,
 * and a group reads each shared partition once for all its members instead
 * of once per member.  0 = automatic (the default:
 * min(8, 32 / G) members), 1 = no grouping, 2..8 = at most that many (never
 * more than 32 / G).  Results are bitwise the same either way; a knob for
 * measurements.  It applies to the later calls of the calling thread only;
 * returns PAGED_EINVAL for other values. */
int paged_attention_set_group_members(int32_t members);

/* Measurement hook: when `count` is 5, every later paged_attention call on
 * this thread records events[0] before its first kernel and events[1..4]
 * after the plan, decode, decode-merge and prefill kernels, on the call's
 * stream, so a caller can read each stage's duration with
 * hipEventElapsedTime.  A NULL entry leaves that point unrecorded (each
 * record adds a few microseconds between kernels, so a caller timing one
 * kernel records only the two events around it).  The handles are
 * hipEvent_t values created by the caller, who keeps them alive while calls
 * use them.  count = 0 (or events = NULL) switches it off.  Returns
 * PAGED_EINVAL for other counts or five NULL entries. */
int paged_attention_set_stage_events(void* const* events, int32_t count);

const char* paged_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
