/*
 * pagedattn.h - C ABI of the MI355X (gfx950) paged-decode library
 * (libpagedattn.so).
 *
 * Two operations, after the pages this library follows:
 *   [KVP]   "PagedAttention：KV Cache 的分页革命" (openeuler.csdn.net)
 *   [INFRA] "【infra之路】10-PagedAttention 与 KV Cache 管理" (jsqmd.com)
 *   [OPS]   the l189.com article on the ops-transformer PagedAttention
 *           operator for the Ascend NPU
 *
 * pa_reshape_and_cache writes each new token's K and V rows into the physical
 * slot named for it ([INFRA] §1.2: the step appends the new token's K and V to
 * the cache; §3.3: the token goes into the next slot of the request's last
 * block, a new block being appended to the table when that one is full).
 *
 * pa_decode is decode-phase attention over a paged cache ([INFRA] §1.1: the new
 * token's query of each head is scored against every cached key, scaled,
 * normalised by a softmax, and the weights average the cached values; §3.3 and
 * §3.4: the cached rows are found through the request's block table, which is
 * passed to the kernel, Q1 of §8).
 *
 * Layouts (all row-major, contiguous, element type `dtype`):
 *   q, out        [num_seqs, num_q_heads, head_dim]
 *   key, value    [num_tokens, num_kv_heads, head_dim]
 *   k_cache,
 *   v_cache       [num_blocks, num_kv_heads, block_size, head_dim]
 *                 (one (block, kv head) tile is block_size*head_dim contiguous
 *                 elements; K and V are separate pools, as [OPS] keeps the K
 *                 and V halves of a page apart)
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]; entry j of row s is
 *                 the physical block holding tokens j*block_size ..
 *                 j*block_size + block_size - 1 of sequence s
 *   context_lens  int32 [num_seqs]; tokens attended by each sequence
 *   slot_mapping  int32 [num_tokens]; slot = block * block_size + offset,
 *                 negative = write nothing for that token
 *
 * Query head h reads KV head h / (num_q_heads / num_kv_heads) (grouped-query
 * attention with contiguous groups; [INFRA] §2.1 names 8 KV heads for 32
 * query heads).
 *
 * Ownership and threading: every pointer argument is a device pointer owned by
 * the caller (except where stated). The library allocates, frees and
 * synchronises nothing; it keeps no state between calls. Work is enqueued on
 * `stream` (a hipStream_t; NULL is the null stream) and runs asynchronously.
 * Calls on different streams touching the same buffers race as any two
 * kernels would.
 *
 * Errors: arguments are checked on the host before anything is enqueued; on a
 * non-zero status nothing was enqueued (except PA_ERR_HIP, which reports a
 * launch failure). Values that live in device memory (table entries in
 * [0, num_blocks), 1 <= context_lens[s] <= max_context_len, distinct slots,
 * zero workspace counters) are preconditions; they are checked only when the
 * environment variable PA_DEBUG is set to a non-zero value, in which case the
 * call copies them to the host (synchronising the stream) and returns
 * PA_ERR_BAD_INDEX on a violation. A context length of 0 yields an all-zero
 * output row.
 *
 * Tuning (read once per process): PA_FLAT_WGS_PER_CU (a positive integer)
 * overrides the number of workgroups per compute unit of the balanced form
 * (default: as many as fit, at most 3). PA_FLAT_SEG_COST (0..1024) overrides
 * the tiles of overhead the balanced form charges each (sequence, KV head) when
 * it divides the work (default 4).
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
  PA_OK = 0,
  PA_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
  PA_ERR_BAD_SHAPE = 2,          /* a size is out of range or inconsistent */
  PA_ERR_UNSUPPORTED = 3,        /* head_dim, block_size, dtype or group not built */
  PA_ERR_WORKSPACE_TOO_SMALL = 4,
  PA_ERR_HIP = 5,                /* the HIP runtime reported an error */
  PA_ERR_BAD_INDEX = 6,          /* PA_DEBUG: a device-side precondition failed */
  PA_ERR_BAD_POINTER = 7,        /* memory the GPU cannot address (e.g. pageable host) */
  PA_ERR_SCRATCH_TOO_SMALL = 8   /* pa_decode_step_noalloc: the call needs more scratch
                                    than PA_NOALLOC_SCRATCH_BYTES */
};

/* Element types of q, out, key, value and the pools (all the same). */
enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 };

/*
 * pa_reshape_and_cache - copy new tokens' K/V rows into the pools.
 *
 * For every token t with slot = slot_mapping[t] >= 0, copies key[t, h, :] to
 * k_cache[slot / block_size, h, slot % block_size, :] and value[t, h, :] to
 * the same place of v_cache, for every KV head h. The copy is bit-exact (no
 * conversion). Slots must be distinct and < num_blocks * block_size (checked
 * under PA_DEBUG only).
 *
 * Supported: head_dim in {64, 128, 256}, block_size in {8, 16, 32, 64},
 * dtype in {PA_F32, PA_F16, PA_BF16}. num_tokens may be 0 (no launch).
 */
int32_t pa_reshape_and_cache(const void *key, const void *value, void *k_cache,
                             void *v_cache, const int32_t *slot_mapping,
                             int32_t num_tokens, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t dtype, void *stream);

/*
 * pa_decode_workspace_size - device scratch bytes pa_decode needs.
 *
 * partition_size selects the form of the decode (see pa_decode): 0 for the
 * balanced single launch, or a fixed partition size. Returns (size_t)-1 for
 * arguments pa_decode would reject. The workspace starts with one int32
 * arrival counter per (sequence, KV head); the balanced form needs them to be
 * zero when a call starts and leaves them zero when it ends, so a workspace
 * must be zero-filled once, before its first use. The fixed-partition form
 * never touches the counters, so one workspace may serve both forms.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t partition_size,
                                int32_t dtype);

/*
 * pa_decode - one decode step of paged attention.
 *
 * out[s, h, :] = sum_i p_i * V_s[i, :] with p = softmax(scale * K_s q[s, h]),
 * where K_s and V_s are the first context_lens[s] rows of KV head
 * h / (num_q_heads / num_kv_heads), gathered through block_tables[s].
 * Accumulation is float32; out is rounded once to `dtype` (nearest even).
 * Table entries past a sequence's last block are never used, and slots past
 * its context never contribute (entries are clamped into the pool, so no read
 * leaves it).
 *
 * The context is processed in pieces whose partial results are combined by a
 * log-sum-exp reduction (split-K in the manner of flash decoding, [INFRA] Q2
 * of §8). partition_size chooses how it is cut:
 *   0     balanced form (the default): one launch whose workgroups each take an
 *         equal share of all (sequence, KV head, 16-token tile) work, however
 *         unequal the context lengths; a (sequence, KV head) split between
 *         workgroups is combined by the last of them to finish. Used for
 *         num_seqs <= 4096 (and while that work stays below 2^31 tiles);
 *         beyond that the call falls back to fixed partitions of 256 tokens.
 *   P > 0 fixed partitions of P tokens (a multiple of 16, at most 4096): one
 *         workgroup per (partition, KV head, sequence), then a second launch
 *         combines the partitions.
 *
 * scale            the softmax scale (1/sqrt(head_dim) for standard attention)
 * max_context_len  max over s of context_lens[s] (host value)
 * workspace        device scratch of at least pa_decode_workspace_size(...)
 *                  bytes, zero-filled before its first use (see above); it
 *                  may be NULL only for the fixed form with max_context_len
 *                  <= partition_size (nothing to combine)
 *
 * Supported: head_dim in {64, 128, 256} (rows of at most 512 bytes, so not
 * 256 with PA_F32); block_size in {8, 16, 32, 64}; num_q_heads / num_kv_heads
 * in {1, 2, 4, 8}; dtype in {PA_F32, PA_F16, PA_BF16}; max_context_len <=
 * max_blocks_per_seq * block_size.
 */
int32_t pa_decode(void *out, const void *q, const void *k_cache,
                  const void *v_cache, const int32_t *block_tables,
                  const int32_t *context_lens, float scale, int32_t num_seqs,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t num_blocks,
                  int32_t max_blocks_per_seq, int32_t max_context_len,
                  int32_t partition_size, int32_t dtype, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * pa_decode_step - one whole decode step in a single launch: the cache write of
 * this step's tokens, then the attention (a decode step appends the new
 * token's K and V to the cache and attends over everything cached,
 * [INFRA] §1.2).
 *
 * Same result as pa_reshape_and_cache(key, value, k_cache, v_cache,
 * slot_mapping, num_seqs, ...) followed by pa_decode(..., partition_size = 0,
 * ...): the pools end with the new rows in place and `out` is bit-identical.
 * Token s of key/value [num_seqs, num_kv_heads, head_dim] belongs to sequence
 * s. Normally it is the sequence's last attended position: slot_mapping[s] is
 * the slot of position context_lens[s] - 1 (table entry (n-1)/block_size,
 * offset (n-1)%block_size), and the attention then reads that position's K/V
 * from key/value, not from the pool, so the write and the reads need no
 * ordering inside the launch. A token may also be written to a slot that no
 * sequence of the call attends (a fresh block past the context): the row is
 * written and not read. Any other slot (an attended position of another
 * sequence, or of its own other than the last) breaks the call's
 * preconditions; checked under PA_DEBUG only. slot_mapping[s] < 0 writes
 * nothing for that sequence (its last position is then read from the pools).
 *
 * Workspace as for pa_decode with partition_size 0 (zero-filled before its
 * first use). Beyond 4096 sequences the call writes first and then decodes
 * with fixed partitions (two launches).
 */
int32_t pa_decode_step(void *out, const void *q, const void *key,
                       const void *value, void *k_cache, void *v_cache,
                       const int32_t *slot_mapping, const int32_t *block_tables,
                       const int32_t *context_lens, float scale,
                       int32_t num_seqs, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks,
                       int32_t max_blocks_per_seq, int32_t max_context_len,
                       int32_t dtype, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Bytes of the static device scratch of pa_decode_step_noalloc (per GPU). */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * pa_decode_step_noalloc - pa_decode_step for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops that must not
 * call hipMalloc, harnesses that forbid it. No workspace argument: the decode's
 * scratch (counters and split partials) is a static device array of
 * PA_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library, one per GPU, held
 * until the process ends. The call allocates and frees nothing.
 *
 * Arguments, layouts, preconditions and the result are those of
 * pa_decode_step; out, the pools and key/value come out bit-identical to a
 * pa_decode_step call with a zero-filled workspace. The call enqueues a small
 * kernel that clears the counters, then the decode step, on `stream`.
 * Returns PA_ERR_SCRATCH_TOO_SMALL (nothing enqueued) when
 * pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
 * max_context_len, 0, dtype) exceeds PA_NOALLOC_SCRATCH_BYTES (e.g. 64
 * sequences of 8 KV heads, GQA-4, head_dim 128 need 5.3 MB), otherwise the
 * codes of pa_decode_step. The first call on a GPU looks up that GPU's copy
 * of the array (hipGetSymbolAddress); later calls reuse the address.
 *
 * Every call on one GPU shares its array: calls that overlap in time on that
 * GPU (on different streams, or from several host threads) race on it and
 * give wrong results; order them on one stream. PA_DEBUG checks copy to the
 * host and synchronise, so they must stay off under graph capture.
 */
int32_t pa_decode_step_noalloc(void *out, const void *q, const void *key,
                               const void *value, void *k_cache, void *v_cache,
                               const int32_t *slot_mapping,
                               const int32_t *block_tables,
                               const int32_t *context_lens, float scale,
                               int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq,
                               int32_t max_context_len, int32_t dtype,
                               void *stream);

/*
 * pa_copy_blocks - copy whole physical blocks inside the pools
 * (copy-on-write: several tables may point at one block, and a request about
 * to write into a shared block first takes a private copy of it, [INFRA] §4.3).
 *
 * block_mapping int32 [num_pairs, 2]: pair i makes block block_mapping[2i+1]
 * an exact copy of block block_mapping[2i], in k_cache and in v_cache (every
 * KV head, every slot: num_kv_heads * block_size * head_dim elements each).
 * Destinations must be distinct and must not be sources in the same call
 * (checked under PA_DEBUG only); a pair naming a block outside [0, num_blocks)
 * copies nothing. Supported shapes as for pa_reshape_and_cache. num_pairs may
 * be 0 (no launch).
 */
int32_t pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *block_mapping,
                       int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t dtype,
                       void *stream);

/*
 * pa_swap_blocks - copy whole blocks from one pair of pools to another, for
 * swapping: a preempted request's blocks move out to host memory and come back
 * when it resumes, the table being the only thing that changes ([INFRA] §4.3).
 *
 * Pair i of block_mapping int32 [num_pairs, 2] (device memory) copies block
 * block_mapping[2i] of (src_k, src_v) to block block_mapping[2i+1] of
 * (dst_k, dst_v), every KV head and slot, bit for bit. Either pool pair may be
 * pinned host memory the GPU can address (hipHostMalloc, e.g. torch's
 * pin_memory=True); the kernel then reads or writes it over the host link.
 * Each pool pointer is looked up with hipPointerGetAttributes (a few
 * microseconds of host time per call): host pointers are translated to their
 * device addresses, and memory that is neither device memory nor registered
 * host memory gives PA_ERR_BAD_POINTER before anything is launched.
 * src pools are [src_num_blocks, ...], dst pools [dst_num_blocks, ...]; the
 * two pairs must not overlap. Destinations must be distinct and in range
 * (checked under PA_DEBUG only); a pair outside either pool copies nothing.
 * block_mapping may be device memory or pinned host memory.
 */
int32_t pa_swap_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                       const int32_t *block_mapping, int32_t num_pairs,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t src_num_blocks, int32_t dst_num_blocks,
                       int32_t dtype, void *stream);

/*
 * pa_prefill - multi-token (chunked-prefill) paged attention: each query token
 * of a chunk attends to its sequence's cached tokens up to and including its
 * own position ([INFRA] §1.1, the per-step attention, for every token of the
 * chunk; [OPS] calls the operator with a whole sequence of queries).
 *
 * Queries of all sequences are packed along one token axis:
 *   q, out           [num_tokens, num_q_heads, head_dim], dtype
 *   query_start_loc  int32 [num_seqs + 1]: sequence s owns tokens
 *                    query_start_loc[s] .. query_start_loc[s+1]-1 (its chunk,
 *                    L_s tokens; 0 <= L_s <= max_query_len)
 *   context_lens     int32 [num_seqs]: cached tokens of sequence s INCLUDING
 *                    the chunk, whose K/V must already be in the pools
 *                    (pa_reshape_and_cache); L_s <= context_lens[s]
 *   k_cache, v_cache, block_tables, num_blocks, max_blocks_per_seq as for
 *   pa_decode.
 * Token t of sequence s sits at position context_lens[s] - L_s + t and
 * attends to positions 0 .. context_lens[s] - L_s + t; query head h reads KV
 * head h / (num_q_heads / num_kv_heads). out = softmax(scale * q.K^T) V per
 * (token, head), accumulated in fp32 and rounded once to dtype.
 *
 * Built: dtype PA_F16 or PA_BF16, head_dim 64 or 128, block_size 8-64,
 * num_q_heads / num_kv_heads in {1, 2, 4, 8}, a finite scale > 0; otherwise
 * PA_ERR_UNSUPPORTED.
 * No workspace; nothing allocated. Device-resident preconditions (monotone
 * query_start_loc ending at num_tokens, chunk and context lengths, table
 * entries in range) are checked only under PA_DEBUG=1 (PA_ERR_BAD_INDEX).
 * Without it, table entries are clamped into [0, num_blocks) (no read leaves
 * the pools), and a sequence whose chunk lies outside [0, num_tokens), is
 * longer than its context, or whose context is longer than its table row gets
 * no output rows. max_blocks_per_seq * block_size must stay below 2^31.
 * Tokens of sequences with L_s = 0 do not exist; nothing else is written.
 */
int32_t pa_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *block_tables, const int32_t *context_lens,
                   const int32_t *query_start_loc, float scale, int32_t num_seqs,
                   int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                   int32_t max_blocks_per_seq, int32_t max_query_len, int32_t dtype,
                   void *stream);

/* A static, human-readable name of a status code. */
const char *pa_status_str(int32_t status);

/* Library ABI version (bumped on any signature change). */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
