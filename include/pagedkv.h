/*
 * pagedkv.h - C ABI of the paged-KV decode-attention library (gfx950).
 *
 * The library computes decode-step attention over a paged KV cache:
 * a pool of fixed-size KV blocks, a per-sequence block table mapping
 * logical block i of a sequence to a physical block, appends of new
 * tokens' K/V through that table, and causal scaled-dot-product attention
 * that gathers every cached block through the table while it computes.
 *
 * Sources (the pages this library implements):
 *  - "Inference Engineering" capstone lab (openarchlab, inference lab):
 *    class KVPool (write / gather / release) and function forward
 *    (attention core) in its NumPy listing; mapping-table rows 6-7.
 *  - foundations-of-llms chapter 5 "Inference & optimisation":
 *    section 2.1 (KV cache: append k_t, v_t, then attend q_t over K, V),
 *    section 3.1 (grouped-query attention), section 3.2 (PagedAttention:
 *    fixed-size blocks allocated on demand, a block table read by the
 *    attention kernel), section 4.1 (online softmax).
 *  - LLM inference serving tutorial (ARIS): section 1.7 (idempotent
 *    reclaim, no double free), section 4.1 (bytes per token),
 *    section 4.2 (block-table indirection, internal fragmentation).
 *
 * Conventions for every entry point
 *  - Return value: PKV_OK (0) or a negative PKV_ERR_* code. Arguments are
 *    validated before anything is launched or mutated, so an error leaves
 *    no partial effect. pkv_strerror() names a code.
 *  - Device pointers are plain addresses in the current HIP device's
 *    memory, owned by the caller; the library never allocates, frees or
 *    retains device memory. Host pointers (kvpool_*) are owned by the
 *    caller and only read or written during the call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default
 *    stream). Kernels are enqueued asynchronously on it; outputs are valid
 *    once the caller synchronises with the stream. The library keeps no
 *    per-call state, so calls on different streams may run concurrently as
 *    long as their output buffers differ.
 *  - Data the host cannot check without a device round trip (block ids in
 *    the table, seq_lens, q_start) is checked on the device: an attention
 *    row whose sequence length is out of range, or whose table holds an id
 *    outside [0, num_blocks), is written as NaN (out and lse) instead of
 *    reading out of bounds; kv_append skips a token whose table entry is out
 *    of range.
 *
 * Memory layouts (row-major, innermost last)
 *  - k_cache, v_cache: [num_blocks][n_kv][block_size][head_dim] elements of
 *    `dtype` (the lab pool's [block][head][slot][dim] layout): one (block,
 *    kv head) tile of block_size x head_dim elements is contiguous.
 *  - block_table: int32 [num_seqs][table_stride]; entry i of row s is the
 *    physical block holding positions [i*block_size, (i+1)*block_size) of
 *    sequence s. Entries at or past ceil(seq_lens[s]/block_size) are never
 *    read (pad them with -1).
 *  - q, out: [rows][n_q][head_dim] of `dtype`; lse: float [rows][n_q]
 *    (natural-log log-sum-exp of the scaled scores), nullable.
 *  - Query head h reads kv head h / (n_q / n_kv) (contiguous groups).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define PKV_OK                       0
#define PKV_ERR_NULL_POINTER        -1  /* a required pointer is NULL */
#define PKV_ERR_INVALID_ARGUMENT    -2  /* a size or shape is out of range */
#define PKV_ERR_UNSUPPORTED         -3  /* no kernel instantiation for this shape/dtype */
#define PKV_ERR_OUT_OF_BLOCKS       -4  /* the pool has fewer free blocks than requested */
#define PKV_ERR_INVALID_FREE        -5  /* freeing an id that is out of range, already free, or repeated */
#define PKV_ERR_WORKSPACE_TOO_SMALL -6  /* workspace_bytes below paged_attn_workspace_size() */
#define PKV_ERR_TABLE_FULL          -7  /* a sequence needs more blocks than its table row holds */
#define PKV_ERR_HIP                 -8  /* a HIP launch failed (hipGetLastError) */
#define PKV_ERR_NO_MEMORY           -9  /* host allocation for the pool object failed */
#define PKV_ERR_INVALID_BLOCK      -10  /* a block id to share or copy is out of range, not allocated, or repeated */
#define PKV_ERR_SCRATCH_LIMIT      -11  /* the call needs more split-K workspace than the static scratch holds */

/* ---- element types ----------------------------------------------------- */
#define PKV_F32  0   /* IEEE binary32 */
#define PKV_BF16 1   /* bfloat16 (upper half of binary32), stored as 16 bits */

/* Human-readable name of a status code (static string, never NULL). */
const char* pkv_strerror(int status);

/* ======================================================================
 * Block pool (host). The allocator hands out block ids, not bytes; K/V
 * storage is the caller's k_cache / v_cache.
 *
 * Source: lab page, class KVPool - a sorted free list from which a
 * sequence takes the lowest id each time a position reaches the end of its
 * last block, with every block returned (and the list re-sorted) when the
 * sequence ends; chapter 5 section 3.2 (blocks allocated on demand);
 * serving tutorial section 1.7 (reclaim is idempotent: no double free, no
 * leak). The lab asserts when the pool runs dry; here that is
 * PKV_ERR_OUT_OF_BLOCKS with nothing changed.
 *
 * Ordering: ids are handed out lowest *rank* first, where alloc_order[i]
 * has rank i (NULL = identity order 0..num_blocks-1, the lab's policy).
 * Not thread-safe: one thread owns a pool.
 * ==================================================================== */
typedef struct kvpool kvpool_t;

/* Create a pool of num_blocks (>= 1) blocks of block_size (>= 1) tokens.
 * alloc_order: NULL or a permutation of 0..num_blocks-1 (copied).
 * Errors: NULL_POINTER (out), INVALID_ARGUMENT (sizes, not a permutation),
 * NO_MEMORY. */
int kvpool_create(int32_t num_blocks, int32_t block_size,
                  const int32_t* alloc_order, kvpool_t** out);

/* Destroy a pool (NULL is accepted and ignored). */
int kvpool_destroy(kvpool_t* pool);

/* Take the n lowest-rank free blocks, written to out_ids[0..n) in rank
 * order. All or nothing: OUT_OF_BLOCKS if fewer than n are free. n = 0 is
 * a no-op. */
int kvpool_alloc(kvpool_t* pool, int32_t n, int32_t* out_ids);

/* Drop one reference to each of n blocks; a block whose last reference
 * goes rejoins the free set (a block from kvpool_alloc has one reference).
 * All or nothing: INVALID_FREE if any id is out of range, currently free,
 * or listed twice. */
int kvpool_free(kvpool_t* pool, int32_t n, const int32_t* ids);

/* Sequence helper: roll a row back to `length` tokens - keep its first
 * ceil(length / block_size) blocks and drop the row's reference to every
 * block after them (blocks no other row holds rejoin the free set); their
 * entries become -1 and *num_held is updated. A row already that short is
 * unchanged, so repeating the call is a no-op. Source: chapter 5 section 5
 * (speculative decoding: the target model verifies gamma drafted tokens in
 * one pass; a rejected draft and every draft after it are discarded) and
 * the serving tutorial's question on speculative decoding (the KV of
 * rejected candidates is rolled back and never counted as committed).
 * Positions past the new length inside the last kept block keep their old
 * contents; attention never reads past seq_lens and the next append
 * overwrites them. Errors: NULL_POINTER, INVALID_ARGUMENT, INVALID_FREE. */
int kvpool_truncate(kvpool_t* pool, int32_t* row, int32_t* num_held, int32_t length);

/* ----------------------------------------------------------------------
 * Shared blocks. Source: serving tutorial section 4.2 (a physical block
 * can be shared through reference counts by a common prefix or by beam /
 * parallel-sampling branches; a shared, still-writable tail block that one
 * holder is about to change is copied and that holder's table remapped
 * instead of writing the shared copy), section 1.7 (a shared block goes
 * back to the allocator only when its last holder releases it), and its
 * question on best-of-n (the prompt's KV is held once, only the branches'
 * own tokens grow with the number of branches); lab-scale demo D08 (two
 * sequences of 6 and 7 tokens with block size 4 sharing one full block
 * need 3 physical blocks instead of 4). The attention entry points need
 * nothing extra: table rows may name the same block.
 * -------------------------------------------------------------------- */

/* Add one reference to each of n allocated blocks. All or nothing:
 * INVALID_BLOCK if an id is out of range, free, or listed twice. */
int kvpool_share(kvpool_t* pool, int32_t n, const int32_t* ids);

/* Holders of block `id` (0 = free). INVALID_ARGUMENT if out of range. */
int kvpool_refcount(const kvpool_t* pool, int32_t id, int32_t* out);

/* Sequence helper: make an empty row (*dst_held == 0) share the first
 * ceil(length / block_size) blocks of another row (its first `length`
 * tokens), one more reference each; *dst_held is set to that count. A
 * length that ends inside a block shares that block too; the first write
 * into it goes through kvpool_cow. Errors: INVALID_ARGUMENT (dst not
 * empty, length past the source's blocks), TABLE_FULL, INVALID_BLOCK. */
int kvpool_fork(kvpool_t* pool, const int32_t* src_row, int32_t src_held,
                int32_t* dst_row, int32_t* dst_held, int32_t row_capacity, int32_t length);

/* Sequence helper, before writing positions [start, start + count) of a
 * row: every block of the row in that range held by more than one row is
 * replaced in this row by a newly allocated block (lowest rank first, in
 * row order), dropping one reference to the old block. The (old, new)
 * pairs go to copy_src / copy_dst (capacity entries each; at most
 * ceil(count / block_size) + 1 are needed) and *num_copies; the caller
 * copies their contents with kv_copy_blocks before appending. All or
 * nothing: INVALID_BLOCK (a row entry in range is not an allocated block),
 * INVALID_ARGUMENT (capacity too small), OUT_OF_BLOCKS. Blocks past
 * num_held are not touched (kvpool_ensure allocates them unshared). */
int kvpool_cow(kvpool_t* pool, int32_t* row, int32_t num_held, int32_t start, int32_t count,
               int32_t* copy_src, int32_t* copy_dst, int32_t capacity, int32_t* num_copies);

/* Number of free blocks. */
int kvpool_num_free(const kvpool_t* pool, int32_t* out);

/* Free ids in the order they would be handed out (out has room for
 * num_blocks; *count receives the number written). */
int kvpool_free_ids(const kvpool_t* pool, int32_t* out, int32_t* count);

/* Sequence helper: grow a table row so it covers `length` tokens, i.e.
 * holds ceil(length / block_size) blocks. row[0..*num_held) are the blocks
 * the sequence already holds; new ids are appended in rank order and
 * *num_held is updated. TABLE_FULL if the row would need more than
 * row_capacity entries; OUT_OF_BLOCKS if the pool is short (row unchanged
 * in both cases). */
int kvpool_ensure(kvpool_t* pool, int32_t* row, int32_t* num_held,
                  int32_t row_capacity, int32_t length);

/* Sequence helper: drop the row's reference to each of its blocks (blocks
 * no other row holds rejoin the free set), set its entries to -1 and
 * *num_held to 0. Releasing an empty row is a no-op, so calling this twice
 * is safe. */
int kvpool_release(kvpool_t* pool, int32_t* row, int32_t* num_held);

/* ======================================================================
 * kv_append - write new tokens' K/V into the pool through the table.
 *
 * Source: lab page, KVPool.write (token at position p goes to slot p % B
 * of block table[p / B], for every kv head); chapter 5 section 2.1 (append
 * k_t, v_t to the cache). Stage 1 of the decode step.
 *
 * k_new, v_new: device, [total_new][n_kv][head_dim] of dtype, the new
 *   tokens of all sequences packed in sequence order.
 * new_start: device int32 [num_seqs + 1], prefix sums: sequence s owns new
 *   rows new_start[s] .. new_start[s+1]-1; new_start[num_seqs] == total_new.
 * start_pos: device int32 [num_seqs], position of sequence s's first new
 *   token (its cached length before the append).
 * The table rows must already cover start_pos[s] + (new tokens of s)
 * (kvpool_ensure). Only the addressed slots are written.
 * Errors: NULL_POINTER, INVALID_ARGUMENT (negative/zero sizes, dtype),
 * HIP. total_new == 0 launches nothing. */
int kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
              const int32_t* block_table, int32_t table_stride,
              const int32_t* start_pos, const int32_t* new_start,
              int32_t num_seqs, int32_t total_new, int32_t num_blocks,
              int32_t n_kv, int32_t head_dim, int32_t block_size, int32_t dtype,
              void* stream);

/* ======================================================================
 * kv_copy_blocks - copy whole blocks inside both pools: block src_ids[i]'s
 * K and V (all kv heads, all slots) onto block dst_ids[i], i < n.
 *
 * Source: serving tutorial section 4.2 (copy-on-write: the holder about to
 * write a shared block gets a copy of it). Pair the call with kvpool_cow,
 * whose (old, new) pairs it takes, before kv_append into those blocks.
 *
 * src_ids, dst_ids: device int32 [n]. Every dst must differ from every
 * other dst and from every src of the call (kvpool_cow's pairs do), else
 * the result is undefined. A pair naming an id outside [0, num_blocks), or
 * the same block twice, is skipped. Shapes as kv_append.
 * Errors: NULL_POINTER, INVALID_ARGUMENT (sizes, dtype), HIP. n == 0
 * launches nothing. */
int kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_ids, const int32_t* dst_ids,
                   int32_t n, int32_t num_blocks, int32_t n_kv, int32_t head_dim,
                   int32_t block_size, int32_t dtype, void* stream);

/* ======================================================================
 * Attention workspace. Both attention entry points split each sequence's
 * keys into ranges of split_tokens keys, compute a partial softmax state
 * per range, and merge the ranges in a second pass (chapter 5 section 4.1:
 * online softmax; the merged result equals the plain softmax).
 *
 * split_tokens: 0 = let the library choose (paged_attn_split_tokens tells
 *   which); otherwise a positive multiple of block_size.
 * num_q_rows: decode = num_seqs; chunk = total query rows.
 * Writes the required byte count to *bytes (may be 0 for shapes that need
 * no partials). Errors: NULL_POINTER, INVALID_ARGUMENT. */
int paged_attn_split_tokens(int32_t num_q_rows, int32_t n_kv, int32_t block_size,
                            int32_t max_seq_len, int32_t requested, int32_t* out);
int paged_attn_workspace_size(int32_t num_q_rows, int32_t n_q, int32_t n_kv,
                              int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                              int32_t split_tokens, size_t* bytes);
/* Workspace for paged_attn_chunk on any of its paths (and for
 * paged_attn_chunk_q8): the larger of paged_attn_workspace_size(total_q,
 * ...) and, when the chunk qualifies for the balanced path (see
 * paged_attn_chunk), its partial slots for a bf16 or an 8-bit pool. Needs
 * the device (the balanced grid is sized from it). Errors: NULL_POINTER,
 * INVALID_ARGUMENT, HIP. */
int paged_attn_chunk_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t n_q,
                                    int32_t n_kv, int32_t head_dim, int32_t block_size,
                                    int32_t max_seq_len, int32_t split_tokens, size_t* bytes);

/* ======================================================================
 * paged_attn_decode - one query token per sequence.
 *
 * Source: chapter 5 section 2.1 (q_t against every cached key and value),
 * section 3.1 (query head h uses kv head h / (n_q/n_kv)), section 3.2
 * (the kernel reads the block table to gather K/V from scattered pages);
 * lab page, forward (scores scaled by `scale`, max-subtracted softmax,
 * weighted sum of V). Stages 2 and 3 of the decode step.
 *
 * seq_lens: device int32 [num_seqs], keys per sequence *after* the append
 *   (the new token included); each must be in [1, max_seq_len] and at
 *   most table_stride * block_size, else that row's output is NaN.
 * q, out: [num_seqs][n_q][head_dim] of dtype; lse: float [num_seqs][n_q]
 *   or NULL. scale: multiplies q.k (the lab uses 1/sqrt(head_dim)).
 * workspace: device, at least paged_attn_workspace_size(num_seqs, ...)
 *   bytes, 256-byte aligned; contents on entry are ignored.
 * Supported: dtype PKV_BF16 or PKV_F32; 1 <= head_dim <= 512;
 *   block_size >= 1; n_q a multiple of n_kv. bf16 with head_dim 128 and
 *   block_size 16 takes the bandwidth-tuned kernel.
 * Errors: NULL_POINTER, INVALID_ARGUMENT (n_q % n_kv != 0, sizes, split),
 * UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP. */
int paged_attn_decode(void* out, float* lse, const void* q,
                      const void* k_cache, const void* v_cache,
                      const int32_t* block_table, int32_t table_stride,
                      const int32_t* seq_lens,
                      int32_t num_seqs, int32_t max_seq_len, int32_t num_blocks,
                      int32_t n_q, int32_t n_kv, int32_t head_dim, int32_t block_size,
                      float scale, int32_t dtype, int32_t split_tokens,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * paged_attn_decode_append - the whole decode step in one pass: each
 * sequence's new token is appended to the pool, then one query token per
 * sequence attends over the cache including it.
 *
 * Source: chapter 5 section 2.1 (a decode step appends k_t, v_t to the
 * cache, then attends q_t over every cached key and value); the append
 * places the token as the lab page's KVPool.write does (position p to slot
 * p % B of block table[p / B], every kv head). Same result as kv_append of
 * one token per sequence at position seq_lens[s] - 1 followed by
 * paged_attn_decode, without the separate append launch: the wave that
 * reads a sequence's last block for a kv head writes the new row first
 * (while the batch has at most half as many (sequence, kv head) pairs as
 * the pass has waves; with more, the append is a small launch of its own
 * inside the call).
 *
 * k_new, v_new: device, [num_seqs][n_kv][head_dim] bf16, 16-byte aligned.
 * seq_lens: keys per sequence after the append (the new token is at
 *   seq_lens[s] - 1); table rows must cover it (kvpool_ensure). A sequence
 *   whose length is out of range gets NaN rows and no append, and a token
 *   whose table entry is outside the pool is not written (its rows NaN),
 *   as in kv_append and paged_attn_decode.
 * k_cache, v_cache: written at the appended slots only. Other arguments
 *   and the workspace as paged_attn_decode (split_tokens is 0).
 * Supported: dtype PKV_BF16, head_dim 128, block_size 16, n_q / n_kv in
 *   {1, 2, 4, 8}, at most 8192 sequences, 16-byte aligned tensors; other
 *   shapes return UNSUPPORTED (call kv_append, then paged_attn_decode).
 * Errors: NULL_POINTER, INVALID_ARGUMENT, UNSUPPORTED,
 * WORKSPACE_TOO_SMALL, HIP. */
int paged_attn_decode_append(void* out, float* lse, const void* q, void* k_cache, void* v_cache,
                             const void* k_new, const void* v_new, const int32_t* block_table,
                             int32_t table_stride, const int32_t* seq_lens, int32_t num_seqs,
                             int32_t max_seq_len, int32_t num_blocks, int32_t n_q, int32_t n_kv,
                             int32_t head_dim, int32_t block_size, float scale, int32_t dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * paged_attn_decode_append_noalloc - paged_attn_decode_append with its
 * split-K workspace in a static device array of the library instead of a
 * caller buffer: the call allocates nothing (no hipMalloc, no allocating
 * library routine).
 *
 * For callers that cannot allocate device memory: code under stream
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The array holds PKV_NOALLOC_SCRATCH_BYTES (16 MiB); each GPU the library
 * runs on keeps its own copy until the process ends. Its device address is
 * looked up on the first call on each device. A batch whose partition needs
 * more (about (waves + num_seqs * n_kv) * (n_q / n_kv) partials of
 * 8 + 4 * head_dim bytes: up to ~800 sequences at 8 kv heads and group 4)
 * returns PKV_ERR_SCRATCH_LIMIT before anything is launched; use
 * paged_attn_decode_append with a workspace for those. Nothing in the array
 * has to start at zero. All calls on one GPU share its array, so calls that
 * overlap in time on one GPU (different streams, or threads) race: serialise
 * them. Arguments, results and other errors as paged_attn_decode_append. */
#define PKV_NOALLOC_SCRATCH_BYTES (16u << 20)
int paged_attn_decode_append_noalloc(void* out, float* lse, const void* q, void* k_cache, void* v_cache,
                                     const void* k_new, const void* v_new, const int32_t* block_table,
                                     int32_t table_stride, const int32_t* seq_lens, int32_t num_seqs,
                                     int32_t max_seq_len, int32_t num_blocks, int32_t n_q, int32_t n_kv,
                                     int32_t head_dim, int32_t block_size, float scale, int32_t dtype,
                                     void* stream);

/* ======================================================================
 * paged_attn_chunk - a chunk of C_s consecutive query tokens per sequence
 * (chunked prefill), causal.
 *
 * Source: lab page, forward called on a prompt chunk at offset `start`
 * over the gathered cache (mask: key j allowed iff j <= start + i) and its
 * scheduler's prefill branch; chapter 5 section 4.1 (tiling with online
 * softmax). Query i of sequence s sits at absolute position
 * seq_lens[s] - C_s + i and attends keys 0 .. that position.
 *
 * q_start: device int32 [num_seqs + 1], prefix sums of C_s; q, out are
 *   [total_q][n_q][head_dim]; lse float [total_q][n_q] or NULL.
 * max_q_len: host bound on every C_s. seq_lens[s] >= C_s is required
 *   (else NaN rows). Other arguments as paged_attn_decode; the workspace
 *   is sized by paged_attn_chunk_workspace_size (or, for the chunk kernels
 *   only, paged_attn_workspace_size with num_q_rows = total_q).
 * Paths: bf16, head_dim 128, block_size 16, split_tokens 0 and
 *   max_q_len * (n_q / n_kv) <= 32 (verification-sized chunks) with a
 *   workspace of paged_attn_chunk_workspace_size bytes: the decode pass's
 *   balanced partition over every (sequence, kv head, block) tile, all of a
 *   kv head's (query, head) rows at once; otherwise one workgroup per
 *   (query tile, kv head, sequence) on the matrix cores, or the generic
 *   split path. All give the result defined above.
 * Errors: as paged_attn_decode. */
int paged_attn_chunk(void* out, float* lse, const void* q, const int32_t* q_start,
                     const void* k_cache, const void* v_cache,
                     const int32_t* block_table, int32_t table_stride,
                     const int32_t* seq_lens,
                     int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                     int32_t max_seq_len, int32_t num_blocks,
                     int32_t n_q, int32_t n_kv, int32_t head_dim, int32_t block_size,
                     float scale, int32_t dtype, int32_t split_tokens,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * paged_attn_chunk_append - a chunk step in one call: each sequence's C_s
 * new tokens (rows q_start[s] .. q_start[s+1]-1 of k_new / v_new, the last
 * C_s of its seq_lens[s] keys) are appended to the pool, then the chunk
 * attends as paged_attn_chunk.
 *
 * Source: the lab page's prefill branch and forward on a prompt chunk at
 * offset start (write the chunk's K/V, then attend causally over the cache
 * including it); chapter 5 section 5 (a verification pass appends the
 * drafts and attends them as one chunk). Same result as kv_append of the
 * chunk at start_pos = seq_lens - C_s followed by paged_attn_chunk, without
 * the caller building start_pos / new_start (positions come from seq_lens
 * and q_start). On the matrix-core chunk kernel (bf16, head_dim 128,
 * block_size 16, split_tokens 0, 16-byte aligned k_new / v_new) the append
 * is fused into it: each workgroup writes its own query tile's tokens and
 * reads the chunk's keys from k_new / v_new. Otherwise the append is
 * launched first inside the call.
 *
 * k_new, v_new: device, [total_q][n_kv][head_dim] of dtype. A sequence that
 *   the chunk pass rejects (seq_lens[s] < C_s, out of range) gets no
 *   append; a token whose table entry is outside the pool is not written.
 * Other arguments, workspace and errors as paged_attn_chunk. */
int paged_attn_chunk_append(void* out, float* lse, const void* q, const int32_t* q_start,
                            void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* block_table, int32_t table_stride, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                            int32_t num_blocks, int32_t n_q, int32_t n_kv, int32_t head_dim,
                            int32_t block_size, float scale, int32_t dtype, int32_t split_tokens,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * 8-bit K/V (quantised cache).
 *
 * Source: chapter 5 section 4 (post-training quantisation, symmetric
 * absmax onto the integer grid [-q_max, q_max], q_max = 2^(b-1) - 1 = 127
 * for 8 bits: s = max|w| / q_max, w_q = clamp(round(w / s)), the value is
 * read back as s * w_q; group-wise: one scale per group of consecutive
 * elements, group sizes 32/64/128), applied here to the cache with one
 * group per (token, kv head) - the head_dim values a token writes for one
 * kv head; serving tutorial section 7 (KV-cache quantisation is a design
 * point of its own: per-token granularity, capacity and bandwidth) and
 * section 4.1 (scales are storage beyond the ideal K/V payload); the lab
 * page notes it did not run a quantised KV cache.
 *
 * Layout: k_codes, v_codes int8 [num_blocks][n_kv][block_size][head_dim]
 * (two's complement codes in [-127, 127]); k_scale, v_scale float
 * [num_blocks][n_kv][block_size], the scale of each (block, kv head, slot).
 * Storage per token and kv head: head_dim + 4 bytes for K and the same for
 * V (264 bytes at head_dim 128, against 512 for bf16).
 * ==================================================================== */

/* kv_append_q8 - quantise new tokens' K/V and write them through the table
 * (kv_append's addressing; its argument meanings). For every new token and
 * kv head, separately for K and V: s = max(max_i |x_i|, 1e-8) / 127 and
 * code_i = clamp(rint(x_i / s), -127, 127), computed in fp32 with correctly
 * rounded division and ties-to-even rounding; the codes go to the slot's
 * row, s to its scale. new_dtype: PKV_BF16 or PKV_F32 (k_new, v_new
 * [total_new][n_kv][head_dim]); inputs must be finite. Any head_dim and
 * block_size. Errors: NULL_POINTER, INVALID_ARGUMENT, HIP. */
int kv_append_q8(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                 const void* k_new, const void* v_new, int32_t new_dtype,
                 const int32_t* block_table, int32_t table_stride,
                 const int32_t* start_pos, const int32_t* new_start,
                 int32_t num_seqs, int32_t total_new, int32_t num_blocks,
                 int32_t n_kv, int32_t head_dim, int32_t block_size, void* stream);

/* paged_attn_decode_q8 - paged_attn_decode over an 8-bit cache: keys and
 * values are read as s * code; q and out are bf16; fp32 accumulation.
 * Supported: head_dim 128, block_size 16, n_q / n_kv in {1, 2, 4, 8},
 * 1..8192 sequences (else UNSUPPORTED); q, out, both code pools and both
 * scale arrays 16-byte aligned (else INVALID_ARGUMENT). The workspace is sized by
 * paged_attn_workspace_size with split_tokens 0 (the size covers both the
 * bf16 and the 8-bit pass). Invalid lengths or table entries give NaN rows
 * as in paged_attn_decode. Other arguments as paged_attn_decode. */
int paged_attn_decode_q8(void* out, float* lse, const void* q,
                         const void* k_codes, const void* v_codes,
                         const float* k_scale, const float* v_scale,
                         const int32_t* block_table, int32_t table_stride,
                         const int32_t* seq_lens,
                         int32_t num_seqs, int32_t max_seq_len, int32_t num_blocks,
                         int32_t n_q, int32_t n_kv, int32_t head_dim, int32_t block_size,
                         float scale, void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * paged_attn_decode_q8_append - the decode step in one call over an 8-bit
 * pool: each sequence's new token (bf16) is quantised into the pool at
 * position seq_lens[s] - 1, then paged_attn_decode_q8 runs over it.
 *
 * Source: chapter 5 section 2.1 (append k_t, v_t, then attend) and
 * section 4 (absmax quantisation, as kv_append_q8). Same result as
 * kv_append_q8 (bf16 input) of one token per sequence followed by
 * paged_attn_decode_q8: codes and scales bit-identical, outputs
 * bit-identical. The append rides in the split pass while the batch has at
 * most half as many (sequence, kv head) pairs as the pass has waves, else
 * it is a small launch of its own before it.
 *
 * k_new, v_new: device, [num_seqs][n_kv][head_dim] bf16, 16-byte aligned.
 * k_codes, v_codes, k_scale, v_scale: as paged_attn_decode_q8, written at
 *   the appended slots only. A sequence whose length is out of range gets
 *   NaN rows and no append; a token whose table entry is outside the pool
 *   is not written. Other arguments and errors as paged_attn_decode_q8. */
int paged_attn_decode_q8_append(void* out, float* lse, const void* q, void* k_codes, void* v_codes,
                                float* k_scale, float* v_scale, const void* k_new, const void* v_new,
                                const int32_t* block_table, int32_t table_stride, const int32_t* seq_lens,
                                int32_t num_seqs, int32_t max_seq_len, int32_t num_blocks, int32_t n_q,
                                int32_t n_kv, int32_t head_dim, int32_t block_size, float scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/* paged_attn_chunk_q8 - paged_attn_chunk over an 8-bit cache: keys and
 * values read as s * code; q and out bf16; fp32 accumulation. Source:
 * chapter 5 section 5 (a verification pass attends the drafted tokens as
 * one causal chunk) and section 2.2 (chunked prefill) over the cache of
 * chapter 5 section 4 (absmax codes) - the serving tutorial's section 7
 * treats KV quantisation as a design point that combines with the others.
 * Query i of sequence s sits at position seq_lens[s] - C_s + i (as
 * paged_attn_chunk). Supported: head_dim 128, block_size 16, n_q / n_kv in
 * {1, 2, 4, 8}, and either
 *  - max_q_len * (n_q / n_kv) <= 32 (verification-sized chunks): the
 *    balanced partition over every (sequence, kv head, block) tile, codes
 *    exact in bf16, the scales applied to scores and weights in fp32; or
 *  - larger chunks with max_seq_len <= 32768: the blocks each sequence
 *    holds are first written to the workspace as bf16 s * code (the fp32
 *    product rounded to bf16: one more rounding than the path above), then
 *    the matrix-core chunk kernel of paged_attn_chunk runs over them;
 * else UNSUPPORTED. q, out, code pools and scale arrays 16-byte aligned
 * (else INVALID_ARGUMENT). workspace: paged_attn_chunk_q8_workspace_size
 * bytes, 256-byte aligned. Append the chunk first with kv_append_q8
 * (positions seq_lens - C_s), or call paged_attn_chunk_q8_append. Invalid lengths or table entries give NaN
 * rows. Errors as paged_attn_chunk. */
/* Workspace for paged_attn_chunk_q8 (either of its paths): the balanced
 * partition's partial slots (needs the device: the grid is sized from it),
 * or for larger chunks num_seqs * ceil(max_seq_len / block_size) staged
 * bf16 blocks of K and of V plus their table. 0 for shapes it does not
 * support. Errors: NULL_POINTER, INVALID_ARGUMENT, HIP. */
int paged_attn_chunk_q8_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t n_q,
                                       int32_t n_kv, int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                                       size_t* bytes);
int paged_attn_chunk_q8(void* out, float* lse, const void* q, const int32_t* q_start,
                        const void* k_codes, const void* v_codes, const float* k_scale, const float* v_scale,
                        const int32_t* block_table, int32_t table_stride, const int32_t* seq_lens,
                        int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                        int32_t num_blocks, int32_t n_q, int32_t n_kv, int32_t head_dim, int32_t block_size,
                        float scale, void* workspace, size_t workspace_bytes, void* stream);

/* paged_attn_chunk_q8_append - the chunk step over an 8-bit cache in one
 * call: each sequence's C_s new bf16 rows (rows q_start[s] ..
 * q_start[s+1]-1 of k_new / v_new, [total_q][n_kv][head_dim]) quantised
 * into the pool as kv_append_q8 does, at the last C_s of its seq_lens[s]
 * positions, then paged_attn_chunk_q8. Source: as paged_attn_chunk_append
 * (the lab page's prefill branch; chapter 5 section 5's verification pass)
 * over the cache of chapter 5 section 4. Same result as kv_append_q8 at
 * start_pos = seq_lens - C_s followed by paged_attn_chunk_q8; a sequence
 * the chunk pass rejects gets no append, a token whose table entry is
 * outside the pool is not written. Every argument and the workspace are
 * checked before anything is written. Other arguments, support and errors
 * as paged_attn_chunk_q8. */
int paged_attn_chunk_q8_append(void* out, float* lse, const void* q, const int32_t* q_start,
                               void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                               const void* k_new, const void* v_new, const int32_t* block_table,
                               int32_t table_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t total_q,
                               int32_t max_q_len, int32_t max_seq_len, int32_t num_blocks, int32_t n_q,
                               int32_t n_kv, int32_t head_dim, int32_t block_size, float scale,
                               void* workspace, size_t workspace_bytes, void* stream);

/* kv_copy_blocks_q8 - kv_copy_blocks for an 8-bit cache: block src_ids[i]'s
 * codes and scales (K and V) onto block dst_ids[i]. Source: serving tutorial
 * section 4.2 (copy-on-write of a shared block) with the 8-bit layout above;
 * pair it with kvpool_cow as for kv_copy_blocks. Same pair rules and errors
 * as kv_copy_blocks. */
int kv_copy_blocks_q8(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                      const int32_t* src_ids, const int32_t* dst_ids, int32_t n, int32_t num_blocks,
                      int32_t n_kv, int32_t head_dim, int32_t block_size, void* stream);

/* ======================================================================
 * sample_tokens - pick the next token of each row of logits.
 *
 * Source: lab page, function sample (temperature 0 = greedy, softmax of
 * logits / T, top-k, then top-p on the renormalised result, then a draw
 * with the filtered probabilities); chapter 5's filter-and-sample listing
 * (sort the scaled logits, mask past k, mask where the cumulative
 * probability before a token reaches p - never the first); serving
 * tutorial demos D01/D02 (greedy takes the lowest index among tied maxima;
 * top-k keeps exactly k; top-p keeps the shortest prefix reaching p, the
 * boundary token included; top-k then top-p is not top-p then top-k).
 *
 * Per row: T = temperature[row] (0: greedy on the raw logits; < 0 or NaN:
 * token -1); z = logit / T in fp32; order by decreasing z, ties to the
 * lower index; top_k[row] > 0 keeps the first k of that order; masses
 * exp(z - max z); top_p[row] < 1 keeps the prefix of the order up to the
 * first token at which the cumulative mass reaches top_p times the kept
 * total; token = the first index, in vocabulary order, whose cumulative
 * kept mass exceeds u[row] times the kept total. u is the caller's uniform
 * random number in [0, 1) (the only randomness; this call draws none).
 *
 * logits: device float [rows][ld] (the first vocab entries of each row are
 *   used; finite values); temperature, top_p, u: device float [rows];
 *   top_k: device int32 [rows]; token: device int32 [rows] (output);
 *   kept: device int32 [rows][2] or NULL - tokens kept after top-k and
 *   after top-p. workspace: device memory of at least
 *   sample_workspace_size(rows, vocab) bytes, 8-byte aligned, owned by the
 *   caller, holding per-chunk results between the call's two kernels
 *   (contents on entry are ignored; calls sharing one workspace must not
 *   overlap). Rows with a top-k of at most 256 tokens (and greedy rows) are
 *   finished from per-chunk candidates; rows with top-k off and a vocabulary
 *   of at most 64 x 8192 from per-chunk maxima and fp64 mass histograms
 *   (falling back to the next path when more than 12288 tokens share the
 *   histogram bin of the top-p boundary); other rows by one workgroup over
 *   the whole row. All paths give the result defined above. Errors: NULL_POINTER,
 *   INVALID_ARGUMENT (vocab < 1 or above 8192 x 8192, ld < vocab,
 *   rows x ceil(vocab / 8192) or rows x 4 above INT32_MAX, workspace not 8-byte
 *   aligned), WORKSPACE_TOO_SMALL, HIP. */
int sample_tokens(int32_t* token, int32_t* kept, const float* logits, int32_t rows, int32_t vocab,
                  int64_t ld, const float* temperature, const int32_t* top_k, const float* top_p,
                  const float* u, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace sample_tokens needs: rows x ceil(vocab / 8192) chunks,
 * each with 2048 fp64 histogram bins (which also hold the 256 candidate
 * slots of 8 bytes) and a 16-byte header, plus per row 12288 8-byte slots
 * and 64 bytes of counters, when there are at most 64 chunks; else the 256
 * candidate slots per chunk only.
 * Errors: NULL_POINTER, INVALID_ARGUMENT (as for sample_tokens). */
int sample_workspace_size(int32_t rows, int32_t vocab, size_t* bytes);

/* ======================================================================
 * Profiling hook (not part of the computation): when both events are
 * non-NULL, paged_attn_decode launches its first-pass (split) kernel and
 * paged_attn_chunk its matrix-core kernel so that the kernel's own dispatch
 * records `before` when the kernel starts executing and `after` when it
 * has finished (hipExtLaunchKernel's event pair); elapsed time between them
 * is that kernel's duration, without the latency of separate event
 * packets. Pass NULLs to disable. Events are hipEvent_t passed as void*.
 * Process-wide; not thread-safe. */
int pkv_set_profile_events(void* before, void* after);

/* Read-only streaming probe (measurement only, not part of the
 * computation): reads device memory and folds it into a checksum, to give
 * the attention passes' HBM rates something to be compared with.
 *  - order == NULL: reads `bytes` (a multiple of 16) contiguous bytes at `a`
 *    with `workgroups` workgroups of 256 threads; sink holds
 *    workgroups * 256 uint32.
 *  - order != NULL: `workgroups` single-wave workgroups; tile t of order
 *    (t < tiles) names tile order[t] of tile_bytes (4096 or 2048) bytes in
 *    `a` and the same tile of `b` (the K and V tile of one (block, kv head):
 *    4 KiB for a bf16 pool, 2 KiB of codes for an 8-bit pool, at head_dim
 *    128 and block_size 16); wave w reads its own contiguous run of the
 *    order, one tile in flight while the previous is folded (the decode
 *    split pass's access pattern without its arithmetic). The caller keeps
 *    every order[t] inside both buffers. sink holds workgroups * 64 uint32.
 * a and b 16-byte aligned. Errors: NULL_POINTER, INVALID_ARGUMENT, HIP. */
int pkv_stream_read(const void* a, const void* b, size_t bytes, const int32_t* order, int32_t tiles,
                    int32_t tile_bytes, int32_t workgroups, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
