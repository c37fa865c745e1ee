/*
 * pagedattn_blocks.h -- host-side block manager of the paged KV cache, and
 * the device copy it asks for.
 *
 * The manager owns the assignment of fixed 16-token physical blocks to
 * sequences: a free list, a block table per sequence mapping logical
 * blocks to physical ones, and a reference count per physical block so
 * that sequences can share blocks ("03 -- Engines Papers", section 2: the
 * block table; copy-on-write sharing with a refcount for parallel sampling
 * and beam search; the block manager's allocate/free in the whiteboard
 * trace; the fraction of KV memory in use as the measure that matters).
 * It produces what the attention path consumes: block tables, context
 * lengths, the slot of every new token (slot = 16 * block + offset), and
 * shared-prefix groups for cascade attention (pa_plan_cascade).
 *
 * All manager calls are host-only, synchronous, and not thread-safe (one
 * manager per scheduler thread). Status codes are pa_status values
 * (pagedattn.h); PA_ENOMEM when no block is free, in which case the
 * manager is left unchanged.
 */
#ifndef PAGEDATTN_BLOCKS_H
#define PAGEDATTN_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#include "pagedattn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager; /* opaque */

/* A manager of num_blocks physical blocks for sequences of at most
 * max_blocks_per_seq blocks (16 * max_blocks_per_seq tokens). Returns NULL
 * if an argument is not positive or memory runs out. Blocks are handed out
 * lowest id first. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t max_blocks_per_seq);
void pa_bm_destroy(pa_block_manager* bm);

/* A new sequence `seq` holding num_tokens >= 0 tokens (a prompt). Writes the
 * slots of its tokens to slots[0 .. num_tokens) unless slots is NULL.
 * PA_EINVAL if seq exists or the length exceeds the table. */
int pa_bm_add(pa_block_manager* bm, int64_t seq, int32_t num_tokens, int32_t* slots);

/* A new sequence `seq` whose first prefix_blocks blocks are those of
 * sequence `owner` (a cached prompt prefix: shared, refcount + 1 each;
 * they must be full), followed by num_tokens tokens of its own (slots of
 * those written to slots unless NULL). */
int pa_bm_add_shared(pa_block_manager* bm, int64_t seq, int64_t owner, int32_t prefix_blocks,
                     int32_t num_tokens, int32_t* slots);

/* A new sequence `child` sharing every block of `parent`, the last one
 * included even if partly filled (parallel sampling, beam search). */
int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);

/* Append num_tokens tokens to seq and write their slots. If the sequence's
 * last block is shared and partly filled, it is first replaced by a private
 * copy (copy-on-write): the pair (source block, destination block) is
 * written to copy_pair[0..1] and *num_copies is set to 1, else 0. The
 * caller copies those blocks of the cache (pa_copy_blocks) before it
 * appends the new rows (pa_kv_append). copy_pair may be NULL only when no
 * copy is needed. */
int pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t num_tokens, int32_t* slots,
                 int32_t* copy_pair, int32_t* num_copies);

/* Release a sequence: each of its blocks loses a reference and returns to
 * the free list at zero. */
int pa_bm_free(pa_block_manager* bm, int64_t seq);

/* Tokens held by seq (-1 if it does not exist). */
int32_t pa_bm_length(const pa_block_manager* bm, int64_t seq);

/* Block-table rows and context lengths of a batch: row i (stride
 * row_stride >= the longest sequence's block count) lists seqs[i]'s
 * physical blocks, padded with -1; context_lens[i] its tokens. */
int pa_bm_tables(const pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* tables,
                 int32_t row_stride, int32_t* context_lens);

/* Shared-prefix groups of a batch for pa_plan_cascade: sequences of the
 * batch (batch indices 0..n-1) whose tables start with the same physical
 * block form a group (two members or more), with prefix_blocks = the
 * number of leading table entries all members share, counting full
 * blocks only. Output arrays hold up to n entries (offsets n + 1). */
int pa_bm_prefix_groups(const pa_block_manager* bm, const int64_t* seqs, int32_t n,
                        int32_t* group_offsets, int32_t* group_members,
                        int32_t* group_prefix_blocks, int32_t* num_groups,
                        int32_t* num_members);

/* Occupancy of the pool. utilization = tokens held in used blocks /
 * (used blocks * 16): the share of allocated KV memory that holds tokens
 * (a block shared by several sequences counts once). */
typedef struct pa_bm_stats {
    int32_t num_blocks;
    int32_t free_blocks;
    int32_t used_blocks;
    int32_t shared_blocks;   /* refcount > 1 */
    int32_t num_sequences;
    int32_t pad;
    int64_t logical_tokens;  /* sum of the sequences' lengths */
    int64_t stored_tokens;   /* tokens held in used blocks, shared ones once */
    double utilization;
} pa_bm_stats;
int pa_bm_get_stats(const pa_block_manager* bm, pa_bm_stats* stats);

/* Reference count of a physical block (-1 if out of range). */
int32_t pa_bm_refcount(const pa_block_manager* bm, int32_t block);

/* Check a batch's metadata on the host before it reaches the kernels, for
 * callers that build tables themselves: every table entry a context needs
 * lies in [0, num_blocks); context lengths fit the table; query spans
 * (query_start_loc, NULL = one token each) are ordered, within their
 * contexts; every slot_mapping entry of a query token (num_tokens entries,
 * -1 = skipped) is the slot of that token's position, and no two tokens
 * share a slot; with refcounts (NULL = unchecked) no token is appended
 * into a block of refcount > 1. Returns PA_OK, or PA_EINVAL with the
 * offending sequence in *bad_seq (token row for slot errors). Host arrays. */
int pa_validate_batch(int32_t num_blocks, int32_t max_blocks_per_seq,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* query_start_loc, const int32_t* slot_mapping,
                      int32_t num_seqs, int32_t num_tokens, const int32_t* refcounts,
                      int32_t* bad_seq);

/* Device: copy whole blocks of the cache (K and V for every KV head, and
 * the fp8 scales) from pairs[2k] to pairs[2k + 1] for k < num_pairs, on
 * stream: the copies copy-on-write asks for. pairs is a device array;
 * destinations must be distinct and not also sources. */
int pa_copy_blocks(const pa_shape* shape, void* k_cache, void* v_cache, float* k_scale,
                   float* v_scale, const int32_t* pairs, int num_pairs, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_BLOCKS_H */
