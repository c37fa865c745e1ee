/*
 * pagedattn.h -- C ABI of the MI355X (gfx950) paged-attention library.
 *
 * The library computes attention of each sequence's query tokens over a KV
 * cache held in fixed 16-token physical blocks that a per-sequence block
 * table maps from logical positions ("03 -- Engines Papers", section 2:
 * key trick, block table, and the kernel that must gather K/V from
 * non-contiguous blocks; "The LLM inference engine playbook", Theme 3).
 * Query heads are grouped onto KV heads (GQA; "References", GQA entry).
 * A batch may mix single-token decodes with chunked-prefill spans
 * ("03 -- Engines Papers", section 3). The key blocks of the whole batch
 * are split into pieces of equal work (blocks plus a fixed cost for each
 * context a piece starts), one per resident wave, so long and short
 * contexts finish together; a context cut by a piece boundary is
 * completed by a log-sum-exp merge of its pieces' partial results (the
 * split-K decode pattern of the playbook's Theme 4; the LSE merge of
 * "03 -- Engines Papers", section 12). The cache may be stored as FP8 E4M3
 * with one scale per (block, KV head) (playbook, Themes 3 and 6).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array argument is a DEVICE pointer owned by the caller. The
 *   library never allocates device memory, frees or synchronizes; every
 *   call only enqueues kernels on `stream` (a hipStream_t passed as void*,
 *   NULL = the null stream) and returns. Scratch memory is the caller's
 *   `workspace`, sized by pa_workspace_bytes.
 * - A call whose batch holds chunked-prefill spans beside single-token
 *   tiles runs its span kernel on `stream` and its decode kernels on a
 *   second stream of the library's, forked from `stream` after the work
 *   queued before the call and joined back into it before the call's
 *   merge (or, for pa_paged_attn_partial, before it returns), so the two
 *   kinds of tile run side by side ("03 -- Engines Papers", section 3).
 *   Work queued on `stream` after the call still waits for all of it, and
 *   a graph capture of `stream` captures both branches. The library makes
 *   that stream (default priority) and two events once per device, in the
 *   first pa_workspace_bytes call for a batch that can hold spans (else in
 *   the first such attention call: callers that capture graphs size their
 *   workspace first), and keeps them until the process ends; calls from
 *   several host threads on one device take a lock around the fork and
 *   join. pa_paged_attn_hybrid_noalloc never makes them: it uses them if
 *   they exist, else runs every kernel on `stream`. Results are the same
 *   either way.
 * - Return value: PA_OK (0) or a negative pa_status. Arguments are checked
 *   on the host before anything is enqueued; a failed check enqueues
 *   nothing. Data-dependent contract breaches (a block id out of range, a
 *   context longer than 16 * max_blocks_per_seq, two tokens appending to
 *   one slot, an append into a block shared with another sequence) are
 *   NOT detected by the kernels.
 * - Layouts (row-major, contiguous):
 *     q, out       [T][Hq][D]           dtype q_dtype (out has q's dtype)
 *     k_cache      [num_blocks][Hkv][16][D]   token rows of D values
 *     v_cache      [num_blocks][Hkv][D][16]   D rows of 16 token values
 *                  (dim-major, unlike K: a departure from the token-major
 *                  [16][D] block the plainest reading of the pages gives,
 *                  so that the P.V matrix-core operand comes straight from
 *                  16-byte loads; the price is that an append writes a
 *                  token's V as D values 32 bytes apart)
 *     k_scale, v_scale [num_blocks][Hkv] float32 (FP8 caches only, else NULL)
 *     block_tables [num_seqs][max_blocks_per_seq] int32
 *     context_lens [num_seqs] int32: keys each sequence attends over, which
 *                  INCLUDE its query tokens of this step (append first)
 *     query_start_loc [num_seqs + 1] int32, exclusive prefix sums of the
 *                  per-sequence query counts n_i; qsl[0] = 0, qsl[S] = T
 *     lse          [T][Hq] float32, natural log of the softmax normalizer
 * - Semantics: sequence i's n_i query tokens are the LAST n_i positions of
 *   its context; query j (0-based in the span) sits at position
 *   L_i - n_i + j and sees keys 0 .. L_i - n_i + j inclusive. Query head h
 *   reads KV head h / (Hq / Hkv). A stored FP8 byte c in block b, KV head g
 *   means e4m3fn(c) * scale[b][g]. A sequence with context length 0 yields
 *   a zero output row and lse = -inf.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16

typedef enum pa_dtype {
    PA_F32 = 0,        /* IEEE binary32 */
    PA_BF16 = 1,       /* bfloat16 */
    PA_FP8_E4M3FN = 2  /* OCP FP8 E4M3FN (bias 7, max 448, no inf) */
} pa_dtype;

typedef enum pa_status {
    PA_OK = 0,
    PA_EINVAL = -1,     /* bad pointer, shape, dtype combination or size */
    PA_EWORKSPACE = -2, /* workspace NULL or smaller than pa_workspace_bytes */
    PA_EHIP = -3,       /* a HIP runtime call or kernel launch failed */
    PA_ENOTSUP = -4,    /* valid request this build does not implement */
    PA_ENOMEM = -5,     /* no free physical block (block manager) */
    PA_ESCRATCH = -6    /* batch needs more than the static scratch buffer
                           of pa_paged_attn_hybrid_noalloc holds */
} pa_status;

/* Problem shape shared by all calls on one cache. Supported today:
 * head_dim in {64, 128}; block_size == 16; Hq % Hkv == 0 with
 * G = Hq / Hkv <= 16; (q_dtype, kv_dtype) in {(F32, F32), (BF16, BF16),
 * (BF16, FP8_E4M3FN)}; partition_size 0 (split each call's key blocks into
 * equal pieces, one per resident wave) or a
 * positive multiple of 16 (pieces of that many tokens). Query rows are
 * grouped into tiles: a span of at most 16 / G tokens (every decode) is one
 * narrow tile of G * n_i rows; a longer span is cut into wide tiles of
 * 128 / G tokens (F32 caches: into narrow tiles of 16 / G tokens). A call
 * may hold at most 8192 tiles, counted as num_seqs for a decode call and,
 * for a hybrid call, num_seqs + min(num_seqs + ceil(num_q_tokens /
 * (128 / G)), num_q_tokens) (F32: min(num_seqs + ceil(num_q_tokens /
 * (16 / G)), num_q_tokens)), plus 2 * num_seqs when cascade is 1; beyond
 * that it returns PA_ENOTSUP, as it does when num_q_tokens * num_q_heads
 * reaches 2^31 - 1 (output rows are indexed with 32 bits). */
typedef struct pa_shape {
    int32_t num_q_heads;        /* Hq */
    int32_t num_kv_heads;       /* Hkv */
    int32_t head_dim;           /* D */
    int32_t block_size;         /* must be PA_BLOCK_SIZE */
    int32_t num_blocks;         /* physical blocks in the pool */
    int32_t max_blocks_per_seq; /* row stride of block_tables */
    int32_t q_dtype;            /* pa_dtype of q, out, and new K/V rows */
    int32_t kv_dtype;           /* pa_dtype of the caches */
    int32_t partition_size;     /* split-KV piece in tokens, 0 = balanced */
    int32_t cascade;            /* 1: plans may hold shared-prefix groups
                                   (pa_plan_cascade); reserves their room */
    int32_t fp8_qk;             /* 1 (fp8 cache only): both products of the
                                   decode kernel on the fp8 matrix cores:
                                   S = K q^T with q quantized per (token,
                                   head) into two e4m3 terms, value and
                                   residual, and O += V^T P with P (times the
                                   block's V scale and a power-of-two output
                                   scale) as two e4m3 terms against the
                                   stored V bytes ("Inference engines",
                                   recent developments: the QK and score-V
                                   matmuls themselves in FP8); spans keep the
                                   exact bf16 products; results within the
                                   fp8 tolerance, not bitwise those of 0 */
} pa_shape;

/* Bytes of device workspace the attention calls need for this batch (work
 * list, per-segment counters, split partials). Returns 0 when the shape is
 * invalid. num_q_tokens = T (num_seqs for a decode call); max_query_len =
 * largest n_i (1 for a decode call). The decode and hybrid calls below are
 * pa_plan followed by pa_paged_attn_run. */
size_t pa_workspace_bytes(const pa_shape* shape, int num_seqs, int num_q_tokens,
                          int max_context_len, int max_query_len);

/* Decode: one query token per sequence (T = num_seqs, token i belongs to
 * sequence i). Computes out (and lse if non-NULL) for every sequence.
 * max_context_len must be >= every context_lens[i] (it sizes the launch;
 * the library never reads lengths back to the host). Paged KV storage and
 * its gather: "03 -- Engines Papers", section 2; split-K decode with a
 * log-sum-exp merge for long contexts: playbook Theme 4 and the first
 * page's section 12. */
int pa_paged_attn_decode(const pa_shape* shape, void* out, float* lse, const void* q,
                         const void* k_cache, const void* v_cache, const float* k_scale,
                         const float* v_scale, const int32_t* block_tables,
                         const int32_t* context_lens, int num_seqs, int max_context_len,
                         float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Hybrid batch: sequences with n_i >= 1 query tokens each (chunked-prefill
 * spans and decodes together, "03 -- Engines Papers", section 3), T =
 * num_q_tokens = query_start_loc[num_seqs]. Each span attends causally over
 * its paged context as stated above. max_query_len >= every n_i. */
int pa_paged_attn_hybrid(const pa_shape* shape, void* out, float* lse, const void* q,
                         const void* k_cache, const void* v_cache, const float* k_scale,
                         const float* v_scale, const int32_t* block_tables,
                         const int32_t* context_lens, const int32_t* query_start_loc,
                         int num_seqs, int num_q_tokens, int max_query_len,
                         int max_context_len, float scale, void* workspace,
                         size_t workspace_bytes, void* stream);

/* pa_paged_attn_hybrid for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments and results as pa_paged_attn_hybrid (bit for
 * bit), without the workspace: the plan, the pieces' partial results and
 * the merge use a buffer of PA_NOALLOC_SCRATCH_BYTES that the library holds
 * in static device memory, one per GPU it runs on, for the life of the
 * process. The call allocates and frees nothing. Batches whose workspace
 * (pa_workspace_bytes) exceeds that size return PA_ESCRATCH before anything
 * is enqueued. Every call on one GPU shares that GPU's buffer: calls that
 * overlap on one GPU (different streams, or threads) race, so a caller
 * orders them, for instance on one stream. Nothing in the buffer needs to
 * start at zero: each call's plan writes every record the call reads. */
#define PA_NOALLOC_SCRATCH_BYTES (128u << 20)
int pa_paged_attn_hybrid_noalloc(const pa_shape* shape, void* out, float* lse, const void* q,
                                 const void* k_cache, const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* block_tables,
                                 const int32_t* context_lens, const int32_t* query_start_loc,
                                 int num_seqs, int num_q_tokens, int max_query_len,
                                 int max_context_len, float scale, void* stream);

/* Plan a batch: turn (query spans, context lengths) into the work list the
 * attention kernel streams -- tiles of up to 16 query rows, one stream of
 * 16-token key blocks over all (tile, KV head) segments, cut into pieces
 * balanced over the device's resident waves (or of partition_size tokens).
 * Writes only `workspace`. The request trace on "03 -- Engines Papers"
 * plans once per step from the active sequences before the model runs; a
 * plan stays valid for every pa_paged_attn_run that passes the same shape,
 * batch sizes and the same context_lens / query_start_loc contents (every
 * layer of one step), enqueued after it. query_start_loc NULL = decode
 * (num_q_tokens == num_seqs). Calls that overlap on one workspace race. */
int pa_plan(const pa_shape* shape, const int32_t* context_lens, const int32_t* query_start_loc,
            int num_seqs, int num_q_tokens, int max_query_len, int max_context_len,
            void* workspace, size_t workspace_bytes, void* stream);

/* pa_plan for a batch in which groups of single-token sequences share the
 * physical blocks of a common prefix -- a parallel-sampling group, requests
 * that hit the same cached prompt -- through copy-on-write ("03 -- Engines
 * Papers", section 2). Cascade attention (same page, section 12): each
 * group's prefix is read once for all of its members, in tiles of up to
 * max(32 / G, 1) members (two 16-row matrix-core tiles of G heads per
 * member), and each member reads only the
 * blocks after the prefix; the run's merge pass combines the two parts of
 * every member by log-sum-exp. The outputs are the same attention as
 * without groups, up to rounding.
 *
 * Group g's members are group_members[group_offsets[g] ..
 * group_offsets[g + 1]) (sequence indices; device arrays, group_offsets
 * [num_groups + 1] with group_offsets[0] = 0 and group_offsets[num_groups]
 * = num_members); they share their first group_prefix_blocks[g] block-table
 * entries (device [num_groups]). The prefix is read through the first
 * member's block table. A member that has more than one query token, or no
 * key past the prefix, reads its whole context itself instead. Contract
 * (not checked by the kernels): the members' tables do hold the same
 * physical blocks there, and a sequence is in at most one group.
 * shape->cascade must be 1; num_groups, num_members <= num_seqs. */
int pa_plan_cascade(const pa_shape* shape, const int32_t* context_lens,
                    const int32_t* query_start_loc, int num_seqs, int num_q_tokens,
                    int max_query_len, int max_context_len, int num_groups, int num_members,
                    const int32_t* group_offsets, const int32_t* group_members,
                    const int32_t* group_prefix_blocks, void* workspace, size_t workspace_bytes,
                    void* stream);

/* pa_plan for a hybrid batch whose spans are speculative candidates
 * verified in one pass ("03 -- Engines Papers", sections 5 to 7: the draft
 * tokens form a candidate tree checked under a tree attention mask).
 * tree_mask: device [num_q_tokens] uint64, one word per query token; in a
 * span of at most 64 tokens, token j sees every key before the span and
 * span token k <= j only where bit k of its word is set (bits above j are
 * ignored; a chain j -> j-1 -> ... is the causal mask). Spans of more than
 * 64 tokens, and decodes of one token with bit 0 set, attend as in
 * pa_plan. The plan copies the masks into the workspace. */
int pa_plan_tree(const pa_shape* shape, const int32_t* context_lens,
                 const int32_t* query_start_loc, int num_seqs, int num_q_tokens, int max_query_len,
                 int max_context_len, const uint64_t* tree_mask, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Attention with a plan made by pa_plan (same arguments as the plan, plus
 * the tensors). Enqueues the attention pass (one launch per tile class
 * present) and then the merge pass: pieces that cut a segment write partial
 * results to the workspace, and the merge combines them by log-sum-exp. */
int pa_paged_attn_run(const pa_shape* shape, void* out, float* lse, const void* q,
                      const void* k_cache, const void* v_cache, const float* k_scale,
                      const float* v_scale, const int32_t* block_tables,
                      const int32_t* context_lens, const int32_t* query_start_loc, int num_seqs,
                      int num_q_tokens, int max_query_len, int max_context_len, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/* The two passes of pa_paged_attn_run as separate calls, for callers that
 * schedule or time them apart. pa_paged_attn_partial writes the rows of
 * every (tile, KV head) segment one wave saw whole, and partial results
 * (log-sum-exp and normalized output) for segments cut by a piece boundary;
 * pa_paged_attn_merge (the second pass) combines those partials by
 * log-sum-exp into out / lse. Same batch arguments as the plan. */
int pa_paged_attn_partial(const pa_shape* shape, void* out, float* lse, const void* q,
                          const void* k_cache, const void* v_cache, const float* k_scale,
                          const float* v_scale, const int32_t* block_tables,
                          const int32_t* context_lens, const int32_t* query_start_loc,
                          int num_seqs, int num_q_tokens, int max_query_len, int max_context_len,
                          float scale, void* workspace, size_t workspace_bytes, void* stream);
int pa_paged_attn_merge(const pa_shape* shape, void* out, float* lse, const int32_t* context_lens,
                        const int32_t* query_start_loc, int num_seqs, int num_q_tokens,
                        int max_query_len, int max_context_len, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Decode with this step's K/V rows appended in the same attention pass.
 * Equivalent to pa_kv_append of k_new / v_new ([num_seqs][Hkv][D] in
 * q_dtype, 16-byte aligned) at slot block_tables[i][(L_i - 1) / 16] * 16 +
 * (L_i - 1) % 16 with L_i = context_lens[i] (the context including the new
 * token; the slot of the new position through the block table, "03 --
 * Engines Papers", section 2), followed by the attention of the same call
 * without append: the cache bytes written and out / lse are bit for bit
 * those. The wave that reads a sequence's last block for a KV head puts
 * the new token into the tile it loaded and writes it to the cache, so the
 * step needs no append launch (one launch fewer per layer). Needs a decode
 * plan (query_start_loc NULL; cascade plans allowed); sequences with L_i = 0
 * append nothing; contexts past max_context_len are not supported (as for
 * the attention). run_append: both passes with a plan made earlier;
 * partial_append: the first pass only (pa_paged_attn_merge completes it);
 * decode_append: plan and both passes. */
int pa_paged_attn_run_append(const pa_shape* shape, void* out, float* lse, const void* q,
                             const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int num_seqs, int max_context_len, float scale, void* workspace,
                             size_t workspace_bytes, void* stream);
int pa_paged_attn_partial_append(const pa_shape* shape, void* out, float* lse, const void* q,
                                 const void* k_new, const void* v_new, void* k_cache,
                                 void* v_cache, const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int num_seqs, int max_context_len, float scale,
                                 void* workspace, size_t workspace_bytes, void* stream);
int pa_paged_attn_decode_append(const pa_shape* shape, void* out, float* lse, const void* q,
                                const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, const float* k_scale, const float* v_scale,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int num_seqs, int max_context_len, float scale, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Append this step's new K/V rows into their slots before attention runs
 * on the same stream. k_new, v_new: [num_tokens][Hkv][D] in q_dtype.
 * slot_mapping: [num_tokens] int32, slot = physical_block * 16 + offset
 * (the logical-to-physical mapping of the block table, "03 -- Engines
 * Papers", section 2); a negative slot skips its token. Same-dtype caches
 * receive the values bit for bit; an FP8 cache receives
 * e4m3fn(fp32(new) / scale[block][head]) rounded to nearest-even and
 * saturated to +-448 (NaN -> 0x7F), using the block's existing scale.
 * Slots must be distinct and must not lie in a block another sequence
 * still shares (copy-on-write, same section). */
int pa_kv_append(const pa_shape* shape, void* k_cache, void* v_cache, const float* k_scale,
                 const float* v_scale, const void* k_new, const void* v_new,
                 const int32_t* slot_mapping, int num_tokens, void* stream);

/* Decode n FP8 E4M3FN bytes to float32 with the device's conversion path
 * (the one the attention kernels use), for inspecting a cache. */
int pa_fp8_e4m3fn_to_f32(const uint8_t* in, float* out, int n, void* stream);

/* Workspace introspection, for tools and tests that read a plan back from
 * device memory. Fills *info with the bounds and byte offsets of the
 * workspace regions that pa_plan, pa_plan_cascade and pa_plan_tree write for
 * this batch: the same computation that pa_workspace_bytes and the plan
 * calls make (`decode` = 1 for a plan made with query_start_loc NULL).
 * Region contents, all int32 fields in this order:
 *   header   [64]: tiles, cut segments, cascade records, tree flag, then per
 *            stream s (0 wide: chunked-prefill spans; 1 narrow: decodes,
 *            short spans, cascade suffixes; 2 group: shared-prefix group
 *            tiles) at 4 + 4 s: blocks per KV head, work per piece (blocks
 *            plus a fixed cost per segment started), pieces
 *   tiles    [max_tiles] x 12: seq, first query token, query tokens, blocks,
 *            context length, first query row, span tokens, flags (1 suffix,
 *            2 group), first block, 3 unused
 *   pieces   per stream [max_pieces] x 16: tile, KV head, first block,
 *            blocks in the piece, then a copy of that tile's 12 fields
 *   splits   [max_splits] x 8: first row, query tokens, KV head, first and
 *            last piece, stream, 2 unused (past the header's count: k0 = -1)
 *   cascade  cas_seq: 6 x [num_seqs] (member prefix blocks, suffix tile,
 *            group tile, place in the group tile, member copy, group's
 *            first tile); cas_recs [max_cas_recs] x 8: query row, KV head,
 *            suffix first and last piece, prefix first and last piece, place
 *            in the group tile, unused
 * Host only; enqueues nothing. Returns PA_OK, or PA_EINVAL for an invalid
 * shape or size. */
typedef struct pa_layout_info {
    int32_t waves[3];          /* resident workgroups of the wide, narrow and
                                  group streams' kernels */
    int32_t narrow_tokens;     /* query tokens per narrow tile */
    int32_t wide_tokens;       /* query tokens per wide tile (0: no spans) */
    int32_t part_blocks;       /* partition_size / 16 (0: balanced) */
    int32_t members_per_tile;  /* cascade members per group tile */
    int32_t wide_row_tiles;    /* 16-row tiles of a wide slot */
    int32_t header_words;      /* int32 words of the header */
    int32_t part_cost[3];      /* when balancing: a segment's start in blocks
                                  of work, per stream (the group stream's is
                                  nonzero only in batches without spans) */
    int32_t span_shared;       /* span workgroups when the span launch runs
                                  beside the narrow and group launches (one
                                  per compute unit; 0: never) */
    int32_t group_row_tiles;   /* 16-row tiles of a group tile and of a
                                  group-stream slot */
    int64_t max_tiles, max_pieces[3], max_splits, max_cas_recs;
    int64_t off_tiles, off_splits, off_tree, off_cas_seq, off_cas_recs;
    int64_t off_cas_lse[2], off_cas_o[2];
    int64_t off_pieces[3], off_part_lse[3], off_part_o[3];
    int64_t total;             /* bytes */
} pa_layout_info;
int pa_workspace_layout(const pa_shape* shape, int num_seqs, int num_q_tokens,
                        int max_context_len, int max_query_len, int decode,
                        pa_layout_info* info);

/* Static text for a status code. */
const char* pa_status_string(int status);

/* Library ABI version (major * 100 + minor): 200 added pa_shape.cascade
 * and pa_plan_cascade; 201 added pa_plan_tree; 202 added pa_shape.fp8_qk;
 * 203 added pa_workspace_layout; 204 added pa_paged_attn_hybrid_noalloc;
 * 205 gave pa_layout_info a third block stream; 206 gave piece records
 * their block counts and pa_layout_info the per-stream part costs; 207
 * runs P.V on the fp8 matrix cores too when fp8_qk is set; 208 added
 * pa_paged_attn_run_append, pa_paged_attn_partial_append and
 * pa_paged_attn_decode_append; 209 runs a batch's span launch beside its
 * narrow and group launches (a second stream of the library's) and gave
 * pa_layout_info span_shared; 210 gave shared-prefix group tiles two
 * 16-row tiles (pa_layout_info.group_row_tiles); 211 charges each group
 * segment a start cost when pieces are balanced in batches without spans
 * (plans change, calls and results do not). */
int pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
