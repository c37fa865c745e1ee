// pa_internal.h -- structures shared by the host launchers and the gfx950
// kernels of the paged-attention library. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

// A tile: query rows and the 16-token key blocks they read.
//  - span tile (flags 0): the G heads of `ntok` consecutive query tokens of
//    one sequence's span; blocks 0 .. nb-1 (causal: up to the tile's last
//    query position; at least one, so a tile with no keys still gets a wave
//    that writes its zero rows).
//  - suffix tile (TILE_SUFFIX): a single-token sequence in a shared-prefix
//    group; blocks b0 .. b0+nb-1, the keys after the shared prefix.
//  - group tile (TILE_GROUP): the single query tokens of up to `ntok`
//    members of a shared-prefix group (group_members[qtok0 ..]), G rows
//    each; blocks 0 .. nb-1 of the prefix, read once for all of them
//    (cascade attention, "03 -- Engines Papers", section 12).
enum { TILE_SUFFIX = 1, TILE_GROUP = 2 };
struct TileDesc {
    int32_t seq;    // the sequence whose block table the tile reads
    int32_t qtok0;  // first query token of the tile, relative to the span;
                    // group tile: first entry in group_members
    int32_t ntok;   // query tokens in the tile (group tile: members)
    int32_t nb;     // key blocks the tile reads (>= 1)
    int32_t L;      // the sequence's context length (clamped); group tile:
                    // 16 * nb, the prefix
    int32_t qs;     // the sequence's first query token row
    int32_t nspan;  // the sequence's query tokens
    int32_t flags;  // TILE_SUFFIX, TILE_GROUP or 0
    int32_t b0;     // first logical block
    int32_t pad[3];
};

// Where a piece of the block stream begins: segment (tile, kv head), block j
// (counted from the tile's b0), the piece's length in blocks, and a copy of
// that tile's record so a wave starts with one load.
struct PieceStart {
    int32_t tile;
    int32_t kvh;
    int32_t j;
    int32_t nblocks;
    TileDesc td;
};

// A segment cut by piece boundaries: its rows and the pieces holding its
// partial results. Pieces are numbered within the substream of the
// segment's KV head: k0 wrote its tail slot, k0+1 .. k1 their head slots;
// piece k of KV head h is piece k * Hkv + h of the stream.
struct SplitSeg {
    int32_t row0;    // first query token row of the tile
    int32_t ntok;    // query tokens in the tile
    int32_t kvh;
    int32_t k0;
    int32_t k1;
    int32_t stream;  // STREAM_WIDE, STREAM_NARROW or STREAM_GROUP
    int32_t pad[2];
};

// Three block streams: tiles of chunked-prefill spans (wide: up to
// kSpanRows query rows, run by a workgroup of kSpanWaves waves that share
// every K/V block through LDS); tiles of at most 16 rows (narrow: decodes,
// short spans and cascade suffixes; one wave each); and shared-prefix group
// tiles (one wave each, as the narrow ones). Each is cut into its own
// pieces and run by its own launch, so a stream's pieces balance among
// segments of like cost: a group's long prefix does not share a piece
// count with the one-block suffixes of its members.
enum { STREAM_WIDE = 0, STREAM_NARROW = 1, STREAM_GROUP = 2, NUM_STREAMS = 3 };
constexpr int kSpanRows = 128;                // query rows of a wide tile
constexpr int kSpanRowTiles = kSpanRows / 16;  // 16-row tiles of a wide tile (and slot)
#ifndef PA_SPAN_WAVES
#define PA_SPAN_WAVES 4
#endif
constexpr int kSpanWaves = PA_SPAN_WAVES;      // waves of a span workgroup
static_assert(kSpanWaves == 4 || kSpanWaves == 8, "two or one row tiles per wave");
// 16-row tiles of a shared-prefix group tile (and of the group stream's
// partial slots): a group tile holds the single query tokens of
// 16 * kGroupRowTiles / G members, and each of its waves reads the group's
// prefix blocks once for all of them.
#ifndef PA_GROUP_ROW_TILES
#define PA_GROUP_ROW_TILES 2
#endif
constexpr int kGroupRowTiles = PA_GROUP_ROW_TILES;
static_assert(kGroupRowTiles == 1 || kGroupRowTiles == 2, "one or two row tiles per group tile");
// row tiles of a partial slot of stream st
constexpr int slot_row_tiles(int st) {
    return st == STREAM_WIDE ? kSpanRowTiles : st == STREAM_GROUP ? kGroupRowTiles : 1;
}
// Kernel kinds: the cache dtype, or an fp8 cache whose S = K q^T runs on
// the fp8 matrix cores (pa_shape.fp8_qk).
constexpr int KIND_FP8_QK = 3;

// Header words at the start of the workspace: per stream s, the blocks of
// each KV head's substream, the piece size (in blocks of cost when
// balancing) and the piece count at HDR_STREAM + 4 s.
enum {
    HDR_NTILES = 0,
    HDR_NSPLIT = 1,
    HDR_NCAS = 2,  // cascade records
    HDR_TREE = 3,  // 1: the plan holds tree verification masks
    HDR_STREAM = 4,
    HDR_TOTAL = 0,
    HDR_R = 1,
    HDR_NPIECES = 2,
    HDR_WORDS = 64
};

// Partial results: two slots per piece (the segment it enters mid-way, the
// segment it leaves unfinished), 16 rows each.
enum { SLOT_HEAD = 0, SLOT_TAIL = 1 };

constexpr int kMaxTiles = 8192;  // tiles per call (the plan keeps them in LDS)

// A single-token sequence in a shared-prefix group, for one KV head: its G
// rows combine two parts by log-sum-exp, the prefix (rows row_off .. of
// group tile gtile) and the suffix (rows 0 .. of its suffix tile). A part
// read whole by one piece was written to the dense per-row buffer of its
// kind; a cut part lies in the slots of pieces k0 .. k1 of its stream's KV
// head substream.
struct CascadeRec {
    int32_t row;     // the sequence's query token row
    int32_t kvh;
    int32_t suf_k0, suf_k1;
    int32_t pre_k0, pre_k1;
    int32_t pre_pos;  // the member's place in the group tile (rows pre_pos * G ..)
    int32_t pad;
};

// Per-row buffers of whole cascade parts: [T * Hq] lse (log2 units) and
// [T * Hq][D] normalized outputs, one pair for prefixes, one for suffixes.
enum { CAS_PRE = 0, CAS_SUF = 1 };

struct PlanArgs {
    const int32_t* context_lens;
    const int32_t* qsl;  // nullptr: one query token per sequence
    int32_t num_seqs;
    int32_t num_tokens;
    int32_t max_context_len;  // contexts are clamped to this
    int32_t narrow_tokens;    // query tokens per narrow tile (16 / G, 1 for decode)
    int32_t wide_tokens;      // query tokens per wide tile (kSpanRows / G; 0: no spans)
    int32_t num_kv_heads;
    int32_t part_blocks;  // blocks per piece; 0 = balance over the stream's waves
    // when balancing: the cost of a segment's start in blocks of work (its
    // row setup, the first block's latency, its epilogue), per stream
    int32_t part_cost[NUM_STREAMS];
    int32_t waves[NUM_STREAMS];  // resident workgroups of each stream's kernel
    // span workgroups when the span stream runs beside the others (0: the
    // span stream always gets waves[STREAM_WIDE]); used when the single-token
    // streams' work is at least kSpanShareRatio times the span stream's
    int32_t span_shared;
    int32_t min_blocks[NUM_STREAMS];  // smallest piece of each stream when balancing
    int32_t max_tiles;
    int64_t max_pieces[NUM_STREAMS];
    TileDesc* tiles;
    PieceStart* pieces[NUM_STREAMS];
    SplitSeg* splits;    // [max_splits] segments the merge completes
    int64_t max_splits;  // at most one per (tile, KV head), one per inner piece boundary
    int32_t* hdr;
    // shared-prefix groups (num_groups 0: none)
    int32_t num_groups;
    int32_t members_per_tile;  // single-token members per group tile
    const int32_t* group_offsets;        // [num_groups + 1]
    const int32_t* group_members;        // sequence ids
    const int32_t* group_prefix_blocks;  // [num_groups]
    int32_t* cas_prefix;  // [num_seqs] shared blocks of a cascade member, else 0
    int32_t* cas_tile;    // [num_seqs] a member's suffix tile
    int32_t* cas_gtile;   // [num_seqs] a member's group tile
    int32_t* cas_pos;     // [num_seqs] a member's place in its group tile
    int32_t* cas_members;  // [num_seqs] copy of group_members for the attention pass
    int32_t* cas_gbase;    // [num_seqs] a group's first tile (-1: none)
    CascadeRec* cas_recs;  // [num_seqs * Hkv]
    int32_t max_cas_recs;
    // tree verification masks ([num_tokens], nullptr: causal spans), copied
    // into the workspace so that the runs need no extra argument
    const uint64_t* tree_mask;
    uint64_t* tree_ws;
};

struct AttnArgs {
    void* out;
    float* lse;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int32_t* qsl;
    const TileDesc* tiles;
    const PieceStart* pieces;  // this stream's pieces
    const int32_t* hdr;
    int32_t stream;
    float* part_lse;  // [pieces][2][row tiles * 16], log2 units
    float* part_o;    // [pieces][2][row tiles][D/16][64 lanes] float4, normalized
    const int32_t* group_members;  // group tiles' members (sequence ids, workspace copy)
    const int32_t* cas_prefix;     // [num_seqs] shared blocks of a cascade member
    float* cas_lse[2];             // CAS_PRE, CAS_SUF per-row buffers
    float* cas_o[2];
    const uint64_t* tree;          // [num_tokens] masks (used when hdr[HDR_TREE])
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t num_blocks;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    float scale_log2;  // softmax scale times log2(e)
    // decode with append: this step's K/V rows [num_seqs][Hkv][D] (q dtype),
    // put at position context_lens - 1 of each sequence (nullptr: none)
    const void* k_new;
    const void* v_new;
};

struct MergeArgs {
    void* out;
    float* lse;
    const SplitSeg* splits;
    const int32_t* hdr;
    const float* part_lse[NUM_STREAMS];
    const float* part_o[NUM_STREAMS];
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t max_splits;  // workgroups [0, max_splits) complete cut segments
    int32_t wide_nt;     // row tiles of the wide stream's slots (kSpanRowTiles)
    const CascadeRec* cas_recs;  // the rest combine cascade parts
    const float* cas_lse[2];
    const float* cas_o[2];
};

struct AppendArgs {
    void* k_cache;
    void* v_cache;
    const float* k_scale;
    const float* v_scale;
    const void* k_new;
    const void* v_new;
    const int32_t* slot_mapping;
    int32_t num_tokens;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t num_blocks;
};

struct CopyArgs {
    void* k_cache;
    void* v_cache;
    float* k_scale;  // nullptr unless fp8
    float* v_scale;
    const int32_t* pairs;  // [num_pairs][2] source, destination
    int64_t block_bytes;   // bytes of one block in one cache (all KV heads)
    int32_t num_blocks;
    int32_t num_kv_heads;
};

// Launchers (host side), defined next to their kernels.
// The span kernel (wide stream): workgroups that fit on the device at once.
int span_resident_groups(int kind, int head_dim);
// Span workgroups that run beside the narrow launches of the same call (one
// per compute unit, leaving each SIMD a wave slot for a narrow wave), or 0
// when the span kernel's resources leave no such room.
int span_shared_groups(int kind, int head_dim);
hipError_t launch_span(int kind, int head_dim, const AttnArgs& a, int64_t max_pieces,
                       hipStream_t s);
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_attention(int kind, int head_dim, const AttnArgs& a, int64_t max_pieces,
                            hipStream_t s);  // a.stream selects the wide or narrow kernel
// The group stream (g) then the narrow stream (n) in one narrow launch
// (decode batches with shared-prefix groups); max_pieces: the larger bound.
hipError_t launch_narrow_pair(int kind, int head_dim, const AttnArgs& g, const AttnArgs& n,
                              int64_t max_pieces, hipStream_t s);
// Workgroups of the attention kernel of a stream that fit on the device at
// once (narrow: waves; wide: span workgroups), or 0 if the device cannot be
// queried.
int resident_waves(int kind, int head_dim, int stream);
// records: cut-segment workgroups (a.max_splits) plus cascade records
hipError_t launch_merge(int q_dtype, int head_dim, const MergeArgs& a, int64_t records,
                        bool wide, hipStream_t s);
hipError_t launch_append(int new_dtype, int kv_dtype, const AppendArgs& a, hipStream_t s);
hipError_t launch_copy_blocks(const CopyArgs& a, int num_pairs, hipStream_t s);
hipError_t launch_fp8_decode(const uint8_t* in, float* out, int n, hipStream_t s);

// The span stream runs on one workgroup per compute unit, beside the narrow
// and group launches, when those streams' balanced work (blocks plus start
// costs per KV head) is at least this many times the span stream's: then the
// decodes' HBM-bound time hides the span tiles' longer run at half their
// residency. Below it the span tiles keep the whole device.
constexpr int kSpanShareRatio = 2;

// Smallest piece (in 16-token blocks) when pieces are balanced over the
// resident waves. One block: a wave that walked several short segments one
// after another (one-block suffixes of cascade members, say) would pay a
// chain of dependent loads for each, while other waves idle.
#ifndef PA_MIN_PIECE_BLOCKS
#define PA_MIN_PIECE_BLOCKS 1
#endif
constexpr int kMinPieceBlocks = PA_MIN_PIECE_BLOCKS;
// Smallest piece of the group stream when balancing. A piece that cuts a
// group tile writes its 16 kGroupRowTiles rows of partial results (16 KB at
// D = 128 with two row tiles) per cut, as much as two bf16 blocks of K and
// V; shorter pieces would write more than they read.
#ifndef PA_GROUP_MIN_PIECE_BLOCKS
#define PA_GROUP_MIN_PIECE_BLOCKS 8
#endif
constexpr int kGroupMinPieceBlocks = PA_GROUP_MIN_PIECE_BLOCKS;

}  // namespace pa

// Record sizes published by pa_workspace_layout's description.
static_assert(sizeof(pa::TileDesc) == 12 * 4, "tile record format");
static_assert(sizeof(pa::PieceStart) == 16 * 4, "piece record format");
static_assert(sizeof(pa::SplitSeg) == 8 * 4, "cut-segment record format");
static_assert(sizeof(pa::CascadeRec) == 8 * 4, "cascade record format");
