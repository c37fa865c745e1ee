// pa_api.hip -- the C ABI: argument checks, workspace layout, launches.
// Every function here only checks host-known arguments and enqueues
// kernels on the caller's stream (and, for a batch with spans beside
// single-token tiles, on the library's side stream, forked from and joined
// back into the caller's); nothing allocates device memory or synchronizes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "pa_internal.h"
#include "pagedattn_blocks.h"

#ifndef PA_WIDE_SPANS
#define PA_WIDE_SPANS 1
#endif

// The cost of a segment's start, in blocks of work, when pieces are
// balanced (the plan cuts pieces at equal blocks + cost). A span segment
// starts by loading 128 query rows and ends by writing 128 output rows, some
// six blocks' worth of K/V traffic (the span kernel gained 7% at 6). A
// narrow segment's setup mostly hides under its first loads: a cost of 3,
// measured with a pause before each run, left the Llama-3-8B-shaped batch
// unchanged, gained 0.3-1% on the long-context and fp8 batches and lost 1%
// on the hybrid batch and 10% on a tiny one, so narrow segments carry none.
// A group tile's segment starts with a chain of dependent loads (its members'
// entries, their query rows, the block ids, the first blocks and their
// scales): timed per wave on the parallel-sampling batch, 5.9 us per segment
// against 0.73 us per fp8 block, so about eight blocks. It is charged where
// the group and narrow pieces share one launch (batches without spans),
// whose end is its slowest wave's; beside a span launch it measured slower.
#ifndef PA_PART_COST
#define PA_PART_COST 0
#endif
#ifndef PA_PART_COST_WIDE
#define PA_PART_COST_WIDE 6
#endif
#ifndef PA_PART_COST_GROUP
#define PA_PART_COST_GROUP 8
#endif

// Scratch of pa_paged_attn_hybrid_noalloc, in static device memory: each
// GPU the library runs on holds its own copy until the process ends. Host
// code never passes this name to a kernel (on the host it is only a stand-in
// for the symbol); it uses the device address that hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

// A call whose batch holds span tiles and single-token tiles runs the span
// launch on the caller's stream and the narrow and group launches on a
// second stream of the library's, so that the two run side by side (1); or
// every launch on the caller's stream, one after another (0).
#ifndef PA_SIDE_STREAM
#define PA_SIDE_STREAM 1
#endif
// A decode batch with shared-prefix groups runs its group and narrow streams
// in one launch (1) or in one launch each (0).
#ifndef PA_NARROW_PAIR
#define PA_NARROW_PAIR 1
#endif

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int cdiv(int a, int b) { return (a + b - 1) / b; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Layout {
    int part_blocks = 0;  // blocks per piece, 0 = balanced over resident waves
    int narrow_tokens = 0, wide_tokens = 0;
    int waves[pa::NUM_STREAMS] = {};
    int part_cost[pa::NUM_STREAMS] = {};
    int span_shared = 0;  // span workgroups beside the narrow launches (0: none)
    int64_t max_tiles = 0;
    int64_t max_pieces[pa::NUM_STREAMS] = {};
    int64_t max_splits = 0;  // bound of the cut-segment list
    size_t off_tiles = 0, off_splits = 0, total = 0;
    size_t off_pieces[pa::NUM_STREAMS] = {};
    size_t off_lse[pa::NUM_STREAMS] = {};
    size_t off_o[pa::NUM_STREAMS] = {};
    // cascade (shared-prefix groups), when the shape allows them
    bool cascade = false;
    int members_per_tile = 0;
    int64_t max_cas_recs = 0;
    size_t off_cas_seq = 0;  // 6 int arrays of num_seqs
    size_t off_cas_recs = 0;
    size_t off_cas_lse[2] = {0, 0}, off_cas_o[2] = {0, 0};
    size_t off_tree = 0;  // [num_tokens] uint64 tree masks
};

int check_shape(const pa_shape* s) {
    if (!s) return PA_EINVAL;
    if (s->num_q_heads <= 0 || s->num_kv_heads <= 0) return PA_EINVAL;
    if (s->num_q_heads % s->num_kv_heads) return PA_EINVAL;
    if (s->num_q_heads / s->num_kv_heads > 16) return PA_ENOTSUP;
    if (s->head_dim != 64 && s->head_dim != 128) return PA_EINVAL;
    if (s->block_size != PA_BLOCK_SIZE) return PA_EINVAL;
    if (s->num_blocks <= 0 || s->max_blocks_per_seq <= 0) return PA_EINVAL;
    const bool ok = (s->q_dtype == PA_F32 && s->kv_dtype == PA_F32) ||
                    (s->q_dtype == PA_BF16 && s->kv_dtype == PA_BF16) ||
                    (s->q_dtype == PA_BF16 && s->kv_dtype == PA_FP8_E4M3FN);
    if (!ok) return PA_EINVAL;
    if (s->partition_size < 0 || s->partition_size % PA_BLOCK_SIZE) return PA_EINVAL;
    if (s->cascade != 0 && s->cascade != 1) return PA_EINVAL;
    if (s->fp8_qk != 0 && (s->fp8_qk != 1 || s->kv_dtype != PA_FP8_E4M3FN)) return PA_EINVAL;
    return PA_OK;
}

// The attention kernels' kind: the cache dtype, or fp8 with QK on the fp8
// matrix cores.
int kernel_kind(const pa_shape* s) {
    return s->kv_dtype == PA_FP8_E4M3FN && s->fp8_qk ? pa::KIND_FP8_QK : s->kv_dtype;
}

// Upper bound of resident attention waves when no device can be queried
// (256 compute units x 32 waves).
constexpr int kWaveBound = 8192;

// Workspace: [header][tiles][cut segments] then, per stream, [piece
// starts][partial lse][partial outputs].
// Spans of more than narrow_tokens query tokens get wide tiles; a batch
// whose max_query_len is below that has none and no wide region.
Layout make_layout(const pa_shape* s, int num_seqs, int num_tokens, int max_context_len,
                   int max_query_len, bool decode) {
    Layout l;
    const int G = s->num_q_heads / s->num_kv_heads;
    l.narrow_tokens = decode ? 1 : (16 / G > 1 ? 16 / G : 1);
    l.wide_tokens = pa::kSpanRows / G > 1 ? pa::kSpanRows / G : 1;
    l.part_blocks = s->partition_size / PA_BLOCK_SIZE;
    // wide tiles for spans longer than a narrow tile (0: every span in narrow
    // tiles). The span kernel computes on the bf16 matrix cores, so f32
    // caches, which need f32 products, keep their spans in narrow tiles.
    const bool spans = PA_WIDE_SPANS && !decode && max_query_len > l.narrow_tokens &&
                       s->kv_dtype != PA_F32;
    if (!spans) l.wide_tokens = 0;
    if (spans && PA_SIDE_STREAM) l.span_shared = pa::span_shared_groups(kernel_kind(s), s->head_dim);
    l.cascade = s->cascade != 0;
    // a group tile holds the single query tokens of up to 16 / G members
    l.members_per_tile = 16 * pa::kGroupRowTiles / G > 1 ? 16 * pa::kGroupRowTiles / G : 1;
    // (spans are disjoint, so no stream has more tiles than query tokens)
    const int64_t T = num_tokens;
    const int64_t tiles_of[pa::NUM_STREAMS] = {
        spans ? std::min((int64_t)num_seqs + cdiv(num_tokens, l.wide_tokens), T) : 0,
        // narrow: one per sequence, or every span cut into narrow tiles
        spans || decode ? (int64_t)num_seqs
                        : std::min((int64_t)num_seqs + cdiv(num_tokens, l.narrow_tokens), T),
        // shared-prefix groups' tiles (at most one per group plus one per
        // members_per_tile members, each sequence in at most one group)
        l.cascade ? 2 * (int64_t)num_seqs : 0};
    l.max_tiles = tiles_of[0] + tiles_of[1] + tiles_of[2];
    const int64_t blocks_per_tile = cdiv(max_context_len > 0 ? max_context_len : 1, PA_BLOCK_SIZE);
    size_t off = align_up(sizeof(int32_t) * pa::HDR_WORDS);
    l.off_tiles = off;
    off = align_up(off + sizeof(pa::TileDesc) * (size_t)l.max_tiles);
    int64_t splits = 0;
    for (int st = 0; st < pa::NUM_STREAMS; ++st) {
        const int w = pa::resident_waves(kernel_kind(s), s->head_dim, st);
        l.waves[st] = w > 0 ? w : kWaveBound;
        l.part_cost[st] = st == pa::STREAM_WIDE                ? PA_PART_COST_WIDE
                          : st == pa::STREAM_GROUP && !spans ? PA_PART_COST_GROUP
                                                              : PA_PART_COST;
        // pieces per KV head substream: ceil(B / R) with B <= tiles * blocks
        // per tile, and R = P / 16, or R >= Hkv * B / waves when balanced
        const int64_t H = s->num_kv_heads;
        const int64_t per_head = l.part_blocks > 0
                                     ? cdiv(tiles_of[st] * blocks_per_tile, (int64_t)l.part_blocks)
                                     : cdiv((int64_t)l.waves[st], H);
        int64_t mp = H * per_head;
        if (tiles_of[st] == 0) mp = 0;
        l.max_pieces[st] = mp;
        // a cut segment holds an inner piece boundary of its substream (at
        // most per_head - 1 each), and each (tile, KV head) is one segment
        if (mp > 0) splits += std::min(mp - H, tiles_of[st] * H);
    }
    l.max_splits = splits;
    l.off_splits = off;
    off = align_up(off + sizeof(pa::SplitSeg) * (size_t)(splits > 0 ? splits : 1));
    l.off_tree = off;
    off = align_up(off + sizeof(uint64_t) * (size_t)(num_tokens > 0 ? num_tokens : 1));
    if (l.cascade) {
        const size_t rows = (size_t)num_tokens * s->num_q_heads;
        l.max_cas_recs = (int64_t)num_seqs * s->num_kv_heads;
        l.off_cas_seq = off;
        off = align_up(off + sizeof(int32_t) * 6 * (size_t)num_seqs);
        l.off_cas_recs = off;
        off = align_up(off + sizeof(pa::CascadeRec) * (size_t)l.max_cas_recs);
        for (int k = 0; k < 2; ++k) {
            l.off_cas_lse[k] = off;
            off = align_up(off + sizeof(float) * rows);
            l.off_cas_o[k] = off;
            off = align_up(off + sizeof(float) * rows * s->head_dim);
        }
    }
    for (int st = 0; st < pa::NUM_STREAMS; ++st) {
        const int nt = pa::slot_row_tiles(st);
        const size_t slots = (size_t)l.max_pieces[st] * 2;
        l.off_pieces[st] = off;
        off = align_up(off + sizeof(pa::PieceStart) * (size_t)l.max_pieces[st]);
        l.off_lse[st] = off;
        off = align_up(off + sizeof(float) * slots * 16 * nt);
        l.off_o[st] = off;
        off = align_up(off + sizeof(float) * slots * 16 * nt * s->head_dim);
    }
    l.total = off;
    return l;
}

// Checks shared by plan and run; fills the layout.
int check_batch(const pa_shape* s, const int32_t* context_lens, const int32_t* qsl,
                int num_seqs, int num_tokens, int max_query_len, int max_context_len,
                void* workspace, size_t workspace_bytes, Layout* l) {
    int rc = check_shape(s);
    if (rc != PA_OK) return rc;
    if (num_seqs < 0 || num_tokens < 0 || max_context_len < 0) return PA_EINVAL;
    if (qsl == nullptr && num_tokens != num_seqs) return PA_EINVAL;
    if (qsl != nullptr && num_seqs > 0 && num_tokens > 0 && max_query_len < 1) return PA_EINVAL;
    if ((int64_t)max_context_len > (int64_t)PA_BLOCK_SIZE * s->max_blocks_per_seq)
        return PA_EINVAL;
    if (num_seqs > 0 && !context_lens) return PA_EINVAL;
    // the kernels index output rows (query token x query head) with 32 bits
    if ((int64_t)num_tokens * s->num_q_heads >= (int64_t)INT32_MAX) return PA_ENOTSUP;
    *l = make_layout(s, num_seqs, num_tokens, max_context_len, max_query_len, qsl == nullptr);
    if (l->max_tiles > pa::kMaxTiles) return PA_ENOTSUP;
    if (!workspace || workspace_bytes < l->total) return PA_EWORKSPACE;
    if (((uintptr_t)workspace % kAlign) != 0) return PA_EINVAL;
    return PA_OK;
}

// Checks of the attention inputs and outputs (host-known properties only).
int check_io(const pa_shape* s, const void* out, const void* q, const void* k_cache,
             const void* v_cache, const float* k_scale, const float* v_scale,
             const int32_t* block_tables) {
    if (!out || !q || !k_cache || !v_cache || !block_tables) return PA_EINVAL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_EINVAL;
    if (s->kv_dtype == PA_FP8_E4M3FN && (!k_scale || !v_scale)) return PA_EINVAL;
    return PA_OK;
}

// Shared-prefix groups handed to a plan (device arrays, host counts).
struct Groups {
    int num_groups = 0, num_members = 0;
    const int32_t* offsets = nullptr;
    const int32_t* members = nullptr;
    const int32_t* prefix_blocks = nullptr;
    const uint64_t* tree_mask = nullptr;  // tree verification masks
};

int plan_impl(const pa_shape* s, const int32_t* context_lens, const int32_t* qsl, int num_seqs,
              int num_tokens, int max_query_len, int max_context_len, const Groups& grp,
              void* workspace, size_t workspace_bytes, void* stream) {
    Layout l;
    int rc = check_batch(s, context_lens, qsl, num_seqs, num_tokens, max_query_len,
                         max_context_len, workspace, workspace_bytes, &l);
    if (rc != PA_OK) return rc;
    if (grp.num_groups < 0 || grp.num_members < 0) return PA_EINVAL;
    if (grp.num_groups > 0) {
        if (!l.cascade) return PA_EINVAL;  // the shape reserved no room for groups
        if (grp.num_groups > num_seqs || grp.num_members > num_seqs) return PA_EINVAL;
        if (!grp.offsets || !grp.members || !grp.prefix_blocks) return PA_EINVAL;
    }
    if (num_seqs == 0 || num_tokens == 0) return PA_OK;
    char* ws = (char*)workspace;
    pa::PlanArgs pl{};
    pl.context_lens = context_lens;
    pl.qsl = qsl;
    pl.num_seqs = num_seqs;
    pl.num_tokens = num_tokens;
    pl.max_context_len = max_context_len;
    pl.narrow_tokens = l.narrow_tokens;
    pl.wide_tokens = l.wide_tokens;
    pl.num_kv_heads = s->num_kv_heads;
    pl.part_blocks = l.part_blocks;
    for (int st = 0; st < pa::NUM_STREAMS; ++st)
        pl.min_blocks[st] = st == pa::STREAM_GROUP ? pa::kGroupMinPieceBlocks : pa::kMinPieceBlocks;
    pl.span_shared = l.span_shared;
    pl.max_tiles = (int32_t)l.max_tiles;
    pl.tiles = (pa::TileDesc*)(ws + l.off_tiles);
    for (int st = 0; st < pa::NUM_STREAMS; ++st) {
        pl.part_cost[st] = l.part_cost[st];
        pl.waves[st] = l.waves[st];
        pl.max_pieces[st] = l.max_pieces[st];
        pl.pieces[st] = (pa::PieceStart*)(ws + l.off_pieces[st]);
    }
    pl.splits = (pa::SplitSeg*)(ws + l.off_splits);
    pl.max_splits = l.max_splits;
    pl.hdr = (int32_t*)ws;
    pl.tree_mask = grp.tree_mask;
    pl.tree_ws = (uint64_t*)(ws + l.off_tree);
    if (l.cascade) {
        pl.num_groups = grp.num_groups;
        pl.members_per_tile = l.members_per_tile;
        pl.group_offsets = grp.offsets;
        pl.group_members = grp.members;
        pl.group_prefix_blocks = grp.prefix_blocks;
        int32_t* cs = (int32_t*)(ws + l.off_cas_seq);
        pl.cas_prefix = cs;
        pl.cas_tile = cs + num_seqs;
        pl.cas_gtile = cs + 2 * (size_t)num_seqs;
        pl.cas_pos = cs + 3 * (size_t)num_seqs;
        pl.cas_members = cs + 4 * (size_t)num_seqs;
        pl.cas_gbase = cs + 5 * (size_t)num_seqs;
        pl.cas_recs = (pa::CascadeRec*)(ws + l.off_cas_recs);
        pl.max_cas_recs = (int32_t)l.max_cas_recs;
    }
    return pa::launch_plan(pl, (hipStream_t)stream) == hipSuccess ? PA_OK : PA_EHIP;
}

// The library's second stream on a device (default priority), with the two
// events that fork it from the caller's stream and join it back. Made once
// per device, by pa_workspace_bytes for a batch that can hold spans or else
// by the first such call, and kept until the process ends. The mutex keeps
// one call's record / wait / launch sequence together when several host
// threads enqueue work on one device.
struct SideStream {
    std::once_flag once;
    std::atomic<bool> ok{false};
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    std::mutex m;
};
constexpr int kMaxSideDevices = 64;
SideStream g_side[kMaxSideDevices];

// The current device's side stream; made here if `create`, else only
// returned when it exists (nullptr: the call runs on the caller's stream).
SideStream* side_stream(bool create) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
    SideStream& d = g_side[dev];
    if (create) {
        std::call_once(d.once, [&d] {
            d.ok.store(hipStreamCreateWithFlags(&d.s, hipStreamNonBlocking) == hipSuccess &&
                           hipEventCreateWithFlags(&d.fork, hipEventDisableTiming) ==
                               hipSuccess &&
                           hipEventCreateWithFlags(&d.join, hipEventDisableTiming) == hipSuccess,
                       std::memory_order_release);
        });
    }
    return d.ok.load(std::memory_order_acquire) ? &d : nullptr;
}

// Which passes of the attention a call enqueues.
enum Passes { PASS_ATTENTION = 1, PASS_MERGE = 2, PASS_BOTH = 3 };

int run_impl(const pa_shape* s, void* out, float* lse, const void* q, const void* k_cache,
             const void* v_cache, const float* k_scale, const float* v_scale,
             const int32_t* block_tables, const int32_t* context_lens, const int32_t* qsl,
             int num_seqs, int num_tokens, int max_query_len, int max_context_len, float scale,
             void* workspace, size_t workspace_bytes, void* stream, int passes,
             const void* k_new = nullptr, const void* v_new = nullptr,
             bool side_create = true) {
    Layout l;
    int rc = check_batch(s, context_lens, qsl, num_seqs, num_tokens, max_query_len,
                         max_context_len, workspace, workspace_bytes, &l);
    if (rc != PA_OK) return rc;
    if (num_seqs == 0 || num_tokens == 0) return PA_OK;
    if (passes & PASS_ATTENTION) {
        rc = check_io(s, out, q, k_cache, v_cache, k_scale, v_scale, block_tables);
        if (rc != PA_OK) return rc;
        if ((k_new || v_new) &&
            (!k_new || !v_new || qsl || !aligned16(k_new) || !aligned16(v_new)))
            return PA_EINVAL;  // the append goes with decode plans only
    } else if (!out || !aligned16(out)) {
        return PA_EINVAL;
    }
    char* ws = (char*)workspace;
    hipStream_t hs = (hipStream_t)stream;
    if (passes & PASS_ATTENTION) {
        pa::AttnArgs aa{};
        aa.out = out;
        aa.lse = lse;
        aa.q = q;
        aa.k_cache = k_cache;
        aa.v_cache = v_cache;
        aa.k_scale = k_scale;
        aa.v_scale = v_scale;
        aa.block_tables = block_tables;
        aa.context_lens = context_lens;
        aa.qsl = qsl;
        aa.tiles = (const pa::TileDesc*)(ws + l.off_tiles);
        aa.hdr = (const int32_t*)ws;
        aa.num_q_heads = s->num_q_heads;
        aa.num_kv_heads = s->num_kv_heads;
        aa.group = s->num_q_heads / s->num_kv_heads;
        aa.num_blocks = s->num_blocks;
        aa.max_blocks_per_seq = s->max_blocks_per_seq;
        aa.max_context_len = max_context_len;
        aa.scale_log2 = scale * 1.44269504088896340736f;
        aa.num_seqs = num_seqs;
        aa.tree = (const uint64_t*)(ws + l.off_tree);

        if (l.cascade) {
            aa.cas_prefix = (const int32_t*)(ws + l.off_cas_seq);
            aa.group_members = (const int32_t*)(ws + l.off_cas_seq) + 4 * (size_t)num_seqs;
            for (int k = 0; k < 2; ++k) {
                aa.cas_lse[k] = (float*)(ws + l.off_cas_lse[k]);
                aa.cas_o[k] = (float*)(ws + l.off_cas_o[k]);
            }
        }
        // spans first (matrix-core heavy), then the single-token tiles. A
        // layout with span_shared > 0 forks the narrow and group launches
        // onto the side stream, so that they run beside the span launch
        // (the plan then cuts the span stream for one workgroup per compute
        // unit whenever the other streams hold most of the work), and joins
        // it back before the merge.
        SideStream* side = nullptr;
        if (l.span_shared > 0 && l.max_pieces[pa::STREAM_WIDE] > 0 &&
            (l.max_pieces[pa::STREAM_NARROW] > 0 || l.max_pieces[pa::STREAM_GROUP] > 0))
            side = side_stream(side_create);
        std::unique_lock<std::mutex> side_lock;
        if (side) {
            side_lock = std::unique_lock<std::mutex>(side->m);
            if (hipEventRecord(side->fork, hs) != hipSuccess ||
                hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess)
                return PA_EHIP;
        }
        bool failed = false;
        // no spans, group and narrow pieces: one launch for both streams
        const bool pair = PA_NARROW_PAIR && l.max_pieces[pa::STREAM_WIDE] == 0 &&
                          l.max_pieces[pa::STREAM_NARROW] > 0 &&
                          l.max_pieces[pa::STREAM_GROUP] > 0;
        if (pair) {
            pa::AttnArgs ga = aa, na = aa;
            ga.stream = pa::STREAM_GROUP;
            na.stream = pa::STREAM_NARROW;
            for (pa::AttnArgs* x : {&ga, &na}) {
                x->pieces = (const pa::PieceStart*)(ws + l.off_pieces[x->stream]);
                x->part_lse = (float*)(ws + l.off_lse[x->stream]);
                x->part_o = (float*)(ws + l.off_o[x->stream]);
            }
            ga.k_new = ga.v_new = nullptr;
            na.k_new = k_new;
            na.v_new = v_new;
            failed = pa::launch_narrow_pair(
                         kernel_kind(s), s->head_dim, ga, na,
                         std::max(l.max_pieces[pa::STREAM_GROUP], l.max_pieces[pa::STREAM_NARROW]),
                         hs) != hipSuccess;
        }
        for (int st = 0; st < pa::NUM_STREAMS && !failed && !pair; ++st) {
            if (l.max_pieces[st] == 0) continue;
            aa.stream = st;
            aa.pieces = (const pa::PieceStart*)(ws + l.off_pieces[st]);
            aa.part_lse = (float*)(ws + l.off_lse[st]);
            aa.part_o = (float*)(ws + l.off_o[st]);
            // the new rows go with the stream that holds the decodes' last
            // blocks (group tiles hold shared prefixes only)
            aa.k_new = st == pa::STREAM_NARROW ? k_new : nullptr;
            aa.v_new = st == pa::STREAM_NARROW ? v_new : nullptr;
            const hipStream_t ls = side && st != pa::STREAM_WIDE ? side->s : hs;
            failed = pa::launch_attention(kernel_kind(s), s->head_dim, aa, l.max_pieces[st], ls) !=
                     hipSuccess;
        }
        // the join is enqueued even after a failed launch, so that a graph
        // capture that forked the side stream gets it back
        if (side && (hipEventRecord(side->join, side->s) != hipSuccess ||
                     hipStreamWaitEvent(hs, side->join, 0) != hipSuccess))
            failed = true;
        if (failed) return PA_EHIP;
    }
    if (passes & PASS_MERGE) {
        pa::MergeArgs ma{};
        ma.out = out;
        ma.lse = lse;
        ma.splits = (const pa::SplitSeg*)(ws + l.off_splits);
        ma.hdr = (const int32_t*)ws;
        for (int st = 0; st < pa::NUM_STREAMS; ++st) {
            ma.part_lse[st] = (const float*)(ws + l.off_lse[st]);
            ma.part_o[st] = (const float*)(ws + l.off_o[st]);
        }
        ma.num_q_heads = s->num_q_heads;
        ma.num_kv_heads = s->num_kv_heads;
        ma.group = s->num_q_heads / s->num_kv_heads;
        ma.wide_nt = pa::kSpanRowTiles;
        ma.max_splits = (int32_t)l.max_splits;
        int64_t records = l.max_splits;
        if (l.cascade) {
            ma.cas_recs = (const pa::CascadeRec*)(ws + l.off_cas_recs);
            for (int k = 0; k < 2; ++k) {
                ma.cas_lse[k] = (const float*)(ws + l.off_cas_lse[k]);
                ma.cas_o[k] = (const float*)(ws + l.off_cas_o[k]);
            }
            records += l.max_cas_recs;
        }
        if (records > 0 && pa::launch_merge(s->q_dtype, s->head_dim, ma, records,
                                            l.max_pieces[pa::STREAM_WIDE] > 0, hs) != hipSuccess)
            return PA_EHIP;
    }
    return PA_OK;
}

// Workspace bytes of a batch; *spans_beside: its span launch may run beside
// the single-token launches (on the side stream).
size_t workspace_bytes_of(const pa_shape* shape, int num_seqs, int num_q_tokens,
                          int max_context_len, int max_query_len, bool* spans_beside) {
    if (check_shape(shape) != PA_OK || num_seqs < 0 || num_q_tokens < 0 || max_context_len < 0)
        return 0;
    const bool decode = max_query_len <= 1 && num_q_tokens == num_seqs;
    // a decode-shaped hybrid call may use either layout: size for the larger
    Layout a = make_layout(shape, num_seqs, num_q_tokens, max_context_len, max_query_len, decode);
    Layout b = make_layout(shape, num_seqs, num_q_tokens, max_context_len, max_query_len, false);
    *spans_beside = b.span_shared > 0;
    return a.total > b.total ? a.total : b.total;
}

// One hybrid call: plan, attention and merge on the caller's stream (and
// the side stream). side_create false: the side stream is used only if it
// already exists (the no-alloc entry point makes nothing).
int hybrid_impl(const pa_shape* shape, void* out, float* lse, const void* q, const void* k_cache,
                const void* v_cache, const float* k_scale, const float* v_scale,
                const int32_t* block_tables, const int32_t* context_lens,
                const int32_t* query_start_loc, int num_seqs, int num_q_tokens,
                int max_query_len, int max_context_len, float scale, void* workspace,
                size_t workspace_bytes, void* stream, bool side_create) {
    if (check_shape(shape) != PA_OK) return check_shape(shape);
    if (!query_start_loc) return PA_EINVAL;
    if (num_seqs > 0 && num_q_tokens > 0) {
        int rc0 = check_io(shape, out, q, k_cache, v_cache, k_scale, v_scale, block_tables);
        if (rc0 != PA_OK) return rc0;
    }
    int rc = plan_impl(shape, context_lens, query_start_loc, num_seqs, num_q_tokens,
                       max_query_len, max_context_len, Groups{}, workspace, workspace_bytes, stream);
    if (rc != PA_OK) return rc;
    return run_impl(shape, out, lse, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                    context_lens, query_start_loc, num_seqs, num_q_tokens, max_query_len,
                    max_context_len, scale, workspace, workspace_bytes, stream, PASS_BOTH,
                    nullptr, nullptr, side_create);
}

}  // namespace

extern "C" {

size_t pa_workspace_bytes(const pa_shape* shape, int num_seqs, int num_q_tokens,
                          int max_context_len, int max_query_len) {
    bool spans_beside = false;
    const size_t n = workspace_bytes_of(shape, num_seqs, num_q_tokens, max_context_len,
                                        max_query_len, &spans_beside);
    // a batch that can hold spans beside single-token tiles uses the side
    // stream: make it now, before the caller can capture a call
    if (spans_beside) side_stream(true);
    return n;
}

int pa_plan(const pa_shape* shape, const int32_t* context_lens, const int32_t* query_start_loc,
            int num_seqs, int num_q_tokens, int max_query_len, int max_context_len,
            void* workspace, size_t workspace_bytes, void* stream) {
    return plan_impl(shape, context_lens, query_start_loc, num_seqs, num_q_tokens, max_query_len,
                     max_context_len, Groups{}, workspace, workspace_bytes, stream);
}

int pa_plan_cascade(const pa_shape* shape, const int32_t* context_lens,
                    const int32_t* query_start_loc, int num_seqs, int num_q_tokens,
                    int max_query_len, int max_context_len, int num_groups, int num_members,
                    const int32_t* group_offsets, const int32_t* group_members,
                    const int32_t* group_prefix_blocks, void* workspace, size_t workspace_bytes,
                    void* stream) {
    Groups grp;
    grp.num_groups = num_groups;
    grp.num_members = num_members;
    grp.offsets = group_offsets;
    grp.members = group_members;
    grp.prefix_blocks = group_prefix_blocks;
    return plan_impl(shape, context_lens, query_start_loc, num_seqs, num_q_tokens, max_query_len,
                     max_context_len, grp, workspace, workspace_bytes, stream);
}

int pa_plan_tree(const pa_shape* shape, const int32_t* context_lens,
                 const int32_t* query_start_loc, int num_seqs, int num_q_tokens, int max_query_len,
                 int max_context_len, const uint64_t* tree_mask, void* workspace,
                 size_t workspace_bytes, void* stream) {
    if (!query_start_loc || !tree_mask) return PA_EINVAL;
    Groups grp;
    grp.tree_mask = tree_mask;
    return plan_impl(shape, context_lens, query_start_loc, num_seqs, num_q_tokens, max_query_len,
                     max_context_len, grp, workspace, workspace_bytes, stream);
}

int pa_paged_attn_run(const pa_shape* shape, void* out, float* lse, const void* q,
                      const void* k_cache, const void* v_cache, const float* k_scale,
                      const float* v_scale, const int32_t* block_tables,
                      const int32_t* context_lens, const int32_t* query_start_loc, int num_seqs,
                      int num_q_tokens, int max_query_len, int max_context_len, float scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
    return run_impl(shape, out, lse, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                    context_lens, query_start_loc, num_seqs, num_q_tokens, max_query_len,
                    max_context_len, scale, workspace, workspace_bytes, stream, PASS_BOTH);
}

int pa_paged_attn_partial(const pa_shape* shape, void* out, float* lse, const void* q,
                          const void* k_cache, const void* v_cache, const float* k_scale,
                          const float* v_scale, const int32_t* block_tables,
                          const int32_t* context_lens, const int32_t* query_start_loc,
                          int num_seqs, int num_q_tokens, int max_query_len, int max_context_len,
                          float scale, void* workspace, size_t workspace_bytes, void* stream) {
    return run_impl(shape, out, lse, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                    context_lens, query_start_loc, num_seqs, num_q_tokens, max_query_len,
                    max_context_len, scale, workspace, workspace_bytes, stream, PASS_ATTENTION);
}

int pa_paged_attn_merge(const pa_shape* shape, void* out, float* lse, const int32_t* context_lens,
                        const int32_t* query_start_loc, int num_seqs, int num_q_tokens,
                        int max_query_len, int max_context_len, void* workspace,
                        size_t workspace_bytes, void* stream) {
    return run_impl(shape, out, lse, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                    context_lens, query_start_loc, num_seqs, num_q_tokens, max_query_len,
                    max_context_len, 0.f, workspace, workspace_bytes, stream, PASS_MERGE);
}

int pa_paged_attn_decode(const pa_shape* shape, void* out, float* lse, const void* q,
                         const void* k_cache, const void* v_cache, const float* k_scale,
                         const float* v_scale, const int32_t* block_tables,
                         const int32_t* context_lens, int num_seqs, int max_context_len,
                         float scale, void* workspace, size_t workspace_bytes, void* stream) {
    // check everything before enqueueing the plan
    if (check_shape(shape) != PA_OK) return check_shape(shape);
    if (num_seqs > 0) {
        int rc0 = check_io(shape, out, q, k_cache, v_cache, k_scale, v_scale, block_tables);
        if (rc0 != PA_OK) return rc0;
    }
    int rc = plan_impl(shape, context_lens, nullptr, num_seqs, num_seqs, 1, max_context_len,
                       Groups{}, workspace, workspace_bytes, stream);
    if (rc != PA_OK) return rc;
    return run_impl(shape, out, lse, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                    context_lens, nullptr, num_seqs, num_seqs, 1, max_context_len, scale,
                    workspace, workspace_bytes, stream, PASS_BOTH);
}

int pa_paged_attn_run_append(const pa_shape* shape, void* out, float* lse, const void* q,
                             const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int num_seqs, int max_context_len, float scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
    return run_impl(shape, out, lse, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                    context_lens, nullptr, num_seqs, num_seqs, 1, max_context_len, scale,
                    workspace, workspace_bytes, stream, PASS_BOTH, k_new, v_new);
}

int pa_paged_attn_partial_append(const pa_shape* shape, void* out, float* lse, const void* q,
                                 const void* k_new, const void* v_new, void* k_cache,
                                 void* v_cache, const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int num_seqs, int max_context_len, float scale,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    return run_impl(shape, out, lse, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                    context_lens, nullptr, num_seqs, num_seqs, 1, max_context_len, scale,
                    workspace, workspace_bytes, stream, PASS_ATTENTION, k_new, v_new);
}

int pa_paged_attn_decode_append(const pa_shape* shape, void* out, float* lse, const void* q,
                                const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, const float* k_scale, const float* v_scale,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int num_seqs, int max_context_len, float scale, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (check_shape(shape) != PA_OK) return check_shape(shape);
    if (num_seqs > 0) {
        int rc0 = check_io(shape, out, q, k_cache, v_cache, k_scale, v_scale, block_tables);
        if (rc0 != PA_OK) return rc0;
        if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return PA_EINVAL;
    }
    int rc = plan_impl(shape, context_lens, nullptr, num_seqs, num_seqs, 1, max_context_len,
                       Groups{}, workspace, workspace_bytes, stream);
    if (rc != PA_OK) return rc;
    return run_impl(shape, out, lse, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                    context_lens, nullptr, num_seqs, num_seqs, 1, max_context_len, scale,
                    workspace, workspace_bytes, stream, PASS_BOTH, k_new, v_new);
}

int pa_paged_attn_hybrid(const pa_shape* shape, void* out, float* lse, const void* q,
                         const void* k_cache, const void* v_cache, const float* k_scale,
                         const float* v_scale, const int32_t* block_tables,
                         const int32_t* context_lens, const int32_t* query_start_loc,
                         int num_seqs, int num_q_tokens, int max_query_len,
                         int max_context_len, float scale, void* workspace,
                         size_t workspace_bytes, void* stream) {
    return hybrid_impl(shape, out, lse, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                       context_lens, query_start_loc, num_seqs, num_q_tokens, max_query_len,
                       max_context_len, scale, workspace, workspace_bytes, stream, true);
}

int pa_kv_append(const pa_shape* shape, void* k_cache, void* v_cache, const float* k_scale,
                 const float* v_scale, const void* k_new, const void* v_new,
                 const int32_t* slot_mapping, int num_tokens, void* stream) {
    int rc = check_shape(shape);
    if (rc != PA_OK) return rc;
    if (num_tokens < 0) return PA_EINVAL;
    if (num_tokens == 0) return PA_OK;
    if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping) return PA_EINVAL;
    if (shape->kv_dtype == PA_FP8_E4M3FN && (!k_scale || !v_scale)) return PA_EINVAL;
    pa::AppendArgs a{k_cache,      v_cache,    k_scale,
                     v_scale,      k_new,      v_new,
                     slot_mapping, num_tokens, shape->num_kv_heads,
                     shape->head_dim, shape->num_blocks};
    if (pa::launch_append(shape->q_dtype, shape->kv_dtype, a, (hipStream_t)stream) != hipSuccess)
        return PA_EHIP;
    return PA_OK;
}

int pa_fp8_e4m3fn_to_f32(const uint8_t* in, float* out, int n, void* stream) {
    if (n < 0 || (n > 0 && (!in || !out))) return PA_EINVAL;
    return pa::launch_fp8_decode(in, out, n, (hipStream_t)stream) == hipSuccess ? PA_OK
                                                                                : PA_EHIP;
}

int pa_copy_blocks(const pa_shape* shape, void* k_cache, void* v_cache, float* k_scale,
                   float* v_scale, const int32_t* pairs, int num_pairs, void* stream) {
    int rc = check_shape(shape);
    if (rc != PA_OK) return rc;
    if (num_pairs < 0) return PA_EINVAL;
    if (num_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !pairs || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_EINVAL;
    const bool fp8 = shape->kv_dtype == PA_FP8_E4M3FN;
    if (fp8 && (!k_scale || !v_scale)) return PA_EINVAL;
    const int eb = shape->kv_dtype == PA_F32 ? 4 : shape->kv_dtype == PA_BF16 ? 2 : 1;
    pa::CopyArgs ca{};
    ca.k_cache = k_cache;
    ca.v_cache = v_cache;
    ca.k_scale = fp8 ? k_scale : nullptr;
    ca.v_scale = fp8 ? v_scale : nullptr;
    ca.pairs = pairs;
    ca.block_bytes = (int64_t)shape->num_kv_heads * PA_BLOCK_SIZE * shape->head_dim * eb;
    ca.num_blocks = shape->num_blocks;
    ca.num_kv_heads = shape->num_kv_heads;
    return pa::launch_copy_blocks(ca, num_pairs, (hipStream_t)stream) == hipSuccess ? PA_OK
                                                                                  : PA_EHIP;
}

}  // extern "C"

namespace {

// The scratch array's device address per device, looked up once per
// device, with that device current, on the first no-alloc call there.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

void* scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int pa_paged_attn_hybrid_noalloc(const pa_shape* shape, void* out, float* lse, const void* q,
                                 const void* k_cache, const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* block_tables,
                                 const int32_t* context_lens, const int32_t* query_start_loc,
                                 int num_seqs, int num_q_tokens, int max_query_len,
                                 int max_context_len, float scale, void* stream) {
    if (check_shape(shape) != PA_OK) return check_shape(shape);
    if (num_seqs < 0 || num_q_tokens < 0 || max_context_len < 0) return PA_EINVAL;
    bool spans_beside = false;
    const size_t need = workspace_bytes_of(shape, num_seqs, num_q_tokens, max_context_len,
                                           max_query_len, &spans_beside);
    if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ESCRATCH;
    void* ws = scratch_address();
    if (!ws) return PA_EHIP;
    return hybrid_impl(shape, out, lse, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                       context_lens, query_start_loc, num_seqs, num_q_tokens, max_query_len,
                       max_context_len, scale, ws, (size_t)PA_NOALLOC_SCRATCH_BYTES, stream,
                       false);
}

int pa_workspace_layout(const pa_shape* shape, int num_seqs, int num_q_tokens,
                        int max_context_len, int max_query_len, int decode,
                        pa_layout_info* info) {
    if (!info || check_shape(shape) != PA_OK || num_seqs < 0 || num_q_tokens < 0 ||
        max_context_len < 0)
        return PA_EINVAL;
    const Layout l = make_layout(shape, num_seqs, num_q_tokens, max_context_len, max_query_len,
                                 decode != 0);
    pa_layout_info r{};
    for (int st = 0; st < pa::NUM_STREAMS; ++st) {
        r.waves[st] = l.waves[st];
        r.part_cost[st] = l.part_cost[st];
        r.max_pieces[st] = l.max_pieces[st];
        r.off_pieces[st] = (int64_t)l.off_pieces[st];
        r.off_part_lse[st] = (int64_t)l.off_lse[st];
        r.off_part_o[st] = (int64_t)l.off_o[st];
    }
    r.span_shared = l.span_shared;
    r.narrow_tokens = l.narrow_tokens;
    r.wide_tokens = l.wide_tokens;
    r.part_blocks = l.part_blocks;
    r.members_per_tile = l.members_per_tile;
    r.wide_row_tiles = pa::kSpanRowTiles;
    r.group_row_tiles = pa::kGroupRowTiles;
    r.header_words = pa::HDR_WORDS;
    r.max_tiles = l.max_tiles;
    r.max_splits = l.max_splits;
    r.max_cas_recs = l.max_cas_recs;
    r.off_tiles = (int64_t)l.off_tiles;
    r.off_splits = (int64_t)l.off_splits;
    r.off_tree = (int64_t)l.off_tree;
    r.off_cas_seq = (int64_t)l.off_cas_seq;
    r.off_cas_recs = (int64_t)l.off_cas_recs;
    for (int k = 0; k < 2; ++k) {
        r.off_cas_lse[k] = (int64_t)l.off_cas_lse[k];
        r.off_cas_o[k] = (int64_t)l.off_cas_o[k];
    }
    r.total = (int64_t)l.total;
    *info = r;
    return PA_OK;
}

const char* pa_status_string(int status) {
    switch (status) {
    case PA_OK: return "ok";
    case PA_EINVAL: return "invalid argument";
    case PA_EWORKSPACE: return "workspace missing or too small";
    case PA_EHIP: return "HIP runtime or launch error";
    case PA_ENOTSUP: return "not supported";
    case PA_ENOMEM: return "no free block";
    case PA_ESCRATCH: return "batch needs more than the static scratch buffer holds";
    default: return "unknown status";
    }
}

int pa_version(void) { return 211; }

}  // extern "C"
