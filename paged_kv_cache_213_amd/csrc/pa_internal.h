// pa_internal.h -- structures shared by the host launchers and the gfx950
// kernels of the paged-attention library. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

// One unit of attention work before the KV-head fan-out: the query rows of
// one tile of a sequence's span, over one partition of its keys.
struct WorkItem {
    int32_t seq;    // sequence index
    int32_t qtok0;  // first query token of the tile, relative to the span
    int32_t part;   // partition index: keys [part * P, (part + 1) * P)
    int32_t ntok;   // query tokens in the tile (1 for a decode)
};

// Header words at the start of the workspace.
enum { HDR_NITEMS = 0, HDR_COUNTER = 1, HDR_WORDS = 64 };

struct PlanArgs {
    const int32_t* context_lens;
    const int32_t* qsl;  // nullptr: one query token per sequence
    int32_t num_seqs;
    int32_t num_tokens;
    int32_t max_context_len;  // contexts are clamped to this
    int32_t part_size;
    int32_t tile_tokens;
    int64_t max_items;  // capacity of `items`
    WorkItem* items;
    int32_t* hdr;
    int32_t* tok_np;  // per query token: partitions of its tile
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
    const WorkItem* items;
    int32_t* hdr;
    float* part_lse;  // [T][Hq][max_parts], log2 units
    float* part_o;    // [T][Hq][max_parts][D], normalized
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t num_blocks;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    int32_t part_size;
    int32_t max_parts;
    float scale_log2;  // softmax scale times log2(e)
};

struct MergeArgs {
    void* out;
    float* lse;
    const int32_t* tok_np;
    const float* part_lse;
    const float* part_o;
    int32_t num_tokens;
    int32_t num_q_heads;
    int32_t max_parts;
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

// Launchers (host side), defined next to their kernels.
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_attention(int kv_dtype, int head_dim, const AttnArgs& a, int64_t max_units,
                            hipStream_t s);
hipError_t launch_merge(int q_dtype, int head_dim, const MergeArgs& a, hipStream_t s);
hipError_t launch_append(int new_dtype, int kv_dtype, const AppendArgs& a, hipStream_t s);
hipError_t launch_fp8_decode(const uint8_t* in, float* out, int n, hipStream_t s);

constexpr int kDefaultPartition = 512;

}  // namespace pa
