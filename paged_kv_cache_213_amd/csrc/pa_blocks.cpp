// pa_blocks.cpp -- host block manager of the paged KV cache: free list,
// per-sequence block tables, reference counts with copy-on-write, slot
// mapping, shared-prefix groups, and a host-side check of batch metadata.
// The structures follow "03 -- Engines Papers", section 2 (block table,
// copy-on-write with a refcount) and its whiteboard trace (allocate/free).
#include <stdint.h>

#include <algorithm>
#include <functional>
#include <map>
#include <queue>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pagedattn_blocks.h"

namespace {

constexpr int kB = PA_BLOCK_SIZE;

struct Seq {
    std::vector<int32_t> blocks;  // logical block -> physical block
    int32_t len = 0;              // tokens
};

}  // namespace

struct pa_block_manager {
    int32_t num_blocks = 0;
    int32_t max_blocks = 0;
    // free blocks, lowest id first: allocation stays compact and repeatable
    std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_list;
    std::vector<int32_t> refcount;
    std::vector<int32_t> fill;  // tokens held by each block
    std::unordered_map<int64_t, Seq> seqs;

    int32_t take() {
        const int32_t b = free_list.top();
        free_list.pop();
        refcount[b] = 1;
        fill[b] = 0;
        return b;
    }
    void release(int32_t b) {
        if (--refcount[b] == 0) {
            fill[b] = 0;
            free_list.push(b);
        }
    }
    // Blocks a sequence of len tokens needs.
    static int32_t blocks_for(int64_t len) { return (int32_t)((len + kB - 1) / kB); }

    // Append n tokens to s (whose last block is private or full): new blocks
    // as needed, slots written. The caller has checked the free blocks.
    void write_tokens(Seq& s, int32_t n, int32_t* slots) {
        for (int32_t k = 0; k < n; ++k) {
            const int32_t pos = s.len + k;
            if (pos % kB == 0 && pos / kB == (int32_t)s.blocks.size()) s.blocks.push_back(take());
            const int32_t b = s.blocks[pos / kB];
            fill[b] = std::max(fill[b], pos % kB + 1);
            if (slots) slots[k] = b * kB + pos % kB;
        }
        s.len += n;
    }
};

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t max_blocks_per_seq) {
    if (num_blocks <= 0 || max_blocks_per_seq <= 0) return nullptr;
    pa_block_manager* bm = new (std::nothrow) pa_block_manager;
    if (!bm) return nullptr;
    try {
        bm->num_blocks = num_blocks;
        bm->max_blocks = max_blocks_per_seq;
        bm->refcount.assign(num_blocks, 0);
        bm->fill.assign(num_blocks, 0);
        std::vector<int32_t> ids(num_blocks);
        for (int32_t i = 0; i < num_blocks; ++i) ids[i] = i;
        bm->free_list = decltype(bm->free_list)(std::greater<int32_t>(), std::move(ids));
    } catch (...) {
        delete bm;
        return nullptr;
    }
    return bm;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_add(pa_block_manager* bm, int64_t seq, int32_t num_tokens, int32_t* slots) {
    if (!bm || num_tokens < 0 || bm->seqs.count(seq)) return PA_EINVAL;
    const int32_t need = pa_block_manager::blocks_for(num_tokens);
    if (need > bm->max_blocks) return PA_EINVAL;
    if (need > (int32_t)bm->free_list.size()) return PA_ENOMEM;
    Seq& s = bm->seqs[seq];
    bm->write_tokens(s, num_tokens, slots);
    return PA_OK;
}

int pa_bm_add_shared(pa_block_manager* bm, int64_t seq, int64_t owner, int32_t prefix_blocks,
                     int32_t num_tokens, int32_t* slots) {
    if (!bm || num_tokens < 0 || prefix_blocks < 0 || bm->seqs.count(seq)) return PA_EINVAL;
    auto it = bm->seqs.find(owner);
    if (it == bm->seqs.end()) return PA_EINVAL;
    const Seq& o = it->second;
    // only full blocks of the owner can be shared as a prefix
    if ((int64_t)prefix_blocks * kB > o.len) return PA_EINVAL;
    const int64_t len = (int64_t)prefix_blocks * kB + num_tokens;
    if (pa_block_manager::blocks_for(len) > bm->max_blocks) return PA_EINVAL;
    if (pa_block_manager::blocks_for(len) - prefix_blocks > (int32_t)bm->free_list.size())
        return PA_ENOMEM;
    Seq s;
    s.blocks.assign(o.blocks.begin(), o.blocks.begin() + prefix_blocks);
    for (int32_t b : s.blocks) ++bm->refcount[b];
    s.len = prefix_blocks * kB;
    bm->write_tokens(s, num_tokens, slots);
    bm->seqs.emplace(seq, std::move(s));
    return PA_OK;
}

int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
    if (!bm || parent == child || bm->seqs.count(child)) return PA_EINVAL;
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end()) return PA_EINVAL;
    Seq s = it->second;
    for (int32_t b : s.blocks) ++bm->refcount[b];
    bm->seqs.emplace(child, std::move(s));
    return PA_OK;
}

int pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t num_tokens, int32_t* slots,
                 int32_t* copy_pair, int32_t* num_copies) {
    if (!bm || num_tokens < 0) return PA_EINVAL;
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return PA_EINVAL;
    Seq& s = it->second;
    const int64_t len = (int64_t)s.len + num_tokens;
    if (pa_block_manager::blocks_for(len) > bm->max_blocks) return PA_EINVAL;
    // copy-on-write: the partly filled last block is shared
    const bool cow = num_tokens > 0 && s.len % kB != 0 && bm->refcount[s.blocks.back()] > 1;
    if (cow && !copy_pair) return PA_EINVAL;
    const int32_t need =
        pa_block_manager::blocks_for(len) - (int32_t)s.blocks.size() + (cow ? 1 : 0);
    if (need > (int32_t)bm->free_list.size()) return PA_ENOMEM;
    if (num_copies) *num_copies = 0;
    if (cow) {
        const int32_t src = s.blocks.back();
        const int32_t dst = bm->take();
        bm->fill[dst] = s.len % kB;
        --bm->refcount[src];  // still held by the other sharers
        s.blocks.back() = dst;
        copy_pair[0] = src;
        copy_pair[1] = dst;
        if (num_copies) *num_copies = 1;
    }
    bm->write_tokens(s, num_tokens, slots);
    return PA_OK;
}

int pa_bm_free(pa_block_manager* bm, int64_t seq) {
    if (!bm) return PA_EINVAL;
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return PA_EINVAL;
    for (int32_t b : it->second.blocks) bm->release(b);
    bm->seqs.erase(it);
    return PA_OK;
}

int32_t pa_bm_length(const pa_block_manager* bm, int64_t seq) {
    if (!bm) return -1;
    auto it = bm->seqs.find(seq);
    return it == bm->seqs.end() ? -1 : it->second.len;
}

int pa_bm_tables(const pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* tables,
                 int32_t row_stride, int32_t* context_lens) {
    if (!bm || n < 0 || (n > 0 && (!seqs || !tables || !context_lens)) || row_stride <= 0)
        return PA_EINVAL;
    for (int32_t i = 0; i < n; ++i) {
        auto it = bm->seqs.find(seqs[i]);
        if (it == bm->seqs.end() || (int32_t)it->second.blocks.size() > row_stride)
            return PA_EINVAL;
    }
    for (int32_t i = 0; i < n; ++i) {
        const Seq& s = bm->seqs.find(seqs[i])->second;
        int32_t* row = tables + (int64_t)i * row_stride;
        std::fill(row, row + row_stride, -1);
        std::copy(s.blocks.begin(), s.blocks.end(), row);
        context_lens[i] = s.len;
    }
    return PA_OK;
}

int pa_bm_prefix_groups(const pa_block_manager* bm, const int64_t* seqs, int32_t n,
                        int32_t* group_offsets, int32_t* group_members,
                        int32_t* group_prefix_blocks, int32_t* num_groups,
                        int32_t* num_members) {
    if (!bm || n < 0 || !group_offsets || !num_groups || !num_members ||
        (n > 0 && (!seqs || !group_members || !group_prefix_blocks)))
        return PA_EINVAL;
    std::vector<const Seq*> s(n);
    for (int32_t i = 0; i < n; ++i) {
        auto it = bm->seqs.find(seqs[i]);
        if (it == bm->seqs.end()) return PA_EINVAL;
        s[i] = &it->second;
    }
    // batch indices by first physical block, in batch order
    std::map<int32_t, std::vector<int32_t>> by_first;
    for (int32_t i = 0; i < n; ++i)
        if (!s[i]->blocks.empty()) by_first[s[i]->blocks[0]].push_back(i);
    int32_t g = 0, m = 0;
    group_offsets[0] = 0;
    for (auto& kv : by_first) {
        const std::vector<int32_t>& mem = kv.second;
        if (mem.size() < 2) continue;
        // leading entries all members share, full blocks only
        int32_t pb = INT32_MAX;
        for (int32_t i : mem) pb = std::min(pb, s[i]->len / kB);
        for (int32_t j = 0; j < pb; ++j) {
            const int32_t b = s[mem[0]]->blocks[j];
            bool same = true;
            for (int32_t i : mem) same = same && s[i]->blocks[j] == b;
            if (!same) {
                pb = j;
                break;
            }
        }
        if (pb < 1) continue;
        for (int32_t i : mem) group_members[m++] = i;
        group_prefix_blocks[g] = pb;
        group_offsets[++g] = m;
    }
    *num_groups = g;
    *num_members = m;
    return PA_OK;
}

int pa_bm_get_stats(const pa_block_manager* bm, pa_bm_stats* st) {
    if (!bm || !st) return PA_EINVAL;
    *st = pa_bm_stats{};
    st->num_blocks = bm->num_blocks;
    st->free_blocks = (int32_t)bm->free_list.size();
    st->used_blocks = bm->num_blocks - st->free_blocks;
    for (int32_t b = 0; b < bm->num_blocks; ++b) {
        if (bm->refcount[b] > 1) ++st->shared_blocks;
        if (bm->refcount[b] > 0) st->stored_tokens += bm->fill[b];
    }
    st->num_sequences = (int32_t)bm->seqs.size();
    for (const auto& kv : bm->seqs) st->logical_tokens += kv.second.len;
    st->utilization =
        st->used_blocks > 0 ? (double)st->stored_tokens / ((double)st->used_blocks * kB) : 1.0;
    return PA_OK;
}

int32_t pa_bm_refcount(const pa_block_manager* bm, int32_t block) {
    if (!bm || block < 0 || block >= bm->num_blocks) return -1;
    return bm->refcount[block];
}

int pa_validate_batch(int32_t num_blocks, int32_t max_blocks_per_seq,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* query_start_loc, const int32_t* slot_mapping,
                      int32_t num_seqs, int32_t num_tokens, const int32_t* refcounts,
                      int32_t* bad_seq) {
    int32_t dummy;
    if (!bad_seq) bad_seq = &dummy;
    *bad_seq = -1;
    if (num_blocks <= 0 || max_blocks_per_seq <= 0 || num_seqs < 0 || num_tokens < 0)
        return PA_EINVAL;
    if (num_seqs > 0 && (!block_tables || !context_lens)) return PA_EINVAL;
    if (!query_start_loc && num_tokens != num_seqs) return PA_EINVAL;
    if (query_start_loc && (query_start_loc[0] != 0 || query_start_loc[num_seqs] != num_tokens))
        return PA_EINVAL;
    std::unordered_set<int32_t> seen;
    for (int32_t i = 0; i < num_seqs; ++i) {
        const int32_t L = context_lens[i];
        const int32_t q0 = query_start_loc ? query_start_loc[i] : i;
        const int32_t n = query_start_loc ? query_start_loc[i + 1] - q0 : 1;
        const int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
        bool ok = L >= 0 && (int64_t)L <= (int64_t)kB * max_blocks_per_seq && n >= 0 && n <= L;
        for (int32_t j = 0; ok && j < (L + kB - 1) / kB; ++j)
            ok = row[j] >= 0 && row[j] < num_blocks;
        if (!ok) {
            *bad_seq = i;
            return PA_EINVAL;
        }
        if (!slot_mapping) continue;
        for (int32_t k = 0; k < n; ++k) {
            const int32_t slot = slot_mapping[q0 + k];
            if (slot < 0) continue;  // skipped token
            const int32_t pos = L - n + k;
            const int32_t want = row[pos / kB] * kB + pos % kB;
            const bool shared = refcounts && refcounts[row[pos / kB]] > 1;
            if (slot != want || shared || !seen.insert(slot).second) {
                *bad_seq = q0 + k;
                return PA_EINVAL;
            }
        }
    }
    return PA_OK;
}

}  // extern "C"
