// blocks.cpp — host block manager of the per-layer memory policy ([Novita] §關鍵技術 1: each
// layer takes a full cache or a sliding window over one paged memory, with its own block-table
// strategy; [primer] §4.1: a sequence's blocks need not be contiguous and come from a pool).
//
// Layers with the same policy form a group with one block table and one slot mapping per
// step. A full group gives a sequence a new block at every page. A window group's row is a
// ring: ceil(S / P) sink columns kept for good, then R columns that the pages past them
// cycle through (page j in column sink_pages + (j - sink_pages) mod R), so a sequence never
// holds more than sink_pages + R blocks of the group and a block is reused once the window
// has left it. Free blocks are a stack per group: a released block is the next one handed out.
// Host code only (no device calls); not thread-safe.
#include <stdint.h>

#include <new>
#include <vector>

#include "../../include/pagedkv.h"

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Group {
    int32_t window = 0;  // 0: full cache
    int32_t sinks = 0;
    int32_t ring = 0;  // R (window groups)
    int32_t sink_pages = 0;
    int32_t cols = 0;  // row width of the table
    int32_t num_blocks = 0;
    std::vector<int32_t> free_ids;  // back() is handed out next
    std::vector<int32_t> table;     // [max_seqs][cols]; -1: no block yet
    int64_t in_use = 0;

    int64_t column(int64_t page) const {
        if (ring == 0 || page < sink_pages) return page;
        return sink_pages + (page - sink_pages) % ring;
    }
    // distinct columns of pages [0, ceil(L / P))
    int64_t blocks_for(int64_t L, int32_t P) const {
        const int64_t pages = ceil_div(L, P);
        if (ring == 0) return pages;
        const int64_t cap = (int64_t)sink_pages + ring;
        return pages < cap ? pages : cap;
    }
};

}  // namespace

struct pkv_block_manager {
    int32_t P = 0;
    int32_t max_seqs = 0;
    int32_t max_pages = 0;
    std::vector<Group> groups;
    std::vector<int64_t> len;
};

extern "C" {

int32_t pkv_ring_pages(int32_t window, int32_t block_size) {
    if (window <= 0 || block_size <= 0) return 0;
    return (int32_t)(((int64_t)window + 2LL * block_size - 2) / block_size);
}

int64_t pkv_policy_blocks(int64_t context_len, int32_t block_size, int32_t window, int32_t num_sinks,
                          int32_t ring_pages) {
    if (context_len < 0 || block_size <= 0 || num_sinks < 0 || ring_pages < 0) return -1;
    Group g;
    if (window > 0) {
        g.window = window;
        g.ring = ring_pages > 0 ? ring_pages : pkv_ring_pages(window, block_size);
        g.sink_pages = (int32_t)ceil_div(num_sinks, block_size);
    }
    return g.blocks_for(context_len, block_size);
}

pkv_status pkv_bm_create(int32_t block_size, int32_t max_seqs, int32_t max_pages_per_seq,
                         const pkv_layer_group* groups, int32_t num_groups, pkv_block_manager** out) {
    if (!groups || !out) return PKV_ERR_NULL;
    if (block_size % 16 != 0 || block_size < 16 || block_size > 256) return PKV_ERR_UNSUPPORTED;
    if (max_seqs <= 0 || max_pages_per_seq <= 0 || num_groups <= 0) return PKV_ERR_SHAPE;
    for (int32_t g = 0; g < num_groups; ++g) {
        const pkv_layer_group& c = groups[g];
        if (c.num_sinks < 0 || c.num_blocks < 0 || c.ring_pages < 0) return PKV_ERR_SHAPE;
        if (c.window > 0 && c.ring_pages > 0 && c.ring_pages < pkv_ring_pages(c.window, block_size))
            return PKV_ERR_MODE;
        if ((int64_t)c.num_blocks * block_size > INT32_MAX) return PKV_ERR_UNSUPPORTED;
    }
    pkv_block_manager* bm = new (std::nothrow) pkv_block_manager;
    if (!bm) return PKV_ERR_SHAPE;
    try {
        bm->P = block_size;
        bm->max_seqs = max_seqs;
        bm->max_pages = max_pages_per_seq;
        bm->len.assign((size_t)max_seqs, 0);
        bm->groups.resize((size_t)num_groups);
        for (int32_t g = 0; g < num_groups; ++g) {
            const pkv_layer_group& c = groups[g];
            Group& G = bm->groups[(size_t)g];
            G.num_blocks = c.num_blocks;
            if (c.window > 0) {
                G.window = c.window;
                G.sinks = c.num_sinks;
                G.ring = c.ring_pages > 0 ? c.ring_pages : pkv_ring_pages(c.window, block_size);
                G.sink_pages = (int32_t)ceil_div(c.num_sinks, block_size);
                if ((int64_t)G.sink_pages + G.ring > INT32_MAX) {
                    delete bm;
                    return PKV_ERR_UNSUPPORTED;
                }
                G.cols = G.sink_pages + G.ring;
            } else {
                G.cols = max_pages_per_seq;
            }
            G.free_ids.resize((size_t)c.num_blocks);
            for (int32_t i = 0; i < c.num_blocks; ++i) G.free_ids[(size_t)i] = c.num_blocks - 1 - i;
            G.table.assign((size_t)max_seqs * (size_t)G.cols, -1);
        }
    } catch (const std::bad_alloc&) {
        delete bm;
        return PKV_ERR_SHAPE;
    }
    *out = bm;
    return PKV_OK;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int32_t pkv_bm_table_cols(const pkv_block_manager* bm, int32_t group) {
    if (!bm || group < 0 || group >= (int32_t)bm->groups.size()) return 0;
    return bm->groups[(size_t)group].cols;
}

int32_t pkv_bm_ring_pages(const pkv_block_manager* bm, int32_t group) {
    if (!bm || group < 0 || group >= (int32_t)bm->groups.size()) return 0;
    return bm->groups[(size_t)group].ring;
}

pkv_status pkv_bm_append(pkv_block_manager* bm, const int32_t* seq_ids, const int32_t* num_new, int32_t n,
                         int32_t* slots, int32_t* context_lens) {
    if (!bm) return PKV_ERR_NULL;
    if (n < 0) return PKV_ERR_SHAPE;
    if (n == 0) return PKV_OK;
    if (!seq_ids) return PKV_ERR_NULL;
    const int32_t P = bm->P;
    // Validate everything and count the blocks each group needs before changing anything.
    std::vector<char> seen((size_t)bm->max_seqs, 0);
    std::vector<int64_t> need(bm->groups.size(), 0);
    int64_t total = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t s = seq_ids[i];
        const int64_t cnt = num_new ? num_new[i] : 1;
        if (s < 0 || s >= bm->max_seqs || seen[(size_t)s] || cnt < 0) return PKV_ERR_SHAPE;
        seen[(size_t)s] = 1;
        const int64_t L0 = bm->len[(size_t)s], L1 = L0 + cnt;
        if (L1 > INT32_MAX) return PKV_ERR_SHAPE;
        for (size_t g = 0; g < bm->groups.size(); ++g) {
            const Group& G = bm->groups[g];
            if (G.ring == 0 && ceil_div(L1, P) > G.cols) return PKV_ERR_SHAPE;
            need[g] += G.blocks_for(L1, P) - G.blocks_for(L0, P);
        }
        total += cnt;
    }
    if (total > INT32_MAX) return PKV_ERR_SHAPE;
    if (total > 0 && !slots) return PKV_ERR_NULL;
    for (size_t g = 0; g < bm->groups.size(); ++g)
        if (need[g] > (int64_t)bm->groups[g].free_ids.size()) return PKV_ERR_NO_BLOCKS;

    int64_t k = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t s = seq_ids[i];
        const int64_t L0 = bm->len[(size_t)s], L1 = L0 + (num_new ? num_new[i] : 1);
        for (int64_t t = L0; t < L1; ++t, ++k) {
            const int64_t page = t / P;
            for (size_t g = 0; g < bm->groups.size(); ++g) {
                Group& G = bm->groups[g];
                int32_t& e = G.table[(size_t)s * G.cols + (size_t)G.column(page)];
                if (e < 0) {
                    e = G.free_ids.back();
                    G.free_ids.pop_back();
                    ++G.in_use;
                }
                const bool live = G.window == 0 || t < G.sinks || t >= L1 - G.window;
                slots[(size_t)g * (size_t)total + (size_t)k] = live ? (int32_t)(e * P + t % P) : -1;
            }
        }
        bm->len[(size_t)s] = L1;
        if (context_lens) context_lens[i] = (int32_t)L1;
    }
    return PKV_OK;
}

pkv_status pkv_bm_release(pkv_block_manager* bm, int32_t seq_id) {
    if (!bm) return PKV_ERR_NULL;
    if (seq_id < 0 || seq_id >= bm->max_seqs) return PKV_ERR_SHAPE;
    for (Group& G : bm->groups) {
        int32_t* row = G.table.data() + (size_t)seq_id * G.cols;
        // highest column first, so that the lowest column's block is handed out first again
        for (int32_t c = G.cols - 1; c >= 0; --c) {
            if (row[c] < 0) continue;
            G.free_ids.push_back(row[c]);
            row[c] = -1;
            --G.in_use;
        }
    }
    bm->len[(size_t)seq_id] = 0;
    return PKV_OK;
}

pkv_status pkv_bm_block_tables(const pkv_block_manager* bm, int32_t group, const int32_t* seq_ids, int32_t n,
                               int32_t* table) {
    if (!bm) return PKV_ERR_NULL;
    if (group < 0 || group >= (int32_t)bm->groups.size() || n < 0) return PKV_ERR_SHAPE;
    if (n == 0) return PKV_OK;
    if (!seq_ids || !table) return PKV_ERR_NULL;
    const Group& G = bm->groups[(size_t)group];
    for (int32_t i = 0; i < n; ++i)
        if (seq_ids[i] < 0 || seq_ids[i] >= bm->max_seqs) return PKV_ERR_SHAPE;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t* row = G.table.data() + (size_t)seq_ids[i] * G.cols;
        for (int32_t c = 0; c < G.cols; ++c) table[(size_t)i * G.cols + c] = row[c];
    }
    return PKV_OK;
}

int64_t pkv_bm_context_len(const pkv_block_manager* bm, int32_t seq_id) {
    if (!bm || seq_id < 0 || seq_id >= bm->max_seqs) return -1;
    return bm->len[(size_t)seq_id];
}

int64_t pkv_bm_blocks_in_use(const pkv_block_manager* bm, int32_t group) {
    if (!bm || group < 0 || group >= (int32_t)bm->groups.size()) return -1;
    return bm->groups[(size_t)group].in_use;
}

}  // extern "C"
