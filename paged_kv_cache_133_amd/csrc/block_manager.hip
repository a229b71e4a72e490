// Host-side block manager of the paged cache: physical blocks handed out from a free list,
// a logical -> physical block list per sequence, and a reference count per block for
// prefix sharing ("Paged KV Cache and Packed Sequence", 2.1-2.2 and 5.2-5.3):
//  * the free list is popped from its end (LIFO) and a sequence gets a new block only when a
//    token crosses into a new logical block (2.2: most decode steps allocate nothing);
//  * fork gives a child sequence the parent's blocks and raises their counts (beam search,
//    parallel sampling); release lowers the counts of all of a sequence's blocks first and
//    recycles a block only at zero (5.2);
//  * appending into a shared, partly filled last block copies it first (copy on write): the
//    manager takes a fresh block and reports (source, destination) for the caller's device
//    copy (pkv_kv_cache_copy_blocks) before the new rows are written;
//  * the table of a batch is written into a fixed-width [n][max_blocks_per_seq] int32 array
//    on the host, ready for one copy to the device (5.3: allocation stays on the host; the
//    device step, captured or not, only reads the table).
// All calls are on the host, need no GPU, and change nothing when they fail.
#include <algorithm>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"
#include "pkv_internal.h"

struct pkv_block_manager {
    int64_t num_blocks;
    int32_t block_size;
    int32_t max_blocks_per_seq;
    std::vector<int32_t> free_list;          // back = next block handed out
    std::vector<int32_t> ref;                // owners of each physical block
    struct Seq {
        std::vector<int32_t> blocks;
        int64_t len = 0;
    };
    std::unordered_map<int64_t, Seq> seqs;
};

namespace {

int bm_fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    pkv::set_error_v(code, fmt, ap);
    va_end(ap);
    return code;
}

}  // namespace

extern "C" {

pkv_block_manager* pkv_bm_create(int64_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq) {
    if (num_blocks <= 0 || num_blocks > 0x7fffffffLL || block_size <= 0 || max_blocks_per_seq <= 0) {
        bm_fail(PKV_ERR_SHAPE, "bm_create: num_blocks, block_size and max_blocks_per_seq must be positive");
        return nullptr;
    }
    auto* bm = new pkv_block_manager();
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->max_blocks_per_seq = max_blocks_per_seq;
    bm->free_list.resize((size_t)num_blocks);
    for (int64_t i = 0; i < num_blocks; ++i) bm->free_list[(size_t)i] = (int32_t)i;
    bm->ref.assign((size_t)num_blocks, 0);
    return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int64_t pkv_bm_num_free(const pkv_block_manager* bm) { return bm ? (int64_t)bm->free_list.size() : -1; }

int pkv_bm_add(pkv_block_manager* bm, int64_t seq) {
    if (!bm) return bm_fail(PKV_ERR_NULL, "bm_add: NULL manager");
    if (seq < 0) return bm_fail(PKV_ERR_SHAPE, "bm_add: sequence ids are >= 0 (negative ids mark padding rows)");
    if (bm->seqs.count(seq)) return bm_fail(PKV_ERR_SHAPE, "bm_add: sequence %lld exists", (long long)seq);
    bm->seqs.emplace(seq, pkv_block_manager::Seq());
    return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
    if (!bm) return bm_fail(PKV_ERR_NULL, "bm_fork: NULL manager");
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end()) return bm_fail(PKV_ERR_SHAPE, "bm_fork: no sequence %lld", (long long)parent);
    if (child < 0 || bm->seqs.count(child))
        return bm_fail(PKV_ERR_SHAPE, "bm_fork: child id %lld is negative or exists", (long long)child);
    pkv_block_manager::Seq c = it->second;
    for (int32_t blk : c.blocks) ++bm->ref[(size_t)blk];
    bm->seqs.emplace(child, std::move(c));
    return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* bm, int64_t seq, int32_t num_tokens, int64_t* slots_out,
                  int64_t* copy_out, int32_t* num_copies) {
    if (num_copies) *num_copies = 0;
    if (!bm) return bm_fail(PKV_ERR_NULL, "bm_append: NULL manager");
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return bm_fail(PKV_ERR_SHAPE, "bm_append: no sequence %lld", (long long)seq);
    if (num_tokens < 0) return bm_fail(PKV_ERR_SHAPE, "bm_append: negative token count");
    if (num_tokens == 0) return PKV_OK;
    auto& s = it->second;
    const int64_t bs = bm->block_size;
    const int64_t len1 = s.len + num_tokens;
    const int64_t need = (len1 + bs - 1) / bs;                 // logical blocks after the append
    if (need > bm->max_blocks_per_seq)
        return bm_fail(PKV_ERR_SHAPE, "bm_append: %lld tokens need %lld blocks (max_blocks_per_seq %d)",
                       (long long)len1, (long long)need, bm->max_blocks_per_seq);
    // A partly filled, shared last block is copied before anything is written into it.
    const bool cow = s.len % bs != 0 && bm->ref[(size_t)s.blocks.back()] > 1;
    const int64_t fresh = need - (int64_t)s.blocks.size() + (cow ? 1 : 0);
    if (fresh > (int64_t)bm->free_list.size())
        return bm_fail(PKV_ERR_WORKSPACE, "bm_append: kv cache full (%lld blocks needed, %lld free)",
                       (long long)fresh, (long long)bm->free_list.size());
    if (cow && (!copy_out || !num_copies))
        return bm_fail(PKV_ERR_NULL, "bm_append: a copy on write needs copy_out and num_copies");
    if (cow) {
        const int32_t src = s.blocks.back();
        const int32_t dst = bm->free_list.back();
        bm->free_list.pop_back();
        bm->ref[(size_t)dst] = 1;
        --bm->ref[(size_t)src];
        s.blocks.back() = dst;
        copy_out[0] = src;
        copy_out[1] = dst;
        *num_copies = 1;
    }
    while ((int64_t)s.blocks.size() < need) {
        const int32_t blk = bm->free_list.back();
        bm->free_list.pop_back();
        bm->ref[(size_t)blk] = 1;
        s.blocks.push_back(blk);
    }
    for (int32_t i = 0; i < num_tokens; ++i) {
        const int64_t pos = s.len + i;
        if (slots_out) slots_out[i] = (int64_t)s.blocks[(size_t)(pos / bs)] * bs + pos % bs;
    }
    s.len = len1;
    return PKV_OK;
}

int pkv_bm_decode_step(pkv_block_manager* bm, const int64_t* seqs, int32_t n, int64_t* slots_out,
                       int64_t* copies_out, int32_t* num_copies, int32_t* table, int32_t* seq_lens,
                       int32_t pad_block) {
    if (num_copies) *num_copies = 0;
    if (!bm) return bm_fail(PKV_ERR_NULL, "bm_decode_step: NULL manager");
    if (n < 0) return bm_fail(PKV_ERR_SHAPE, "bm_decode_step: negative row count");
    if (n == 0) return PKV_OK;
    if (!seqs || !copies_out || !num_copies || !table)
        return bm_fail(PKV_ERR_NULL, "bm_decode_step: NULL array");
    // Check everything first so that a failure changes nothing: every id known and listed
    // once, every sequence within max_blocks_per_seq, and enough free blocks for the new
    // blocks and the copies on write (a shared block is copied only while another row of
    // the step, or a sequence outside it, still holds it).
    const int64_t bs = bm->block_size;
    std::unordered_map<int64_t, int32_t> seen;
    std::unordered_map<int32_t, int32_t> dropped;
    int64_t fresh = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (seqs[i] < 0) continue;
        auto it = bm->seqs.find(seqs[i]);
        if (it == bm->seqs.end())
            return bm_fail(PKV_ERR_SHAPE, "bm_decode_step: no sequence %lld", (long long)seqs[i]);
        if (seen[seqs[i]]++)
            return bm_fail(PKV_ERR_SHAPE, "bm_decode_step: sequence %lld listed twice", (long long)seqs[i]);
        const auto& s = it->second;
        if (s.len % bs == 0) {
            if ((int64_t)s.blocks.size() + 1 > bm->max_blocks_per_seq)
                return bm_fail(PKV_ERR_SHAPE, "bm_decode_step: sequence %lld would exceed max_blocks_per_seq",
                               (long long)seqs[i]);
            ++fresh;
        } else {
            const int32_t last = s.blocks.back();
            if (bm->ref[(size_t)last] - dropped[last] > 1) {
                ++fresh;
                ++dropped[last];
            }
        }
    }
    if (fresh > (int64_t)bm->free_list.size())
        return bm_fail(PKV_ERR_WORKSPACE, "bm_decode_step: kv cache full (%lld blocks needed, %lld free)",
                       (long long)fresh, (long long)bm->free_list.size());
    int32_t copies = 0;
    const int32_t w = bm->max_blocks_per_seq;
    for (int32_t i = 0; i < n; ++i) {
        int32_t* row = table + (int64_t)i * w;
        if (seqs[i] < 0) {                          // padding row
            if (slots_out) slots_out[i] = -1;
            std::fill(row, row + w, pad_block);
            if (seq_lens) seq_lens[i] = 0;
            continue;
        }
        int64_t slot = -1, copy[2];
        int32_t nc = 0;
        const int rc = pkv_bm_append(bm, seqs[i], 1, &slot, copy, &nc);
        if (rc != PKV_OK) return rc;                // not reached: checked above
        if (nc) {
            copies_out[2 * copies] = copy[0];
            copies_out[2 * copies + 1] = copy[1];
            ++copies;
        }
        if (slots_out) slots_out[i] = slot;
        const auto& s = bm->seqs.at(seqs[i]);
        std::fill(row, row + w, pad_block);
        std::copy(s.blocks.begin(), s.blocks.end(), row);
        if (seq_lens) seq_lens[i] = (int32_t)std::min<int64_t>(s.len, 0x7fffffff);
    }
    *num_copies = copies;
    return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* bm, int64_t seq) {
    if (!bm) return bm_fail(PKV_ERR_NULL, "bm_free: NULL manager");
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return bm_fail(PKV_ERR_SHAPE, "bm_free: no sequence %lld", (long long)seq);
    // every count first, then the blocks that reached zero back to the free list
    for (int32_t blk : it->second.blocks) --bm->ref[(size_t)blk];
    for (int32_t blk : it->second.blocks)
        if (bm->ref[(size_t)blk] == 0) {
            bm->ref[(size_t)blk] = -1;                 // pushed once even if listed twice
            bm->free_list.push_back(blk);
        }
    for (int32_t blk : it->second.blocks)
        if (bm->ref[(size_t)blk] < 0) bm->ref[(size_t)blk] = 0;
    bm->seqs.erase(it);
    return PKV_OK;
}

int pkv_bm_length(const pkv_block_manager* bm, int64_t seq, int64_t* len) {
    if (!bm || !len) return bm_fail(PKV_ERR_NULL, "bm_length: NULL argument");
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return bm_fail(PKV_ERR_SHAPE, "bm_length: no sequence %lld", (long long)seq);
    *len = it->second.len;
    return PKV_OK;
}

int pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block, int32_t* count) {
    if (!bm || !count) return bm_fail(PKV_ERR_NULL, "bm_ref_count: NULL argument");
    if (block < 0 || block >= bm->num_blocks) return bm_fail(PKV_ERR_SHAPE, "bm_ref_count: no block %d", block);
    *count = bm->ref[(size_t)block];
    return PKV_OK;
}

int pkv_bm_table(const pkv_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* table,
                 int32_t* seq_lens, int32_t pad_block) {
    if (!bm) return bm_fail(PKV_ERR_NULL, "bm_table: NULL manager");
    if (n < 0) return bm_fail(PKV_ERR_SHAPE, "bm_table: negative count");
    if (n > 0 && (!seqs || !table)) return bm_fail(PKV_ERR_NULL, "bm_table: NULL array");
    for (int32_t i = 0; i < n; ++i)
        if (!bm->seqs.count(seqs[i])) return bm_fail(PKV_ERR_SHAPE, "bm_table: no sequence %lld", (long long)seqs[i]);
    const int32_t w = bm->max_blocks_per_seq;
    for (int32_t i = 0; i < n; ++i) {
        const auto& s = bm->seqs.at(seqs[i]);
        int32_t* row = table + (int64_t)i * w;
        std::fill(row, row + w, pad_block);
        std::copy(s.blocks.begin(), s.blocks.end(), row);
        if (seq_lens) seq_lens[i] = (int32_t)std::min<int64_t>(s.len, 0x7fffffff);
    }
    return PKV_OK;
}

}  // extern "C"
