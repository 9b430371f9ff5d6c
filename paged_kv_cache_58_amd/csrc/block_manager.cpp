// Host-side block manager for the paged KV cache: the caller side that turns
// sequences of token ids into block tables and slot mappings.
//
// What it implements (the block manager of "Implémentation du cache" in the
// nano-vLLM article; PagedAttention's shared prefix blocks and copy-on-write
// in the CS336 lecture 10 notes, "核心概念与定义"):
//  * a fixed pool of num_blocks blocks of block_size token slots, handed out
//    from a free list;
//  * every full block carries a chained hash: the hash of the previous full
//    block of its sequence combined with the block's own token ids, so two
//    sequences whose prompts share a prefix of whole blocks map those blocks
//    to the same physical blocks (the token ids are compared as well, so a
//    hash collision never shares a block wrongly);
//  * a reference count per block: a shared block returns to the free list
//    only when its last sequence releases it;
//  * forking a sequence (several samples of one prompt) shares all of its
//    blocks; the first append into a shared, partly filled last block copies
//    it first (copy-on-write): the manager gives it a fresh block and queues
//    the (source, destination) pair for the block-copy kernel.
//
// Pure C++ with no HIP headers; not thread-safe (one driver thread owns a
// manager).  Exposed through the pa_bm_* calls of pa.h.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pa.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

// 64-bit mix of a running hash with one value (splitmix64's finaliser applied
// to the xor): the chained block hash folds the previous block's hash and then
// each token id of the block.
inline uint64_t mix64(uint64_t h, uint64_t v) {
    uint64_t z = h ^ (v + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2));
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

constexpr uint64_t kHashSeed = 0x6A09E667F3BCC908ull;

uint64_t chain_hash(uint64_t prev, const int32_t *tokens, int n) {
    uint64_t h = mix64(kHashSeed, prev);
    for (int i = 0; i < n; ++i) h = mix64(h, static_cast<uint32_t>(tokens[i]));
    return h;
}

struct Block {
    int32_t ref = 0;
    bool hashed = false;
    uint64_t hash = 0;
    std::vector<int32_t> tokens;  // token ids of a hashed (full) block
};

struct Seq {
    std::vector<int32_t> blocks;
    int64_t num_tokens = 0;
    uint64_t last_hash = 0;       // chained hash of the last full block (0: none yet)
    std::vector<int32_t> tail;    // token ids of the partly filled last block
};

}  // namespace

struct pa_block_manager {
    int32_t block_size;
    std::vector<Block> blocks;
    std::deque<int32_t> free_list;
    std::unordered_map<uint64_t, int32_t> by_hash;
    std::unordered_map<int64_t, Seq> seqs;
    std::vector<std::pair<int32_t, int32_t>> copies;  // pending copy-on-write pairs

    int32_t take_free() {
        const int32_t b = free_list.front();
        free_list.pop_front();
        blocks[b].ref = 1;
        return b;
    }
    void release(int32_t b) {
        Block &blk = blocks[b];
        if (--blk.ref > 0) return;
        if (blk.hashed) {
            auto it = by_hash.find(blk.hash);
            if (it != by_hash.end() && it->second == b) by_hash.erase(it);
        }
        blk.hashed = false;
        blk.tokens.clear();
        free_list.push_back(b);
    }
    // Registers a block that has just become full under its chained hash,
    // unless another block already holds those tokens under that hash.
    void register_full(int32_t b, uint64_t h, const int32_t *tokens) {
        Block &blk = blocks[b];
        blk.hashed = true;
        blk.hash = h;
        blk.tokens.assign(tokens, tokens + block_size);
        by_hash.emplace(h, b);
    }
    // The block holding exactly these tokens under hash h, or -1.
    int32_t lookup(uint64_t h, const int32_t *tokens) const {
        auto it = by_hash.find(h);
        if (it == by_hash.end()) return -1;
        const Block &blk = blocks[it->second];
        if (!blk.hashed || blk.ref <= 0 ||
            !std::equal(blk.tokens.begin(), blk.tokens.end(), tokens))
            return -1;
        return it->second;
    }
};

PA_EXPORT pa_block_manager *pa_bm_create(int32_t num_blocks, int32_t block_size) {
    if (num_blocks <= 0 || block_size <= 0) return nullptr;
    auto *m = new (std::nothrow) pa_block_manager();
    if (!m) return nullptr;
    m->block_size = block_size;
    m->blocks.resize(num_blocks);
    for (int32_t b = 0; b < num_blocks; ++b) m->free_list.push_back(b);
    return m;
}

PA_EXPORT void pa_bm_destroy(pa_block_manager *m) { delete m; }

PA_EXPORT int32_t pa_bm_num_free(const pa_block_manager *m) {
    return m ? static_cast<int32_t>(m->free_list.size()) : 0;
}

PA_EXPORT int32_t pa_bm_ref_count(const pa_block_manager *m, int32_t block) {
    if (!m || block < 0 || block >= static_cast<int32_t>(m->blocks.size())) return -1;
    return m->blocks[block].ref;
}

PA_EXPORT pa_status pa_bm_add_sequence(pa_block_manager *m, int64_t seq_id,
                                       const int32_t *tokens, int32_t num_tokens,
                                       int32_t *num_cached) {
    if (!m || (num_tokens > 0 && !tokens) || num_tokens < 0) return PA_ERR_NULL;
    if (m->seqs.count(seq_id)) return PA_ERR_SHAPE;
    const int bs = m->block_size;
    const int n_full = num_tokens / bs;
    const int n_tail = num_tokens - n_full * bs;
    // how many blocks must come from the free list
    int need = n_tail > 0 ? 1 : 0;
    {
        uint64_t prev = 0;
        bool sharing = true;
        for (int j = 0; j < n_full; ++j) {
            const int32_t *tk = tokens + static_cast<int64_t>(j) * bs;
            prev = chain_hash(prev, tk, bs);
            if (sharing && m->lookup(prev, tk) >= 0) continue;
            sharing = false;  // past the first miss nothing is shared
            ++need;
        }
    }
    if (need > static_cast<int>(m->free_list.size())) return PA_ERR_WORKSPACE;

    Seq s;
    uint64_t prev = 0;
    bool sharing = true;
    int cached = 0;
    for (int j = 0; j < n_full; ++j) {
        const int32_t *tk = tokens + static_cast<int64_t>(j) * bs;
        const uint64_t h = chain_hash(prev, tk, bs);
        int32_t b = sharing ? m->lookup(h, tk) : -1;
        if (b >= 0) {
            ++m->blocks[b].ref;
            cached += bs;
        } else {
            sharing = false;
            b = m->take_free();
            m->register_full(b, h, tk);
        }
        s.blocks.push_back(b);
        prev = h;
    }
    s.last_hash = prev;
    if (n_tail > 0) {
        s.blocks.push_back(m->take_free());
        s.tail.assign(tokens + static_cast<int64_t>(n_full) * bs, tokens + num_tokens);
    }
    s.num_tokens = num_tokens;
    m->seqs.emplace(seq_id, std::move(s));
    if (num_cached) *num_cached = cached;
    return PA_OK;
}

PA_EXPORT pa_status pa_bm_append_token(pa_block_manager *m, int64_t seq_id, int32_t token,
                                       int32_t *slot) {
    if (!m || !slot) return PA_ERR_NULL;
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PA_ERR_SHAPE;
    Seq &s = it->second;
    const int bs = m->block_size;
    const int64_t t = s.num_tokens;
    if (t % bs == 0) {  // the last block is full (or there is none): a fresh block
        if (m->free_list.empty()) return PA_ERR_WORKSPACE;
        s.blocks.push_back(m->take_free());
    } else {
        int32_t &last = s.blocks.back();
        if (m->blocks[last].ref > 1) {  // shared partial block: copy it before writing
            if (m->free_list.empty()) return PA_ERR_WORKSPACE;
            const int32_t fresh = m->take_free();
            m->copies.emplace_back(last, fresh);
            m->release(last);
            last = fresh;
        }
    }
    *slot = s.blocks.back() * bs + static_cast<int32_t>(t % bs);
    s.tail.push_back(token);
    s.num_tokens = t + 1;
    if (s.num_tokens % bs == 0) {  // the block just filled: it becomes shareable
        const uint64_t h = chain_hash(s.last_hash, s.tail.data(), bs);
        const int32_t b = s.blocks.back();
        if (m->lookup(h, s.tail.data()) < 0) m->register_full(b, h, s.tail.data());
        s.last_hash = h;
        s.tail.clear();
    }
    return PA_OK;
}

PA_EXPORT pa_status pa_bm_fork(pa_block_manager *m, int64_t parent, int64_t child) {
    if (!m) return PA_ERR_NULL;
    auto it = m->seqs.find(parent);
    if (it == m->seqs.end() || m->seqs.count(child)) return PA_ERR_SHAPE;
    Seq s = it->second;
    for (int32_t b : s.blocks) ++m->blocks[b].ref;
    m->seqs.emplace(child, std::move(s));
    return PA_OK;
}

PA_EXPORT pa_status pa_bm_free_sequence(pa_block_manager *m, int64_t seq_id) {
    if (!m) return PA_ERR_NULL;
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PA_ERR_SHAPE;
    // release the last block first, so a prefix shared with others stays
    for (auto b = it->second.blocks.rbegin(); b != it->second.blocks.rend(); ++b) m->release(*b);
    m->seqs.erase(it);
    return PA_OK;
}

PA_EXPORT int64_t pa_bm_num_tokens(const pa_block_manager *m, int64_t seq_id) {
    if (!m) return -1;
    auto it = m->seqs.find(seq_id);
    return it == m->seqs.end() ? -1 : it->second.num_tokens;
}

PA_EXPORT pa_status pa_bm_block_table(const pa_block_manager *m, int64_t seq_id, int32_t *out,
                                      int32_t max_blocks) {
    if (!m || !out) return PA_ERR_NULL;
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PA_ERR_SHAPE;
    const auto &bl = it->second.blocks;
    if (static_cast<int32_t>(bl.size()) > max_blocks) return PA_ERR_SHAPE;
    std::copy(bl.begin(), bl.end(), out);
    std::fill(out + bl.size(), out + max_blocks, -1);
    return PA_OK;
}

PA_EXPORT int32_t pa_bm_take_copies(pa_block_manager *m, int32_t *src, int32_t *dst,
                                    int32_t max_pairs) {
    if (!m || !src || !dst || max_pairs <= 0) return 0;
    const int32_t n = std::min<int32_t>(max_pairs, static_cast<int32_t>(m->copies.size()));
    for (int32_t i = 0; i < n; ++i) {
        src[i] = m->copies[i].first;
        dst[i] = m->copies[i].second;
    }
    m->copies.erase(m->copies.begin(), m->copies.begin() + n);
    return n;
}
