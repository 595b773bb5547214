// Host-side KV block manager: the block pool's free list, per-sequence block
// tables, and the prefix cache, as the pages lay them out ("09 -- Mini
// Inference Engine (The Capstone)", the engine diagram's KV cache manager:
// block pool with a free list, prefix hash -> block ids, block tables per
// sequence; Week 4 -- a block is taken from the free list when a sequence's
// last block fills and all of a sequence's blocks return on completion; Week 5
// -- rolling hash hash(previous block's hash, block tokens) per full block, a
// global hash -> block map, prompt blocks found there are shared instead of
// recomputed, blocks reference-counted and freed only at count zero).
//
// Choices the pages leave open, made here:
//   - a freed block whose contents are cached keeps its cache entry while it
//     sits in the free list (least recently freed first out), so a later
//     prompt can still find it; the entry is dropped when the block is taken
//     for other contents;
//   - a cache hit is confirmed on the block's stored tokens and on its parent
//     block, so a hit means exactly an equal token prefix (a 64-bit hash
//     collision cannot alias two prefixes);
//   - blocks enter the cache only once the caller reports their tokens
//     computed (pa_bm_mark_computed), never while their K/V is still unwritten;
//   - when every prompt token would come from the cache, the last block is
//     recomputed privately: the final prompt token needs a forward pass, and a
//     shared block is never written;
//   - a sequence frees its blocks last one first, so a shared prefix stays in
//     the free list longer than the tails behind it.
// Every call is atomic: on failure nothing changes.  One mutex per manager.
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

struct pa_block_manager {
    struct Block {
        int32_t ref = 0;
        bool in_free = false;
        int32_t prev = -1, next = -1;   // free list links
        bool cached = false;            // holds a cache entry
        uint64_t hash = 0;
        int32_t parent = -1;            // previous block of the cached prefix (-1: first)
        std::vector<int32_t> tokens;    // the block's tokens while cached
    };
    struct Seq {
        std::vector<int32_t> table;     // physical block ids
        std::vector<int32_t> tokens;    // every token of the sequence so far
        int32_t computed = 0;           // tokens whose K/V the caller reported written
        int32_t registered = 0;         // full blocks already offered to the cache
    };

    int32_t num_blocks, block_size;
    bool prefix;
    std::vector<Block> blocks;
    int32_t head = -1, tail = -1, nfree = 0;
    std::unordered_map<uint64_t, int32_t> cache;
    std::unordered_map<int64_t, Seq> seqs;
    int64_t hit_blocks = 0, queried_blocks = 0;
    std::mutex mu;

    pa_block_manager(int32_t nb, int32_t bs, bool pc) : num_blocks(nb), block_size(bs), prefix(pc), blocks(nb) {
        for (int32_t i = 0; i < nb; ++i) push_free(i);
    }

    void push_free(int32_t id) {
        Block& b = blocks[id];
        b.in_free = true;
        b.prev = tail;
        b.next = -1;
        if (tail >= 0) blocks[tail].next = id; else head = id;
        tail = id;
        ++nfree;
    }
    void remove_free(int32_t id) {
        Block& b = blocks[id];
        if (b.prev >= 0) blocks[b.prev].next = b.next; else head = b.next;
        if (b.next >= 0) blocks[b.next].prev = b.prev; else tail = b.prev;
        b.prev = b.next = -1;
        b.in_free = false;
        --nfree;
    }
    // Take the least recently freed block for new contents.
    int32_t take() {
        const int32_t id = head;
        remove_free(id);
        Block& b = blocks[id];
        if (b.cached) {
            auto it = cache.find(b.hash);
            if (it != cache.end() && it->second == id) cache.erase(it);
            b.cached = false;
            b.tokens.clear();
        }
        b.ref = 1;
        return id;
    }
    void release(int32_t id) {
        if (--blocks[id].ref == 0) push_free(id);
    }

    static uint64_t mix(uint64_t h, uint64_t v) {
        h ^= v + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
        h ^= h >> 31;
        h *= 0xBF58476D1CE4E5B9ull;
        h ^= h >> 29;
        return h;
    }
    // Rolling hash of a full block: (previous block's hash, its tokens).
    uint64_t block_hash(uint64_t prev, const int32_t* t) const {
        uint64_t h = mix(0x6A09E667F3BCC908ull, prev);
        for (int32_t i = 0; i < block_size; ++i) h = mix(h, (uint32_t)t[i]);
        return h;
    }
    // Cached block holding exactly these tokens after `parent`, or -1.
    int32_t lookup(uint64_t h, int32_t parent, const int32_t* t) const {
        auto it = cache.find(h);
        if (it == cache.end()) return -1;
        const Block& b = blocks[it->second];
        if (!b.cached || b.parent != parent || memcmp(b.tokens.data(), t, block_size * sizeof(int32_t)) != 0)
            return -1;
        return it->second;
    }
};

namespace {

int32_t blocks_for(int64_t tokens, int32_t bs) { return (int32_t)((tokens + bs - 1) / bs); }

}  // namespace

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t prefix_caching) {
    if (num_blocks <= 0 || block_size <= 0 || (int64_t)num_blocks * block_size > INT32_MAX) return nullptr;
    return new (std::nothrow) pa_block_manager(num_blocks, block_size, prefix_caching != 0);
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int32_t pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, const int32_t* tokens,
                           int32_t num_tokens, int32_t* num_cached_tokens) {
    if (m == nullptr || num_cached_tokens == nullptr || (num_tokens > 0 && tokens == nullptr)) return PA_ERR_NULL;
    if (num_tokens < 0) return PA_ERR_SHAPE;
    std::lock_guard<std::mutex> lock(m->mu);
    if (m->seqs.count(seq_id)) return PA_ERR_SHAPE;
    const int32_t bs = m->block_size;
    const int32_t need = blocks_for(num_tokens, bs);
    // Prefix lookup over the prompt's full blocks, stopping at the first miss.
    std::vector<int32_t> hits;
    if (m->prefix) {
        uint64_t h = 0;
        int32_t parent = -1;
        for (int32_t b = 0; b < num_tokens / bs; ++b) {
            h = m->block_hash(h, tokens + (int64_t)b * bs);
            const int32_t id = m->lookup(h, parent, tokens + (int64_t)b * bs);
            if (id < 0) break;
            hits.push_back(id);
            parent = id;
        }
        if (!hits.empty() && (int64_t)hits.size() * bs == num_tokens) hits.pop_back();
    }
    int32_t revived = 0;
    for (int32_t id : hits) revived += m->blocks[id].in_free ? 1 : 0;
    if (m->nfree - revived < need - (int32_t)hits.size()) return PA_ERR_CAPACITY;
    pa_block_manager::Seq s;
    s.table.reserve(need);
    for (int32_t id : hits) {
        if (m->blocks[id].in_free) m->remove_free(id);
        ++m->blocks[id].ref;
        s.table.push_back(id);
    }
    while ((int32_t)s.table.size() < need) s.table.push_back(m->take());
    s.tokens.assign(tokens, tokens + num_tokens);
    s.computed = (int32_t)hits.size() * bs;
    s.registered = (int32_t)hits.size();
    if (m->prefix) {
        m->queried_blocks += num_tokens / bs;
        m->hit_blocks += (int64_t)hits.size();
    }
    m->seqs.emplace(seq_id, std::move(s));
    *num_cached_tokens = (int32_t)hits.size() * bs;
    return PA_OK;
}

int32_t pa_bm_append(pa_block_manager* m, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                     int32_t* slots_out) {
    if (m == nullptr || (num_tokens > 0 && tokens == nullptr)) return PA_ERR_NULL;
    if (num_tokens < 0) return PA_ERR_SHAPE;
    std::lock_guard<std::mutex> lock(m->mu);
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PA_ERR_SHAPE;
    pa_block_manager::Seq& s = it->second;
    const int32_t bs = m->block_size;
    const int64_t total = (int64_t)s.tokens.size() + num_tokens;
    if (total > INT32_MAX) return PA_ERR_SHAPE;
    const int32_t extra = blocks_for(total, bs) - (int32_t)s.table.size();
    if (extra > m->nfree) return PA_ERR_CAPACITY;
    for (int32_t i = 0; i < extra; ++i) s.table.push_back(m->take());
    const int32_t base = (int32_t)s.tokens.size();
    s.tokens.insert(s.tokens.end(), tokens, tokens + num_tokens);
    if (slots_out != nullptr)
        for (int32_t i = 0; i < num_tokens; ++i) {
            const int32_t p = base + i;
            slots_out[i] = s.table[p / bs] * bs + p % bs;
        }
    return PA_OK;
}

int32_t pa_bm_mark_computed(pa_block_manager* m, int64_t seq_id, int32_t num_computed_tokens) {
    if (m == nullptr) return PA_ERR_NULL;
    std::lock_guard<std::mutex> lock(m->mu);
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PA_ERR_SHAPE;
    pa_block_manager::Seq& s = it->second;
    if (num_computed_tokens < 0 || num_computed_tokens > (int32_t)s.tokens.size()) return PA_ERR_SHAPE;
    if (num_computed_tokens > s.computed) s.computed = num_computed_tokens;
    if (!m->prefix) return PA_OK;
    const int32_t bs = m->block_size;
    // Offer each newly completed full block to the cache, chaining the hash
    // from the block before it.
    uint64_t h = 0;
    for (int32_t b = 0; b < s.registered; ++b) h = m->block_hash(h, s.tokens.data() + (int64_t)b * bs);
    for (int32_t b = s.registered; b < s.computed / bs; ++b) {
        const int32_t* t = s.tokens.data() + (int64_t)b * bs;
        h = m->block_hash(h, t);
        pa_block_manager::Block& blk = m->blocks[s.table[b]];
        if (!blk.cached && m->cache.find(h) == m->cache.end()) {
            blk.cached = true;
            blk.hash = h;
            blk.parent = b > 0 ? s.table[b - 1] : -1;
            blk.tokens.assign(t, t + bs);
            m->cache.emplace(h, s.table[b]);
        }
        s.registered = b + 1;
    }
    return PA_OK;
}

int32_t pa_bm_free_sequence(pa_block_manager* m, int64_t seq_id) {
    if (m == nullptr) return PA_ERR_NULL;
    std::lock_guard<std::mutex> lock(m->mu);
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PA_ERR_SHAPE;
    const std::vector<int32_t>& t = it->second.table;
    for (auto b = t.rbegin(); b != t.rend(); ++b) m->release(*b);
    m->seqs.erase(it);
    return PA_OK;
}

int32_t pa_bm_block_table(pa_block_manager* m, int64_t seq_id, int32_t* table_out, int32_t capacity,
                          int32_t* num_blocks_out, int32_t* num_tokens_out) {
    if (m == nullptr || num_blocks_out == nullptr) return PA_ERR_NULL;
    std::lock_guard<std::mutex> lock(m->mu);
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PA_ERR_SHAPE;
    const std::vector<int32_t>& t = it->second.table;
    *num_blocks_out = (int32_t)t.size();
    if (num_tokens_out != nullptr) *num_tokens_out = (int32_t)it->second.tokens.size();
    if ((int32_t)t.size() > capacity) return PA_ERR_SHAPE;
    if (!t.empty()) {
        if (table_out == nullptr) return PA_ERR_NULL;
        memcpy(table_out, t.data(), t.size() * sizeof(int32_t));
    }
    return PA_OK;
}

int32_t pa_bm_num_free_blocks(pa_block_manager* m) {
    if (m == nullptr) return -1;
    std::lock_guard<std::mutex> lock(m->mu);
    return m->nfree;
}

int32_t pa_bm_stats(pa_block_manager* m, int64_t* hit_blocks, int64_t* queried_blocks,
                    int32_t* cached_blocks) {
    if (m == nullptr || hit_blocks == nullptr || queried_blocks == nullptr || cached_blocks == nullptr)
        return PA_ERR_NULL;
    std::lock_guard<std::mutex> lock(m->mu);
    *hit_blocks = m->hit_blocks;
    *queried_blocks = m->queried_blocks;
    *cached_blocks = (int32_t)m->cache.size();
    return PA_OK;
}

int32_t pa_bm_block_refcount(pa_block_manager* m, int32_t block_id) {
    if (m == nullptr || block_id < 0 || block_id >= m->num_blocks) return -1;
    std::lock_guard<std::mutex> lock(m->mu);
    return m->blocks[block_id].ref;
}

}  // extern "C"
