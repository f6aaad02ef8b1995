// block_manager.cpp -- host-side paged block pool, block tables and prefix
// cache (C ABI in include/pkv_block_manager.h).
//
// Pages cited:
//   [A] "KV-Cache Engineering: Paged Attention, Prefix Cache,
//        Disaggregation (2026)" -- prefix caching, cross-layer sharing
//   [B] "KV Cache Engineering: PagedAttention, Continuous Batching,
//        Attention Variants, and the Bandwidth Wall" -- "PagedAttention",
//        "Prefix Caching"
//   [C] "KV-Cache Engineering: The Memory Wall of LLM Serving" -- "When the
//        cache fills"
//
// Data structures: per block a reference count, its prefix key if it is
// cached, and its place in the eviction list; the free blocks in an
// ordered set (lowest id first); the evictable cached blocks in a list
// (least recently released first) with O(1) removal on a re-hit; the key ->
// block map; per sequence its table, token count, the keys of its full
// blocks and the tokens of its partly filled last block (all a later
// append needs to key that block once it fills).
#include <algorithm>
#include <array>
#include <cstdint>
#include <list>
#include <mutex>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"
#include "../../include/pkv_block_manager.h"

namespace {

// 128-bit cumulative key of a token prefix: two 64-bit lanes, each a chain
// of the splitmix64 output function (a bijective 64-bit mixer) over the
// lane state combined with the next token id.
struct Key {
    uint64_t a, b;
    bool operator==(const Key& o) const { return a == o.a && b == o.b; }
};

struct KeyHash {
    size_t operator()(const Key& k) const { return (size_t)(k.a ^ (k.b >> 1)); }
};

inline uint64_t mix64(uint64_t x)
{
    x ^= x >> 30;
    x *= 0xBF58476D1CE4E5B9ull;
    x ^= x >> 27;
    x *= 0x94D049BB133111EBull;
    x ^= x >> 31;
    return x;
}

Key root_key(int64_t ns)
{
    return Key{mix64((uint64_t)ns ^ 0x243F6A8885A308D3ull),
               mix64(~(uint64_t)ns ^ 0x13198A2E03707344ull)};
}

Key extend(Key k, const int32_t* toks, int32_t n)
{
    for (int32_t i = 0; i < n; ++i) {
        const uint64_t t = (uint32_t)toks[i];
        k.a = mix64(k.a + 0x9E3779B97F4A7C15ull + t);
        k.b = mix64(k.b ^ (t * 0xD6E8FEB86659FD93ull + 0xA0761D6478BD642Full));
    }
    return k;
}

struct Block {
    int32_t ref = 0;
    bool keyed = false;
    bool in_lru = false;
    Key key{0, 0};
    std::list<int32_t>::iterator lru_pos;
};

struct Seq {
    std::vector<int32_t> table;
    std::vector<Key> keys;          // keys of the full blocks, in order
    std::vector<int32_t> partial;   // tokens of the partly filled last block
    int32_t n = 0;                  // tokens
};

} // namespace

struct pkv_block_manager {
    int32_t bs;
    Key root;
    std::vector<Block> blocks;
    std::set<int32_t> free_set;
    std::list<int32_t> lru;
    std::unordered_map<Key, int32_t, KeyHash> cache;
    std::unordered_map<int64_t, Seq> seqs;
    std::vector<std::array<int32_t, 3>> copies;
    int64_t hits = 0, lookups = 0, evictions = 0, cow = 0;
    std::mutex mu;

    int64_t available() const { return (int64_t)free_set.size() + (int64_t)lru.size(); }

    int32_t allocate()
    {
        int32_t blk;
        if (!free_set.empty()) {
            blk = *free_set.begin();
            free_set.erase(free_set.begin());
        } else {
            blk = lru.front();
            lru.pop_front();
            Block& v = blocks[blk];
            v.in_lru = false;
            cache.erase(v.key);
            v.keyed = false;
            ++evictions;
        }
        blocks[blk].ref = 1;
        return blk;
    }

    void take(int32_t blk)
    {
        Block& v = blocks[blk];
        if (v.ref == 0 && v.in_lru) {
            lru.erase(v.lru_pos);
            v.in_lru = false;
        }
        ++v.ref;
    }

    void key_block(int32_t blk, const Key& k)
    {
        if (cache.find(k) != cache.end())
            return;
        cache.emplace(k, blk);
        blocks[blk].keyed = true;
        blocks[blk].key = k;
    }

    void release_block(int32_t blk)
    {
        Block& v = blocks[blk];
        if (--v.ref > 0)
            return;
        if (v.keyed) {
            v.lru_pos = lru.insert(lru.end(), blk);
            v.in_lru = true;
        } else {
            free_set.insert(blk);
        }
    }

    int add(int64_t id, const int32_t* toks, int32_t n, int32_t* cached)
    {
        if (seqs.count(id))
            return PKV_EINVAL;
        std::vector<int32_t> matched;
        std::vector<Key> keys;
        Key k = root;
        const int32_t cand = (n - 1) / bs;
        for (int32_t j = 0; j < cand; ++j) {
            k = extend(k, toks + (int64_t)j * bs, bs);
            auto it = cache.find(k);
            ++lookups;
            if (it == cache.end())
                break;
            ++hits;
            matched.push_back(it->second);
            keys.push_back(k);
        }
        const int64_t nblk = ((int64_t)n + bs - 1) / bs;
        int64_t in_lru = 0;
        for (int32_t b : matched)
            in_lru += blocks[b].ref == 0 ? 1 : 0;
        if (nblk - (int64_t)matched.size() > available() - in_lru)
            return PKV_ENOSPACE;
        Seq s;
        s.table.reserve(nblk);
        for (int32_t b : matched) {
            take(b);
            s.table.push_back(b);
        }
        s.keys = keys;
        for (int64_t j = (int64_t)matched.size(); j < nblk; ++j) {
            const int32_t blk = allocate();
            s.table.push_back(blk);
            if ((j + 1) * bs <= n) {
                const Key kj = extend(j ? s.keys.back() : root, toks + j * bs, bs);
                s.keys.push_back(kj);
                key_block(blk, kj);
            }
        }
        s.n = n;
        const int32_t full = n / bs;
        s.partial.assign(toks + (int64_t)full * bs, toks + n);
        seqs.emplace(id, std::move(s));
        *cached = (int32_t)matched.size() * bs;
        return PKV_OK;
    }

    int append(int64_t id, const int32_t* toks, int32_t n)
    {
        auto it = seqs.find(id);
        if (it == seqs.end())
            return PKV_EINVAL;
        Seq& s = it->second;
        int64_t need = 0;
        if (s.n % bs != 0 && n > 0 && blocks[s.table.back()].ref > 1)
            need += 1;
        need += ((int64_t)s.n + n + bs - 1) / bs - ((int64_t)s.n + bs - 1) / bs;
        if (need > available())
            return PKV_ENOSPACE;
        for (int32_t i = 0; i < n; ++i) {
            if (s.n % bs == 0) {
                s.table.push_back(allocate());
            } else if (blocks[s.table.back()].ref > 1) {
                const int32_t src = s.table.back();
                const int32_t dst = allocate();
                copies.push_back({src, dst, s.n % bs});
                ++cow;
                --blocks[src].ref;
                s.table.back() = dst;
            }
            s.partial.push_back(toks[i]);
            ++s.n;
            if (s.n % bs == 0) {
                const Key k = extend(s.keys.empty() ? root : s.keys.back(), s.partial.data(), bs);
                s.keys.push_back(k);
                key_block(s.table.back(), k);
                s.partial.clear();
            }
        }
        return PKV_OK;
    }
};

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size, int64_t hash_namespace)
{
    if (num_blocks < 1 || block_size < 1)
        return nullptr;
    try {
        pkv_block_manager* bm = new pkv_block_manager();
        bm->bs = block_size;
        bm->root = root_key(hash_namespace);
        bm->blocks.resize(num_blocks);
        for (int32_t b = 0; b < num_blocks; ++b)
            bm->free_set.insert(bm->free_set.end(), b);
        return bm;
    } catch (...) {
        return nullptr;
    }
}

void pkv_bm_destroy(pkv_block_manager* bm)
{
    delete bm;
}

int pkv_bm_add(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t n,
               int32_t* cached_tokens)
{
    if (!bm || !tokens || !cached_tokens || n < 1)
        return PKV_EINVAL;
    std::lock_guard<std::mutex> g(bm->mu);
    try {
        return bm->add(seq, tokens, n, cached_tokens);
    } catch (const std::bad_alloc&) {
        return PKV_ENOMEM;
    }
}

int pkv_bm_append(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t n)
{
    if (!bm || n < 0 || (n > 0 && !tokens))
        return PKV_EINVAL;
    std::lock_guard<std::mutex> g(bm->mu);
    try {
        return bm->append(seq, tokens, n);
    } catch (const std::bad_alloc&) {
        return PKV_ENOMEM;
    }
}

int32_t pkv_bm_append_batch(pkv_block_manager* bm, const int64_t* seqs, int32_t n_seqs,
                            const int32_t* token_start, const int32_t* tokens)
{
    if (!bm || n_seqs < 0 || (n_seqs > 0 && (!seqs || !token_start || !tokens)))
        return PKV_EINVAL;
    std::lock_guard<std::mutex> g(bm->mu);
    for (int32_t i = 0; i < n_seqs; ++i) {
        const int32_t n = token_start[i + 1] - token_start[i];
        if (n < 0)
            return i;
        int st;
        try {
            st = bm->append(seqs[i], tokens + token_start[i], n);
        } catch (const std::bad_alloc&) {
            st = PKV_ENOMEM;
        }
        if (st != PKV_OK)
            return i == 0 ? st : i;
    }
    return n_seqs;
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child)
{
    if (!bm)
        return PKV_EINVAL;
    std::lock_guard<std::mutex> g(bm->mu);
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end() || bm->seqs.count(child))
        return PKV_EINVAL;
    try {
        Seq s = it->second;
        for (int32_t b : s.table)
            ++bm->blocks[b].ref;
        bm->seqs.emplace(child, std::move(s));
    } catch (const std::bad_alloc&) {
        return PKV_ENOMEM;
    }
    return PKV_OK;
}

int pkv_bm_release(pkv_block_manager* bm, int64_t seq)
{
    if (!bm)
        return PKV_EINVAL;
    std::lock_guard<std::mutex> g(bm->mu);
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end())
        return PKV_EINVAL;
    const std::vector<int32_t>& t = it->second.table;
    for (auto b = t.rbegin(); b != t.rend(); ++b)
        bm->release_block(*b);
    bm->seqs.erase(it);
    return PKV_OK;
}

int32_t pkv_bm_take_copies(pkv_block_manager* bm, int32_t* out, int32_t max_copies)
{
    if (!bm || max_copies < 0 || (max_copies > 0 && !out))
        return PKV_EINVAL;
    std::lock_guard<std::mutex> g(bm->mu);
    const int32_t n = (int32_t)std::min<size_t>(bm->copies.size(), (size_t)max_copies);
    for (int32_t i = 0; i < n; ++i)
        for (int c = 0; c < 3; ++c)
            out[3 * i + c] = bm->copies[i][c];
    bm->copies.erase(bm->copies.begin(), bm->copies.begin() + n);
    return n;
}

int32_t pkv_bm_context_len(pkv_block_manager* bm, int64_t seq)
{
    if (!bm)
        return PKV_EINVAL;
    std::lock_guard<std::mutex> g(bm->mu);
    auto it = bm->seqs.find(seq);
    return it == bm->seqs.end() ? PKV_EINVAL : it->second.n;
}

int32_t pkv_bm_table(pkv_block_manager* bm, int64_t seq, int32_t* row, int32_t width)
{
    if (!bm || !row || width < 0)
        return PKV_EINVAL;
    std::lock_guard<std::mutex> g(bm->mu);
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end())
        return PKV_EINVAL;
    const std::vector<int32_t>& t = it->second.table;
    if ((int64_t)t.size() > width)
        return PKV_EINVAL;
    for (int32_t j = 0; j < width; ++j)
        row[j] = j < (int32_t)t.size() ? t[j] : -1;
    return (int32_t)t.size();
}

int pkv_bm_export(pkv_block_manager* bm, const int64_t* seqs, int32_t n_seqs,
                  int32_t* block_tables, int32_t width, int32_t* context_lens)
{
    if (!bm || n_seqs < 0 || width < 0 || (n_seqs > 0 && (!seqs || !block_tables || !context_lens)))
        return PKV_EINVAL;
    std::lock_guard<std::mutex> g(bm->mu);
    for (int32_t i = 0; i < n_seqs; ++i) {
        auto it = bm->seqs.find(seqs[i]);
        if (it == bm->seqs.end() || (int64_t)it->second.table.size() > width)
            return PKV_EINVAL;
    }
    for (int32_t i = 0; i < n_seqs; ++i) {
        const Seq& s = bm->seqs.find(seqs[i])->second;
        int32_t* row = block_tables + (int64_t)i * width;
        const int32_t nb = (int32_t)s.table.size();
        for (int32_t j = 0; j < width; ++j)
            row[j] = j < nb ? s.table[j] : -1;
        context_lens[i] = s.n;
    }
    return PKV_OK;
}

int pkv_bm_stats(pkv_block_manager* bm, int64_t* out, int32_t n)
{
    if (!bm || !out || n < 0 || n > 8)
        return PKV_EINVAL;
    std::lock_guard<std::mutex> g(bm->mu);
    const int64_t v[8] = {(int64_t)bm->free_set.size(), (int64_t)bm->lru.size(),
                          (int64_t)bm->cache.size(), (int64_t)bm->seqs.size(),
                          bm->hits, bm->lookups, bm->evictions, bm->cow};
    for (int32_t i = 0; i < n; ++i)
        out[i] = v[i];
    return PKV_OK;
}

int32_t pkv_bm_ref(pkv_block_manager* bm, int32_t block)
{
    if (!bm)
        return PKV_EINVAL;
    std::lock_guard<std::mutex> g(bm->mu);
    if (block < 0 || block >= (int32_t)bm->blocks.size())
        return PKV_EINVAL;
    return bm->blocks[block].ref;
}

int32_t pkv_bm_lru(pkv_block_manager* bm, int32_t* out, int32_t max)
{
    if (!bm || max < 0 || (max > 0 && !out))
        return PKV_EINVAL;
    std::lock_guard<std::mutex> g(bm->mu);
    int32_t i = 0;
    for (int32_t b : bm->lru) {
        if (i >= max)
            break;
        out[i++] = b;
    }
    return (int32_t)bm->lru.size();
}

} // extern "C"
