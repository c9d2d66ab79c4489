// Host block manager of the paged KV cache: which physical block and slot each token
// of each sequence uses, with reference counts, copy-on-write, prefix caching and LRU
// eviction of cold cached blocks. Plain C++ on the host; its outputs (block tables,
// context lengths, slot mappings, copy pairs) are the inputs of the device calls.
//
// Rules ([P2] = "vLLM 核心源码深度解析：PagedAttention 的 KV Cache 管理、Scheduler 调度引擎
// 与 Continuous Batching 实现全解", [P3] = "论文专题讲解：vLLM / PagedAttention：为什么
// KV cache 需要分页管理", [P1] = "vLLM 源码解析：PagedAttention 如何让大模型推理提速 10 倍"):
//  - token position p of a sequence lives in logical block p / bs at offset p % bs
//    ([P2] "Block Table 数据结构"); its slot is physical_block * bs + offset;
//  - free blocks form a stack: allocation pops, release pushes, both O(1) ([P2]
//    "内存分配与回收流程");
//  - blocks are taken on demand: ceil(n / bs) for an n-token prompt, one more when a
//    decoded token finds its last block full ([P3] "Block table：为什么它能减少碎片");
//  - reference counts; a write into a block shared by several sequences first copies
//    it to a fresh block (copy-on-write), and the copy pair is returned for the device
//    ([P3] "共享前缀和 copy-on-write", [P1] section 五);
//  - prefix caching: a full block is found again by its token prefix ([P2]
//    "Copy-on-Write 与 Prefix Caching"). The key of logical block j chains the key of
//    block j-1 with block j's tokens (64-bit), and a hit also compares the stored
//    parent key and the block's own tokens, so a false hit needs a 64-bit collision of
//    the parent key;
//  - a cached block whose count drops to zero stays cold (evictable) at the back of an
//    LRU list; when no block is free, allocation evicts the front ([P2]
//    "BlockAllocator 源码核心：vLLM 的显存管理心脏"); a sequence releases its blocks last
//    first, so a prompt's first blocks leave the cache last;
//  - every operation checks that its blocks are available before it changes anything.
// Not thread-safe: one manager per scheduler thread.
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace {

constexpr uint64_t kRootKey = 0x243F6A8885A308D3ull;   // parent key of logical block 0

uint64_t mix64(uint64_t x) {   // the splitmix64 finaliser
    x ^= x >> 30;
    x *= 0xBF58476D1CE4E5B9ull;
    x ^= x >> 27;
    x *= 0x94D049BB133111EBull;
    x ^= x >> 31;
    return x;
}

uint64_t chain_key(uint64_t parent, const int32_t* tokens, int bs) {
    uint64_t h = mix64(parent ^ 0x9E3779B97F4A7C15ull);
    for (int i = 0; i < bs; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tokens[i] ^ ((uint64_t)i << 32));
    return h;
}

struct Sequence {
    std::vector<int32_t> table;
    int64_t len = 0;
    bool tracked = false;            // token ids known: full blocks can be cached
    std::vector<int32_t> tokens;
    std::vector<uint64_t> keys;      // chain key of each full block (tracked only)
};

}  // namespace

struct pkv_block_manager {
    int num_blocks = 0, bs = 0;
    std::vector<int32_t> free;       // a stack: back() is handed out next
    std::vector<int32_t> ref;
    // LRU list of cold blocks (cached, unreferenced): head = least recently released
    std::vector<int32_t> prev, next;
    int32_t head = -1, tail = -1;
    int cold = 0;
    // prefix cache: key -> block, plus each cached block's key, parent key and tokens
    std::unordered_map<uint64_t, int32_t> cache;
    std::vector<uint8_t> cached;
    std::vector<uint64_t> key, parent;
    std::vector<int32_t> block_tokens;
    std::unordered_map<int64_t, Sequence> seqs;

    int available() const { return (int)free.size() + cold; }

    void lru_push(int32_t b) {
        prev[b] = tail;
        next[b] = -1;
        if (tail >= 0) next[tail] = b; else head = b;
        tail = b;
        ++cold;
    }
    void lru_unlink(int32_t b) {
        if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
        if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
        prev[b] = next[b] = -1;
        --cold;
    }
    // A block for a new owner (count 1): from the free stack, else the least recently
    // released cold block, dropped from the cache. Callers check availability first.
    int32_t take() {
        int32_t b;
        if (!free.empty()) {
            b = free.back();
            free.pop_back();
        } else {
            b = head;
            lru_unlink(b);
            cache.erase(key[b]);
            cached[b] = 0;
        }
        ref[b] = 1;
        return b;
    }
    void hold(int32_t b) {
        if (ref[b] == 0) lru_unlink(b);   // a cold block revived by a prefix hit
        ++ref[b];
    }
    void release(int32_t b) {
        if (--ref[b] == 0) {
            if (cached[b]) lru_push(b); else free.push_back(b);
        }
    }
    // The cached block holding `tokens` behind parent key `pk`, or -1.
    int32_t lookup(uint64_t pk, const int32_t* tokens, uint64_t* k_out) const {
        const uint64_t k = chain_key(pk, tokens, bs);
        *k_out = k;
        const auto it = cache.find(k);
        if (it == cache.end()) return -1;
        const int32_t b = it->second;
        if (parent[b] != pk ||
            std::memcmp(&block_tokens[(size_t)b * bs], tokens, sizeof(int32_t) * bs) != 0)
            return -1;
        return b;
    }
    // Cache block b under key k (parent key pk, tokens) unless the key is taken or the
    // block is already cached.
    void enter(int32_t b, uint64_t k, uint64_t pk, const int32_t* tokens) {
        if (cached[b] || cache.count(k)) return;
        cache.emplace(k, b);
        cached[b] = 1;
        key[b] = k;
        parent[b] = pk;
        std::memcpy(&block_tokens[(size_t)b * bs], tokens, sizeof(int32_t) * bs);
    }
};

extern "C" {

pkv_block_manager* pkv_bm_create(int num_blocks, int block_size, const int32_t* order) {
    if (num_blocks < 0 || block_size <= 0) return nullptr;
    pkv_block_manager* m = new (std::nothrow) pkv_block_manager();
    if (!m) return nullptr;
    try {
        m->num_blocks = num_blocks;
        m->bs = block_size;
        m->ref.assign(num_blocks, 0);
        m->prev.assign(num_blocks, -1);
        m->next.assign(num_blocks, -1);
        m->cached.assign(num_blocks, 0);
        m->key.assign(num_blocks, 0);
        m->parent.assign(num_blocks, 0);
        m->block_tokens.assign((size_t)num_blocks * block_size, 0);
        m->free.resize(num_blocks);
        std::vector<uint8_t> seen(num_blocks, 0);
        for (int i = 0; i < num_blocks; ++i) {
            const int32_t b = order ? order[i] : i;
            if (b < 0 || b >= num_blocks || seen[b]) {   // not a permutation
                delete m;
                return nullptr;
            }
            seen[b] = 1;
            m->free[num_blocks - 1 - i] = b;   // order[0] on top of the stack
        }
    } catch (...) {
        delete m;
        return nullptr;
    }
    return m;
}

void pkv_bm_destroy(pkv_block_manager* m) { delete m; }

int pkv_bm_available(const pkv_block_manager* m) { return m ? m->available() : PKV_E_NULL; }

int pkv_bm_can_allocate(const pkv_block_manager* m, int num_tokens) {
    if (!m) return PKV_E_NULL;
    if (num_tokens < 0) return PKV_E_SHAPE;
    return ((int64_t)num_tokens + m->bs - 1) / m->bs <= m->available() ? 1 : 0;
}

int pkv_bm_add_sequence(pkv_block_manager* m, int64_t seq_id, int num_tokens,
                        const int32_t* token_ids, int* cached_tokens) {
    if (!m) return PKV_E_NULL;
    if (num_tokens < 0) return PKV_E_SHAPE;
    if (m->seqs.count(seq_id)) return PKV_E_SEQUENCE;
    const int bs = m->bs;
    const int full = num_tokens / bs;
    const int nblocks = (num_tokens + bs - 1) / bs;
    // plan: leading full blocks found in the cache
    std::vector<int32_t> hits;
    std::vector<uint64_t> keys;
    uint64_t pk = kRootKey;
    if (token_ids) {
        for (int j = 0; j < full; ++j) {
            uint64_t k;
            const int32_t b = m->lookup(pk, token_ids + (size_t)j * bs, &k);
            if (b < 0) break;
            hits.push_back(b);
            keys.push_back(k);
            pk = k;
        }
    }
    const int misses = nblocks - (int)hits.size();
    int cold_hits = 0;
    for (int32_t b : hits) cold_hits += m->ref[b] == 0;
    if (misses > m->available() - cold_hits) return PKV_E_NOSPACE;
    try {
        Sequence s;
        s.table.reserve(nblocks);
        for (int32_t b : hits) {
            m->hold(b);
            s.table.push_back(b);
        }
        for (int i = 0; i < misses; ++i) s.table.push_back(m->take());
        s.len = num_tokens;
        s.tracked = token_ids != nullptr;
        if (s.tracked) {
            s.tokens.assign(token_ids, token_ids + num_tokens);
            s.keys = keys;
            for (int j = (int)hits.size(); j < full; ++j) {
                const int32_t* t = token_ids + (size_t)j * bs;
                const uint64_t k = chain_key(pk, t, bs);
                m->enter(s.table[j], k, pk, t);
                s.keys.push_back(k);
                pk = k;
            }
        }
        m->seqs.emplace(seq_id, std::move(s));
    } catch (...) {
        return PKV_E_LAUNCH;   // out of host memory
    }
    if (cached_tokens) *cached_tokens = (int)hits.size() * bs;
    return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* m, int64_t parent_id, int64_t child_id) {
    if (!m) return PKV_E_NULL;
    const auto it = m->seqs.find(parent_id);
    if (it == m->seqs.end() || m->seqs.count(child_id)) return PKV_E_SEQUENCE;
    try {
        Sequence child = it->second;   // copies table, tokens and keys
        for (int32_t b : child.table) m->hold(b);
        m->seqs.emplace(child_id, std::move(child));
    } catch (...) {
        return PKV_E_LAUNCH;
    }
    return PKV_OK;
}

int pkv_bm_append_token(pkv_block_manager* m, int64_t seq_id, int32_t token_id, int64_t* slot,
                        int32_t* copy_src, int32_t* copy_dst) {
    if (!m) return PKV_E_NULL;
    const auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PKV_E_SEQUENCE;
    Sequence& s = it->second;
    const int bs = m->bs;
    const int64_t pos = s.len;
    const size_t j = (size_t)(pos / bs);
    const int off = (int)(pos % bs);
    const bool fresh = j == s.table.size();
    const bool shared = !fresh && m->ref[s.table[j]] > 1;
    if ((fresh || shared) && m->available() == 0) return PKV_E_NOSPACE;
    int32_t src = -1, dst = -1;
    try {
        if (s.tracked) s.tokens.push_back(token_id);
        if (fresh) {
            s.table.push_back(m->take());
        } else if (shared) {
            src = s.table[j];
            dst = m->take();
            m->release(src);
            s.table[j] = dst;
        }
    } catch (...) {
        return PKV_E_LAUNCH;
    }
    s.len = pos + 1;
    if (s.tracked && (pos + 1) % bs == 0) {
        const uint64_t pk = j == 0 ? kRootKey : s.keys[j - 1];
        const int32_t* t = s.tokens.data() + j * bs;
        const uint64_t k = chain_key(pk, t, bs);
        m->enter(s.table[j], k, pk, t);
        s.keys.push_back(k);
    }
    if (slot) *slot = (int64_t)s.table[j] * bs + off;
    if (copy_src) *copy_src = src;
    if (copy_dst) *copy_dst = dst;
    return PKV_OK;
}

int pkv_bm_append_tokens(pkv_block_manager* m, const int64_t* seq_ids, const int32_t* token_ids,
                         int n, int64_t* slots, int32_t* copy_pairs) {
    if (!m) return PKV_E_NULL;
    if (n < 0) return PKV_E_SHAPE;
    if (n > 0 && (!seq_ids || !slots)) return PKV_E_NULL;
    for (int i = 0; i < n; ++i) {
        int32_t src = -1, dst = -1;
        const int rc = pkv_bm_append_token(m, seq_ids[i], token_ids ? token_ids[i] : 0,
                                           &slots[i], &src, &dst);
        if (rc == PKV_E_NOSPACE) return i;   // sequences i .. n-1 are untouched
        if (rc != PKV_OK) return rc;
        if (copy_pairs) {
            copy_pairs[2 * i] = src;
            copy_pairs[2 * i + 1] = dst;
        }
    }
    return n;
}

int pkv_bm_free_sequence(pkv_block_manager* m, int64_t seq_id) {
    if (!m) return PKV_E_NULL;
    const auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PKV_E_SEQUENCE;
    const std::vector<int32_t>& t = it->second.table;
    for (size_t i = t.size(); i-- > 0;) m->release(t[i]);
    m->seqs.erase(it);
    return PKV_OK;
}

int64_t pkv_bm_num_tokens(const pkv_block_manager* m, int64_t seq_id) {
    if (!m) return PKV_E_NULL;
    const auto it = m->seqs.find(seq_id);
    return it == m->seqs.end() ? PKV_E_SEQUENCE : it->second.len;
}

int pkv_bm_block_table(const pkv_block_manager* m, int64_t seq_id, int32_t* out, int capacity) {
    if (!m) return PKV_E_NULL;
    const auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PKV_E_SEQUENCE;
    const std::vector<int32_t>& t = it->second.table;
    const int n = (int)t.size();
    if (out)
        for (int i = 0; i < n && i < capacity; ++i) out[i] = t[i];
    return n;
}

int pkv_bm_refcount(const pkv_block_manager* m, int32_t block) {
    if (!m) return PKV_E_NULL;
    if (block < 0 || block >= m->num_blocks) return PKV_E_SHAPE;
    return m->ref[block];
}

int pkv_bm_build_tables(const pkv_block_manager* m, const int64_t* seq_ids, int num_seqs,
                        int width, int32_t* tables, int32_t* context_lens) {
    if (!m) return PKV_E_NULL;
    if (num_seqs < 0 || width < 0) return PKV_E_SHAPE;
    if (num_seqs > 0 && (!seq_ids || !tables || !context_lens)) return PKV_E_NULL;
    // one lookup per sequence, everything checked before anything is written
    std::vector<const Sequence*> found;
    try {
        found.resize(num_seqs);
    } catch (...) {
        return PKV_E_LAUNCH;
    }
    for (int i = 0; i < num_seqs; ++i) {
        const auto it = m->seqs.find(seq_ids[i]);
        if (it == m->seqs.end()) return PKV_E_SEQUENCE;
        if ((int)it->second.table.size() > width || it->second.len > 0x7fffffff)
            return PKV_E_SHAPE;
        found[i] = &it->second;
    }
    for (int i = 0; i < num_seqs; ++i) {
        const Sequence& s = *found[i];
        int32_t* row = tables + (size_t)i * width;
        const size_t n = s.table.size();
        if (n) std::memcpy(row, s.table.data(), n * sizeof(int32_t));
        for (size_t j = n; j < (size_t)width; ++j) row[j] = -1;
        context_lens[i] = (int32_t)s.len;
    }
    return PKV_OK;
}

}  // extern "C"
