// Host-side block manager of the paged KV cache (C ABI in pagedkv.h).
//
// What it keeps ("2.1 PagedAttention", source walk-through of the V1 engine, sections
// on the two core classes, the free list and reference counts): every physical block
// has a reference count; free blocks sit in a doubly linked queue so that allocation
// can take n blocks from its head and a prefix-cache hit can pull a free-but-cached
// block out of the middle; a block whose count drops to zero keeps its contents and
// goes back to the queue -- to the tail if it carries a prefix hash (evicted late,
// roughly LRU), to the head otherwise (reused first).  Requests free their blocks
// tail first.  Full blocks are indexed by a hash chained over the previous block's
// hash and the block's tokens ("Inside vLLM, part 2", prefix caching); a cached
// block loses its hash only when the queue hands it out again.  Copy-on-write
// ("2.1 PagedAttention", section 6): writing into a block that others still
// reference first moves the writer to a private copy.
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace {

constexpr int32_t kNil = -1;

struct BlockState {
    int32_t ref = 0;
    int32_t prev = kNil, next = kNil;   // links of the free queue
    bool in_queue = false;
    bool hashed = false;
    uint64_t hash = 0;
};

struct Pool {
    std::vector<BlockState> b;
    int32_t head = kNil, tail = kNil, nfree = 0;
    std::unordered_map<uint64_t, int32_t> cached;   // block hash -> block id

    explicit Pool(int32_t n) : b((size_t)n) {
        for (int32_t i = 0; i < n; ++i) push_back(i);   // ids in ascending order
    }
    void push_back(int32_t i) {
        BlockState& s = b[(size_t)i];
        s.prev = tail;
        s.next = kNil;
        if (tail != kNil) b[(size_t)tail].next = i; else head = i;
        tail = i;
        s.in_queue = true;
        ++nfree;
    }
    void push_front(int32_t i) {
        BlockState& s = b[(size_t)i];
        s.prev = kNil;
        s.next = head;
        if (head != kNil) b[(size_t)head].prev = i; else tail = i;
        head = i;
        s.in_queue = true;
        ++nfree;
    }
    void unlink(int32_t i) {
        BlockState& s = b[(size_t)i];
        if (s.prev != kNil) b[(size_t)s.prev].next = s.next; else head = s.next;
        if (s.next != kNil) b[(size_t)s.next].prev = s.prev; else tail = s.prev;
        s.prev = s.next = kNil;
        s.in_queue = false;
        --nfree;
    }
    void drop_hash(int32_t i) {
        BlockState& s = b[(size_t)i];
        if (!s.hashed) return;
        auto it = cached.find(s.hash);
        if (it != cached.end() && it->second == i) cached.erase(it);
        s.hashed = false;
        s.hash = 0;
    }
    bool valid(int32_t i) const { return i >= 0 && (size_t)i < b.size(); }
};

// 64-bit FNV-1a over little-endian bytes.
uint64_t fnv1a(uint64_t h, const void* p, size_t n) {
    const unsigned char* c = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i < n; ++i) {
        h ^= c[i];
        h *= 0x100000001b3ULL;
    }
    return h;
}

}  // namespace

struct pkv_block_pool {
    Pool pool;
    explicit pkv_block_pool(int32_t n) : pool(n) {}
};

extern "C" {

pkv_block_pool* pkv_pool_create(int32_t num_blocks) {
    if (num_blocks <= 0) return nullptr;
    return new (std::nothrow) pkv_block_pool(num_blocks);
}

void pkv_pool_destroy(pkv_block_pool* p) { delete p; }

int32_t pkv_pool_num_free(const pkv_block_pool* p) { return p ? p->pool.nfree : -1; }

int32_t pkv_pool_ref_count(const pkv_block_pool* p, int32_t id) {
    if (!p || !p->pool.valid(id)) return -1;
    return p->pool.b[(size_t)id].ref;
}

pkv_status pkv_pool_allocate(pkv_block_pool* p, int32_t n, int32_t* ids) {
    if (!p) return PKV_ERR_NULL;
    if (n < 0) return PKV_ERR_SHAPE;
    if (n == 0) return PKV_OK;
    if (!ids) return PKV_ERR_NULL;
    Pool& P = p->pool;
    if (n > P.nfree) return PKV_ERR_NO_BLOCKS;   // nothing taken: the caller preempts
    for (int32_t k = 0; k < n; ++k) {
        const int32_t i = P.head;
        P.unlink(i);
        P.drop_hash(i);                           // its old contents are about to go
        P.b[(size_t)i].ref = 1;
        ids[k] = i;
    }
    return PKV_OK;
}

pkv_status pkv_pool_free(pkv_block_pool* p, const int32_t* ids, int32_t n) {
    if (!p) return PKV_ERR_NULL;
    if (n < 0) return PKV_ERR_SHAPE;
    if (n > 0 && !ids) return PKV_ERR_NULL;
    Pool& P = p->pool;
    // validate before changing anything: every id in range, listed no more often
    // than it is referenced
    std::unordered_map<int32_t, int32_t> times;
    for (int32_t k = 0; k < n; ++k) {
        if (!P.valid(ids[k])) return PKV_ERR_SHAPE;
        if (++times[ids[k]] > P.b[(size_t)ids[k]].ref) return PKV_ERR_SHAPE;
    }
    for (int32_t k = 0; k < n; ++k) {
        const int32_t i = ids[k];
        if (--P.b[(size_t)i].ref == 0) {
            if (P.b[(size_t)i].hashed) P.push_back(i); else P.push_front(i);
        }
    }
    return PKV_OK;
}

pkv_status pkv_pool_touch(pkv_block_pool* p, const int32_t* ids, int32_t n) {
    if (!p) return PKV_ERR_NULL;
    if (n < 0) return PKV_ERR_SHAPE;
    if (n > 0 && !ids) return PKV_ERR_NULL;
    Pool& P = p->pool;
    for (int32_t k = 0; k < n; ++k)
        if (!P.valid(ids[k])) return PKV_ERR_SHAPE;
    for (int32_t k = 0; k < n; ++k) {
        const int32_t i = ids[k];
        if (P.b[(size_t)i].ref == 0 && P.b[(size_t)i].in_queue) P.unlink(i);
        ++P.b[(size_t)i].ref;
    }
    return PKV_OK;
}

pkv_status pkv_pool_cache_blocks(pkv_block_pool* p, const int32_t* ids, const uint64_t* hashes,
                                 int32_t n) {
    if (!p) return PKV_ERR_NULL;
    if (n < 0) return PKV_ERR_SHAPE;
    if (n > 0 && (!ids || !hashes)) return PKV_ERR_NULL;
    Pool& P = p->pool;
    for (int32_t k = 0; k < n; ++k)
        if (!P.valid(ids[k])) return PKV_ERR_SHAPE;
    for (int32_t k = 0; k < n; ++k) {
        const int32_t i = ids[k];
        BlockState& s = P.b[(size_t)i];
        if (s.hashed) continue;                    // already indexed
        if (P.cached.count(hashes[k])) continue;   // another block holds these contents
        s.hashed = true;
        s.hash = hashes[k];
        P.cached.emplace(hashes[k], i);
    }
    return PKV_OK;
}

int32_t pkv_pool_longest_hit(const pkv_block_pool* p, const uint64_t* hashes, int32_t n,
                             int32_t* ids) {
    if (!p || n < 0 || (n > 0 && (!hashes || !ids))) return -1;
    int32_t k = 0;
    for (; k < n; ++k) {
        auto it = p->pool.cached.find(hashes[k]);
        if (it == p->pool.cached.end()) break;     // a prefix: stop at the first miss
        ids[k] = it->second;
    }
    return k;
}

pkv_status pkv_pool_cow(pkv_block_pool* p, int32_t id, int32_t* out_id, int32_t* copy_needed) {
    if (!p || !out_id || !copy_needed) return PKV_ERR_NULL;
    Pool& P = p->pool;
    if (!P.valid(id) || P.b[(size_t)id].ref <= 0) return PKV_ERR_SHAPE;
    if (P.b[(size_t)id].ref == 1) {                // sole owner: write in place
        *out_id = id;
        *copy_needed = 0;
        return PKV_OK;
    }
    int32_t fresh = kNil;
    const pkv_status st = pkv_pool_allocate(p, 1, &fresh);
    if (st != PKV_OK) return st;
    --P.b[(size_t)id].ref;                         // the writer leaves the shared block
    *out_id = fresh;
    *copy_needed = 1;
    return PKV_OK;
}

int32_t pkv_pool_free_queue(const pkv_block_pool* p, int32_t* ids, int32_t capacity) {
    if (!p || capacity < 0 || (capacity > 0 && !ids)) return -1;
    int32_t k = 0;
    for (int32_t i = p->pool.head; i != kNil; i = p->pool.b[(size_t)i].next) {
        if (k < capacity) ids[k] = i;
        ++k;
    }
    return k;
}

uint64_t pkv_block_hash(uint64_t parent, const int32_t* tokens, int32_t n) {
    uint64_t h = 0xcbf29ce484222325ULL;
    h = fnv1a(h, &parent, sizeof(parent));
    if (tokens && n > 0) h = fnv1a(h, tokens, (size_t)n * sizeof(int32_t));
    return h;
}

}  // extern "C"
