// Random operation streams on the host block pool (pkv_pool_*) under AddressSanitizer
// and UndefinedBehaviorSanitizer, with the pool's invariants checked after every step:
// the free queue holds exactly the blocks whose reference count is zero, each once,
// and its length is the free count; every reference a simulated request holds is
// counted.  Any memory error in the linked queue or the hash index aborts the run.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "pagedkv.h"

static uint64_t g_state = 0x2545F4914F6CDD1Dull;
static uint64_t rnd() {                  // splitmix64
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static void fail(const char* what, int step) {
    fprintf(stderr, "step %d: %s\n", step, what);
    abort();
}

int main() {
    for (int round = 0; round < 40; ++round) {
        const int32_t n = 1 + (int32_t)(rnd() % 300);
        pkv_block_pool* p = pkv_pool_create(n);
        if (!p) fail("create", 0);
        std::vector<std::vector<int32_t>> reqs;     // blocks each live request references
        std::vector<int32_t> refs((size_t)n, 0);
        uint64_t next_hash = 1;
        for (int step = 0; step < 4000; ++step) {
            const int op = (int)(rnd() % 7);
            if (op == 0 || op == 1) {                // allocate for a new request
                const int32_t k = (int32_t)(rnd() % 8);
                std::vector<int32_t> ids((size_t)std::max(k, 1));
                const pkv_status s = pkv_pool_allocate(p, k, ids.data());
                if (s == PKV_OK) {
                    ids.resize((size_t)k);
                    for (int32_t i : ids) refs[(size_t)i]++;
                    reqs.push_back(ids);
                } else if (s != PKV_ERR_NO_BLOCKS) {
                    fail("allocate status", step);
                }
            } else if (op == 2 && !reqs.empty()) {   // a request finishes: tail first
                const size_t r = rnd() % reqs.size();
                std::vector<int32_t> ids = reqs[r];
                std::reverse(ids.begin(), ids.end());
                if (pkv_pool_free(p, ids.data(), (int32_t)ids.size()) != PKV_OK) fail("free", step);
                for (int32_t i : ids) refs[(size_t)i]--;
                reqs.erase(reqs.begin() + (long)r);
            } else if (op == 3 && !reqs.empty()) {   // a new request shares a prefix (hit)
                const std::vector<int32_t>& src = reqs[rnd() % reqs.size()];
                std::vector<int32_t> ids(src.begin(), src.begin() + (long)(rnd() % (src.size() + 1)));
                if (pkv_pool_touch(p, ids.data(), (int32_t)ids.size()) != PKV_OK) fail("touch", step);
                for (int32_t i : ids) refs[(size_t)i]++;
                reqs.push_back(ids);
            } else if (op == 4 && !reqs.empty()) {   // index a request's blocks by hash
                const std::vector<int32_t>& ids = reqs[rnd() % reqs.size()];
                std::vector<uint64_t> h(ids.size());
                for (auto& x : h) x = (rnd() % 4 == 0) ? 1 + rnd() % 16 : next_hash++;
                if (pkv_pool_cache_blocks(p, ids.data(), h.data(), (int32_t)ids.size()) != PKV_OK)
                    fail("cache", step);
                std::vector<int32_t> hit(h.size() + 1);
                if (pkv_pool_longest_hit(p, h.data(), (int32_t)h.size(), hit.data()) < 0)
                    fail("longest_hit", step);
            } else if (op == 5 && !reqs.empty()) {   // copy-on-write before a write
                std::vector<int32_t>& ids = reqs[rnd() % reqs.size()];
                if (ids.empty()) continue;
                const size_t j = rnd() % ids.size();
                int32_t out = -1, copy = -1;
                const pkv_status s = pkv_pool_cow(p, ids[j], &out, &copy);
                if (s == PKV_OK) {
                    if (copy) {
                        refs[(size_t)ids[j]]--;
                        refs[(size_t)out]++;
                        ids[j] = out;
                    } else if (out != ids[j]) {
                        fail("cow in place", step);
                    }
                } else if (s != PKV_ERR_NO_BLOCKS) {
                    fail("cow status", step);
                }
            } else if (op == 6) {                    // bad arguments are rejected, nothing changes
                const int32_t bad[2] = {n, -1};
                if (pkv_pool_free(p, bad, 1) != PKV_ERR_SHAPE) fail("free range", step);
                if (pkv_pool_touch(p, bad + 1, 1) != PKV_ERR_SHAPE) fail("touch range", step);
                if (pkv_pool_ref_count(p, n) != -1) fail("ref_count range", step);
            }
            // invariants
            std::vector<int32_t> q((size_t)n + 1);
            const int32_t len = pkv_pool_free_queue(p, q.data(), n + 1);
            if (len != pkv_pool_num_free(p)) fail("queue length", step);
            std::vector<char> seen((size_t)n, 0);
            for (int32_t k = 0; k < len; ++k) {
                const int32_t i = q[(size_t)k];
                if (i < 0 || i >= n || seen[(size_t)i]) fail("queue entry", step);
                seen[(size_t)i] = 1;
            }
            for (int32_t i = 0; i < n; ++i) {
                if (pkv_pool_ref_count(p, i) != refs[(size_t)i]) fail("reference count", step);
                if ((refs[(size_t)i] == 0) != (seen[(size_t)i] != 0)) fail("queue membership", step);
            }
        }
        pkv_pool_destroy(p);
    }
    const int32_t toks[3] = {1, 2, 3};
    if (pkv_block_hash(0, toks, 3) == pkv_block_hash(0, toks, 2)) abort();
    printf("block pool: 40 pools x 4000 random steps, invariants held\n");
    return 0;
}
