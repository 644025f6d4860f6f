// Drives every C entry point of libpagedkv's host layer (argument checks, geometry,
// workspace sizing, split set-up) over edge-case and random arguments, in a host-only
// build whose kernel launchers are stubs, under AddressSanitizer and
// UndefinedBehaviorSanitizer: any out-of-bounds access, signed overflow or invalid
// shift in the size arithmetic aborts the run.  Pointers are dummies: the stubs never
// touch memory, and no call reaches the device.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "pagedkv.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {            // splitmix64
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static const int32_t kEdges[] = {0, 1, 2, 3, 4, 7, 8, 16, 31, 32, 33, 63, 64, 65, 100, 128, 255, 256,
                                 1000, 4096, 65535, 65536, 1 << 20, 1 << 30, INT32_MAX, -1,
                                 INT32_MIN};
static int32_t pick() {
    const uint64_t r = next_u64();
    if (r % 3 == 0) return kEdges[(r >> 8) % (sizeof(kEdges) / sizeof(kEdges[0]))];
    if (r % 3 == 1) return (int32_t)((r >> 8) % 300);
    return (int32_t)(r >> 32);
}
static int32_t pick_small(const int32_t* v, int n) { return v[next_u64() % (uint64_t)n]; }

static void* P = (void*)0x1000;
static int n_ok = 0, n_err = 0;

static void note(pkv_status s) {
    if ((int)s < 0 || (int)s > 8) {
        fprintf(stderr, "status out of range: %d\n", (int)s);
        abort();
    }
    if (pkv_status_string(s) == nullptr) abort();
    (s == PKV_OK ? n_ok : n_err)++;
}

int main() {
    const int32_t dims[] = {64, 128, 96, 0, -64};
    const int32_t bss[] = {4, 8, 16, 32, 12, 64, 0};
    const int32_t dts[] = {0, 1, 2};
    for (int it = 0; it < 200000; ++it) {
        const pkv_dtype dt = (pkv_dtype)pick_small(dts, 3);
        const int32_t nb = next_u64() % 2 ? pick() : 1 + (int32_t)(next_u64() % 100000);
        const int32_t hkv = next_u64() % 2 ? pick() : 1 + (int32_t)(next_u64() % 16);
        const int32_t bs = pick_small(bss, 7), d = pick_small(dims, 5);
        const int32_t g = 1 + (int32_t)(next_u64() % 10);
        const int32_t hq = next_u64() % 4 ? (int32_t)((int64_t)hkv * g) : pick();
        const int32_t S = next_u64() % 2 ? pick() : (int32_t)(next_u64() % 5000);
        const int32_t mb = next_u64() % 2 ? pick() : 1 + (int32_t)(next_u64() % 20000);
        const int32_t maxctx = next_u64() % 2 ? pick() : (int32_t)(next_u64() % 300000);
        const int32_t pt = next_u64() % 2 ? 0 : pick();
        const float scale = next_u64() % 8 ? 0.088f : (next_u64() % 2 ? 0.f / 0.f : 1.f / 0.f);
        void* ptr = next_u64() % 16 ? P : nullptr;
        const size_t need = paged_attention_decode_workspace_bytes(S, hq, hkv, d, maxctx, pt);
        const size_t wsb = next_u64() % 2 ? need : (size_t)(next_u64() % (need + 2));
        void* ws = next_u64() % 8 ? P : nullptr;
        const int32_t T = pick();

        note(paged_kv_write(dt, ptr, P, nb, hkv, bs, d, P, P, (const int64_t*)P, T, nullptr));
        note(copy_blocks(dt, P, ptr, nb, hkv, bs, d, (const int64_t*)P, T, nullptr));
        note(paged_attention_decode(dt, ptr, P, P, P, nb, hkv, bs, d, (const int32_t*)P, mb,
                                    (const int32_t*)P, S, maxctx, hq, scale, pt, ws, wsb, nullptr));
        note(paged_attention_decode_noalloc(dt, ptr, P, P, P, nb, hkv, bs, d, (const int32_t*)P, mb,
                                            (const int32_t*)P, S, maxctx, hq, scale, pt, nullptr));
        const int32_t L = pick();
        note(contiguous_attention_decode(dt, ptr, P, P, P, S, L, hkv, d, (const int32_t*)P, maxctx,
                                         hq, scale, ws, wsb, nullptr));
        const int32_t nq = 1 + (int32_t)(next_u64() % 10);
        const size_t mqw = paged_attention_decode_multi_query_workspace_bytes(S, nq, hq, hkv, d);
        note(paged_attention_decode_multi_query(dt, ptr, P, P, P, nb, hkv, bs, d, (const int32_t*)P,
                                                mb, (const int32_t*)P, S, nq, maxctx, hq, scale, ws,
                                                next_u64() % 2 ? mqw : wsb, nullptr));
        const int32_t ng = next_u64() % 3 ? 1 + (int32_t)(next_u64() % 8) : pick();
        const int32_t mgs = pick(), mpl = pick();
        const size_t spw = paged_attention_decode_shared_prefix_workspace_bytes(S, hq, hkv, d, maxctx,
                                                                                mpl);
        note(paged_attention_decode_shared_prefix(
            dt, ptr, P, P, P, nb, hkv, bs, d, (const int32_t*)P, mb, (const int32_t*)P, S, maxctx,
            hq, scale, (const int32_t*)P, (const int32_t*)P, (const int32_t*)P, (const int32_t*)P,
            ng, mgs, mpl, ws, next_u64() % 2 ? spw : wsb, nullptr));
        const int32_t nc = pick(), mq = pick();
        const size_t pfw = paged_attention_prefill_chunk_workspace_bytes(hq, hkv, d);
        note(paged_attention_prefill_chunk(dt, ptr, P, (const int32_t*)P, nc, mq, P, P, nb, hkv, bs,
                                           d, (const int32_t*)P, mb, (const int32_t*)P, maxctx, hq,
                                           scale, next_u64() % 2 ? ws : nullptr,
                                           next_u64() % 2 ? pfw : wsb, nullptr));
        note(pkv_validate(nb, bs, (const int32_t*)ptr, mb, (const int32_t*)P, S, (const int64_t*)P, T,
                          (const int64_t*)P, pick(), (int32_t*)P, nullptr));
        note(pkv_validate_chunks((const int32_t*)ptr, (const int32_t*)P, pick(), pick(),
                                 next_u64() % 2 ? (int32_t*)P : nullptr, nullptr));
        // swap_blocks reads its host block mapping: a real host array, ids checked first
        std::vector<int64_t> map((size_t)2 * 8);
        for (auto& x : map) x = (int64_t)(int32_t)pick();
        const int32_t np = (int32_t)(next_u64() % 9);
        note(swap_blocks(dt, P, P, nb, P, P, nb, hkv, bs, d, map.data(), np, nullptr) );
    }
    printf("api calls: %d ok, %d rejected\n", n_ok, n_err);
    return 0;
}
