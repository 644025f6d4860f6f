// Chunked-prefill attention over a paged KV cache on the gfx950 matrix cores.
//
// What is computed ("Inside vLLM, part 2", chunked prefill): a long prompt is
// processed a bounded chunk of tokens per step; the chunk's queries attend
// causally to the whole cached prefix and to the chunk itself.  Chunk c holds
// n_q queries, the last n_q positions of its context; query i at position
// p = ctx - n_q + i sees keys t <= p.  Keys are read through the block table
// ("2.1 PagedAttention", sections 3 and 5).
//
// Mapping: one workgroup (4 waves) owns 128 packed query rows of one
// (chunk, kv head): row r = (query r / G, head r % G) of the G query heads that
// share the kv head, so every K/V tile is loaded once for all G heads.  Per
// 64-key tile:
//   S^T = K Q^T       v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q rows
//                     held in registers; the C layout gives each lane one query
//                     row (column) and 16 keys per 32-key block, so the row-wise
//                     softmax is lane-local plus one permlane32 swap;
//   O^T += V^T P^T    A = V^T from LDS in the key order in which the C registers
//                     of S^T hold them, B = bf16 P^T straight from those registers.
// Head dim 128 (dma_attend_tiles, pkv_attn_tiles.h): K/V tiles go from the pool
// straight into LDS with direct loads, both row-major with XOR-permuted chunks, and
// V^T is read with the transposing LDS read; step j loads V of tile j+1 and K of
// tile j+2 and runs the S^T products of tile j+1 beside the softmax of tile j, with
// one barrier per tile.  Head dim 64 (attend below): two register stages hold the
// K/V of tiles j+1 and j+2 while tile j's products run, and V is written transposed
// with a 16-byte XOR swizzle that keeps the transposing writes and the operand reads
// free of bank conflicts.  Workgroups are ordered so that all query tiles of one
// (chunk, kv head) run on the same XCD and share its L2.
// Keys past the context get -inf scores by selection (whatever stale data their K
// rows hold) and their V rows repeat the last token's row, so stale or NaN slots
// never reach the output.
//
// Balanced key split.  With one workgroup per query tile, a batch whose work items
// all fit in one round of resident workgroups lasts as long as its longest chunk.
// Given a workspace, and when the items fit in one round but the longest holds over
// 5/4 of an even share, the kernel instead cuts the 64-key tiles of all items,
// ordered by (chunk, kv head, query tile, tile), into one contiguous range per
// resident workgroup.  An item inside one range is finished in place; an item cut
// by range ends leaves partial states (normalised bf16 output, reference maximum,
// sum) in two slots per workgroup, and the workgroup that starts it records which
// workgroups hold its pieces; prefill_merge_kernel combines them by log-sum-exp.
// Every workgroup derives the same plan from the chunk lengths, so no host pass has
// to agree on it.
#include "pkv_attn_tiles.h"
#include "pkv_split.h"

#include <mutex>
#include <type_traits>

namespace pkv {

// ---- the plan of the balanced split -----------------------------------------------

// Chunk c as the kernels see it: first query row, queries, clamped context, and the
// query tiles that hold work (none for a malformed chunk: n_q > ctx, or a negative
// first row).
struct PfChunk {
    int q0, nq, ctx, nqt;
};
template <int QP>
__device__ __forceinline__ PfChunk pf_chunk(const PrefillArgs& a, int c, int num_q_tiles) {
    PfChunk k;
    k.q0 = as_const(a.cu_q_lens)[c];
    k.nq = as_const(a.cu_q_lens)[c + 1] - k.q0;
    const int ctx = as_const(a.context_lens)[c];
    k.ctx = max(0, min(ctx, min(a.max_context_len, a.max_blocks_per_seq * a.g.block_size)));
    k.nqt = (k.q0 < 0 || k.nq <= 0 || k.nq > k.ctx) ? 0 : min((k.nq + QP - 1) / QP, num_q_tiles);
    return k;
}
// 64-key tiles query tile qt (< nqt) reads: keys up to the causal limit of its last row.
template <int QP>
__device__ __forceinline__ int pf_tiles(const PfChunk& k, int qt) {
    return (k.ctx - k.nq + min(k.nq, (qt + 1) * QP) + kKeyTile - 1) / kKeyTile;
}
// Tiles of all query tiles of a chunk (one kv head); maxn takes the largest item.
template <int QP>
__device__ __forceinline__ int pf_chunk_tiles(const PfChunk& k, int& maxn) {
    int t = 0;
    for (int qt = 0; qt < k.nqt; ++qt) {
        const int n = pf_tiles<QP>(k, qt);
        t += n;
        maxn = max(maxn, n);
    }
    return t;
}
__device__ __forceinline__ int wave_max_int(int x) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) x = max(x, __shfl_xor(x, d));
    return __builtin_amdgcn_readfirstlane(x);
}

struct PfPlan {
    int64_t T;       // tiles of all items (all kv heads)
    int maxn;        // tiles of the largest item
    int items;       // items with work
};
// Totals over the batch; every wave computes them alike (lanes over chunks).
template <int QP>
__device__ __forceinline__ PfPlan pf_totals(const PrefillArgs& a, int num_chunks, int num_q_tiles) {
    const int lane = threadIdx.x & 63;
    PfPlan p{0, 0, 0};
    for (int c0 = 0; c0 < num_chunks; c0 += 64) {
        int ct = 0, mx = 0, ni = 0;
        if (c0 + lane < num_chunks) {
            const PfChunk k = pf_chunk<QP>(a, c0 + lane, num_q_tiles);
            ct = pf_chunk_tiles<QP>(k, mx);
            ni = k.nqt;
        }
        p.T += wave_sum_int(ct);
        p.maxn = max(p.maxn, wave_max_int(mx));
        p.items += wave_sum_int(ni);
    }
    p.T *= a.g.num_kv_heads;
    p.items *= a.g.num_kv_heads;
    return p;
}
// The split pays only when the items fit in one round of workgroups and the largest
// exceeds an even share by a quarter.
__device__ __forceinline__ bool pf_balanced(const PfPlan& p, int64_t W) {
    return p.T > 0 && p.items <= W && 4 * (int64_t)p.maxn > 5 * ((p.T + W - 1) / W);
}
// Ranges of the split: one per workgroup, but never more than tiles (so none is empty).
__device__ __forceinline__ int pf_ranges(const PfPlan& p, int num_wgs) {
    return (int)min((int64_t)num_wgs, p.T);
}
// Tiles (all kv heads) of the chunks before chunk `upto`, or, with upto < 0, the chunk
// holding tile b and the tiles before it (one inclusive scan per 64 chunks).
template <int QP>
__device__ __forceinline__ void pf_locate(const PrefillArgs& a, int num_chunks, int num_q_tiles,
                                          int upto, int64_t b, int& c, int64_t& before) {
    const int lane = threadIdx.x & 63;
    int64_t carry = 0;
    c = num_chunks;
    before = 0;
    for (int c0 = 0; c0 < num_chunks; c0 += 64) {
        int ct = 0, mx = 0;
        if (c0 + lane < num_chunks)
            ct = pf_chunk_tiles<QP>(pf_chunk<QP>(a, c0 + lane, num_q_tiles), mx) *
                 a.g.num_kv_heads;
        if (upto >= 0) {
            if (c0 >= upto) break;
            carry += wave_sum_int(c0 + lane < upto ? ct : 0);
            continue;
        }
        int incl = ct;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        const uint64_t hit = __ballot(carry + incl > b);
        if (hit) {
            const int ln = __ffsll((unsigned long long)hit) - 1;
            c = c0 + ln;
            before = carry + __builtin_amdgcn_readlane(incl - ct, ln);
            return;
        }
        carry += __builtin_amdgcn_readlane(incl, 63);
    }
    before = carry;
}

// ---- attention of one query tile over a range of its key tiles -------------------

template <int D>
struct PfLds {
    char k[2][kKeyTile * PrefillShape<D>::KPITCH];
    char vt[2][D * PrefillShape<D>::VPITCH];
};

// Query tile qt of (chunk k, kv head h) over its key tiles [k0, k1): the normalised
// output when slot < 0, else the state of each row (normalised output, reference
// maximum m, sum l) into partial slot `slot`.  Every wave of the workgroup calls it alike (it has barriers).
template <int D, int G>
__device__ __forceinline__ void attend(const PrefillArgs& a, const PfChunk& k, int c, int h,
                                       int qt, int k0, int k1, int64_t slot, PfLds<D>& lds) {
    using P = PrefillShape<D>;
    constexpr int QP = kRowsPerWg / G;           // query positions per workgroup

    // An empty asm hides the thread id from loop-invariant code motion: otherwise the
    // per-lane addresses of a workgroup's later pieces are computed once, before its
    // first piece, and held in registers through every tile loop (which spills).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int lane = tid & 63;
    const int n = lane & 31;
    const int half = lane >> 5;
    const int Hq = a.num_q_heads;
    const int bs = a.g.block_size;
    const int mb = a.max_blocks_per_seq;

    const int q0 = k.q0, nq = k.nq, ctx = k.ctx;
    const int32_t* table = a.block_tables + (int64_t)c * mb;
    const char* kb = a.k_pool + (int64_t)h * a.g.head_stride_bytes;
    const char* vb = a.v_pool + (int64_t)h * a.g.head_stride_bytes;

    // this lane's query row
    const int r = w * 32 + n;
    const int qi = r / G;
    const int hh = r - qi * G;
    const int qpos_local = qt * QP + qi;
    const bool row_valid = (r < QP * G) && (qpos_local < nq);
    const int64_t qidx = (int64_t)q0 + qpos_local;
    // last key the row sees (causal limit); -1 hides every key from rows past the chunk
    const int last_key = row_valid ? ctx - nq + qpos_local : -1;

    u32x4 qreg[P::KSTEPS];
    {
        const char* qp = reinterpret_cast<const char*>(a.q) +
                         (qidx * Hq + (int64_t)h * G + hh) * P::RB + half * 16;
#pragma unroll
        for (int ks = 0; ks < P::KSTEPS; ++ks)
            qreg[ks] = row_valid ? *reinterpret_cast<const u32x4*>(qp + ks * 32)
                                 : u32x4{0u, 0u, 0u, 0u};
    }
    // Every row of the wave sees all keys below full_end: the smallest position
    // among its rows bounds them.  Rows past the chunk then compute on zero queries
    // and are never stored; each output column depends on its own row only.
    const int full_end = min(ctx - nq + qt * QP + (w * 32) / G + 1, ctx);

    floatx16_t oacc[P::DT];
#pragma unroll
    for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
    float m = kNoMax, l = 0.f;           // running max (log2 units) and sum of the row
    const float sl2 = a.scale_log2;

    // keys [t_begin, t_end): the range's tiles, up to the last key any row may see
    const int t_begin = k0 * kKeyTile;
    const int t_end = min(k1 * kKeyTile, ctx - nq + min(nq, (qt + 1) * QP));

    // Two K/V stages in registers and two sets of block ids, alternating with the
    // parity of the tile: at tile j, the table reads of tile j+3 go out first, then the
    // K/V reads of tile j+2 (with ids read during tile j-1), so each wait of the
    // in-order load counter covers only what it needs.
    KvStage<D> st0, st1;
    TileIds<D> ids0, ids1;
    TileOffs<D> offs;
    tile_offsets<D>(offs, bs, tid);
    load_ids<D>(ids0, table, a.g, ctx, t_begin, tid);
    load_tile<D>(st0, ids0, offs, a.g, kb, vb, ctx, t_begin, tid);
    load_ids<D>(ids1, table, a.g, ctx, t_begin + kKeyTile, tid);
    if (t_begin + kKeyTile < t_end)
        load_tile<D>(st1, ids1, offs, a.g, kb, vb, ctx, t_begin + kKeyTile, tid);
    load_ids<D>(ids0, table, a.g, ctx, t_begin + 2 * kKeyTile, tid);
    store_tile<D>(st0, lds.k[0], lds.vt[0], tid);
    __syncthreads();

    // one tile: prefetch tile t0 + 128 into `next2` (ids in `use`; the ids of tile
    // t0 + 192 into `load`), attend tile t0 from LDS, then move tile t0 + 64 (in
    // `next1`) into LDS
    auto step = [&](int t0, int buf, KvStage<D>& next2, const KvStage<D>& next1,
                    const TileIds<D>& use, TileIds<D>& load) {
        const char* tk = lds.k[buf];
        const char* tv = lds.vt[buf];
        if (t0 + 2 * kKeyTile < t_end) {
            load_ids<D>(load, table, a.g, ctx, t0 + 3 * kKeyTile, tid);
            load_tile<D>(next2, use, offs, a.g, kb, vb, ctx, t0 + 2 * kKeyTile, tid);
        }
        // ---- S^T = K Q^T ----------------------------------------------------------
        floatx16_t sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[mt][e] = 0.f;
#pragma unroll
            for (int ks = 0; ks < P::KSTEPS; ++ks) {
                const u32x4 ka = *reinterpret_cast<const u32x4*>(
                    tk + (mt * 32 + n) * P::KPITCH + ks * 32 + half * 16);
                sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8_t, ka), __builtin_bit_cast(bf16x8_t, qreg[ks]),
                    sacc[mt], 0, 0, 0);
            }
        }

        // ---- online softmax; lane holds keys t0 + 32mt + 8(e/4) + 4half + e%4 -----
        // On unmasked tiles with a positive scale the max is taken on raw scores and
        // the scale folds into the exponent's fma; otherwise scores are scaled first
        // and hidden keys set to -inf.
        const bool scaled = t0 + kKeyTile > full_end || !(sl2 > 0.f);   // wave-uniform
        const float mul = scaled ? 1.f : sl2;
        if (scaled) {
            const int lim = last_key - t0 - 4 * half;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    sacc[mt][e] = (mt * 32 + 8 * (e >> 2) + (e & 3) <= lim) ? sacc[mt][e] * sl2
                                                                            : -INFINITY;
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, sacc[mt][e]);
        // The reference maximum m moves only when some row of the wave outgrew it by
        // more than kLazyMax (log2 units): probabilities stay below 2^kLazyMax, far
        // inside the bf16 and fp32 ranges, and the rescales of O become rare.
        const float mx = fmaxf(m, swap32_max(mloc) * mul);
        if (__builtin_amdgcn_ballot_w64(mx > m + kLazyMax)) {
            const float alpha = fast_exp2(m - mx);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
            m = mx;
        }
        const float mn = m;
        u32x4 pk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int mt = u >> 1, e0 = (u & 1) * 8;
            float p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = fast_exp2(__builtin_fmaf(sacc[mt][e0 + j], mul, -mn));
            pk[u] = u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                          pack_bf16(p[6], p[7])};
            l = sum_bf16x8(pk[u], l);
        }

        // ---- O^T += V^T P^T ---------------------------------------------------------
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x4 va = *reinterpret_cast<const u32x4*>(
                    tv + vt_off<D>(dt * 32 + n, 2 * u + half));
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8_t, va), __builtin_bit_cast(bf16x8_t, pk[u]),
                    oacc[dt], 0, 0, 0);
            }

        // the other buffer held tile j-1, which every wave finished before the last
        // barrier; the barrier below publishes tile j+1 and frees this buffer
        if (t0 + kKeyTile < t_end) store_tile<D>(next1, lds.k[buf ^ 1], lds.vt[buf ^ 1], tid);
        __syncthreads();
    };
    for (int t0 = t_begin; t0 < t_end; t0 += 2 * kKeyTile) {
        step(t0, 0, st0, st1, ids0, ids1);
        if (t0 + kKeyTile >= t_end) break;
        step(t0 + kKeyTile, 1, st1, st0, ids1, ids0);
    }

    // ---- store: lane holds d = 32dt + 8(e/4) + 4half + e%4 of its row ---------------
    // The normalised row goes to the output, or for a piece of a cut item to its
    // partial slot, with the row's (reference maximum, sum) beside it (both halves of
    // the wave hold the same maximum).
    const float lt = swap32_sum(l);
    if (!row_valid) return;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* orow;
    if (slot >= 0) {
        orow = a.part_o + (slot * kRowsPerWg + r) * D;
        if (half == 0)
            *reinterpret_cast<float2*>(a.part_ml + (slot * kRowsPerWg + r) * 2) = make_float2(m, lt);
    } else {
        orow = reinterpret_cast<uint16_t*>(a.out) + (qidx * Hq + (int64_t)h * G + hh) * D;
    }
#pragma unroll
    for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d = dt * 32 + 8 * g4 + 4 * half;
            uint2 wv;
            wv.x = pack_bf16(oacc[dt][4 * g4 + 0] * inv, oacc[dt][4 * g4 + 1] * inv);
            wv.y = pack_bf16(oacc[dt][4 * g4 + 2] * inv, oacc[dt][4 * g4 + 3] * inv);
            *reinterpret_cast<uint2*>(orow + d) = wv;
        }
}

template <int G>
__device__ __forceinline__ void attend_dma(const PrefillArgs& a, const PfChunk& k, int c, int h,
                                           int qt, int k0, int k1, int64_t slot, PfLdsDma& lds) {
    constexpr int D = 128, RB = 256;
    using P = PrefillShape<D>;
    constexpr int QP = kRowsPerWg / G;

    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 31;
    const int half = lane >> 5;
    const int Hq = a.num_q_heads;
    const int mb = a.max_blocks_per_seq;

    const int q0 = k.q0, nq = k.nq, ctx = k.ctx;
    const int32_t* table = a.block_tables + (int64_t)c * mb;
    const char* kb = a.k_pool + (int64_t)h * a.g.head_stride_bytes;
    const char* vb = a.v_pool + (int64_t)h * a.g.head_stride_bytes;

    const int r = w * 32 + n;
    const int qi = r / G;
    const int hh = r - qi * G;
    const int qpos_local = qt * QP + qi;
    const bool row_valid = (r < QP * G) && (qpos_local < nq);
    const int last_key = row_valid ? ctx - nq + qpos_local : -1;

    u32x4 qreg[P::KSTEPS];
    // the tile loop loads the rows beside the first tiles' block ids; a row past the
    // chunk (or past the packed rows) reads the chunk's last query row, with no branch
    // (whose waits would also wait for those ids): every key is masked for it
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     (((int64_t)q0 + min(qpos_local, nq - 1)) * Hq + (int64_t)h * G + hh) * RB +
                     half * 16;
    auto load_q = [&](u32x4 (&qr)[P::KSTEPS]) {
#pragma unroll
        for (int ks = 0; ks < P::KSTEPS; ++ks) qr[ks] = *reinterpret_cast<const u32x4*>(qp + ks * 32);
    };
    const int full_end = min(ctx - nq + qt * QP + (w * 32) / G + 1, ctx);

    floatx16_t oacc[P::DT];
#pragma unroll
    for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
    float m = kNoMax, l = 0.f;
    const float sl2 = a.scale_log2;

    const int t_begin = k0 * kKeyTile;
    const int t_end = min(k1 * kKeyTile, ctx - nq + min(nq, (qt + 1) * QP));

    dma_attend_tiles(lds, table, a.g, kb, vb, ctx, t_begin, t_end, full_end, last_key, sl2, load_q,
                     qreg, oacc, m, l);

    const float lt = swap32_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (slot >= 0 && row_valid && half == 0)
        *reinterpret_cast<float2*>(a.part_ml + (slot * kRowsPerWg + r) * 2) = make_float2(m, lt);
    // The rows leave through LDS (the tile loop ends with a barrier after its last reads,
    // so the buffers are free): lane (n, half) puts its bf16 elements of row n into a
    // staged copy of the wave's 32 rows, then each store writes 256 contiguous bytes of
    // one row (lane 16 i' + j: bytes 16 j .. 16 j + 15 of row 4 i + i'), instead of 16
    // bytes of each of 32 rows.
    constexpr int kPitch = 272;                // bytes per staged row: 256 + 16
    static_assert(4 * 32 * kPitch <= (int)sizeof(PfLdsDma), "staging fits the tile buffers");
    char* stage = reinterpret_cast<char*>(&lds) + w * 32 * kPitch;
#pragma unroll
    for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            uint2 wv;
            wv.x = pack_bf16(oacc[dt][4 * g4 + 0] * inv, oacc[dt][4 * g4 + 1] * inv);
            wv.y = pack_bf16(oacc[dt][4 * g4 + 2] * inv, oacc[dt][4 * g4 + 3] * inv);
            *reinterpret_cast<uint2*>(stage + n * kPitch + 64 * dt + 16 * g4 + 8 * half) = wv;
        }
    const int j16 = lane & 15;
    u32x4 rowv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        rowv[i] = *reinterpret_cast<const u32x4*>(stage + (4 * i + (lane >> 4)) * kPitch + 16 * j16);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r2 = w * 32 + 4 * i + (lane >> 4);
        const int qi2 = r2 / G;
        const int hh2 = r2 - qi2 * G;
        if (r2 < QP * G && qt * QP + qi2 < nq) {
            uint16_t* dst = slot >= 0
                                ? a.part_o + (slot * kRowsPerWg + r2) * D
                                : reinterpret_cast<uint16_t*>(a.out) +
                                      (((int64_t)q0 + qt * QP + qi2) * Hq + (int64_t)h * G + hh2) * D;
            *reinterpret_cast<u32x4*>(dst + 8 * j16) = rowv[i];
        }
    }
    __syncthreads();                           // the next piece's loads reuse the buffers
}

// The workgroup's LDS and its tile loop for head dimension D.
template <int D>
struct PfTiles {
    using Lds = PfLds<D>;
};
template <>
struct PfTiles<128> {
    using Lds = PfLdsDma;
};
template <int D, int G, typename L>
__device__ __forceinline__ void attend_any(const PrefillArgs& a, const PfChunk& k, int c, int h,
                                           int qt, int k0, int k1, int64_t slot, L& lds) {
    if constexpr (D == 128)
        attend_dma<G>(a, k, c, h, qt, k0, k1, slot, lds);
    else
        attend<D, G>(a, k, c, h, qt, k0, k1, slot, lds);
}

template <int D, int G>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a, int num_chunks,
                                                         int num_q_tiles, int num_items) {
    constexpr int QP = kRowsPerWg / G;
    // two LDS tile buffers: tile j is read from buffer j % 2 while tile j+1 is
    // written into the other one, so one barrier per tile suffices
    __shared__ __attribute__((aligned(16))) typename PfTiles<D>::Lds lds;

    const int Hkv = a.g.num_kv_heads;
    // The walk over this workgroup's tiles [u, e) in the batch order.  The host keeps
    // every tile count below 2^30, so the walk runs in 32 bits; readfirstlane keeps its
    // state in scalar registers (the divisions that start it run on the vector unit).
    int c, h, qt, k0, u, e, w = 0;
    int64_t tiles = 1, nw = 1;           // the split's tiles and ranges (when it splits)
    PfPlan p{0, 0, 0};
    if (a.part_o != nullptr) p = pf_totals<QP>(a, num_chunks, num_q_tiles);
    if (a.part_o != nullptr && pf_balanced(p, a.num_wgs)) {
        // W = min(workgroups, tiles) ranges, none empty (the merge reads a slot of every
        // workgroup between an item's first and last owner), in order over the XCDs:
        // neighbouring ranges (the query tiles of one (chunk, kv head)) share one XCD's L2
        const int W = pf_ranges(p, a.num_wgs);
        const int Wr = (W + kXcds - 1) / kXcds * kXcds;   // <= the grid size
        if ((int)blockIdx.x >= Wr) return;
        w = (blockIdx.x % kXcds) * (Wr / kXcds) + blockIdx.x / kXcds;
        if (w >= W) return;
        tiles = p.T;
        nw = W;
        const Split sp = even_split(p.T, W);
        u = __builtin_amdgcn_readfirstlane((int)range_begin(sp, w));
        e = __builtin_amdgcn_readfirstlane((int)range_begin(sp, w + 1));
        if (u >= e) return;
        int64_t before;
        pf_locate<QP>(a, num_chunks, num_q_tiles, -1, u, c, before);
        if (c >= num_chunks) return;
        const PfChunk k = pf_chunk<QP>(a, c, num_q_tiles);
        int mx = 0;
        const int ct = pf_chunk_tiles<QP>(k, mx);
        if (ct <= 0) return;
        int rem = u - (int)before;
        h = __builtin_amdgcn_readfirstlane(rem / ct);
        rem -= h * ct;
        for (qt = 0; qt < k.nqt; ++qt) {
            const int nt = pf_tiles<QP>(k, qt);
            if (rem < nt) break;
            rem -= nt;
        }
        if (h >= Hkv || qt >= k.nqt) return;
        k0 = __builtin_amdgcn_readfirstlane(rem);
    } else {
        // one item per workgroup, XCD-aware: consecutive items (the query tiles of one
        // (chunk, kv head)) get workgroup ids that are equal modulo the XCD count
        const int nwg = gridDim.x;
        const int item = (blockIdx.x % kXcds) * (nwg / kXcds) + blockIdx.x / kXcds;
        if (item >= num_items) return;
        qt = __builtin_amdgcn_readfirstlane(item % num_q_tiles);
        h = __builtin_amdgcn_readfirstlane((item / num_q_tiles) % Hkv);
        c = __builtin_amdgcn_readfirstlane(item / (num_q_tiles * Hkv));
        const PfChunk k = pf_chunk<QP>(a, c, num_q_tiles);
        if (qt >= k.nqt) return;
        k0 = 0;
        u = 0;
        e = pf_tiles<QP>(k, qt);
    }
    PfChunk k = pf_chunk<QP>(a, c, num_q_tiles);
    // the next item with work after (c, h, qt); there is one while tiles remain
    auto next_item = [&]() {
        if (++qt == k.nqt) {
            qt = 0;
            if (++h == Hkv) {
                h = 0;
                do {
                    if (++c >= num_chunks) return;
                    k = pf_chunk<QP>(a, c, num_q_tiles);
                } while (k.nqt == 0);
            }
        }
    };
    // A range that starts inside an item continues a piece of an earlier workgroup: that
    // piece (slot 0) is attended last, so every workgroup starts at the first key of an
    // item and the query tiles of one (chunk, kv head) on an XCD walk the same keys at
    // about the same time, which keeps their shared K/V tiles in its L2.
    int dc = -1, dh = 0, dqt = 0, dk0 = 0, dk1 = 0;
    if (k0 > 0) {
        dc = c;
        dh = h;
        dqt = qt;
        dk0 = k0;
        dk1 = min(pf_tiles<QP>(k, qt), k0 + (e - u));
        u += dk1 - k0;
        k0 = 0;
        if (u < e) next_item();
    }
    while (u < e && c < num_chunks) {
        const int nt = pf_tiles<QP>(k, qt);
        const int k1 = min(nt, e - u);           // every piece here starts its item
        // a cut item: the piece starting at its first tile goes to slot 1 of the
        // workgroup (a piece continuing one from an earlier workgroup goes to slot 0)
        const int64_t slot = k1 == nt ? -1 : 2 * (int64_t)w + 1;
        // the workgroup that starts an item tells the merge which workgroups hold its
        // pieces (none when it finishes the item itself)
        if (a.part_o != nullptr && threadIdx.x == 0) {
            const int pieces =
                k1 == nt ? 0 : (int)(unit_owner(even_split(tiles, nw), (int64_t)u + nt - 1) - w + 1);
            const int item = (c * Hkv + h) * num_q_tiles + qt;
            *reinterpret_cast<int2*>(a.item_desc + 2 * item) = make_int2(w, pieces);
        }
        attend_any<D, G>(a, k, c, h, qt, 0, k1, slot, lds);
        u += k1;
        if (u < e) next_item();
    }
    if (dc >= 0)
        attend_any<D, G>(a, pf_chunk<QP>(a, dc, num_q_tiles), dc, dh, dqt, dk0, dk1, 2 * (int64_t)w,
                         lds);
}

// One workgroup per work item; nothing to do unless the kernel cut the item.  Thread
// t combines quarter t % 4 of row t / 4 over the item's pieces (four per round of
// loads), weighting each piece's normalised output by l 2^(m - M) with M the running
// maximum.
constexpr int kMergeThreads = 512;
template <int D, int G>
__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(PrefillArgs a, int num_q_tiles,
                                                                      int num_items) {
    constexpr int QP = kRowsPerWg / G;
    constexpr int PARTS = kMergeThreads / kRowsPerWg;   // threads per row
    constexpr int PART = D / PARTS;            // elements per thread
    constexpr int NV = PART / 8;               // 16-byte vectors per thread and piece
    constexpr int PB = 4;                      // pieces per round of loads
    const int item = blockIdx.x;
    if (item >= num_items) return;
    const int Hkv = a.g.num_kv_heads;
    const int qt = item % num_q_tiles;
    const int h = (item / num_q_tiles) % Hkv;
    const int c = item / (num_q_tiles * Hkv);
    // the descriptor slot exists for every item of the grid (item < num_wgs), so it is
    // read beside the chunk's bounds and discarded when the item has no work
    const int2 desc = *reinterpret_cast<const int2*>(a.item_desc + 2 * item);
    const PfChunk k = pf_chunk<QP>(a, c, num_q_tiles);
    if (qt >= k.nqt) return;                   // no work item, no descriptor
    const int w0 = __builtin_amdgcn_readfirstlane(desc.x);
    int np = __builtin_amdgcn_readfirstlane(desc.y);
    if (np <= 0) return;                       // finished in place
    // the kernel writes a descriptor for every item with work; the bounds keep even a
    // stale one inside the workspace's slots
    if (w0 < 0 || w0 >= a.num_wgs) return;
    np = min(np, a.num_wgs - w0);
    const int r = threadIdx.x / PARTS, part = threadIdx.x % PARTS;
    const int qi = r / G, hh = r - qi * G;
    if (r >= QP * G || qt * QP + qi >= k.nq) return;
    auto slot_of = [&](int j) -> int64_t { return j == 0 ? 2 * (int64_t)w0 + 1 : 2 * (int64_t)(w0 + j); };
    float M = kNoMax, L = 0.f;
    float acc[PART];
#pragma unroll
    for (int i = 0; i < PART; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < np; j0 += PB) {
        float2 ml[PB];
        u32x4 v[PB][NV];
#pragma unroll
        for (int b = 0; b < PB; ++b) {
            const int64_t s = slot_of(min(j0 + b, np - 1)) * kRowsPerWg + r;
            ml[b] = *reinterpret_cast<const float2*>(a.part_ml + s * 2);
            const u32x4* src = reinterpret_cast<const u32x4*>(a.part_o + s * D + part * PART);
#pragma unroll
            for (int i = 0; i < NV; ++i) v[b][i] = src[i];
        }
        float Mn = M;
#pragma unroll
        for (int b = 0; b < PB; ++b) {
            if (j0 + b >= np) ml[b] = make_float2(kNoMax, 0.f);   // clamped repeats weigh 0
            Mn = fmaxf(Mn, ml[b].x);
        }
        const float sc = fast_exp2(M - Mn);
        float wt[PB];
        L *= sc;
#pragma unroll
        for (int b = 0; b < PB; ++b) {
            wt[b] = ml[b].y * fast_exp2(ml[b].x - Mn);
            L += wt[b];
        }
        M = Mn;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float lo = acc[8 * i + 2 * q] * sc, hi = acc[8 * i + 2 * q + 1] * sc;
#pragma unroll
                for (int b = 0; b < PB; ++b) {
                    const uint32_t x = v[b][i][q];
                    lo = fmaf(wt[b], bf16lo(x), lo);
                    hi = fmaf(wt[b], bf16hi(x), hi);
                }
                acc[8 * i + 2 * q] = lo;
                acc[8 * i + 2 * q + 1] = hi;
            }
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) +
                     (((int64_t)k.q0 + qt * QP + qi) * a.num_q_heads + (int64_t)h * G + hh) * D +
                     part * PART;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        u32x4 o;
        o.x = pack_bf16(acc[8 * i + 0] * inv, acc[8 * i + 1] * inv);
        o.y = pack_bf16(acc[8 * i + 2] * inv, acc[8 * i + 3] * inv);
        o.z = pack_bf16(acc[8 * i + 4] * inv, acc[8 * i + 5] * inv);
        o.w = pack_bf16(acc[8 * i + 6] * inv, acc[8 * i + 7] * inv);
        reinterpret_cast<u32x4*>(orow)[i] = o;
    }
}

// resident workgroups of the prefill kernel on the current device (a multiple of the
// XCD count), cached per device
template <int D, int G>
static int prefill_wgs_t() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(prefill_kernel<D, G>), 256, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cache[dev] = max(kXcds, max(1, per_cu) * max(1, cus) / kXcds * kXcds);
    }
    return cache[dev];
}

template <int D, int G>
static hipError_t launch_prefill_t(const PrefillArgs& args, int num_chunks, int max_q_len,
                                   int max_context_len, hipStream_t st) {
    constexpr int QP = kRowsPerWg / G;
    const int nqt = (max_q_len + QP - 1) / QP;
    const int64_t items = (int64_t)nqt * args.g.num_kv_heads * num_chunks;
    if (items > (int64_t)1 << 30) return hipErrorInvalidValue;
    PrefillArgs a = args;
    // the split is possible only when every item fits in one round of resident
    // workgroups (and its tile counts stay far inside 32 bits)
    if (a.part_o != nullptr &&
        (a.num_wgs <= 0 || items > a.num_wgs ||
         items * ((max_context_len + kKeyTile - 1) / kKeyTile + 1) >= ((int64_t)1 << 30)))
        a.part_o = nullptr;
    int64_t nwg = (items + kXcds - 1) / kXcds * kXcds;   // a multiple of the XCD count
    if (a.part_o != nullptr) nwg = max(nwg, (int64_t)a.num_wgs);
    hipLaunchKernelGGL((prefill_kernel<D, G>), dim3((uint32_t)nwg), dim3(256), 0, st, a, num_chunks,
                       nqt, (int)items);
    if (a.part_o != nullptr)
        hipLaunchKernelGGL((prefill_merge_kernel<D, G>), dim3((uint32_t)items), dim3(kMergeThreads),
                           0, st, a, nqt, (int)items);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_g(const PrefillArgs& a, int group, int num_chunks, int max_q_len,
                                   int max_context_len, hipStream_t st) {
    switch (group) {
        case 1: return launch_prefill_t<D, 1>(a, num_chunks, max_q_len, max_context_len, st);
        case 2: return launch_prefill_t<D, 2>(a, num_chunks, max_q_len, max_context_len, st);
        case 3: return launch_prefill_t<D, 3>(a, num_chunks, max_q_len, max_context_len, st);
        case 4: return launch_prefill_t<D, 4>(a, num_chunks, max_q_len, max_context_len, st);
        case 5: return launch_prefill_t<D, 5>(a, num_chunks, max_q_len, max_context_len, st);
        case 6: return launch_prefill_t<D, 6>(a, num_chunks, max_q_len, max_context_len, st);
        case 7: return launch_prefill_t<D, 7>(a, num_chunks, max_q_len, max_context_len, st);
        case 8: return launch_prefill_t<D, 8>(a, num_chunks, max_q_len, max_context_len, st);
        default: return hipErrorInvalidValue;
    }
}

template <int D>
static int prefill_wgs_g(int group) {
    switch (group) {
        case 1: return prefill_wgs_t<D, 1>();
        case 2: return prefill_wgs_t<D, 2>();
        case 3: return prefill_wgs_t<D, 3>();
        case 4: return prefill_wgs_t<D, 4>();
        case 5: return prefill_wgs_t<D, 5>();
        case 6: return prefill_wgs_t<D, 6>();
        case 7: return prefill_wgs_t<D, 7>();
        case 8: return prefill_wgs_t<D, 8>();
        default: return 0;
    }
}

int prefill_wgs(int head_dim, int group) {
    if (head_dim == 128) return prefill_wgs_g<128>(group);
    if (head_dim == 64) return prefill_wgs_g<64>(group);
    return 0;
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int group, int num_chunks,
                          int max_q_len, hipStream_t st) {
    if (num_chunks == 0 || max_q_len == 0) return hipSuccess;
    if (head_dim == 128)
        return launch_prefill_g<128>(a, group, num_chunks, max_q_len, a.max_context_len, st);
    if (head_dim == 64)
        return launch_prefill_g<64>(a, group, num_chunks, max_q_len, a.max_context_len, st);
    return hipErrorInvalidValue;
}

}  // namespace pkv
