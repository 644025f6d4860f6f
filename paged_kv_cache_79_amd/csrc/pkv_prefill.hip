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
//   O^T += V^T P^T    A = V^T from LDS (stored transposed, keys in the order in
//                     which the C registers of S^T hold them), B = bf16 P^T
//                     straight from those registers.
// Software pipeline: while the matrix cores work on tile j from LDS, the K/V
// global loads of tiles j+1 and j+2 are in flight in two register stages (tile
// j+2's issued at the top of tile j, after the table reads of tile j+3: the
// in-order load counter then lets each wait cover only what it needs); tile j+1
// goes into the second LDS buffer after tile j's products, with one barrier per
// tile.  V is written transposed with a 16-byte XOR swizzle that keeps both the
// transposing writes and the operand reads free of bank conflicts.  Workgroups are
// ordered so that all query tiles of one (chunk, kv head) run on the same XCD and
// share its L2.
// Keys past the context get -inf scores by selection (whatever stale data their K
// rows hold) and their V rows repeat the last token's row, so stale or NaN slots
// never reach the output.
#include "pkv_attn_tiles.h"

namespace pkv {

template <int D, int G>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a, int num_q_tiles,
                                                         int num_items) {
    using P = PrefillShape<D>;
    constexpr int QP = kRowsPerWg / G;           // query positions per workgroup
    // two LDS tile buffers: tile j is read from buffer j % 2 while tile j+1 is
    // written into the other one, so one barrier per tile suffices
    __shared__ __attribute__((aligned(16))) char lds_k[2][kKeyTile * P::KPITCH];
    __shared__ __attribute__((aligned(16))) char lds_vt[2][D * P::VPITCH];

    // XCD-aware order: consecutive work items (the query tiles of one (chunk, kv head))
    // get workgroup ids that are equal modulo the XCD count.
    const int nwg = gridDim.x;
    const int item = (blockIdx.x % kXcds) * (nwg / kXcds) + blockIdx.x / kXcds;
    if (item >= num_items) return;
    const int qt = item % num_q_tiles;
    const int h = (item / num_q_tiles) % a.g.num_kv_heads;
    const int c = item / (num_q_tiles * a.g.num_kv_heads);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int lane = tid & 63;
    const int n = lane & 31;
    const int half = lane >> 5;
    const int Hq = a.num_q_heads;
    const int bs = a.g.block_size;
    const int mb = a.max_blocks_per_seq;

    const int q0 = as_const(a.cu_q_lens)[c];
    const int nq = as_const(a.cu_q_lens)[c + 1] - q0;
    int ctx = as_const(a.context_lens)[c];
    ctx = max(0, min(ctx, min(a.max_context_len, mb * bs)));
    if (qt * QP >= nq || nq > ctx) return;
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

    // keys any row of this workgroup may see
    const int t_stop = ctx - nq + min(nq, (qt + 1) * QP);

    // Two K/V stages in registers and two sets of block ids, alternating with the
    // parity of the tile: at tile j, the table reads of tile j+3 go out first, then the
    // K/V reads of tile j+2 (with ids read during tile j-1), so each wait of the
    // in-order load counter covers only what it needs.
    KvStage<D> st0, st1;
    TileIds<D> ids0, ids1;
    TileOffs<D> offs;
    tile_offsets<D>(offs, bs, tid);
    load_ids<D>(ids0, table, a.g, ctx, 0, tid);
    load_tile<D>(st0, ids0, offs, a.g, kb, vb, ctx, 0, tid);
    load_ids<D>(ids1, table, a.g, ctx, kKeyTile, tid);
    if (kKeyTile < t_stop) load_tile<D>(st1, ids1, offs, a.g, kb, vb, ctx, kKeyTile, tid);
    load_ids<D>(ids0, table, a.g, ctx, 2 * kKeyTile, tid);
    store_tile<D>(st0, lds_k[0], lds_vt[0], tid);
    __syncthreads();

    // one tile: prefetch tile t0 + 128 into `next2` (ids in `use`; the ids of tile
    // t0 + 192 into `load`), attend tile t0 from LDS, then move tile t0 + 64 (in
    // `next1`) into LDS
    auto step = [&](int t0, int buf, KvStage<D>& next2, const KvStage<D>& next1,
                    const TileIds<D>& use, TileIds<D>& load) {
        const char* tk = lds_k[buf];
        const char* tv = lds_vt[buf];
        if (t0 + 2 * kKeyTile < t_stop) {
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
        if (t0 + kKeyTile < t_stop) store_tile<D>(next1, lds_k[buf ^ 1], lds_vt[buf ^ 1], tid);
        __syncthreads();
    };
    for (int t0 = 0; t0 < t_stop; t0 += 2 * kKeyTile) {
        step(t0, 0, st0, st1, ids0, ids1);
        if (t0 + kKeyTile >= t_stop) break;
        step(t0 + kKeyTile, 1, st1, st0, ids1, ids0);
    }

    // ---- normalise and store: lane holds d = 32dt + 8(e/4) + 4half + e%4 ------------
    const float lt = swap32_sum(l);
    if (!row_valid) return;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + (qidx * Hq + (int64_t)h * G + hh) * D;
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

template <int D, int G>
static hipError_t launch_prefill_t(const PrefillArgs& a, int num_chunks, int max_q_len,
                                   hipStream_t st) {
    constexpr int QP = kRowsPerWg / G;
    const int nqt = (max_q_len + QP - 1) / QP;
    const int64_t items = (int64_t)nqt * a.g.num_kv_heads * num_chunks;
    if (items > (int64_t)1 << 30) return hipErrorInvalidValue;
    const int nwg = (int)((items + kXcds - 1) / kXcds * kXcds);   // a multiple of the XCD count
    hipLaunchKernelGGL((prefill_kernel<D, G>), dim3(nwg), dim3(256), 0, st, a, nqt, (int)items);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_g(const PrefillArgs& a, int group, int num_chunks, int max_q_len,
                                   hipStream_t st) {
    switch (group) {
        case 1: return launch_prefill_t<D, 1>(a, num_chunks, max_q_len, st);
        case 2: return launch_prefill_t<D, 2>(a, num_chunks, max_q_len, st);
        case 3: return launch_prefill_t<D, 3>(a, num_chunks, max_q_len, st);
        case 4: return launch_prefill_t<D, 4>(a, num_chunks, max_q_len, st);
        case 5: return launch_prefill_t<D, 5>(a, num_chunks, max_q_len, st);
        case 6: return launch_prefill_t<D, 6>(a, num_chunks, max_q_len, st);
        case 7: return launch_prefill_t<D, 7>(a, num_chunks, max_q_len, st);
        case 8: return launch_prefill_t<D, 8>(a, num_chunks, max_q_len, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int group, int num_chunks,
                          int max_q_len, hipStream_t st) {
    if (num_chunks == 0 || max_q_len == 0) return hipSuccess;
    if (head_dim == 128) return launch_prefill_g<128>(a, group, num_chunks, max_q_len, st);
    if (head_dim == 64) return launch_prefill_g<64>(a, group, num_chunks, max_q_len, st);
    return hipErrorInvalidValue;
}

}  // namespace pkv
