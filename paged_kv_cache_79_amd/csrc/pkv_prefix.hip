// Shared-prefix pass of decode on the gfx950 matrix cores.
//
// What is computed: sequences that share the physical blocks of a common prefix
// ("2.1 PagedAttention", section 6: block tables of several requests point at the
// same physical blocks, read-only) attend to that prefix with the same keys and
// values.  Instead of every sequence streaming the prefix again, the query heads of
// all members of a group that map to one kv head are stacked into the rows of a
// dense product: S^T = K Q^T over the prefix keys, then O^T += V^T P^T.  Every
// member row sees every prefix key (the prefix lies entirely before each member's
// own tokens).  The result per (member, query head, key split) is a partial softmax
// state -- unnormalised o, the running max m (log2 units) and the sum l -- that the
// decode over the member's own tokens merges by log-sum-exp.
//
// Mapping: one workgroup (4 waves) owns 128 packed (member, head) rows of one
// (group, kv head) and one split of the prefix keys; K/V tiles come through the
// same tile pipeline as chunked prefill (pkv_attn_tiles.h: straight into LDS for
// head dim 128, staged through registers otherwise).  Work items are
// ordered (group, kv head, split, row block) and dealt so that the row blocks of
// one split, which read the same keys, share an XCD.
#include "pkv_attn_tiles.h"

namespace pkv {

template <int D, int G>
__global__ __launch_bounds__(256, 2) void prefix_kernel(PrefixArgs a, int num_row_blocks,
                                                        int num_items) {
    using P = PrefillShape<D>;
    constexpr int QP = kRowsPerWg / G;           // members per workgroup

    const int nwg = gridDim.x;
    const int item = (blockIdx.x % kXcds) * (nwg / kXcds) + blockIdx.x / kXcds;
    if (item >= num_items) return;
    const int rb = item % num_row_blocks;
    const int split = (item / num_row_blocks) % a.num_splits;
    const int h = (item / (num_row_blocks * a.num_splits)) % a.g.num_kv_heads;
    const int grp = item / (num_row_blocks * a.num_splits * a.g.num_kv_heads);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int lane = tid & 63;
    const int n = lane & 31;
    const int half = lane >> 5;
    const int Hq = a.num_q_heads;
    const int mb = a.max_blocks_per_seq;

    // group bounds are caller data: clamp them to the batch and the table, and the
    // prefix to whole blocks (the decode side starts each member's own keys there)
    const int first = min(max(as_const(a.group_first_seq)[grp], 0), a.num_seqs);
    const int members = min(as_const(a.group_num_seqs)[grp], a.num_seqs - first);
    const int plen = min(as_const(a.group_prefix_len)[grp], mb * a.g.block_size) &
                     ~(a.g.block_size - 1);
    const int k0 = split * a.split_tokens;
    const int k1 = min(plen, k0 + a.split_tokens);
    if (rb * QP >= members || k0 >= k1) return;
    const int32_t* table = a.block_tables + (int64_t)first * mb;   // the group's prefix blocks
    const char* kb = a.k_pool + (int64_t)h * a.g.head_stride_bytes;
    const char* vb = a.v_pool + (int64_t)h * a.g.head_stride_bytes;

    // this lane's row: member rb*QP + r/G, query head h*G + r%G
    const int r = w * 32 + n;
    const int mi = r / G;
    const int hh = r - mi * G;
    const int member = rb * QP + mi;
    const bool row_valid = (r < QP * G) && (member < members);
    const int64_t seq = (int64_t)first + member;

    u32x4 qreg[P::KSTEPS];
    // A row past the group (or past the packed rows) reads the group's last member's row:
    // its scores stay finite and nothing of it is written, and the loads need no branch
    // (whose waits would also wait for the block ids loaded beside them).
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     (((int64_t)first + min(member, members - 1)) * Hq + (int64_t)h * G + hh) *
                         P::RB +
                     half * 16;
    auto load_q = [&](u32x4 (&qr)[P::KSTEPS]) {
#pragma unroll
        for (int ks = 0; ks < P::KSTEPS; ++ks) qr[ks] = *reinterpret_cast<const u32x4*>(qp + ks * 32);
    };
    // head dim 128: the tile loop loads the rows beside the first tiles' block ids
    if constexpr (D != 128) load_q(qreg);

    floatx16_t oacc[P::DT];
#pragma unroll
    for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
    float m = kNoMax, l = 0.f;           // running max (log2 units) and sum of the row
    const float sl2 = a.scale_log2;

    if constexpr (D == 128) {
        // K/V straight into LDS (dma_attend_tiles); every row sees every key of [k0, k1),
        // and rows past k1 in the last tile read key k1 - 1
        __shared__ __attribute__((aligned(16))) PfLdsDma lds;
        dma_attend_tiles(lds, table, a.g, kb, vb, k1, k0, k1, k1, k1 - 1, sl2, load_q, qreg, oacc,
                         m, l);

        // The partial state.  o goes through LDS, half a row at a time, so that each store
        // writes whole rows: lane 16 i' + j then holds floats 4j .. 4j + 3 of one row
        // (a row's 64 floats at a pitch of 68, which keeps both the writes of the matrix
        // layout and the row reads on distinct banks).
        const float lt = swap32_sum(l);
        if (row_valid && half == 0) {
            const int64_t prow = (seq * Hq + (int64_t)h * G + hh) * a.state_stride + split;
            *reinterpret_cast<float2*>(a.pre_ml + prow * 2) = make_float2(m, lt);
        }
        constexpr int kPitch = 68;
        static_assert(4 * 32 * kPitch * 4 <= (int)sizeof(PfLdsDma), "staging fits the tile buffers");
        __syncthreads();                   // every wave is done with the tile buffers
        float* stage = reinterpret_cast<float*>(reinterpret_cast<char*>(&lds) + w * 32 * kPitch * 4);
        const int j4 = 4 * (lane & 15);
#pragma unroll
        for (int ph = 0; ph < 2; ++ph) {
            // lane (n, half) holds d = 32 dt + 8 g4 + 4 half + e (e < 4) of row n
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const floatx16_t& acc = oacc[2 * ph + u];
                    *reinterpret_cast<float4*>(stage + n * kPitch + 32 * u + 8 * g4 + 4 * half) =
                        make_float4(acc[4 * g4 + 0], acc[4 * g4 + 1], acc[4 * g4 + 2],
                                    acc[4 * g4 + 3]);
                }
            float4 v8[8];                  // all reads first, then the stores
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v8[i] = *reinterpret_cast<const float4*>(stage + (4 * i + (lane >> 4)) * kPitch + j4);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int rr = 4 * i + (lane >> 4);              // row of the wave
                const float4 v = v8[i];
                const int r2 = w * 32 + rr;
                const int mi2 = r2 / G;
                const int member2 = rb * QP + mi2;
                if (r2 < QP * G && member2 < members) {
                    const int64_t prow2 =
                        (((int64_t)first + member2) * Hq + (int64_t)h * G + (r2 - mi2 * G)) *
                            a.state_stride + split;
                    *reinterpret_cast<float4*>(a.pre_o + prow2 * D + 64 * ph + j4) = v;
                }
            }
        }
        return;
    } else {
    __shared__ __attribute__((aligned(16))) char lds_k[2][kKeyTile * P::KPITCH];
    __shared__ __attribute__((aligned(16))) char lds_vt[2][D * P::VPITCH];
    // keys [k0, k1): keys >= k1 of the last tile are masked below (see load_ids).
    // The same pipeline as chunked prefill: two K/V register stages and two id sets
    // alternating with the tile parity, two LDS buffers, one barrier per tile.
    KvStage<D> st0, st1;
    TileIds<D> ids0, ids1;
    TileOffs<D> offs;
    tile_offsets<D>(offs, a.g.block_size, tid);
    load_ids<D>(ids0, table, a.g, k1, k0, tid);
    load_tile<D>(st0, ids0, offs, a.g, kb, vb, k1, k0, tid);
    load_ids<D>(ids1, table, a.g, k1, k0 + kKeyTile, tid);
    if (k0 + kKeyTile < k1) load_tile<D>(st1, ids1, offs, a.g, kb, vb, k1, k0 + kKeyTile, tid);
    load_ids<D>(ids0, table, a.g, k1, k0 + 2 * kKeyTile, tid);
    store_tile<D>(st0, lds_k[0], lds_vt[0], tid);
    __syncthreads();

    auto step = [&](int t0, int buf, KvStage<D>& next2, const KvStage<D>& next1,
                    const TileIds<D>& use, TileIds<D>& load) {
        const char* tk = lds_k[buf];
        const char* tv = lds_vt[buf];
        if (t0 + 2 * kKeyTile < k1) {
            load_ids<D>(load, table, a.g, k1, t0 + 3 * kKeyTile, tid);
            load_tile<D>(next2, use, offs, a.g, kb, vb, k1, t0 + 2 * kKeyTile, tid);
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
        // Only the last tile of the split can hold keys past k1; with a positive scale
        // the max is taken on raw scores and the scale folds into the exponent's fma.
        const bool scaled = t0 + kKeyTile > k1 || !(sl2 > 0.f);   // wave-uniform
        const float mul = scaled ? 1.f : sl2;
        if (scaled) {
            const int lim = k1 - 1 - t0 - 4 * half;
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
        if (t0 + kKeyTile < k1) store_tile<D>(next1, lds_k[buf ^ 1], lds_vt[buf ^ 1], tid);
        __syncthreads();
    };
    for (int t0 = k0; t0 < k1; t0 += 2 * kKeyTile) {
        step(t0, 0, st0, st1, ids0, ids1);
        if (t0 + kKeyTile >= k1) break;
        step(t0 + kKeyTile, 1, st1, st0, ids1, ids0);
    }

    }

    // ---- partial state of the row: lane holds d = 32dt + 8(e/4) + 4half + e%4 -------
    const float lt = swap32_sum(l);
    if (!row_valid) return;
    const int64_t prow = (seq * Hq + (int64_t)h * G + hh) * a.state_stride + split;
    float* po = a.pre_o + prow * D;
#pragma unroll
    for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d = dt * 32 + 8 * g4 + 4 * half;
            *reinterpret_cast<float4*>(po + d) =
                make_float4(oacc[dt][4 * g4 + 0], oacc[dt][4 * g4 + 1], oacc[dt][4 * g4 + 2],
                            oacc[dt][4 * g4 + 3]);
        }
    if (half == 0) *reinterpret_cast<float2*>(a.pre_ml + prow * 2) = make_float2(m, lt);
}

template <int D, int G>
static hipError_t launch_prefix_t(const PrefixArgs& a, int num_groups, int max_group_seqs,
                                  hipStream_t st) {
    constexpr int QP = kRowsPerWg / G;
    const int nrb = (max_group_seqs + QP - 1) / QP;
    const int64_t items = (int64_t)num_groups * a.g.num_kv_heads * a.num_splits * nrb;
    if (items > ((int64_t)1 << 30)) return hipErrorInvalidValue;
    const int nwg = (int)((items + kXcds - 1) / kXcds * kXcds);
    hipLaunchKernelGGL((prefix_kernel<D, G>), dim3(nwg), dim3(256), 0, st, a, nrb, (int)items);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_prefix_g(const PrefixArgs& a, int group, int num_groups,
                                  int max_group_seqs, hipStream_t st) {
    switch (group) {
        case 1: return launch_prefix_t<D, 1>(a, num_groups, max_group_seqs, st);
        case 2: return launch_prefix_t<D, 2>(a, num_groups, max_group_seqs, st);
        case 3: return launch_prefix_t<D, 3>(a, num_groups, max_group_seqs, st);
        case 4: return launch_prefix_t<D, 4>(a, num_groups, max_group_seqs, st);
        case 5: return launch_prefix_t<D, 5>(a, num_groups, max_group_seqs, st);
        case 6: return launch_prefix_t<D, 6>(a, num_groups, max_group_seqs, st);
        case 7: return launch_prefix_t<D, 7>(a, num_groups, max_group_seqs, st);
        case 8: return launch_prefix_t<D, 8>(a, num_groups, max_group_seqs, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefix(const PrefixArgs& a, int head_dim, int group, int num_groups,
                         int max_group_seqs, hipStream_t st) {
    if (num_groups == 0 || max_group_seqs == 0 || a.num_splits == 0) return hipSuccess;
    if (head_dim == 128) return launch_prefix_g<128>(a, group, num_groups, max_group_seqs, st);
    if (head_dim == 64) return launch_prefix_g<64>(a, group, num_groups, max_group_seqs, st);
    return hipErrorInvalidValue;
}

}  // namespace pkv
