// Multi-query paged decode on the gfx950 matrix cores.
//
// What is computed ("Inside vLLM, part 2", speculative decoding: the target model
// checks k proposed tokens in one step, so every sequence brings k + 1 query
// positions, and each attends causally to the paged context): query i of the n
// queries of sequence s sits at position ctx_s - n + i and sees keys t <= that
// position, read through the block table as in decode ("2.1 PagedAttention",
// sections 3 and 5).
//
// Mapping.  The work split is decode's balanced split: every 64-key tile of every
// (sequence, kv head) is one unit, and a persistent grid of resident waves takes
// contiguous ranges of units.  A wave attends all n * G rows of a (sequence, kv
// head) -- G query heads share each K/V read -- with rows packed into the 16
// columns of 16x16x32 bf16 MFMAs (lane 16q + n holds A[n][8q..8q+7],
// B[8q..8q+7][n] and C[4q..4q+3][n]):
//   S^T = K Q^T     K comes straight from the pool in the A layout (lane 16q + n
//                   loads 16 bytes of key n at d = 32c + 8q), Q^T stays in B
//                   registers for the whole segment;
//   softmax         a lane holds 16 keys of its row: lane-local max and sum plus
//                   two permlane swaps across the four lanes of the row;
//   O^T += V^T P^T  P^T is the S^T registers converted to bf16 in place; V is
//                   staged through LDS row-major and read transposed (gfx950
//                   ds_read_b64_tr_b16), keys in P^T's register order.
// Straddling (sequence, kv head) pairs leave partial states that the balanced
// merge combines, as for decode.
#include <mutex>

#include "pkv_split.h"

namespace pkv {

template <int D>
struct MqShape {
    static constexpr int RB = D * 2;                 // bytes of a K/V row (bf16)
    static constexpr int KC = D / 32;                // QK k-steps of 32 over the head dim
    static constexpr int DT = D / 16;                // 16-row tiles of O^T
    static constexpr int CPR = RB / 16;              // 16-byte chunks per row
    static constexpr int VJ = CPR / 8;               // chunks per key per lane in the V load
    static constexpr int VPITCH = RB + 32;           // bytes of a V row in LDS (72 dwords)
    static constexpr int ROWS = 16;                  // MFMA columns: query rows per column group
};

// The V tile sits in LDS row-major (key rows at a 288-byte pitch for D = 128: four
// consecutive rows start 8 banks apart).  The P.V product's A operand is V^T: lane
// 16q + n needs elements d = 16dt + n of the 8 keys of B-operand slots 8q .. 8q + 7,
// which hold keys 4q + j and 16 + 4q + j (j < 4) of the 32-key half, the order the
// S^T registers give the probabilities.  ds_read_b64_tr_b16 gives lane i of each 16
// lanes element i mod 4 of the 8-byte chunks addressed by lanes 4r + i / 4 (r < 4), so
// lane 4r + m of group q addresses key (4q + r) [+ 16], elements 16dt + 4m .. + 3.
typedef short mq_v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) mq_v4i16 mq_lds_v4i16;

// NC groups of 16 rows: the 16 columns of the matrix tiles hold rows n (NC = 1) or
// n and 16 + n (NC = 2, up to 32 rows: 8 queries x 4 heads), sharing every K and V^T
// operand read.
template <int D, int NC>
struct MqState {
    floatx4_t o[NC][MqShape<D>::DT];   // O^T of this lane's row: d = 16 dt + 4q + j
    float m[NC], l[NC];                // running max (log2 units) and sum of the row
};

__device__ __forceinline__ floatx4_t mfma16(u32x4 a, u32x4 b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Attend the nq * G rows of (s, h) to keys [t_begin, t_end) of the sequence.
template <int D, int G, int NC>
__device__ __forceinline__ void attend_mq(const DecodeArgs& a, int s, int h, int ctx, int nq,
                                          int t_begin, int t_end, char* lds_vt,
                                          MqState<D, NC>& st) {
    using P = MqShape<D>;
    const int lane = threadIdx.x;
    const int n = lane & 15, q = lane >> 4;
    const int bs = a.g.block_size, lbs = a.g.log2_bs;
    const int nblk = (ctx + bs - 1) >> lbs;
    const int rows = nq * G;
    const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    const char* kb = a.k_pool + (int64_t)h * a.g.head_stride_bytes;
    const char* vb = a.v_pool + (int64_t)h * a.g.head_stride_bytes;
    const uint64_t bstride = (uint64_t)a.g.block_stride_bytes;

    // Q^T: column n of group cg is row r = 16 cg + n = (query qi, head h*G + hh);
    // padding columns are zero
    u32x4 qreg[NC][P::KC];
    int lim[NC];                       // last key each of this lane's rows sees
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
        const int r = 16 * cg + n;
        const bool live = r < rows;
        const int qi = live ? r / G : nq - 1;
        const int hh = live ? r - (r / G) * G : 0;
        const char* qp = reinterpret_cast<const char*>(a.q) +
                         (((int64_t)s * nq + qi) * a.num_q_heads + h * G + hh) * P::RB + q * 16;
#pragma unroll
        for (int c = 0; c < P::KC; ++c)
            qreg[cg][c] = live ? *reinterpret_cast<const u32x4*>(qp + c * 64) : u32x4{0u, 0u, 0u, 0u};
        lim[cg] = ctx - nq + qi;
    }

    float m[NC], l[NC];
    floatx4_t o[NC][P::DT];
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
        m[cg] = kNoMax;
        l[cg] = 0.f;
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt) o[cg][dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float sl2 = a.scale_log2;
    const int kp = lane >> 3, c0 = lane & 7;

    // NC = 2 (one wave per SIMD, nothing else to hide its loads): loads run one tile
    // ahead in the registers the current tile has finished with -- the next tile's K
    // goes out right after the S^T products, its V right after the V^T stage, and the
    // table entries of the tile after it in between, so that each wait of the in-order
    // load counter covers only the loads it needs.  Keys are clamped to the segment's
    // last key, so the loads past the last tile re-read that row (no branch, which
    // would make the compiler wait for every load).  NC = 1 (two waves per SIMD) loads
    // each tile at the top of its iteration: running ahead would push it past 256
    // registers.
    constexpr bool AHEAD = NC == 2;
    const int klast = t_end - 1;
    u32x4 kreg[4][P::KC];
    u32x4 vreg[4][2][P::VJ];
    auto load_k = [&](int t0, int tab) {
        const int b0 = min(t0, klast) >> lbs;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int key = min(t0 + 16 * mt + n, klast);
            int pb = __shfl(tab, (key >> lbs) - b0);
            pb = ((unsigned)pb < (unsigned)a.g.num_blocks) ? pb : 0;   // never a bad id
            const char* row = kb + (uint64_t)(uint32_t)pb * bstride +
                              (uint32_t)((key & (bs - 1)) * P::RB + q * 16);
#pragma unroll
            for (int c = 0; c < P::KC; ++c)
                kreg[mt][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + c * 64));
        }
    };
    auto load_v = [&](int t0, int tab) {
        const int b0 = min(t0, klast) >> lbs;
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int key = min(t0 + 2 * (8 * p + kp) + r, klast);
                int pb = __shfl(tab, (key >> lbs) - b0);
                pb = ((unsigned)pb < (unsigned)a.g.num_blocks) ? pb : 0;
                const char* row = vb + (uint64_t)(uint32_t)pb * bstride +
                                  (uint32_t)((key & (bs - 1)) * P::RB + c0 * 16);
#pragma unroll
                for (int j = 0; j < P::VJ; ++j)
                    vreg[p][r][j] =
                        __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + j * 128));
            }
    };
    // block ids of the tile at t0 (a tile past the segment re-reads the last one's)
    auto table_of = [&](int t0) { return load_tile_table(table, min(t0, klast), lbs, nblk, lane); };
    int tab_cur = table_of(t_begin);
    int tab_next = 0;
    if constexpr (AHEAD) {
        // issued in the loop's order (K, table, V), or the loop's first wait, which
        // joins this path, would have to cover all of them
        load_k(t_begin, tab_cur);
        __builtin_amdgcn_sched_barrier(0);
        tab_next = table_of(t_begin + kTile);
        __builtin_amdgcn_sched_barrier(0);
        load_v(t_begin, tab_cur);
    }
    for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
        if constexpr (!AHEAD) {
            load_k(t0, tab_cur);
            load_v(t0, tab_cur);
            tab_cur = table_of(t0 + kTile);
        }
        // ---- S^T = K Q^T: lane holds keys t0 + 16mt + 4q + j of its rows --------------
        floatx4_t sacc[NC][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int cg = 0; cg < NC; ++cg) {
                sacc[cg][mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < P::KC; ++c)
                    sacc[cg][mt] = mfma16(kreg[mt][c], qreg[cg][c], sacc[cg][mt]);
            }
        if constexpr (AHEAD) {
            // the next tile's K, then the block ids of the one after it
            load_k(t0 + kTile, tab_next);
            tab_cur = tab_next;
            tab_next = table_of(t0 + 2 * kTile);
        }

        // ---- online softmax over each row's 64 keys (4 lanes x 16) -------------------
        const bool full = t0 + kTile - 1 <= ctx - nq;    // every key visible to every row
        u32x4 pk[NC][2];
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) {
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int key = t0 + 16 * mt + 4 * q + j;
                    const float sc = (full || key <= lim[cg]) ? sacc[cg][mt][j] * sl2 : -INFINITY;
                    sacc[cg][mt][j] = sc;
                    mx = fmaxf(mx, sc);
                }
            mx = swap32_max(swap16_max(mx));
            const float mn = fmaxf(m[cg], mx);
            const float alpha = fast_exp2(m[cg] - mn);
            m[cg] = mn;
            float ps = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                float p[2][4];
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        p[u][j] = fast_exp2(sacc[cg][2 * s2 + u][j] - mn);
                        ps += p[u][j];
                    }
                pk[cg][s2] = u32x4{pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                                   pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};
            }
            l[cg] = fmaf(l[cg], alpha, ps);
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                for (int dt = 0; dt < P::DT; ++dt) o[cg][dt] *= alpha;
            }
        }

        // ---- the V tile into LDS, row-major ----------------------------------------------
        __syncthreads();               // the previous tile's V reads are done
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int j = 0; j < P::VJ; ++j)
                    *reinterpret_cast<u32x4*>(lds_vt + (2 * (8 * p + kp) + r) * P::VPITCH +
                                              (c0 + 8 * j) * 16) = vreg[p][r][j];
        // the next tile's V (tab_cur now holds its block ids)
        if constexpr (AHEAD) load_v(t0 + kTile, tab_cur);
        __syncthreads();

        // ---- O^T += V^T P^T (each V^T operand serves every column group) ---------------
        // operand i = (dt, s2) = (i / 2, i % 2); the LDS reads run kAhead operands ahead
        // of the products, so a product does not wait for its own read
        constexpr int kOps = P::DT * 2, kAhead = 4;
        auto vt_operand = [&](int i) {
            const int dt = i >> 1, s2 = i & 1;
            const char* row = lds_vt + (32 * s2 + 4 * q + (n >> 2)) * P::VPITCH +
                              (16 * dt + 4 * (n & 3)) * 2;
            const mq_v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((mq_lds_v4i16*)row);
            const mq_v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (mq_lds_v4i16*)(row + 16 * P::VPITCH));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            return u32x4{l2.x, l2.y, h2.x, h2.y};
        };
        u32x4 vbuf[kAhead];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) vbuf[i] = vt_operand(i);
#pragma unroll
        for (int i = 0; i < kOps; ++i) {
            const u32x4 va = vbuf[i % kAhead];
            if (i + kAhead < kOps) vbuf[i % kAhead] = vt_operand(i + kAhead);
#pragma unroll
            for (int cg = 0; cg < NC; ++cg)
                o[cg][i >> 1] = mfma16(va, pk[cg][i & 1], o[cg][i >> 1]);
        }
    }
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt) st.o[cg][dt] = o[cg][dt];
        st.m[cg] = m[cg];
        st.l[cg] = swap32_sum(swap16_sum(l[cg]));
    }
}

// Normalised rows of a finished (s, h): lane 16q + n writes d = 16dt + 4q .. +3 of rows
// 16 cg + n.
template <int D, int G, int NC>
__device__ __forceinline__ void write_mq_rows(const DecodeArgs& a, int s, int h, int nq,
                                              const MqState<D, NC>& st) {
    using P = MqShape<D>;
    const int lane = threadIdx.x;
    const int n = lane & 15, q = lane >> 4;
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
        const int r = 16 * cg + n;
        if (r >= nq * G) continue;
        const int qi = r / G, hh = r - (r / G) * G;
        const float inv = st.l[cg] > 0.f ? 1.f / st.l[cg] : 0.f;
        uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) +
                        (((int64_t)s * nq + qi) * a.num_q_heads + h * G + hh) * D + q * 4;
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt)
            *reinterpret_cast<u32x2*>(dst + dt * 16) =
                u32x2{pack_bf16(st.o[cg][dt][0] * inv, st.o[cg][dt][1] * inv),
                      pack_bf16(st.o[cg][dt][2] * inv, st.o[cg][dt][3] * inv)};
    }
}

// Unnormalised state of row r into partial row prow0 + r.
template <int D, int G, int NC>
__device__ __forceinline__ void write_mq_partial(const DecodeArgs& a, int64_t prow0, int nq,
                                                 const MqState<D, NC>& st) {
    using P = MqShape<D>;
    const int lane = threadIdx.x;
    const int n = lane & 15, q = lane >> 4;
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
        const int r = 16 * cg + n;
        if (r >= nq * G) continue;
        const int64_t prow = prow0 + r;
        float* dst = a.part_o + prow * D + q * 4;
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt)
            *reinterpret_cast<float4*>(dst + dt * 16) =
                make_float4(st.o[cg][dt][0], st.o[cg][dt][1], st.o[cg][dt][2], st.o[cg][dt][3]);
        if (q == 0)
            *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(st.m[cg], st.l[cg]);
    }
}

// NC = 1: two waves per SIMD; NC = 2 doubles the accumulators and runs one wave per SIMD.
template <int D, int G, int NC>
__global__ __launch_bounds__(64, 3 - NC) void decode_mq_kernel(DecodeArgs a, int nq) {
    __shared__ __attribute__((aligned(16))) char lds_vt[kTile * MqShape<D>::VPITCH];
    const int64_t w = blockIdx.x;
    const int Hkv = a.g.num_kv_heads;
    const int rows = nq * G;

    int64_t tiles_all, unused;
    int first[4], first_ctx[4];
    count_tiles(a, 0, tiles_all, unused, first, first_ctx);
    const int64_t T = tiles_all * Hkv;
    const int64_t W = min((int64_t)a.num_waves, T);
    if (w >= W) return;
    const Split sp = make_split(a, T, W);
    const int64_t b = range_begin(sp, w), e = range_begin(sp, w + 1);

    int s = 0;
    int64_t before = 0;
    locate_unit(a, b, Hkv, first, s, before);
    // the first unit's counts come from the registers count_tiles filled
    int nt_s = s < 256 ? lane_value(first, s) : unit_tiles<false>(a, s);
    int ctx = s < 256 ? lane_value(first_ctx, s) : clamp_ctx(a, a.context_lens[s]);
    const int64_t rel = b - before * Hkv;
    int h = (int)(rel / nt_s);
    int tile = (int)(rel - (int64_t)h * nt_s);
    int64_t remaining = e - b;
    MqState<D, NC> st;
    while (remaining > 0) {
        const int seg = (int)min((int64_t)(nt_s - tile), remaining);
        attend_mq<D, G, NC>(a, s, h, ctx, nq, tile * kTile, min(ctx, (tile + seg) * kTile), lds_vt,
                            st);
        if (tile == 0) record_unit(a, sp, w, s, h, e - remaining, nt_s, seg == nt_s);
        if (tile == 0 && seg == nt_s) {
            write_mq_rows<D, G, NC>(a, s, h, nq, st);
        } else {
            // slot 1 for a piece that starts the unit, slot 0 for one that starts inside
            // it (the merge's reading order, as for decode)
            write_mq_partial<D, G, NC>(a, (w * 2 + (tile == 0 ? 1 : 0)) * rows, nq, st);
        }
        remaining -= seg;
        if (remaining > 0) {
            tile = 0;
            if (++h == Hkv) {
                h = 0;
                do {
                    ++s;
                    nt_s = unit_tiles<false>(a, s);
                } while (nt_s == 0);
                ctx = clamp_ctx(a, a.context_lens[s]);
            }
        }
    }
}

// --------------------------------------------------------------------------------------
// host side
// --------------------------------------------------------------------------------------
template <int D, int G, int NC>
static int mq_waves_nc() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(decode_mq_kernel<D, G, NC>), 64, 0) !=
                hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cache[dev] = max(1, per_cu) * max(1, cus);
    }
    return cache[dev];
}
// resident waves of the kernel that serves nq queries of G heads
template <int D, int G>
static int mq_waves_t(int nq) {
    return nq * G <= MqShape<D>::ROWS ? mq_waves_nc<D, G, 1>() : mq_waves_nc<D, G, 2>();
}

template <int D, int G>
static hipError_t launch_mq_t(const DecodeArgs& a, int nq, hipStream_t st) {
    if (nq * G <= MqShape<D>::ROWS)
        hipLaunchKernelGGL((decode_mq_kernel<D, G, 1>), dim3(a.num_waves), dim3(64), 0, st, a, nq);
    else
        hipLaunchKernelGGL((decode_mq_kernel<D, G, 2>), dim3(a.num_waves), dim3(64), 0, st, a, nq);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_balanced_merge_mq(a, D, G, nq, st);
}

#define PKV_MQ_DISPATCH(FN, DD, group, ...)    \
    switch (group) {                           \
        case 1: return FN<DD, 1>(__VA_ARGS__); \
        case 2: return FN<DD, 2>(__VA_ARGS__); \
        case 3: return FN<DD, 3>(__VA_ARGS__); \
        case 4: return FN<DD, 4>(__VA_ARGS__); \
        case 5: return FN<DD, 5>(__VA_ARGS__); \
        case 6: return FN<DD, 6>(__VA_ARGS__); \
        case 7: return FN<DD, 7>(__VA_ARGS__); \
        case 8: return FN<DD, 8>(__VA_ARGS__); \
        default: break;                        \
    }

int decode_mq_waves(int head_dim, int group, int nq) {
    if (head_dim == 128) { PKV_MQ_DISPATCH(mq_waves_t, 128, group, nq) }
    if (head_dim == 64) { PKV_MQ_DISPATCH(mq_waves_t, 64, group, nq) }
    return 0;
}

hipError_t launch_decode_mq(const DecodeArgs& a, int head_dim, int group, int nq, int num_seqs,
                            hipStream_t st) {
    if (num_seqs == 0) return hipSuccess;
    if (nq < 1 || nq * group > 2 * MqShape<128>::ROWS) return hipErrorInvalidValue;
    if (head_dim == 128) { PKV_MQ_DISPATCH(launch_mq_t, 128, group, a, nq, st) }
    if (head_dim == 64) { PKV_MQ_DISPATCH(launch_mq_t, 64, group, a, nq, st) }
    return hipErrorInvalidValue;
}

}  // namespace pkv
