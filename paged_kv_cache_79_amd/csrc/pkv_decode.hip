// Paged decode attention for gfx950.
//
// What is computed ("2.1 PagedAttention", sections 3 and 5): every query head
// of a sequence attends to the sequence's whole context, each logical position
// t being read at physical block block_table[t / block_size], slot
// t % block_size of the pool.  The pages' kernel sketch walks the blocks of
// one sequence with a 32-lane warp; here a 64-lane wave consumes contexts in
// tiles of 64 tokens of one (sequence, kv head):
//
//   1. load    every lane issues 16-byte nontemporal loads in the pool's natural
//              order, so one wave instruction covers 1 KiB of contiguous K (or V)
//              of one block; the tile's block ids arrive with one vector load
//              (issued a tile ahead) and are taken with readlane into scalar bases;
//   2. QK      K is restaged through LDS.  bf16: S^T = K Q^T on 16x16x32 MFMAs,
//              the tile's K rows as the A operand and the G query heads of the
//              group in the first G of 16 B-operand columns (grouped-query
//              packing: one K read serves G heads); lane 16qq + n ends with head
//              n's scores of 16 keys.  fp32: lane t owns token t and forms the G
//              dot products against q broadcast from LDS;
//   3. softmax bf16: per head over its four lanes (two permlane swaps); fp32: tile
//              maximum by DPP row rotations + permlane swaps; running max per
//              head, per-lane running sums (summed once per segment);
//   4. PV      bf16: O^T += V^T P^T on 16x16x32 MFMAs.  P^T is the S^T registers
//              rounded to bf16 (no LDS round trip); V is stored row-major into the
//              K buffer once the scores are done and read transposed
//              (ds_read_b64_tr_b16) in the key order of those registers; lane
//              16qq + n ends with elements 16dt + 4qq + j of head n's output.
//              fp32: V stays in the load layout (lane = 4 elements of one token
//              row) and is accumulated with FMAs against probabilities from LDS.
// Tokens at or beyond the valid length are removed by selection (score -inf,
// V row zero), never by arithmetic, so stale or NaN slots cannot leak in.
//
// Work split.  By default (balanced split) a persistent grid of exactly as many
// waves as the device keeps resident divides all tiles of the batch -- ordered
// by (sequence, kv head, tile) -- into contiguous ranges, so that the work per
// wave does not depend on the mix of context lengths.  When two waves share each
// SIMD, the first-dispatched half of the grid runs faster (it wins issue
// arbitration), so that half gets a fixed larger share of the tiles.  A
// (sequence, kv head) that lies inside one wave's range is finished by that
// wave; one that straddles waves leaves partial softmax states that a second
// kernel merges by log-sum-exp.  With a fixed partition size (> 0) the split
// is by sequence position instead and does not depend on the device.
#include <mutex>

#include <type_traits>

#include "pkv_split.h"

namespace pkv {

template <bool BF16, int D>
struct DecodeShape {
    static constexpr int E = BF16 ? 2 : 4;     // element bytes
    static constexpr int RB = D * E;            // bytes of one token row of one head
    static constexpr int CPR = RB / 16;         // 16-byte chunks per row
    static constexpr int R = 64 / CPR;          // rows covered by one wave-wide load
    static constexpr int NL = kTile / R;        // loads per lane per tile (K or V)
    static constexpr int EPC = 16 / E;          // elements per chunk
    static constexpr int KPITCH = RB + 16;      // LDS row pitch (bytes), padded against bank conflicts
    static_assert(R >= 2 && R <= 8, "row groups");
};

template <bool BF16>
struct DecodeLds {
    // fp32: the probabilities of a tile (dwords); bf16 keeps them in registers
    static constexpr int PWORDS = BF16 ? 4 : kTile * 8;
};

// Softmax state of one segment of one (sequence, kv head) for its G query heads,
// after the per-lane pieces have been combined.  fp32: m and l are uniform; lanes of
// row group 0 hold o for their 16-byte chunk of the head dimension.
template <bool BF16, int D, int G>
struct SegState {
    float m[G], l[G], o[G][DecodeShape<BF16, D>::EPC];
};
// bf16: lane 16 qq + n holds head n's max and sum, and O^T tile dt of the matrix-core
// P.V product: elements d = 16 dt + 4 qq + j (j < 4) of head n's row.
template <int D, int G>
struct SegState<true, D, G> {
    float m, l;
    floatx4_t o[D / 16];
};

// The bf16 V tile sits in the K buffer once the scores are done: rows unpadded
// (D * 2 bytes), 16-byte chunk c of key row k at chunk position c ^ v_swz(k).  The
// P.V operand reads (ds_read_b64_tr_b16: per 16 lanes, 8 bytes from each of four
// consecutive keys, four lanes per key) then fall on 64 distinct banks per 32 lanes,
// and the row-wise stores stay conflict-free.
template <int D>
__device__ __forceinline__ int v_swz(int k) {
    constexpr int RB = D * 2, RPL = 256 / RB, CPR = RB / 16;   // rows per 256 bytes
    return 2 * ((k / RPL) & (CPR / 2 - 1));
}
typedef short dec_v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dec_v4i16 dec_lds_v4i16;

// What a segment loads before its first tile: the block ids of that tile (lane j: block
// t_begin / bs + j) and the G query rows of (s_q, h), this lane's 16-byte chunks
// lane + 64 i.  The balanced kernel loads the next segment's while it attends the
// current one, so a wave moving on to the next kv head of its sequence does not wait
// for them.
template <bool BF16, int D, int G>
struct SegInputs {
    static constexpr int QC = G * DecodeShape<BF16, D>::RB / 16;   // 16-byte chunks of the rows
    static constexpr int QN = (QC + 63) / 64;
    int tab;
    u32x4 q[QN];
};
// nblk: table entries the reads may touch (the sequence's blocks, or the whole row when
// the length is not at hand; entries past the context are never used).
template <bool BF16, int D, int G, bool CONTIG = false>
__device__ __forceinline__ void load_seg_inputs(const DecodeArgs& a, int s, int s_q, int h, int nblk,
                                                int t_begin, SegInputs<BF16, D, G>& in) {
    using I = SegInputs<BF16, D, G>;
    const int lane = threadIdx.x;
    if constexpr (CONTIG) {
        in.tab = 0;
    } else {
        in.tab = load_tile_table(a.block_tables + (int64_t)s * a.max_blocks_per_seq, t_begin,
                                 a.g.log2_bs, nblk, lane);
    }
    const u32x4* qsrc = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const char*>(a.q) +
        ((int64_t)s_q * a.num_q_heads + h * G) * DecodeShape<BF16, D>::RB);
#pragma unroll
    for (int i = 0; i < I::QN; ++i) in.q[i] = qsrc[min(lane + 64 * i, I::QC - 1)];
}

// Attend the G query heads of (s, h) to tokens [t_begin, t_end) of the sequence.
// CONTIG: the unpaged baseline -- K/V in the contiguous [S][L][Hkv][D] layout, no table.
// s picks the block-table row (or slab), s_q the query row (the same but for chunked
// prefill, where the queries of one chunk share its table).
// `in`: the segment's inputs, loaded by the caller (null: loaded here).
template <bool BF16, int D, int G, bool CONTIG = false>
__device__ __forceinline__ void attend_segment(const DecodeArgs& a, int s, int s_q, int h, int ctx,
                                               int t_begin, int t_end, char* lds_k,
                                               uint32_t* lds_p, uint32_t* lds_q,
                                               SegState<BF16, D, G>& st,
                                               const SegInputs<BF16, D, G>* in = nullptr) {
    using S = DecodeShape<BF16, D>;
    const int lane = threadIdx.x;
    const int bs = a.g.block_size;
    const int nblk = (ctx + bs - 1) >> a.g.log2_bs;
    const int ra = lane / S::CPR;          // row inside a wave-wide load
    const int rc = lane - ra * S::CPR;     // 16-byte chunk inside the row
    const uint32_t row_stride = CONTIG ? (uint32_t)a.contig_row_stride : (uint32_t)S::RB;
    const uint32_t lane_off = (uint32_t)ra * row_stride + (uint32_t)(rc * 16);
    const int32_t* table = CONTIG ? nullptr : a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    // bf16, head_dim 64, block_size 4: a (block, head) run is 512 bytes, so one wave-wide
    // load spans two blocks and each lane forms its own address
    const bool small_run = !CONTIG && BF16 && D == 64 && bs * S::RB < 64 * 16;
    const int64_t head_base = CONTIG ? (int64_t)s * a.contig_seq_stride + (int64_t)h * S::RB
                                     : (int64_t)h * a.g.head_stride_bytes;
    const char* kb = (const char*)pin_uniform(a.k_pool + head_base);
    const char* vb = (const char*)pin_uniform(a.v_pool + head_base);

    using I = SegInputs<BF16, D, G>;
    SegInputs<BF16, D, G> own;
    if (in == nullptr) {
        load_seg_inputs<BF16, D, G, CONTIG>(a, s, s_q, h, nblk, t_begin, own);
        in = &own;
    }
    int tab_cur = in->tab;
    __syncthreads();  // the previous segment is done with lds_q
    {
        u32x4* qdst = reinterpret_cast<u32x4*>(lds_q);
#pragma unroll
        for (int i = 0; i < I::QN; ++i)
            if (lane + 64 * i < I::QC) qdst[lane + 64 * i] = in->q[i];
    }
    // bf16: QK runs on the matrix cores (16x16x32 MFMA, S^T = K Q^T with the G heads in
    // the first G of 16 columns).  Lane 16 qq + n takes, for k-step c, elements
    // 32c + 8qq .. +7 of head n's q row as the B operand; the columns past G repeat the
    // last head (finite values whose scores nothing reads).
    constexpr int KC = D / 32;
    const int qn = lane & 15, qq = lane >> 4;
    const char* qcol = reinterpret_cast<const char*>(lds_q) + min(qn, G - 1) * S::RB + qq * 16;
    float mh = kNoMax, ll = 0.f;   // bf16: running max and per-lane sum of head qn

    float m[G], l[G], o[G][S::EPC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = kNoMax;
        l[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < S::EPC; ++e) o[hh][e] = 0.f;
    }
    // bf16: O^T of head qn, lane 16 qq + qn holding d = 16 dt + 4 qq + j
    floatx4_t oacc[BF16 ? D / 16 : 1];
#pragma unroll
    for (int dt = 0; dt < (BF16 ? D / 16 : 1); ++dt) oacc[dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
        // ---- 1. loads of this tile; the next tile's table entries go out after them
        u32x4 kreg[S::NL], vreg[S::NL];
        const int tab = tab_cur;
        // refreshed in the loop so the 32-bit offset is not widened and hoisted: the
        // loads then take the scalar base + 32-bit lane offset form
        uint32_t loff = lane_off;
        asm volatile("" : "+v"(loff));
        // Only a sequence's last tile can be partial: its groups of rows past the context
        // re-read the last group inside it (a cache hit, no HBM traffic); their scores
        // and V rows are masked below.
        const int last_row = __builtin_amdgcn_readfirstlane(min(t_end - t0 - 1, kTile - 1)) &
                             ~(S::R - 1);
#pragma unroll
        for (int i = 0; i < S::NL; ++i) {
            const int row = min(i * S::R, last_row);    // uniform
            uint64_t base;
            if constexpr (CONTIG) {
                // row t0 + row of the sequence's slab (the slab holds a whole number of tiles)
                const uint32_t ur = (uint32_t)(t0 + row);
                base = ((uint64_t)__umulhi(ur, row_stride) << 32) | (uint64_t)(ur * row_stride);
            } else if (small_run) {
                const int lr = row + ra;                            // this lane's row of the tile
                int pbl = __shfl(tab, lr >> a.g.log2_bs);
                pbl = ((unsigned)pbl < (unsigned)a.g.num_blocks) ? pbl : 0;   // never a bad id
                const uint64_t off = (uint64_t)(uint32_t)pbl * (uint64_t)a.g.block_stride_bytes +
                                     (uint32_t)((lr & (bs - 1)) * S::RB + rc * 16);
                kreg[i] = __builtin_nontemporal_load((global_ptr<u32x4>)(kb + off));
                vreg[i] = __builtin_nontemporal_load((global_ptr<u32x4>)(vb + off));
                continue;
            } else {
                const int rel = row >> a.g.log2_bs;   // block of this load inside the tile
                int pb = __builtin_amdgcn_readlane(tab, rel);
                pb = ((unsigned)pb < (unsigned)a.g.num_blocks) ? pb : 0;   // never a bad id
                // scalar base: block, head and first row of this load; per-lane part is
                // lane_off.  The 64-bit product is spelled as two 32-bit halves so it stays
                // on the scalar unit.
                const uint32_t ub = (uint32_t)pb, us = (uint32_t)a.g.block_stride_bytes;
                base = (((uint64_t)__umulhi(ub, us) << 32) | (uint64_t)(ub * us)) +
                       (uint64_t)((row & (bs - 1)) * S::RB);
            }
            // K and V are read exactly once: nontemporal loads keep them from
            // displacing reusable lines (tables, q, partials) in the caches
            kreg[i] = __builtin_nontemporal_load((global_ptr<u32x4>)(pin_uniform(kb + base) + loff));
            vreg[i] = __builtin_nontemporal_load((global_ptr<u32x4>)(pin_uniform(vb + base) + loff));
        }
        if constexpr (!CONTIG) tab_cur = load_tile_table(table, t0 + kTile, a.g.log2_bs, nblk, lane);
#pragma unroll
        for (int i = 0; i < S::NL; ++i)
            *reinterpret_cast<u32x4*>(lds_k + (i * S::R + ra) * S::KPITCH + rc * 16) = kreg[i];
        __syncthreads();

        if constexpr (BF16) {
            // ---- 2. QK: S^T = K Q^T; lane 16qq + n ends with head n's scores of keys
            //         16mt + 4qq + j (mt, j < 4)
            floatx4_t sacc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                sacc[mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < KC; ++c) {
                    const u32x4 ka = *reinterpret_cast<const u32x4*>(
                        lds_k + (16 * mt + qn) * S::KPITCH + c * 64 + qq * 16);
                    const u32x4 qb = *reinterpret_cast<const u32x4*>(qcol + c * 64);
                    sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, ka), __builtin_bit_cast(bf16x8_t, qb),
                        sacc[mt], 0, 0, 0);
                }
            }
            // ---- 3. online softmax of head qn over the lanes qn, 16 + qn, 32 + qn, 48 + qn
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool valid = t0 + 16 * mt + 4 * qq + j < t_end;
                    const float sc = valid ? sacc[mt][j] * a.scale_log2 : -INFINITY;
                    sacc[mt][j] = sc;
                    mx = fmaxf(mx, sc);
                }
            mx = swap32_max(swap16_max(mx));
            const float mn = fmaxf(mh, mx);
            const float al = fast_exp2(mh - mn);
            mh = mn;
            // P^T as the B operand of the P.V product, for each 32-key half ks: lane
            // 16qq + n holds head n's probabilities of keys 32ks + 4qq + j and
            // 32ks + 16 + 4qq + j (j < 4), straight from the S^T registers
            float ps = 0.f;
            u32x4 pk[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float p[2][4];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        p[hf][j] = fast_exp2(sacc[2 * ks + hf][j] - mn);
                        ps += p[hf][j];
                    }
                pk[ks] = u32x4{pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                               pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};
            }
            ll = fmaf(ll, al, ps);

            // ---- 4. PV: O^T += V^T P^T on the matrix cores.  V goes into the K buffer
            //         row-major (every K read of the tile is done), tail rows zeroed
            __syncthreads();
            if (t0 + kTile > t_end) {
#pragma unroll
                for (int i = 0; i < S::NL; ++i)
                    if (t0 + i * S::R + ra >= t_end) vreg[i] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int i = 0; i < S::NL; ++i) {
                const int row = i * S::R + ra;
                *reinterpret_cast<u32x4*>(lds_k + row * S::RB + ((rc ^ v_swz<D>(row)) << 4)) =
                    vreg[i];
            }
            __syncthreads();
            if (__builtin_amdgcn_ballot_w64(al != 1.f)) {
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) oacc[dt] *= al;
            }
            // operand i = (dt, ks) = (i / 2, i % 2): lane 16qq + n gets elements
            // d = 16dt + n of the keys of B slots 8qq .. 8qq + 7 from two transposing
            // reads (lane 4r + m of each 16 addresses key 32ks + 4qq + r [+ 16],
            // elements 16dt + 4m .. + 3); the reads run four operands ahead
            constexpr int kOps = (D / 16) * 2, kAhead = 4;
            auto vt_operand = [&](int i) {
                const int dt = i >> 1, ks = i & 1;
                const int row = 32 * ks + 4 * qq + (qn >> 2);
                const int c = 2 * dt + ((qn >> 1) & 1);
                const char* ptr = lds_k + row * S::RB + ((c ^ v_swz<D>(row)) << 4) + (qn & 1) * 8;
                const dec_v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dec_lds_v4i16*)ptr);
                const dec_v4i16 hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((dec_lds_v4i16*)(ptr + 16 * S::RB));
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
                oacc[i >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, va), __builtin_bit_cast(bf16x8_t, pk[i & 1]),
                    oacc[i >> 1], 0, 0, 0);
            }
            // the next tile's K store reuses the buffer
            __syncthreads();
        } else {
            // ---- 2. QK (fp32): lane = token -------------------------------------------------
            float acc[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) acc[hh] = 0.f;
            const char* krow = lds_k + lane * S::KPITCH;
            // q is re-read from LDS every tile: an opaque zero offset stops the compiler
            // from hoisting all G*D q values out of the loop into registers
            uint32_t qoff = 0;
            asm volatile("" : "+v"(qoff));
#pragma unroll
            for (int j = 0; j < S::CPR; ++j) {
                const u32x4 kk = *reinterpret_cast<const u32x4*>(krow + j * 16);
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    const u32x4 qv = *reinterpret_cast<const u32x4*>(
                        reinterpret_cast<const char*>(lds_q) + qoff + (hh * (S::RB / 4) + j * 4) * 4);
                    acc[hh] = fmaf(u2f(kk.x), u2f(qv.x), acc[hh]);
                    acc[hh] = fmaf(u2f(kk.y), u2f(qv.y), acc[hh]);
                    acc[hh] = fmaf(u2f(kk.z), u2f(qv.z), acc[hh]);
                    acc[hh] = fmaf(u2f(kk.w), u2f(qv.w), acc[hh]);
                }
                // keep the LDS reads of two chunks at a time in flight, not all of them
                if (j & 1) __builtin_amdgcn_sched_barrier(0);
            }

            // ---- 3. online softmax ----------------------------------------------------------
            const bool valid = (t0 + lane) < t_end;
            float alpha[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                const float sc = valid ? acc[hh] * a.scale_log2 : -INFINITY;
                const float mn = fmaxf(m[hh], wave_max(sc));
                alpha[hh] = fast_exp2(m[hh] - mn);
                const float p = fast_exp2(sc - mn);
                m[hh] = mn;
                l[hh] = l[hh] * alpha[hh] + p;
                reinterpret_cast<float*>(lds_p)[lane * 8 + hh] = p;
            }
            __syncthreads();

            // ---- 4. PV (fp32): lane = 4 elements of one token row ---------------------------
            if (t0 + kTile > t_end) {  // tail tile: rows past the valid length contribute nothing
#pragma unroll
                for (int i = 0; i < S::NL; ++i)
                    if (t0 + i * S::R + ra >= t_end) vreg[i] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int hh = 0; hh < G; ++hh)
#pragma unroll
                for (int e = 0; e < S::EPC; ++e) o[hh][e] *= alpha[hh];
#pragma unroll
            for (int i = 0; i < S::NL; ++i) {
                const float* pr = reinterpret_cast<const float*>(lds_p) + (i * S::R + ra) * 8;
                const float4 pa = *reinterpret_cast<const float4*>(pr);
                const float4 pz = *reinterpret_cast<const float4*>(pr + 4);
                const float pv[8] = {pa.x, pa.y, pa.z, pa.w, pz.x, pz.y, pz.z, pz.w};
                const float v[4] = {u2f(vreg[i].x), u2f(vreg[i].y), u2f(vreg[i].z),
                                    u2f(vreg[i].w)};
#pragma unroll
                for (int hh = 0; hh < G; ++hh)
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[hh][e] = fmaf(pv[hh], v[e], o[hh][e]);
            }
        }
    }

    // ---- combine lanes -----------------------------------------------------------------
    if constexpr (BF16) {
        // head qn's sum over its four lanes; O^T stays where the products left it
        st.m = mh;
        st.l = swap32_sum(swap16_sum(ll));
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) st.o[dt] = oacc[dt];
    } else {
        // per-lane sums, then the row groups sharing a chunk
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            st.m[hh] = m[hh];
            st.l[hh] = wave_sum(l[hh]);
#pragma unroll
            for (int e = 0; e < S::EPC; ++e) st.o[hh][e] = group_sum<S::R>(o[hh][e]);
        }
    }
}

// Normalised output rows of the G heads of (s, h).
template <bool BF16, int D, int G>
__device__ __forceinline__ void write_rows(const DecodeArgs& a, int s, int h,
                                           const SegState<BF16, D, G>& st) {
    using S = DecodeShape<BF16, D>;
    const int lane = threadIdx.x;
    if constexpr (BF16) {
        // lane 16qq + n: elements 16dt + 4qq .. + 3 of head n's row
        const int n = lane & 15, qq = lane >> 4;
        if (n >= G) return;
        const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
        uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) +
                        ((int64_t)s * a.num_q_heads + h * G + n) * D + 4 * qq;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            *reinterpret_cast<u32x2*>(dst + 16 * dt) =
                u32x2{pack_bf16(st.o[dt][0] * inv, st.o[dt][1] * inv),
                      pack_bf16(st.o[dt][2] * inv, st.o[dt][3] * inv)};
    } else {
        const int ra = lane / S::CPR, rc = lane - (lane / S::CPR) * S::CPR;
        if (ra != 0) return;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float inv = st.l[hh] > 0.f ? 1.f / st.l[hh] : 0.f;
            const int64_t row = ((int64_t)s * a.num_q_heads + h * G + hh) * D + rc * S::EPC;
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + row) =
                make_float4(st.o[hh][0] * inv, st.o[hh][1] * inv, st.o[hh][2] * inv,
                            st.o[hh][3] * inv);
        }
    }
}

// Unnormalised partial state of head hh into row prow0 + hh * prow_step of the state
// arrays o_base (D floats per row) and ml_base ((max, sum): 2 floats per row).
template <bool BF16, int D, int G>
__device__ __forceinline__ void write_state(float* o_base, float* ml_base, int64_t prow0,
                                            int64_t prow_step, const SegState<BF16, D, G>& st) {
    using S = DecodeShape<BF16, D>;
    const int lane = threadIdx.x;
    if constexpr (BF16) {
        const int n = lane & 15, qq = lane >> 4;
        if (n >= G) return;
        const int64_t prow = prow0 + n * prow_step;
        float* dst = o_base + prow * D + 4 * qq;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            *reinterpret_cast<float4*>(dst + 16 * dt) =
                make_float4(st.o[dt][0], st.o[dt][1], st.o[dt][2], st.o[dt][3]);
        if (qq == 0) *reinterpret_cast<float2*>(ml_base + prow * 2) = make_float2(st.m, st.l);
    } else {
        const int ra = lane / S::CPR, rc = lane - (lane / S::CPR) * S::CPR;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const int64_t prow = prow0 + hh * prow_step;
            if (ra == 0) {
                float* dst = o_base + prow * D + rc * S::EPC;
#pragma unroll
                for (int e = 0; e < S::EPC; e += 4)
                    *reinterpret_cast<float4*>(dst + e) = make_float4(
                        st.o[hh][e], st.o[hh][e + 1], st.o[hh][e + 2], st.o[hh][e + 3]);
            }
            if (lane == 0)
                *reinterpret_cast<float2*>(ml_base + prow * 2) = make_float2(st.m[hh], st.l[hh]);
        }
    }
}
// ... into the balanced split's slots of the workspace.
template <bool BF16, int D, int G>
__device__ __forceinline__ void write_partial(const DecodeArgs& a, int64_t prow0, int64_t prow_step,
                                              const SegState<BF16, D, G>& st) {
    write_state<BF16, D, G>(a.part_o, a.part_ml, prow0, prow_step, st);
}

template <bool BF16, int D, int G>
__device__ __forceinline__ void zero_rows(const DecodeArgs& a, int s, int h) {
    const int lane = threadIdx.x;
    const int64_t row0 = ((int64_t)s * a.num_q_heads + h * G) * D;
    if constexpr (BF16) {
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + row0;
        for (int e = lane; e < G * D; e += 64) o[e] = 0;
    } else {
        float* o = reinterpret_cast<float*>(a.out) + row0;
        for (int e = lane; e < G * D; e += 64) o[e] = 0.f;
    }
}

template <bool BF16, int D, int G, bool CONTIG = false, bool PREFIX = false>
__global__ __launch_bounds__(64, (BF16 ? 2 : 1)) void decode_balanced_kernel(DecodeArgs a) {
    using S = DecodeShape<BF16, D>;
    __shared__ __attribute__((aligned(16))) char lds_k[kTile * S::KPITCH];
    __shared__ __attribute__((aligned(16))) uint32_t lds_p[DecodeLds<BF16>::PWORDS];
    __shared__ __attribute__((aligned(16))) uint32_t lds_q[G * S::RB / 4];

    const int lane = threadIdx.x;
    const int64_t w = blockIdx.x;
    const int Hkv = a.g.num_kv_heads;

    // units = 64-token tiles, ordered by (sequence, kv head, tile); with W <= T every
    // wave's range [wT/W, (w+1)T/W) is non-empty
    int64_t tiles_all, unused;
    int first[4], first_ctx[4];
    count_tiles<PREFIX>(a, 0, tiles_all, unused, first, first_ctx);
    const int64_t T = tiles_all * Hkv;
    const int64_t W = min((int64_t)a.num_waves, T);
    if (w >= W) return;
    const Split sp = make_split(a, T, W);
    const int64_t b = range_begin(sp, w), e = range_begin(sp, w + 1);

    int s = 0;
    int64_t before = 0;
    locate_unit<PREFIX>(a, b, Hkv, first, s, before);
    // the first unit's counts come from the registers count_tiles filled (no round trip
    // before the first loads); later units reload theirs
    int nt_s = s < 256 ? lane_value(first, s) : unit_tiles<PREFIX>(a, s);
    int ctx = s < 256 ? lane_value(first_ctx, s) : clamp_ctx(a, a.context_lens[s]);
    const int64_t rel = b - before * Hkv;
    int h = (int)(rel / nt_s);
    int tile = (int)(rel - (int64_t)h * nt_s);
    int64_t remaining = e - b;
    SegState<BF16, D, G> st;
    // Inputs of the current segment when the previous one loaded them, and of the next
    // kv head of the same sequence (same table row and length), loaded ahead.  (Loading
    // the next sequence's ahead as well measured no faster and needs more registers.)
    SegInputs<BF16, D, G> in_cur, in_next;
    bool have_cur = false;
    while (remaining > 0) {
        const int seg = (int)min((int64_t)(nt_s - tile), remaining);
        const int t_first = seq_start<PREFIX>(a, s, ctx);    // 0 unless in the prefix mode
        const int nblk = (ctx + a.g.block_size - 1) >> a.g.log2_bs;
        if (!have_cur)
            load_seg_inputs<BF16, D, G, CONTIG>(a, s, s, h, nblk, t_first + tile * kTile, in_cur);
        const bool ahead = remaining > seg && h + 1 < Hkv;    // uniform
        if (ahead) load_seg_inputs<BF16, D, G, CONTIG>(a, s, s, h + 1, nblk, t_first, in_next);
        attend_segment<BF16, D, G, CONTIG>(a, s, s, h, ctx, t_first + tile * kTile,
                                           min(ctx, t_first + (tile + seg) * kTile), lds_k, lds_p,
                                           lds_q, st, &in_cur);
        // the wave holding a unit's first tile tells the merge where its pieces are
        if (tile == 0) record_unit(a, sp, w, s, h, e - remaining, nt_s, seg == nt_s);
        if (tile == 0 && seg == nt_s) {
            bool own = false;
            if constexpr (PREFIX) own = t_first > 0;
            if (own) {
                // the row's state of its own tokens goes to the last slot of its prefix
                // states; the merge combines them (all loads at once, every row in parallel)
                const int64_t stride = a.pre_splits + 1;
                write_state<BF16, D, G>(a.pre_o, a.pre_ml,
                                        ((int64_t)s * a.num_q_heads + h * G) * stride +
                                            a.pre_splits,
                                        stride, st);
            } else {
                write_rows<BF16, D, G>(a, s, h, st);
            }
        } else {
            // the merge reads the piece of the wave holding the unit's first tile from
            // slot 1 and every later wave's from slot 0: a piece that starts the unit can
            // only be this wave's last segment, one that starts inside it only the first
            write_partial<BF16, D, G>(a, (w * 2 + (tile == 0 ? 1 : 0)) * G, 1, st);
        }
        remaining -= seg;
        have_cur = ahead;
        if (ahead) in_cur = in_next;
        if (remaining > 0) {
            tile = 0;
            if (++h == Hkv) {
                h = 0;
                do {
                    ++s;
                    nt_s = unit_tiles<PREFIX>(a, s);
                } while (nt_s == 0);
                ctx = clamp_ctx(a, a.context_lens[s]);
            }
        }
    }
}

// Waves per workgroup of the balanced merge: one output row each, or (COOP) all of
// them on one row, for batches with fewer rows than the device has merge slots.
constexpr int kMergeRows = 4;

// Merge the pieces of each (sequence, kv head) that straddles waves; write zero rows
// for empty contexts.  The first covering wave holds its piece in its last slot, every
// later covering wave in its first slot.  In the shared-prefix mode the prefix pass's
// states of the row are merged in as well, together with the row's own-token state
// when one wave finished its (sequence, kv head) (a row with no token after its prefix
// is the prefix states alone).  With nq queries per sequence (multi-query decode) the
// output row is (s * nq + i) * Hq + hq, and a (sequence, kv head) has nq * G partial
// rows.  A row's pieces are located by the record the wave holding the unit's first
// tile left (unit_desc): one load, whatever the batch size, and no split arithmetic.
// COOP: the kMergeRows waves of a workgroup take turns over one row's states (wave i
// takes batches i, i + kMergeRows, ...) and combine their sums through LDS, so a row
// with many pieces (long contexts split over tens of waves) needs one round of loads
// per kMergeRows batches instead of one per batch.
template <bool BF16, int D, int G, bool PREFIX = false, bool COOP = false>
__global__ __launch_bounds__(64 * kMergeRows) void decode_balanced_merge_kernel(DecodeArgs a,
                                                                               int nq) {
    constexpr int PER = D / 64;
    constexpr int kBatch = 16;
    const int lane = threadIdx.x & 63;
    const int wi = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int Hkv = a.g.num_kv_heads;
    const int row = COOP ? (int)blockIdx.x : (int)blockIdx.x * kMergeRows + wi;
    if (row >= a.num_seqs * nq * a.num_q_heads) return;     // uniform per workgroup in COOP
    const int sq = row / a.num_q_heads;
    const int hq = row - sq * a.num_q_heads;
    const int s = sq / nq;
    const int h = hq / G;
    const int rows = nq * G, r = (sq - s * nq) * G + (hq - h * G);
    const int2 desc = *reinterpret_cast<const int2*>(a.unit_desc + 2 * ((int64_t)s * Hkv + h));
    const int ctx = clamp_ctx(a, a.context_lens[s]);
    const int start = seq_start<PREFIX>(a, s, ctx);
    const int nt = ntiles_of(ctx - start);
    const int ns =
        PREFIX ? min((start + a.pre_split_tokens - 1) / a.pre_split_tokens, a.pre_splits) : 0;
    const int64_t pre_row0 = ((int64_t)s * a.num_q_heads + hq) * (a.pre_splits + 1);
    const int64_t o = (int64_t)row * D + lane * PER;
    int64_t w0 = 0;
    int npieces = 0, own = 0;
    if (nt > 0) {
        // (wave holding the unit's first tile, waves its tiles span), recorded by that
        // wave; clamped so that a stale record can never address past the workspace
        w0 = min(max(desc.x, 0), a.num_waves - 1);
        const int span = min(max(desc.y, 1), a.num_waves - (int)w0);
        if (span == 1) {
            if (ns == 0) return;               // finished and written by one wave
            own = 1;                           // its state is in the row's last slot
        } else {
            npieces = span;
        }
    }
    // The states of the row: in the shared-prefix mode its ns prefix splits and, when
    // one wave finished the (sequence, kv head), the own-token state in the row's last
    // slot; then the pieces of the covering waves.
    const int npre = ns + own;
    const int nst = npre + npieces;
    if (nst == 0) {
        if (COOP && wi != 0) return;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            if constexpr (BF16)
                reinterpret_cast<uint16_t*>(a.out)[o + k] = 0;
            else
                reinterpret_cast<float*>(a.out)[o + k] = 0.f;
        }
        return;
    }
    auto state = [&](int k, const float*& so, const float*& sml) {
        if (PREFIX && k < npre) {
            const int64_t rr = pre_row0 + (k < ns ? k : a.pre_splits);
            so = a.pre_o + rr * D;
            sml = a.pre_ml + rr * 2;
        } else {
            // the first covering wave holds its piece in slot 1, later ones in slot 0
            const int p = k - npre;
            const int64_t rr = ((w0 + p) * 2 + (p == 0 ? 1 : 0)) * rows + r;
            so = a.part_o + rr * D;
            sml = a.part_ml + rr * 2;
        }
    };
    // states in batches, each batch one round of loads: lane j holds the (max, sum) of
    // state c0 + j while every lane loads its part of all the batch's output rows
    // (unconditionally, clamped to the batch); a running maximum rescales what earlier
    // batches accumulated, as in the online softmax.  A row with few states takes a
    // batch of 4 or 8, so that it issues no more loads than it has states.
    float M = kNoMax, L = 0.f;                 // L: per-lane sum, reduced at the end
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
    auto batches = [&](auto batch_c) {
        constexpr int B = decltype(batch_c)::value;
        const int first_batch = COOP ? wi * B : 0;
        const int batch_step = COOP ? kMergeRows * B : B;
        for (int c0 = first_batch; c0 < nst; c0 += batch_step) {
            const int cnt = min(B, nst - c0);
            float2 ml = make_float2(-INFINITY, 0.f);
            if (lane < cnt) {
                const float *so, *sml;
                state(c0 + lane, so, sml);
                ml = *reinterpret_cast<const float2*>(sml);
            }
            float v[B][PER];
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const float *so, *sml;
                state(c0 + min(j, cnt - 1), so, sml);
#pragma unroll
                for (int k = 0; k < PER; ++k) v[j][k] = so[lane * PER + k];
            }
            const float Mn = fmaxf(M, wave_max(ml.x));
            const float c = fast_exp2(M - Mn);
            M = Mn;
            const float wgt = lane < cnt ? fast_exp2(ml.x - Mn) : 0.f;
            L = fmaf(L, c, wgt * ml.y);
#pragma unroll
            for (int k = 0; k < PER; ++k) acc[k] *= c;
#pragma unroll
            for (int j = 0; j < B; ++j) {
                if (j < cnt) {
                    const float wj = u2f(__builtin_amdgcn_readlane(f2u(wgt), j));
#pragma unroll
                    for (int k = 0; k < PER; ++k) acc[k] = fmaf(wj, v[j][k], acc[k]);
                }
            }
        }
    };
    if (COOP || nst > 8)
        batches(std::integral_constant<int, kBatch>{});
    else if (nst > 4)
        batches(std::integral_constant<int, 8>{});
    else
        batches(std::integral_constant<int, 4>{});
    L = wave_sum(L);
    if constexpr (COOP) {
        // the waves' partial sums, rescaled to the largest of their maxima
        __shared__ float s_ml[kMergeRows][2];
        __shared__ float s_acc[kMergeRows][D];
        if (lane == 0) {
            s_ml[wi][0] = M;
            s_ml[wi][1] = L;
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) s_acc[wi][lane * PER + k] = acc[k];
        __syncthreads();
        if (wi != 0) return;
        float Mt = s_ml[0][0];
#pragma unroll
        for (int i = 1; i < kMergeRows; ++i) Mt = fmaxf(Mt, s_ml[i][0]);
        L = 0.f;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = 0.f;
#pragma unroll
        for (int i = 0; i < kMergeRows; ++i) {
            const float c = fast_exp2(s_ml[i][0] - Mt);    // 0 for a wave that had no state
            L = fmaf(s_ml[i][1], c, L);
#pragma unroll
            for (int k = 0; k < PER; ++k) acc[k] = fmaf(s_acc[i][lane * PER + k], c, acc[k]);
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        if constexpr (BF16)
            reinterpret_cast<uint16_t*>(a.out)[o + k] = f32_to_bf16(acc[k] * inv);
        else
            reinterpret_cast<float*>(a.out)[o + k] = acc[k] * inv;
    }
}

// --------------------------------------------------------------------------------------
// fixed partitions of part_tokens positions
// --------------------------------------------------------------------------------------
// Query row, block-table row and visible length of grid unit `sh`.  Decode: sequence
// sh / Hkv, its table row, its context.  CHUNKED (causal queries of prefill chunks, or
// of the multi-query decode when no matrix-core path serves the shape): slot v of
// chunk c = v / q_per_chunk is query i = v mod q_per_chunk of the chunk if i < n_q; it
// sits at position ctx_c - n_q + i and sees the keys up to it, through chunk c's table
// row.  ok = false for slots past a chunk's queries.
template <bool CHUNKED>
__device__ __forceinline__ void unit_of(const DecodeArgs& a, int v, int& s_tab, int& s_q, int& ctx,
                                        bool& ok) {
    if constexpr (!CHUNKED) {
        s_tab = s_q = v;
        ctx = clamp_ctx(a, a.context_lens[v]);
        ok = true;
    } else {
        const int c = v / a.q_per_chunk, i = v - c * a.q_per_chunk;
        int q0, nq;
        if (a.cu_q_lens != nullptr) {
            q0 = a.cu_q_lens[c];
            nq = a.cu_q_lens[c + 1] - q0;
        } else {
            q0 = c * a.q_per_chunk;
            nq = a.q_per_chunk;
        }
        const int cc = clamp_ctx(a, a.context_lens[c]);
        s_tab = c;
        s_q = q0 + i;
        ok = i < nq && s_q >= 0 && s_q < a.num_q_rows;
        ctx = max(0, min(cc - nq + i + 1, cc));
    }
}

template <bool BF16, int D, int G, bool CHUNKED = false>
__global__ __launch_bounds__(64, (BF16 ? 2 : 1)) void decode_partition_kernel(DecodeArgs a) {
    using S = DecodeShape<BF16, D>;
    __shared__ __attribute__((aligned(16))) char lds_k[kTile * S::KPITCH];
    __shared__ __attribute__((aligned(16))) uint32_t lds_p[DecodeLds<BF16>::PWORDS];
    __shared__ __attribute__((aligned(16))) uint32_t lds_q[G * S::RB / 4];

    const int sh = blockIdx.x;
    const int part = blockIdx.y;
    const int v = sh / a.g.num_kv_heads;
    const int h = sh - v * a.g.num_kv_heads;
    int s_tab, s_q, ctx;
    bool ok;
    unit_of<CHUNKED>(a, v, s_tab, s_q, ctx, ok);
    if (!ok) return;
    const int t_begin = part * a.part_tokens;
    const bool single = a.num_parts == 1;
    if (t_begin >= ctx) {
        if (single) zero_rows<BF16, D, G>(a, s_q, h);
        return;
    }
    SegState<BF16, D, G> st;
    attend_segment<BF16, D, G>(a, s_tab, s_q, h, ctx, t_begin, min(ctx, t_begin + a.part_tokens),
                               lds_k, lds_p, lds_q, st);
    if (single)
        write_rows<BF16, D, G>(a, s_q, h, st);
    else
        write_partial<BF16, D, G>(a, ((int64_t)s_q * a.num_q_heads + h * G) * a.num_parts + part,
                                  a.num_parts, st);
}

// Log-sum-exp merge of the partitions of one (sequence, q head):
// with M the largest partition max, weight w_p = 2^(m_p - M);
// out = sum_p w_p o_p / sum_p w_p l_p.  One wave per output row.
template <bool BF16, int D>
__global__ __launch_bounds__(64) void decode_partition_merge_kernel(DecodeArgs a) {
    constexpr int PER = D / 64;
    const int row = blockIdx.x;
    const int s = row / a.num_q_heads;
    const int lane = threadIdx.x;
    const int ctx = clamp_ctx(a, a.context_lens[s]);
    const int n = (ctx + a.part_tokens - 1) / a.part_tokens;
    const float* ml = a.part_ml + (int64_t)row * a.num_parts * 2;
    const float* po = a.part_o + (int64_t)row * a.num_parts * D;
    float M = kNoMax;
    for (int p = lane; p < n; p += 64) M = fmaxf(M, ml[2 * p]);
    M = wave_max(M);
    float L = 0.f;
    for (int p = lane; p < n; p += 64) L += fast_exp2(ml[2 * p] - M) * ml[2 * p + 1];
    L = wave_sum(L);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
#pragma unroll 8
    for (int p = 0; p < n; ++p) {
        const float w = fast_exp2(ml[2 * p] - M);
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = fmaf(w, po[(int64_t)p * D + lane * PER + k], acc[k]);
    }
    const int64_t o = (int64_t)row * D + lane * PER;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        if constexpr (BF16)
            reinterpret_cast<uint16_t*>(a.out)[o + k] = f32_to_bf16(acc[k] * inv);
        else
            reinterpret_cast<float*>(a.out)[o + k] = acc[k] * inv;
    }
}

// --------------------------------------------------------------------------------------
// host side
// --------------------------------------------------------------------------------------
// The balanced merge over `rows` output rows: one row per wave, or, when the rows are
// fewer than half the waves the split ran on (long contexts: each row has tens of
// pieces), one row per workgroup whose waves share its pieces.
template <bool BF16, int D, int G, bool PREFIX = false>
static void launch_balanced_merge(const DecodeArgs& a, int64_t rows, int nq, hipStream_t st) {
    if (rows * 2 < a.num_waves)
        hipLaunchKernelGGL((decode_balanced_merge_kernel<BF16, D, G, PREFIX, true>),
                           dim3((unsigned)rows), dim3(64 * kMergeRows), 0, st, a, nq);
    else
        hipLaunchKernelGGL((decode_balanced_merge_kernel<BF16, D, G, PREFIX, false>),
                           dim3((unsigned)((rows + kMergeRows - 1) / kMergeRows)),
                           dim3(64 * kMergeRows), 0, st, a, nq);
}

template <bool BF16, int D, int G, bool CONTIG = false, bool PREFIX = false>
static int balanced_waves_t() {
    // resident waves of the balanced kernel on the current device, cached per device
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu,
                reinterpret_cast<const void*>(decode_balanced_kernel<BF16, D, G, CONTIG, PREFIX>),
                64, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cache[dev] = max(1, per_cu) * max(1, cus);
    }
    return cache[dev];
}

template <bool BF16, int D, int G>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
    const int S = a.num_seqs;
    if (a.part_tokens > 0) {
        const dim3 grid((unsigned)(S * a.g.num_kv_heads), (unsigned)a.num_parts);
        hipLaunchKernelGGL((decode_partition_kernel<BF16, D, G>), grid, dim3(64), 0, st, a);
        if (a.num_parts > 1)
            hipLaunchKernelGGL((decode_partition_merge_kernel<BF16, D>), dim3(S * a.num_q_heads),
                               dim3(64), 0, st, a);
    } else {
        hipLaunchKernelGGL((decode_balanced_kernel<BF16, D, G>), dim3(a.num_waves), dim3(64), 0, st,
                           a);
        launch_balanced_merge<BF16, D, G>(a, (int64_t)S * a.num_q_heads, 1, st);
    }
    return hipGetLastError();
}

#define PKV_DISPATCH_G(FN, BF, DD, group, ...)     \
    switch (group) {                               \
        case 1: return FN<BF, DD, 1>(__VA_ARGS__); \
        case 2: return FN<BF, DD, 2>(__VA_ARGS__); \
        case 3: return FN<BF, DD, 3>(__VA_ARGS__); \
        case 4: return FN<BF, DD, 4>(__VA_ARGS__); \
        case 5: return FN<BF, DD, 5>(__VA_ARGS__); \
        case 6: return FN<BF, DD, 6>(__VA_ARGS__); \
        case 7: return FN<BF, DD, 7>(__VA_ARGS__); \
        case 8: return FN<BF, DD, 8>(__VA_ARGS__); \
        default: break;                            \
    }

// the contiguous-layout (unpaged) baseline: balanced split
template <bool BF16, int D, int G>
static hipError_t launch_contig_t(const DecodeArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((decode_balanced_kernel<BF16, D, G, true>), dim3(a.num_waves), dim3(64), 0,
                       st, a);
    launch_balanced_merge<BF16, D, G>(a, (int64_t)a.num_seqs * a.num_q_heads, 1, st);
    return hipGetLastError();
}
template <bool BF16, int D, int G>
static int contig_waves_t() {
    return balanced_waves_t<BF16, D, G, true>();
}

// causal query chunks on the vector units: one single-partition wave per (query, kv head)
template <bool BF16, int D, int G>
static hipError_t launch_chunked_t(const DecodeArgs& a, int64_t units, hipStream_t st) {
    hipLaunchKernelGGL((decode_partition_kernel<BF16, D, G, true>),
                       dim3((unsigned)(units * a.g.num_kv_heads), 1u), dim3(64), 0, st, a);
    return hipGetLastError();
}
template <bool BF16, int D>
static hipError_t launch_chunked_g(const DecodeArgs& a, int group, int64_t units, hipStream_t st) {
    PKV_DISPATCH_G(launch_chunked_t, BF16, D, group, a, units, st)
    return hipErrorInvalidValue;
}
hipError_t launch_decode_chunked(const DecodeArgs& a, bool is_bf16, int head_dim, int group,
                                 int64_t units, hipStream_t st) {
    if (units == 0) return hipSuccess;
    if (is_bf16) {
        if (head_dim == 128) return launch_chunked_g<true, 128>(a, group, units, st);
        if (head_dim == 64) return launch_chunked_g<true, 64>(a, group, units, st);
    } else {
        if (head_dim == 128) return launch_chunked_g<false, 128>(a, group, units, st);
        if (head_dim == 64) return launch_chunked_g<false, 64>(a, group, units, st);
    }
    return hipErrorInvalidValue;
}

// the shared-prefix mode: bf16, balanced split over the tokens after each prefix
template <bool BF16, int D, int G>
static hipError_t launch_prefix_decode_t(const DecodeArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((decode_balanced_kernel<true, D, G, false, true>), dim3(a.num_waves),
                       dim3(64), 0, st, a);
    launch_balanced_merge<true, D, G, true>(a, (int64_t)a.num_seqs * a.num_q_heads, 1, st);
    return hipGetLastError();
}
template <bool BF16, int D, int G>
static int prefix_waves_t() {
    return balanced_waves_t<true, D, G, false, true>();
}

// the merge of the multi-query decode (bf16): nq * G partial rows per (sequence, kv head)
template <bool BF16, int D, int G>
static hipError_t launch_merge_mq_t(const DecodeArgs& a, int nq, hipStream_t st) {
    launch_balanced_merge<true, D, G>(a, (int64_t)a.num_seqs * nq * a.num_q_heads, nq, st);
    return hipGetLastError();
}

hipError_t launch_balanced_merge_mq(const DecodeArgs& a, int head_dim, int group, int nq,
                                    hipStream_t st) {
    if (head_dim == 128) { PKV_DISPATCH_G(launch_merge_mq_t, true, 128, group, a, nq, st) }
    if (head_dim == 64) { PKV_DISPATCH_G(launch_merge_mq_t, true, 64, group, a, nq, st) }
    return hipErrorInvalidValue;
}

template <bool BF16, int D>
static hipError_t launch_decode_g(const DecodeArgs& a, int group, hipStream_t st) {
    PKV_DISPATCH_G(launch_decode_t, BF16, D, group, a, st)
    return hipErrorInvalidValue;
}

template <bool BF16, int D>
static int balanced_waves_g(int group) {
    PKV_DISPATCH_G(balanced_waves_t, BF16, D, group)
    return 0;
}

int decode_prefix_waves(int head_dim, int group) {
    if (head_dim == 128) { PKV_DISPATCH_G(prefix_waves_t, true, 128, group) }
    if (head_dim == 64) { PKV_DISPATCH_G(prefix_waves_t, true, 64, group) }
    return 0;
}

hipError_t launch_decode_prefix(const DecodeArgs& a, int head_dim, int group, int num_seqs,
                                hipStream_t st) {
    if (num_seqs == 0) return hipSuccess;
    if (head_dim == 128) { PKV_DISPATCH_G(launch_prefix_decode_t, true, 128, group, a, st) }
    if (head_dim == 64) { PKV_DISPATCH_G(launch_prefix_decode_t, true, 64, group, a, st) }
    return hipErrorInvalidValue;
}

int decode_contiguous_waves(bool is_bf16, int head_dim, int group) {
    if (is_bf16) {
        if (head_dim == 128) { PKV_DISPATCH_G(contig_waves_t, true, 128, group) }
        if (head_dim == 64) { PKV_DISPATCH_G(contig_waves_t, true, 64, group) }
    } else {
        if (head_dim == 128) { PKV_DISPATCH_G(contig_waves_t, false, 128, group) }
        if (head_dim == 64) { PKV_DISPATCH_G(contig_waves_t, false, 64, group) }
    }
    return 0;
}

hipError_t launch_decode_contiguous(const DecodeArgs& a, bool is_bf16, int head_dim, int group,
                                    int num_seqs, hipStream_t st) {
    if (num_seqs == 0) return hipSuccess;
    if (is_bf16) {
        if (head_dim == 128) { PKV_DISPATCH_G(launch_contig_t, true, 128, group, a, st) }
        if (head_dim == 64) { PKV_DISPATCH_G(launch_contig_t, true, 64, group, a, st) }
    } else {
        if (head_dim == 128) { PKV_DISPATCH_G(launch_contig_t, false, 128, group, a, st) }
        if (head_dim == 64) { PKV_DISPATCH_G(launch_contig_t, false, 64, group, a, st) }
    }
    return hipErrorInvalidValue;
}

int decode_balanced_waves(bool is_bf16, int head_dim, int group) {
    if (is_bf16) {
        if (head_dim == 128) return balanced_waves_g<true, 128>(group);
        if (head_dim == 64) return balanced_waves_g<true, 64>(group);
    } else {
        if (head_dim == 128) return balanced_waves_g<false, 128>(group);
        if (head_dim == 64) return balanced_waves_g<false, 64>(group);
    }
    return 0;
}

hipError_t launch_decode(const DecodeArgs& a, bool is_bf16, int head_dim, int group, int num_seqs,
                         hipStream_t st) {
    if (num_seqs == 0) return hipSuccess;
    if (is_bf16) {
        if (head_dim == 128) return launch_decode_g<true, 128>(a, group, st);
        if (head_dim == 64) return launch_decode_g<true, 64>(a, group, st);
    } else {
        if (head_dim == 128) return launch_decode_g<false, 128>(a, group, st);
        if (head_dim == 64) return launch_decode_g<false, 64>(a, group, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
