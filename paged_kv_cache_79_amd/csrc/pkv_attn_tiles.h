// Tile helpers of the matrix-core attention kernels (chunked prefill and the
// shared-prefix pass of decode): 64-key K/V tiles staged from the paged pool through
// registers into LDS -- K rows as they are, V transposed for the O^T += V^T P^T
// product -- with the block ids of a tile fetched one tile ahead.
#pragma once

#include "pkv_device.h"
#include "pkv_internal.h"

#include <type_traits>

namespace pkv {

constexpr int kRowsPerWg = 128;   // packed (query, head) rows per workgroup
constexpr int kKeyTile = 64;      // keys per tile
constexpr int kXcds = 8;          // MI355X: workgroups are dealt round-robin to 8 XCDs
// Slack of the lazily updated softmax maximum (log2 units): a factor of 256.
constexpr float kLazyMax = 8.f;

template <int D>
struct PrefillShape {
    static constexpr int RB = D * 2;                  // bytes of a K/V row (bf16)
    static constexpr int CPR = RB / 16;               // 16-byte chunks per row
    static constexpr int KPITCH = RB + 16;            // K tile row pitch in LDS (bytes)
    static constexpr int VPITCH = kKeyTile * 2 + 16;  // V^T row pitch in LDS (bytes): 36 dwords
    static constexpr int KSTEPS = D / 16;             // QK k-steps of 16
    static constexpr int DT = D / 32;                 // 32-row output tiles
    static constexpr int KLOADS = kKeyTile * CPR / 256;   // K chunks per thread per tile
    static constexpr int VLOADS = CPR / 8;            // V chunk pairs per thread per tile
};

// Position of key k (0..63) inside the transposed V tile.  Within a group of 16
// keys, the C registers of a 32x32 MFMA hold key 8b+4h+j (b, h in {0,1}, j < 4) at
// B-operand slot 8h+4b+j of the next MFMA: bits 2 and 3 swap.  The map is its own
// inverse.
__device__ __forceinline__ int vt_slot(int k) {
    return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Byte offset of 16-byte group g (8 key slots) of V^T row d.  Groups are XOR-swizzled
// by 2 * (d / 16): the transposing writes (rows 8 apart, in pairs of keys) then spread
// over all 64 banks, and the operand reads (16 consecutive rows, 36 dwords apart) stay
// on distinct banks.
template <int D>
__device__ __forceinline__ int vt_off(int d, int g) {
    return d * PrefillShape<D>::VPITCH + ((g ^ ((d >> 3) & 6)) << 4);
}

// Thread t loads K rows t / CPR + (256 / CPR) i (whole rows per wave) and the V
// rows of key pair t / 8, chunks t % 8 + 8 j (half rows per lane).
template <int D>
__device__ __forceinline__ int k_row(int i, int tid) {
    using P = PrefillShape<D>;
    return i * (256 / P::CPR) + tid / P::CPR;
}

template <int D>
struct KvStage {
    u32x4 k[PrefillShape<D>::KLOADS];
    u32x4 v[2 * PrefillShape<D>::VLOADS];
};

// Physical block ids behind the rows one thread loads from a tile.
template <int D>
struct TileIds {
    int k[PrefillShape<D>::KLOADS];
    int v[2];
};

// Byte offsets, inside a (block, kv head) run, of the K rows one thread loads.  Tiles
// start at multiples of 64 >= block_size, so they are the same for every tile.
template <int D>
struct TileOffs {
    uint32_t k[PrefillShape<D>::KLOADS];
};

template <int D>
__device__ __forceinline__ void tile_offsets(TileOffs<D>& o, int block_size, int tid) {
    using P = PrefillShape<D>;
#pragma unroll
    for (int i = 0; i < P::KLOADS; ++i)
        o.k[i] = (uint32_t)((k_row<D>(i, tid) & (block_size - 1)) * P::RB + (tid % P::CPR) * 16);
}

// Block ids for the tile starting at t0 (validated where they are used: checking
// them here would wait for these table reads, and with them for every global load
// issued before, at the top of each tile).  Keys past the context (only in a sequence's last tile):
//   K rows read the block of the last token at their own offset -- inside the pool,
//      but stale data, whose scores the softmax replaces by -inf;
//   V rows read the last token's row itself -- finite data, which the zero
//      probability of a hidden key then multiplies to exactly zero.
template <int D>
__device__ __forceinline__ void load_ids(TileIds<D>& ids, const int32_t* table, const PoolGeom& g,
                                         int ctx, int t0, int tid) {
    using P = PrefillShape<D>;
#pragma unroll
    for (int i = 0; i < P::KLOADS; ++i) {
        ids.k[i] = table[(uint32_t)min(t0 + k_row<D>(i, tid), ctx - 1) >> g.log2_bs];
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
        ids.v[r] = table[(uint32_t)min(t0 + 2 * (tid >> 3) + r, ctx - 1) >> g.log2_bs];
}

// Row address in the pool; an id outside the pool reads block 0 instead.
__device__ __forceinline__ const u32x4* pool_row(const char* base, int id, uint32_t num_blocks,
                                                 uint32_t stride, uint32_t off) {
    const uint32_t ub = (uint32_t)id < num_blocks ? (uint32_t)id : 0u;
    return reinterpret_cast<const u32x4*>(base + ((uint64_t)ub * stride + off));
}

// Global loads of the 64-key tile starting at t0.  Ordinary (cached) loads: every
// query tile of a (chunk, kv head) reads the same K/V tiles at about the same time,
// and L2 serves the repeats (nontemporal loads, which suit decode's read-once
// stream, cost the prefill 10-14% here).
template <int D>
__device__ __forceinline__ void load_tile(KvStage<D>& st, const TileIds<D>& ids,
                                          const TileOffs<D>& offs, const PoolGeom& g,
                                          const char* kb, const char* vb, int ctx, int t0,
                                          int tid) {
    using P = PrefillShape<D>;
    const uint32_t stride = (uint32_t)g.block_stride_bytes, nb = (uint32_t)g.num_blocks;
#pragma unroll
    for (int i = 0; i < P::KLOADS; ++i)
        st.k[i] = *pool_row(kb, ids.k[i], nb, stride, offs.k[i]);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const uint32_t tok = (uint32_t)min(t0 + 2 * (tid >> 3) + r, ctx - 1);
        const uint32_t off = (tok & (uint32_t)(g.block_size - 1)) * P::RB + (uint32_t)(tid & 7) * 16;
#pragma unroll
        for (int j = 0; j < P::VLOADS; ++j)
            st.v[2 * j + r] = *pool_row(vb, ids.v[r], nb, stride, off + 128 * j);
    }
}

// Staged tile -> LDS: K rows as they are, V transposed (pairs of keys per dword).
template <int D>
__device__ __forceinline__ void store_tile(const KvStage<D>& st, char* lds_k, char* lds_vt, int tid) {
    using P = PrefillShape<D>;
    const int kp = tid >> 3, c0 = tid & 7;
#pragma unroll
    for (int i = 0; i < P::KLOADS; ++i)
        *reinterpret_cast<u32x4*>(lds_k + k_row<D>(i, tid) * P::KPITCH + (tid % P::CPR) * 16) =
            st.k[i];
    const int slot = vt_slot(2 * kp);           // even: keys 2kp, 2kp+1 share one dword
    const int g = slot >> 3, within = (slot & 7) * 2;
#pragma unroll
    for (int j = 0; j < P::VLOADS; ++j) {
        const u32x4 x0 = st.v[2 * j], x1 = st.v[2 * j + 1];
        const uint32_t a0[4] = {x0.x, x0.y, x0.z, x0.w};
        const uint32_t a1[4] = {x1.x, x1.y, x1.z, x1.w};
        const int dbase = (c0 + 8 * j) * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int d = dbase + 2 * q;
            *reinterpret_cast<uint32_t*>(lds_vt + vt_off<D>(d, g) + within) = pair_lo(a0[q], a1[q]);
            *reinterpret_cast<uint32_t*>(lds_vt + vt_off<D>(d + 1, g) + within) = pair_hi(a0[q], a1[q]);
        }
    }
}

// Sum of the 8 bf16 probabilities packed in p, added to acc: the row sums then count
// the same rounded values that the P V product multiplies.
__device__ __forceinline__ float sum_bf16x8(u32x4 p, float acc) {
    constexpr uint32_t kOnes = 0x3F803F80u;      // (1.0, 1.0) in bf16
    acc = dot2_bf16(p.x, kOnes, acc);
    acc = dot2_bf16(p.y, kOnes, acc);
    acc = dot2_bf16(p.z, kOnes, acc);
    return dot2_bf16(p.w, kOnes, acc);
}

// ---- D = 128: K/V tiles straight from the pool into LDS --------------------------
//
// The tile loop above (load_tile / store_tile) stages every K/V tile through 64 registers
// per lane and writes V transposed into LDS with byte permutes.  For D = 128 the tiles
// instead go from the pool into LDS with the gfx950 direct loads (global_load_lds_dwordx4: lane t's 16 bytes land
// at the wave's LDS base + 16 t), K and V both row-major with 256-byte rows, and the
// V^T operand of the P.V product is read with the transposing ds_read_b64_tr_b16.  No
// registers hold a tile in flight, and no vector instruction touches it on its way.
//
// Which 16-byte chunk of a row a lane fetches decides where it lands, so the chunks of
// each row are permuted (a XOR with row bits) to keep the operand reads free of bank
// conflicts:
//   K: chunk c of row r at position c ^ (r % 16).  The S^T = K Q^T operand of lane l is
//      chunk 2 ks + l / 32 of row 32 mt + l % 32: 16 consecutive rows, 16 positions.
//   V: chunk c of row r at position c ^ 4 (r % 4).  A transposing read serves 32 lanes
//      from 4 consecutive rows x 4 consecutive chunks: 16 positions.
struct PfLdsDma {
    char k[2][kKeyTile * 256];
    char v[2][kKeyTile * 256];
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// One wave-wide direct load, lane t: 16 bytes from gbase + voff to LDS lds + 16 t.  It is
// written as inline asm so that the compiler, which cannot tell the LDS buffers apart, does
// not wait for it before every later LDS read; the wait is explicit (wait_dma).  The nops
// cover the hazards of a base or M0 written just before (VALU write of an SGPR that a
// vector memory instruction reads: 5 wait states).
__device__ __forceinline__ void dma16(uint32_t lds, const char* gbase, uint32_t voff) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "{m0}"(lds)
                 : "memory");
}
// Every direct load of this wave has written LDS (and every other vector load is back).
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef short pf_v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) pf_v4i16 pf_lds_v4i16;

// Attend this wave's 32 rows (the lane's query row: column n = lane % 32 of the 32x32
// products; q of the row in qreg, the B operand of each k-step) to keys [t_begin,
// t_end) of one (sequence, kv head), online softmax into (oacc, m, l) as the prefill
// kernels keep them.  The four waves of the workgroup call it alike (it has barriers).
//   ctx       keys the table holds; rows at or past it read key ctx - 1 (finite data
//             that a zero probability then removes)
//   full_end  every row of the wave sees every key below it
//   last_key  the lane's row sees keys <= last_key (-1: none)
//   load_q    fills qreg (plain loads); called once the first tiles' block ids are on
//             their way, so that the q rows and those ids travel together (the ids' wait
//             then does not also wait for the rows, which the first full wait covers)
// Per tile: the direct loads go out first (V of the next tile, K of the one after; their
// block ids were read a tile earlier), then the S^T = K Q^T products of the next tile
// beside the softmax of this one, O^T += V^T P^T, one wait for this wave's loads and one
// barrier.
template <class LoadQ>
__device__ __forceinline__ void dma_attend_tiles(PfLdsDma& lds, const int32_t* table,
                                                 const PoolGeom& geom, const char* kb,
                                                 const char* vb, int ctx, int t_begin, int t_end,
                                                 int full_end, int last_key, float sl2,
                                                 LoadQ&& load_q, u32x4 (&qreg)[8],
                                                 floatx16_t (&oacc)[4], float& m, float& l) {
    constexpr int D = 128, RB = 256;
    using P = PrefillShape<D>;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 31;
    const int half = lane >> 5;
    const int bs = geom.block_size;
    const uint32_t stride = (uint32_t)geom.block_stride_bytes, nbk = (uint32_t)geom.num_blocks;

    // ---- direct loads: wave w moves rows 16 w .. 16 w + 15 of each tile, four loads of
    // four rows; lane t takes row t / 16 of a load and fills chunk position t % 16
    const int dr = lane >> 4, dp = lane & 15;
    uint32_t kvo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kvo[i] = (uint32_t)(16 * (dp ^ ((4 * i + dr) & 15)));
    const uint32_t vvo = (uint32_t)(16 * (dp ^ (4 * dr)));
    const uint32_t drow = (uint32_t)dr * RB;
    // block ids of a tile's four loads (lane i < 4: load i), read ahead of the loads
    auto tile_ids = [&](int t0) {
        const int tb = min(t0 + 16 * w + 4 * min(lane, 3), ctx - 1);
        return table[(uint32_t)tb >> geom.log2_bs];
    };
    auto issue_loads = [&](int t0, int buf, int ids, auto ragged_c, auto kv_c) {
        constexpr bool ragged = decltype(ragged_c)::value;
        constexpr int kv = decltype(kv_c)::value;      // 0: K, 1: V
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tb = t0 + 16 * w + 4 * i;
            const int tbc = min(tb, ctx - 1);
            uint32_t id = (uint32_t)__builtin_amdgcn_readlane(ids, i);
            id = id < nbk ? id : 0u;
            const uint32_t roff = (uint32_t)(tbc & (bs - 1)) * RB;
            const uint64_t boff = (((uint64_t)__umulhi(id, stride) << 32) | (uint64_t)(id * stride)) + roff;
            const uint32_t row = ragged ? (uint32_t)(min(tb + dr, ctx - 1) - tbc) * RB : drow;
            if constexpr (kv == 0)
                dma16(lds_addr(lds.k[buf]) + (uint32_t)((16 * w + 4 * i) * RB), kb + boff,
                      row + kvo[i]);
            else
                dma16(lds_addr(lds.v[buf]) + (uint32_t)((16 * w + 4 * i) * RB), vb + boff,
                      row + vvo);
        }
    };
    // the K (kv 0) or V (kv 1) rows of the tile at t0; rows past the context (only in the
    // last tile) read the last token's row
    auto issue = [&](int t0, int buf, int ids, auto kv_c) {
        if (t0 + kKeyTile > ctx)
            issue_loads(t0, buf, ids, std::true_type{}, kv_c);
        else
            issue_loads(t0, buf, ids, std::false_type{}, kv_c);
    };
    using KT = std::integral_constant<int, 0>;
    using VT = std::integral_constant<int, 1>;

    // ---- operand offsets inside a tile buffer
    uint32_t koff[P::KSTEPS];      // S^T = K Q^T: row n (+32 mt), chunk 2 ks + half
#pragma unroll
    for (int ks = 0; ks < P::KSTEPS; ++ks)
        koff[ks] = (uint32_t)(n * RB + 16 * ((2 * ks + half) ^ (n & 15)));
    // P.V: the transposing read of lane a (of 16-lane group g) addresses key row
    // 4 (g / 2) + a / 4 (+ 16 u, + 8 for the second half of the operand), elements
    // 32 dt + 16 (g % 2) + 4 (a % 4) .. + 3
    uint32_t vtoff[P::DT];
    {
        const int g = lane >> 4, ai = lane & 15, rr = ai >> 2, qq = ai & 3;
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt)
            vtoff[dt] = (uint32_t)((4 * (g >> 1) + rr) * RB +
                                   16 * (4 * (dt ^ rr) + 2 * (g & 1) + (qq >> 1)) + 8 * (qq & 1));
    }

    if (t_begin >= t_end) return;          // uniform over the workgroup
    const int nt = (t_end - t_begin + kKeyTile - 1) / kKeyTile;

    // S^T = K Q^T of the tile in K buffer kbuf, operands read three ahead
    auto qk_plain = [&](int kbuf, floatx16_t (&sacc)[2]) {
        const char* tk = lds.k[kbuf];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[mt][e] = 0.f;
        constexpr int NK = 2 * P::KSTEPS, AH = 3;
        auto kop = [&](int i) {
            return *reinterpret_cast<const u32x4*>(tk + (i / P::KSTEPS) * 32 * RB +
                                                   koff[i % P::KSTEPS]);
        };
        u32x4 kbf[AH];
#pragma unroll
        for (int i = 0; i < AH; ++i) kbf[i] = kop(i);
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const u32x4 ka = kbf[i % AH];
            if (i + AH < NK) kbf[i % AH] = kop(i + AH);
            sacc[i / P::KSTEPS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, ka), __builtin_bit_cast(bf16x8_t, qreg[i % P::KSTEPS]),
                sacc[i / P::KSTEPS], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Prologue: K and V of tile 0, K of tile 1; S of tile 0.  From then on step j issues V
    // of tile j + 1 and K of tile j + 2, and runs the products of tile j + 1 beside the
    // exponentials of tile j.
    int ids1 = 0, ids2 = 0;
    {
        const int ids0 = tile_ids(t_begin);
        if (nt > 1) ids1 = tile_ids(t_begin + kKeyTile);
        __builtin_amdgcn_sched_barrier(0);
        load_q(qreg);
        __builtin_amdgcn_sched_barrier(0);
        issue(t_begin, 0, ids0, KT{});
        issue(t_begin, 0, ids0, VT{});
        if (nt > 1) issue(t_begin + kKeyTile, 1, ids1, KT{});
        if (nt > 2) ids2 = tile_ids(t_begin + 2 * kKeyTile);
    }
    wait_dma();
    // the ids and q rows are back: the compiler places no wait for them in the loop
    asm volatile("" : "+v"(ids2));
#pragma unroll
    for (int ks = 0; ks < P::KSTEPS; ++ks) asm volatile("" : "+v"(qreg[ks]));
    __syncthreads();
    floatx16_t sacc[2];
    qk_plain(0, sacc);
    __syncthreads();                       // every wave is done with K buffer 0

    // step j: tile t0 = t_begin + 64 j, K of tile j + 1 in K buffer kn, V of tile j in
    // V buffer vc (kn = vc ^ 1 = (j + 1) % 2)
    auto step = [&](int t0, int kn, int vc) {
        const bool more1 = t0 + kKeyTile < t_end, more2 = t0 + 2 * kKeyTile < t_end;
        int ids3 = 0;
        if (more1) issue(t0 + kKeyTile, vc ^ 1, ids1, VT{});
        if (more2) {
            issue(t0 + 2 * kKeyTile, vc, ids2, KT{});
            if (t0 + 3 * kKeyTile < t_end) ids3 = tile_ids(t0 + 3 * kKeyTile);
        }

        // ---- online softmax of tile j: the maximum first (mask on the tiles that hide keys)
        const bool scaled = t0 + kKeyTile > full_end || !(sl2 > 0.f);
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

        // ---- S^T of tile j + 1 (K buffer kn; past the last tile its stale contents give
        // products nothing reads) beside the probabilities of tile j: one product, six
        // vector instructions and one operand read at a time
        floatx16_t snx[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) snx[mt][e] = 0.f;
        u32x4 pk[4];
        {
            const char* tk = lds.k[kn];
            constexpr int NK = 2 * P::KSTEPS, AH = 3;
            auto kop = [&](int i) {
                return *reinterpret_cast<const u32x4*>(tk + (i / P::KSTEPS) * 32 * RB +
                                                       koff[i % P::KSTEPS]);
            };
            u32x4 kbf[AH];
#pragma unroll
            for (int i = 0; i < AH; ++i) kbf[i] = kop(i);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int mt = u >> 1, e0 = (u & 1) * 8;
                float p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    p[j] = fast_exp2(__builtin_fmaf(sacc[mt][e0 + j], mul, -mn));
                pk[u] = u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                              pack_bf16(p[6], p[7])};
                l = sum_bf16x8(pk[u], l);
#pragma unroll
                for (int i = 4 * u; i < 4 * u + 4; ++i) {
                    const u32x4 ka = kbf[i % AH];
                    if (i + AH < NK) kbf[i % AH] = kop(i + AH);
                    snx[i / P::KSTEPS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8_t, ka),
                        __builtin_bit_cast(bf16x8_t, qreg[i % P::KSTEPS]), snx[i / P::KSTEPS], 0, 0,
                        0);
                }
            }
            // issue order: the first AH operand reads, then per product: the product, six
            // vector instructions and the read of the operand AH products ahead
            __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                if (i + AH < NK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- O^T += V^T P^T of tile j (V buffer vc), operands read two ahead
        {
            const char* tv = lds.v[vc];
            constexpr int NV = P::DT * 4, AH = 2;
            auto vop = [&](int i) {
                const int dt = i >> 2, u = i & 3;
                const char* p0 = tv + 16 * u * RB + vtoff[dt];
                const pf_v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((pf_lds_v4i16*)p0);
                const pf_v4i16 hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((pf_lds_v4i16*)(p0 + 8 * RB));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                return u32x4{l2.x, l2.y, h2.x, h2.y};
            };
            u32x4 vbf[AH];
#pragma unroll
            for (int i = 0; i < AH; ++i) vbf[i] = vop(i);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const u32x4 va = vbf[i % AH];
                if (i + AH < NV) vbf[i % AH] = vop(i + AH);
                oacc[i >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8_t, va), __builtin_bit_cast(bf16x8_t, pk[i & 3]),
                    oacc[i >> 2], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // this wave's loads (V of tile j + 1, K of tile j + 2) are in LDS; the barrier
        // publishes them and frees the buffers tile j used
        wait_dma();
        asm volatile("" : "+v"(ids3));
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) sacc[mt] = snx[mt];
        ids1 = ids2;
        ids2 = ids3;
    };
    for (int t0 = t_begin; t0 < t_end; t0 += 2 * kKeyTile) {
        step(t0, 1, 0);
        if (t0 + kKeyTile >= t_end) break;
        step(t0 + kKeyTile, 0, 1);
    }
}

}  // namespace pkv
