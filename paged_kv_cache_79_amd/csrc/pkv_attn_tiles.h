// Tile helpers of the matrix-core attention kernels (chunked prefill and the
// shared-prefix pass of decode): 64-key K/V tiles staged from the paged pool through
// registers into LDS -- K rows as they are, V transposed for the O^T += V^T P^T
// product -- with the block ids of a tile fetched one tile ahead.
#pragma once

#include "pkv_device.h"
#include "pkv_internal.h"

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

}  // namespace pkv
