// The balanced split shared by the decode kernels: all 64-token tiles of a batch,
// ordered by (sequence, kv head, tile), divided into contiguous ranges over a
// persistent grid of waves.  A wave recomputes the plan from the context lengths
// alone, so no host pass or device scratch is needed to agree on it.
#pragma once

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kTile = 64;

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int c) {
    return max(0, min(c, min(a.max_context_len, a.max_blocks_per_seq * a.g.block_size)));
}
__device__ __forceinline__ int ntiles_of(int ctx) { return (ctx + kTile - 1) / kTile; }

// Block-table entries of the 64-token tile starting at t0: lane j holds the physical
// block of logical block t0/bs + j (clamped to the sequence's last block), so one
// vector load fetches every entry a tile needs.
__device__ __forceinline__ int load_tile_table(const int32_t* table, int t0, int log2_bs, int nblk,
                                               int lane) {
    return table[min((t0 >> log2_bs) + lane, nblk - 1)];
}

__device__ __forceinline__ int wave_sum_int(int x) {
    x += (int)__builtin_amdgcn_update_dpp(0u, (uint32_t)x, 0x128, 0xF, 0xF, false);
    x += (int)__builtin_amdgcn_update_dpp(0u, (uint32_t)x, 0x124, 0xF, 0xF, false);
    x += (int)__builtin_amdgcn_update_dpp(0u, (uint32_t)x, 0x122, 0xF, 0xF, false);
    x += (int)__builtin_amdgcn_update_dpp(0u, (uint32_t)x, 0x121, 0xF, 0xF, false);
    auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    x = (int)(r[0] + r[1]);
    auto q = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    // every lane holds the total; readfirstlane tells the compiler it is uniform
    return __builtin_amdgcn_readfirstlane((int)(q[0] + q[1]));
}

// First token of sequence s that the decode attends: in the shared-prefix mode the
// tokens before it (whole blocks) were attended by the prefix pass.  seq_start_of takes
// the sequence's prefix length as loaded.
__device__ __forceinline__ int seq_start_of(const DecodeArgs& a, int prefix_len, int ctx) {
    return min(max(prefix_len, 0) & ~(a.g.block_size - 1), ctx);
}
template <bool PREFIX>
__device__ __forceinline__ int seq_start(const DecodeArgs& a, int s, int ctx) {
    if constexpr (!PREFIX) {
        return 0;
    } else {
        return seq_start_of(a, a.seq_prefix[s], ctx);
    }
}
// Tiles of sequence s (per kv head).
template <bool PREFIX>
__device__ __forceinline__ int unit_tiles(const DecodeArgs& a, int s) {
    const int ctx = clamp_ctx(a, a.context_lens[s]);
    return ntiles_of(ctx - seq_start<PREFIX>(a, s, ctx));
}

// Tiles of the whole batch (all sequences, one kv head) and tiles before sequence `upto`.
// Four chunks of 64 sequences per pass, their loads issued together (a lane past the
// batch reads the last sequence and discards it: loads under a branch would each wait
// for their value in turn); the tile counts and clamped lengths of the first 256
// sequences stay in first[q] and first_ctx[q] (sequence 64q + lane) for locate_unit and
// the wave's first unit.
template <bool PREFIX = false>
__device__ __forceinline__ void count_tiles(const DecodeArgs& a, int upto, int64_t& total,
                                            int64_t& before, int (&first)[4],
                                            int (&first_ctx)[4]) {
    const int lane = threadIdx.x & 63;   // lane of the wave (the merge runs several per workgroup)
    total = 0;
    before = 0;
    for (int c0 = 0; c0 < a.num_seqs; c0 += 256) {
        int nt[4], cl[4], craw[4], praw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int sl = min(c0 + q * 64 + lane, a.num_seqs - 1);
            craw[q] = a.context_lens[sl];
            praw[q] = PREFIX ? a.seq_prefix[sl] : 0;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool in = c0 + q * 64 + lane < a.num_seqs;
            cl[q] = in ? clamp_ctx(a, craw[q]) : 0;
            nt[q] = in ? ntiles_of(cl[q] - (PREFIX ? seq_start_of(a, praw[q], cl[q]) : 0)) : 0;
        }
        if (c0 == 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                first[q] = nt[q];
                first_ctx[q] = cl[q];
            }
        }
        int t = 0, u = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            t += nt[q];
            u += c0 + q * 64 + lane < upto ? nt[q] : 0;
        }
        total += wave_sum_int(t);
        before += wave_sum_int(u);
    }
}
// Value of uniform sequence s < 256 among per-lane values kept as count_tiles keeps them
// (sequence 64q + lane in v[q]): no memory access.
__device__ __forceinline__ int lane_value(const int (&v)[4], int s) {
    const int q = s >> 6;
    const int x = q == 0 ? v[0] : q == 1 ? v[1] : q == 2 ? v[2] : v[3];
    return __builtin_amdgcn_readlane(x, s & 63);
}

// Share of the tiles each wave gets, by the XCD it runs on (in 1/256).  The dispatcher
// hands workgroup w to XCD w mod 8, so in a grid that fills every wave slot the waves
// of one XCD are those with one w mod 8.  Per-wave timestamps on two MI355X machines
// (GQA and long-context batches, 24 calls) put the mean finish of the waves of XCDs 0..7
// at 0.956, 1.005, 0.974, 1.026, 0.993, 1.039, 0.975, 1.034 of the average: odd XCDs
// stream about 5% slower.  The weights take three quarters of the inverse.
constexpr int kXcdWeight[8] = {265, 255, 261, 251, 257, 249, 261, 250};
// Sum of the weights of waves 0..n-1.  The partial period is summed with selects over
// the table's entries as immediates: indexing it at run time would compile to a memory
// load, a dependent round trip in every evaluation.
__device__ __forceinline__ int64_t xcd_weight_prefix(int64_t n) {
    int64_t sum = 0;
#pragma unroll
    for (int x = 0; x < 8; ++x) sum += kXcdWeight[x];
    const int r = (int)(n & 7);
    int pre = 0;
#pragma unroll
    for (int x = 0; x < 7; ++x) pre += x < r ? kXcdWeight[x] : 0;
    return (n >> 3) * sum + pre;
}

// The split of T tiles over W waves into contiguous ranges, every range non-empty.
// Weighted (the grid fills every wave slot, W a multiple of 16, and the lightest wave's
// share T w_min / Ptot is at least one tile): wave w gets a share proportional to its
// class weight (lw for the first half of the grid, which wins issue arbitration when
// two waves share a SIMD, gw for the second) times its XCD's weight.  Otherwise the T
// tiles are shared evenly.
struct Split {
    int64_t T, W;
    int64_t Wl;          // lead waves (W / 2); 0 for the even split
    int64_t lw, gw;      // class weights (lead, lag)
    int64_t Ptot;        // total weight of the W waves
    double inv_ptot;     // 1 / Ptot, for the estimates range_begin corrects
};
__device__ __forceinline__ Split even_split(int64_t T, int64_t W) {
    return Split{T, W, 0, 1, 1, W, 1.0 / (double)W};
}
__device__ __forceinline__ Split make_split(const DecodeArgs& a, int64_t T, int64_t W) {
    Split p = even_split(T, W);
    if (W == a.num_waves && W % 16 == 0 && a.lead_share_q10 > 0 && a.lead_share_q10 < 1024) {
        const int64_t lw = a.lead_share_q10, gw = 1024 - a.lead_share_q10;
        const int64_t Ptot = (lw + gw) * xcd_weight_prefix(W / 2);
        constexpr int64_t kXcdMin = 249;       // smallest entry of kXcdWeight
        if (T * (min(lw, gw) * kXcdMin) >= Ptot) {
            p.Wl = W / 2;
            p.lw = lw;
            p.gw = gw;
            p.Ptot = Ptot;
            p.inv_ptot = 1.0 / (double)Ptot;
        }
    }
    return p;
}
// Weight of waves 0..w-1.
__device__ __forceinline__ int64_t split_prefix(const Split& p, int64_t w) {
    if (p.Wl == 0) return w;
    return w <= p.Wl ? p.lw * xcd_weight_prefix(w)
                     : p.lw * xcd_weight_prefix(p.Wl) + p.gw * xcd_weight_prefix(w - p.Wl);
}
// First tile of wave w's range [begin(w), begin(w + 1)): floor(T P(w) / Ptot);
// begin(W) = T.  64-bit integer division is a long software sequence on the GPU, so
// while T and Ptot stay below 2^31 (T P < 2^62) the quotient is estimated with the
// split's double-precision reciprocal (off by at most one) and corrected with exact
// 64-bit products.
__device__ __forceinline__ int64_t range_begin(const Split& p, int64_t w) {
    const int64_t P = split_prefix(p, w);
    if (p.T < ((int64_t)1 << 31) && p.Ptot < ((int64_t)1 << 31)) {
        const int64_t num = p.T * P;
        int64_t c = (int64_t)((double)num * p.inv_ptot);
        while (c * p.Ptot > num) --c;
        while ((c + 1) * p.Ptot <= num) ++c;
        return c;
    }
    return (p.T / p.Ptot) * P + (p.T % p.Ptot) * P / p.Ptot;
}
// Wave whose range holds tile u (0 <= u < T): the last w with begin(w) <= u.  Within
// each class the shares differ only by the XCD weights (a few percent), so spreading
// the class's tiles evenly over its waves lands within a wave or two of the owner,
// which a short walk over exact range starts settles.
__device__ __forceinline__ int64_t unit_owner(const Split& p, int64_t u) {
    int64_t w;
    if (p.Wl == 0) {
        w = (int64_t)(((float)u + 0.5f) * (float)p.W * __builtin_amdgcn_rcpf((float)p.T));
    } else {
        const int64_t bl = range_begin(p, p.Wl);          // first tile of the lag class
        w = u < bl ? (int64_t)(((float)u + 0.5f) * (float)p.Wl * __builtin_amdgcn_rcpf((float)bl))
                   : p.Wl + (int64_t)(((float)(u - bl) + 0.5f) * (float)(p.W - p.Wl) *
                                      __builtin_amdgcn_rcpf((float)(p.T - bl)));
    }
    w = max((int64_t)0, min(w, p.W - 1));
    while (w > 0 && range_begin(p, w) > u) --w;
    while (w + 1 < p.W && range_begin(p, w + 1) <= u) ++w;
    return w;
}

// Record, from the wave w that holds the first tile u0 of unit (s, h) with nt tiles,
// that wave and how many waves the unit's tiles span (one: w finished it, which the
// caller knows without locating the last tile's owner).
__device__ __forceinline__ void record_unit(const DecodeArgs& a, const Split& sp, int64_t w, int s,
                                            int h, int64_t u0, int nt, bool finished) {
    const int64_t w1 = finished ? w : unit_owner(sp, u0 + nt - 1);
    if ((threadIdx.x & 63) == 0)
        *reinterpret_cast<int2*>(a.unit_desc + 2 * ((int64_t)s * a.g.num_kv_heads + h)) =
            make_int2((int)w, (int)(w1 - w + 1));
}

// Sequence holding unit b (the first s with Hkv * (tiles up to s) > b) and the tiles
// of all sequences before it; one wave-wide inclusive scan per 64 sequences, over the
// counts count_tiles kept for the first 256 (no reload) and reloaded beyond.
template <bool PREFIX = false>
__device__ __forceinline__ void locate_unit(const DecodeArgs& a, int64_t b, int Hkv,
                                            const int (&first)[4], int& s, int64_t& before) {
    const int lane = threadIdx.x & 63;   // lane of the wave (the merge runs several per workgroup)
    s = 0;
    before = 0;
    int64_t carry = 0;
    for (int c0 = 0; c0 < a.num_seqs; c0 += 64) {
        const int sl = c0 + lane;
        int nt;
        if (c0 < 256) {
            const int q = c0 >> 6;                 // uniform
            nt = q == 0 ? first[0] : q == 1 ? first[1] : q == 2 ? first[2] : first[3];
        } else {
            const int t = unit_tiles<PREFIX>(a, min(sl, a.num_seqs - 1));
            nt = sl < a.num_seqs ? t : 0;
        }
        int incl = nt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        const uint64_t hit = __ballot((carry + incl) * Hkv > b);
        if (hit) {
            const int ln = __ffsll((unsigned long long)hit) - 1;
            s = c0 + ln;
            // readlane with a uniform lane: the compiler then knows the value is uniform
            before = carry + __builtin_amdgcn_readlane(incl - nt, ln);
            return;
        }
        carry += __builtin_amdgcn_readlane(incl, 63);
    }
}

}  // namespace pkv
