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
// tokens before it (whole blocks) were attended by the prefix pass.
template <bool PREFIX>
__device__ __forceinline__ int seq_start(const DecodeArgs& a, int s, int ctx) {
    if constexpr (!PREFIX) {
        return 0;
    } else {
        const int p = max(a.seq_prefix[s], 0) & ~(a.g.block_size - 1);
        return min(p, ctx);
    }
}
// Tiles of sequence s (per kv head).
template <bool PREFIX>
__device__ __forceinline__ int unit_tiles(const DecodeArgs& a, int s) {
    const int ctx = clamp_ctx(a, a.context_lens[s]);
    return ntiles_of(ctx - seq_start<PREFIX>(a, s, ctx));
}

// Tiles of the whole batch (all sequences, one kv head) and tiles before sequence `upto`.
// Four chunks of 64 sequences per pass, their loads issued together; the counts of
// the first 256 sequences stay in first[q] (sequence 64q + lane) for locate_unit.
// With a.tile_prefix set, the wave numbered `writer` records, for every pass it owns
// (pass p belongs to wave p mod num_waves), each sequence's tiles before it, and wave 0
// the batch's total at index num_seqs: the merge then finds a row's pieces in O(1).
template <bool PREFIX = false>
__device__ __forceinline__ void count_tiles(const DecodeArgs& a, int upto, int64_t& total,
                                            int64_t& before, int (&first)[4], int64_t writer = -1) {
    const int lane = threadIdx.x & 63;   // lane of the wave (the merge runs several per workgroup)
    total = 0;
    before = 0;
    for (int c0 = 0; c0 < a.num_seqs; c0 += 256) {
        int nt[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int sl = c0 + q * 64 + lane;
            nt[q] = sl < a.num_seqs ? unit_tiles<PREFIX>(a, sl) : 0;
        }
        if (c0 == 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) first[q] = nt[q];
        }
        if (a.tile_prefix != nullptr && writer == (int64_t)(c0 >> 8) % a.num_waves) {
            int64_t off = total;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                int incl = nt[q];
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int y = __shfl_up(incl, d);
                    if (lane >= d) incl += y;
                }
                const int sl = c0 + q * 64 + lane;
                if (sl < a.num_seqs) a.tile_prefix[sl] = off + (incl - nt[q]);
                off += __builtin_amdgcn_readlane(incl, 63);
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
    if (a.tile_prefix != nullptr && writer == 0 && lane == 0) a.tile_prefix[a.num_seqs] = total;
}
template <bool PREFIX = false>
__device__ __forceinline__ void count_tiles(const DecodeArgs& a, int upto, int64_t& total,
                                            int64_t& before) {
    int first[4];
    count_tiles<PREFIX>(a, upto, total, before, first);
}

// The split of T tiles over W waves: the first Wl waves share the first F tiles
// evenly, the other W - Wl waves the remaining T - F (every range non-empty).
struct Split {
    int64_t T, W, F, Wl;
};
__device__ __forceinline__ Split make_split(const DecodeArgs& a, int64_t T, int64_t W) {
    Split p{T, W, T, W};                       // even split: one class of waves
    if (W == a.num_waves && W % 2 == 0) {
        const int64_t F = T * a.lead_share_q10 / 1024, Wl = W / 2;
        if (F >= Wl && T - F >= W - Wl) {
            p.F = F;
            p.Wl = Wl;
        }
    }
    return p;
}
// First tile of wave w's range [begin(w), begin(w + 1)); begin(Wl) = F, begin(W) = T.
__device__ __forceinline__ int64_t range_begin(const Split& p, int64_t w) {
    return w <= p.Wl ? w * p.F / p.Wl : p.F + (w - p.Wl) * (p.T - p.F) / (p.W - p.Wl);
}
// Wave whose range holds tile u.
__device__ __forceinline__ int64_t unit_owner(const Split& p, int64_t u) {
    return u < p.F ? ((u + 1) * p.Wl - 1) / p.F
                   : p.Wl + ((u - p.F + 1) * (p.W - p.Wl) - 1) / (p.T - p.F);
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
            nt = sl < a.num_seqs ? unit_tiles<PREFIX>(a, sl) : 0;
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
