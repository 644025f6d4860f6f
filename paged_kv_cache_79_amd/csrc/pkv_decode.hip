// Paged decode attention for gfx950.
//
// What is computed ("2.1 PagedAttention", sections 3 and 5): every query head
// of a sequence attends to the sequence's whole context, each logical position
// t being read at physical block block_table[t / block_size], slot
// t % block_size of the pool.  The pages' kernel sketch walks the blocks of
// one sequence with a 32-lane warp; here a 64-lane wave owns one
// (sequence, kv head, context partition) work item and consumes the context
// in tiles of 64 tokens:
//
//   1. load    every lane issues 16-byte loads in the pool's natural order, so
//              one wave instruction covers 1 KiB of contiguous K (or V) of one
//              block; the block id comes from a scalar (uniform) table read and
//              is folded into a scalar base address;
//   2. QK      K is restaged through LDS so that lane t owns token t of the
//              tile; it forms the dot products of all G query heads of its
//              group (grouped-query packing: one K read serves G heads) with
//              q held in scalar registers -- no cross-lane reduction;
//   3. softmax tile maximum by DPP row rotations + permlane swaps; running
//              max per head, per-lane running sums (summed once at the end);
//   4. PV      V stays in the load layout (lane = 8 elements of one token row);
//              bf16 probabilities of two tokens are paired with the matching
//              V halves (byte permute) and accumulated with v_dot2;
//   5. output  partial (max, sum, unnormalised o) per partition, or the final
//              row when a sequence fits one partition.
// A second kernel merges partitions by log-sum-exp.  Tokens at or beyond the
// valid length are removed by selection (score -inf, V row zero), never by
// arithmetic, so stale or NaN slots cannot leak into the result.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kTile = 64;

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

template <bool BF16, int D, int G>
__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeArgs a) {
    using S = DecodeShape<BF16, D>;
    __shared__ __attribute__((aligned(16))) char lds_k[kTile * S::KPITCH];
    __shared__ __attribute__((aligned(16))) uint32_t lds_p[kTile * 8];

    const int part = blockIdx.x;
    const int sh = blockIdx.y;
    const int s = sh / a.g.num_kv_heads;
    const int h = sh - s * a.g.num_kv_heads;
    const int lane = threadIdx.x;
    const int Hq = a.num_q_heads;
    const int bs = a.g.block_size;
    const int mb = a.max_blocks_per_seq;
    const int hq0 = h * G;

    int ctx = as_const(a.context_lens)[s];
    ctx = max(0, min(ctx, min(a.max_context_len, mb * bs)));
    const int t_begin = part * a.part_tokens;
    const bool single = a.num_parts == 1;

    if (t_begin >= ctx) {
        if (single) {  // empty context: zero rows
            if constexpr (BF16) {
                uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)s * Hq + hq0) * D;
                for (int e = lane; e < G * D; e += 64) o[e] = 0;
            } else {
                float* o = reinterpret_cast<float*>(a.out) + ((int64_t)s * Hq + hq0) * D;
                for (int e = lane; e < G * D; e += 64) o[e] = 0.f;
            }
        }
        return;
    }
    const int t_end = min(ctx, t_begin + a.part_tokens);
    const int nblk = (ctx + bs - 1) >> a.g.log2_bs;
    const int ra = lane / S::CPR;          // row inside a wave-wide load
    const int rc = lane - ra * S::CPR;     // 16-byte chunk inside the row
    const_ptr<int32_t> table = as_const(a.block_tables) + (int64_t)s * mb;
    const char* kb = a.k_pool + (int64_t)h * a.g.head_stride_bytes;
    const char* vb = a.v_pool + (int64_t)h * a.g.head_stride_bytes;
    const_ptr<uint32_t> qrow = as_const(reinterpret_cast<const uint32_t*>(
        reinterpret_cast<const char*>(a.q) + ((int64_t)s * Hq + hq0) * S::RB));

    float m[G], l[G], o[G][S::EPC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = kNoMax;
        l[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < S::EPC; ++e) o[hh][e] = 0.f;
    }

    for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
        // ---- 1. load K and V of the tile (natural layout) -------------------
        uint4 kreg[S::NL], vreg[S::NL];
#pragma unroll
        for (int i = 0; i < S::NL; ++i) {
            const int r0 = t0 + i * S::R;                  // uniform: first token of this load
            const int lb = min(r0 >> a.g.log2_bs, nblk - 1);
            int pb = table[lb];
            pb = ((unsigned)pb < (unsigned)a.g.num_blocks) ? pb : 0;
            const int64_t base = (int64_t)pb * a.g.block_stride_bytes;  // scalar
            const uint32_t off = (uint32_t)(((r0 & (bs - 1)) + ra) * S::RB + rc * 16);
            kreg[i] = *reinterpret_cast<const uint4*>((kb + base) + off);
            vreg[i] = *reinterpret_cast<const uint4*>((vb + base) + off);
        }
#pragma unroll
        for (int i = 0; i < S::NL; ++i)
            *reinterpret_cast<uint4*>(lds_k + (i * S::R + ra) * S::KPITCH + rc * 16) = kreg[i];
        if (t0 + kTile > t_end) {  // tail tile: rows past the valid length contribute nothing
#pragma unroll
            for (int i = 0; i < S::NL; ++i)
                if (t0 + i * S::R + ra >= t_end) vreg[i] = make_uint4(0, 0, 0, 0);
        }
        __syncthreads();

        // ---- 2. QK: lane = token ------------------------------------------
        float acc[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) acc[hh] = 0.f;
        const_ptr<uint32_t> qs = qrow;
        asm volatile("" : "+s"(qs));   // re-read q each tile (keeps it in SGPRs, not hoisted)
        const char* krow = lds_k + lane * S::KPITCH;
#pragma unroll
        for (int j = 0; j < S::CPR; ++j) {
            const uint4 kk = *reinterpret_cast<const uint4*>(krow + j * 16);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                const_ptr<uint32_t> qh = qs + hh * (S::RB / 4) + j * 4;
                if constexpr (BF16) {
                    acc[hh] = dot2_bf16(kk.x, qh[0], acc[hh]);
                    acc[hh] = dot2_bf16(kk.y, qh[1], acc[hh]);
                    acc[hh] = dot2_bf16(kk.z, qh[2], acc[hh]);
                    acc[hh] = dot2_bf16(kk.w, qh[3], acc[hh]);
                } else {
                    acc[hh] = fmaf(u2f(kk.x), u2f(qh[0]), acc[hh]);
                    acc[hh] = fmaf(u2f(kk.y), u2f(qh[1]), acc[hh]);
                    acc[hh] = fmaf(u2f(kk.z), u2f(qh[2]), acc[hh]);
                    acc[hh] = fmaf(u2f(kk.w), u2f(qh[3]), acc[hh]);
                }
            }
        }

        // ---- 3. online softmax --------------------------------------------
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
            if constexpr (BF16) {
                // pair slot of this token: rows i*R+a and (i^1)*R+a share one dword
                const int i = lane / S::R, ar = lane - (lane / S::R) * S::R;
                const int pidx = (i >> 1) * S::R + ar;
                reinterpret_cast<uint16_t*>(lds_p)[(pidx * 8 + hh) * 2 + (i & 1)] = f32_to_bf16(p);
            } else {
                reinterpret_cast<float*>(lds_p)[lane * 8 + hh] = p;
            }
        }
        __syncthreads();

        // ---- 4. PV --------------------------------------------------------
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < S::EPC; ++e) o[hh][e] *= alpha[hh];
        if constexpr (BF16) {
#pragma unroll
            for (int ii = 0; ii < S::NL / 2; ++ii) {
                const uint4 v0 = vreg[2 * ii], v1 = vreg[2 * ii + 1];
                const uint32_t* pp = lds_p + (ii * S::R + ra) * 8;
                const uint4 pa = *reinterpret_cast<const uint4*>(pp);
                const uint4 pz = *reinterpret_cast<const uint4*>(pp + 4);
                const uint32_t pk[8] = {pa.x, pa.y, pa.z, pa.w, pz.x, pz.y, pz.z, pz.w};
                const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};
                const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t lo = pair_lo(w0[w], w1[w]);
                    const uint32_t hi = pair_hi(w0[w], w1[w]);
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) {
                        o[hh][2 * w] = dot2_bf16(pk[hh], lo, o[hh][2 * w]);
                        o[hh][2 * w + 1] = dot2_bf16(pk[hh], hi, o[hh][2 * w + 1]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < S::NL; ++i) {
                const float* pr = reinterpret_cast<const float*>(lds_p) + (i * S::R + ra) * 8;
                const float4 pa = *reinterpret_cast<const float4*>(pr);
                const float4 pz = *reinterpret_cast<const float4*>(pr + 4);
                const float pv[8] = {pa.x, pa.y, pa.z, pa.w, pz.x, pz.y, pz.z, pz.w};
                const float v[4] = {u2f(vreg[i].x), u2f(vreg[i].y), u2f(vreg[i].z), u2f(vreg[i].w)};
#pragma unroll
                for (int hh = 0; hh < G; ++hh)
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[hh][e] = fmaf(pv[hh], v[e], o[hh][e]);
            }
        }
    }

    // ---- 5. combine lanes and write --------------------------------------
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        l[hh] = wave_sum(l[hh]);
#pragma unroll
        for (int e = 0; e < S::EPC; ++e) o[hh][e] = group_sum<S::R>(o[hh][e]);
    }
    if (single) {
        if (ra == 0) {
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                const float inv = l[hh] > 0.f ? 1.f / l[hh] : 0.f;
                const int64_t row = ((int64_t)s * Hq + hq0 + hh) * D + rc * S::EPC;
                if constexpr (BF16) {
                    uint4 w;
                    w.x = pack_bf16(o[hh][0] * inv, o[hh][1] * inv);
                    w.y = pack_bf16(o[hh][2] * inv, o[hh][3] * inv);
                    w.z = pack_bf16(o[hh][4] * inv, o[hh][5] * inv);
                    w.w = pack_bf16(o[hh][6] * inv, o[hh][7] * inv);
                    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + row) = w;
                } else {
                    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + row) =
                        make_float4(o[hh][0] * inv, o[hh][1] * inv, o[hh][2] * inv, o[hh][3] * inv);
                }
            }
        }
    } else {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const int64_t prow = ((int64_t)s * Hq + hq0 + hh) * a.num_parts + part;
            if (ra == 0) {
                float* dst = a.part_o + prow * D + rc * S::EPC;
#pragma unroll
                for (int e = 0; e < S::EPC; e += 4)
                    *reinterpret_cast<float4*>(dst + e) =
                        make_float4(o[hh][e], o[hh][e + 1], o[hh][e + 2], o[hh][e + 3]);
            }
            if (lane == 0)
                *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(m[hh], l[hh]);
        }
    }
}

// Log-sum-exp merge of the partitions of one (sequence, q head):
// with M the largest partition max, weight w_p = 2^(m_p - M);
// out = sum_p w_p o_p / sum_p w_p l_p.  One wave per output row.
template <bool BF16, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
    constexpr int PER = D / 64;
    const int row = blockIdx.x;
    const int s = row / a.num_q_heads;
    const int lane = threadIdx.x;
    int ctx = a.context_lens[s];
    ctx = max(0, min(ctx, min(a.max_context_len, a.max_blocks_per_seq * a.g.block_size)));
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

template <bool BF16, int D, int G>
static hipError_t launch_decode_t(const DecodeArgs& a, int num_seqs, hipStream_t st) {
    const dim3 grid(a.num_parts, num_seqs * a.g.num_kv_heads);
    hipLaunchKernelGGL((decode_partial_kernel<BF16, D, G>), grid, dim3(64), 0, st, a);
    if (a.num_parts > 1)
        hipLaunchKernelGGL((decode_merge_kernel<BF16, D>), dim3(num_seqs * a.num_q_heads), dim3(64),
                           0, st, a);
    return hipGetLastError();
}

template <bool BF16, int D>
static hipError_t launch_decode_g(const DecodeArgs& a, int group, int num_seqs, hipStream_t st) {
    switch (group) {
        case 1: return launch_decode_t<BF16, D, 1>(a, num_seqs, st);
        case 2: return launch_decode_t<BF16, D, 2>(a, num_seqs, st);
        case 3: return launch_decode_t<BF16, D, 3>(a, num_seqs, st);
        case 4: return launch_decode_t<BF16, D, 4>(a, num_seqs, st);
        case 5: return launch_decode_t<BF16, D, 5>(a, num_seqs, st);
        case 6: return launch_decode_t<BF16, D, 6>(a, num_seqs, st);
        case 7: return launch_decode_t<BF16, D, 7>(a, num_seqs, st);
        case 8: return launch_decode_t<BF16, D, 8>(a, num_seqs, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeArgs& a, bool is_bf16, int head_dim, int group, int num_seqs,
                         hipStream_t st) {
    if (num_seqs == 0) return hipSuccess;
    if (is_bf16) {
        if (head_dim == 128) return launch_decode_g<true, 128>(a, group, num_seqs, st);
        if (head_dim == 64) return launch_decode_g<true, 64>(a, group, num_seqs, st);
    } else {
        if (head_dim == 128) return launch_decode_g<false, 128>(a, group, num_seqs, st);
        if (head_dim == 64) return launch_decode_g<false, 64>(a, group, num_seqs, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
