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
// (chunk, kv head): row r = (query r / G, head r % G) of the G query heads
// that share the kv head, so every K/V tile is loaded once for all G heads.
// Per 64-key tile:
//   S^T = K Q^T       v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q rows
//                     held in registers; the C layout gives each lane one query
//                     row (column) and 16 keys per 32-key block, so the
//                     row-wise softmax is lane-local plus one permlane32 swap;
//   O^T += V^T P^T    A = V^T from LDS (stored transposed, keys in the order in
//                     which the C registers of S^T hold them), B = bf16 P^T
//                     straight from those registers.
// Keys past the context are zero in LDS and masked to -inf, so stale or NaN
// slots never reach the matrix cores.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kRowsPerWg = 128;   // packed (query, head) rows per workgroup
constexpr int kKeyTile = 64;      // keys per tile

template <int D>
struct PrefillShape {
    static constexpr int RB = D * 2;             // bytes of a K/V row (bf16)
    static constexpr int CPR = RB / 16;          // 16-byte chunks per row
    static constexpr int KPITCH = RB + 16;       // K tile row pitch in LDS (bytes)
    static constexpr int VPITCH = kKeyTile * 2 + 16;  // V^T row pitch in LDS (bytes)
    static constexpr int KSTEPS = D / 16;        // QK k-steps of 16
    static constexpr int DT = D / 32;            // 32-row output tiles
};

// Position of key k (0..63) inside the transposed V tile.  Within a group of 16
// keys, the C registers of a 32x32 MFMA hold key 8b+4h+j (b, h in {0,1}, j < 4) at
// B-operand slot 8h+4b+j of the next MFMA: bits 2 and 3 swap.  The map is its own
// inverse.
__device__ __forceinline__ int vt_slot(int k) {
    return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D, int G>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
    using P = PrefillShape<D>;
    constexpr int QP = kRowsPerWg / G;           // query positions per workgroup
    __shared__ __attribute__((aligned(16))) char lds_k[kKeyTile * P::KPITCH];
    __shared__ __attribute__((aligned(16))) char lds_vt[D * P::VPITCH];

    const int qt = blockIdx.x;
    const int h = blockIdx.y;
    const int c = blockIdx.z;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
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
    const int nblk = (ctx + bs - 1) >> a.g.log2_bs;
    const int32_t* table = a.block_tables + (int64_t)c * mb;
    const char* kb = a.k_pool + (int64_t)h * a.g.head_stride_bytes;
    const char* vb = a.v_pool + (int64_t)h * a.g.head_stride_bytes;

    // this lane's query row
    const int r = w * 32 + n;
    const int qi = r / G;
    const int hh = r - qi * G;
    const int qpos_local = qt * QP + qi;
    const bool row_valid = (r < QP * G) && (qpos_local < nq);
    const int pos = ctx - nq + qpos_local;       // causal limit (inclusive)
    const int64_t qidx = (int64_t)q0 + qpos_local;

    uint4 qreg[P::KSTEPS];
    {
        const char* qp = reinterpret_cast<const char*>(a.q) +
                         (qidx * Hq + (int64_t)h * G + hh) * P::RB + half * 16;
#pragma unroll
        for (int ks = 0; ks < P::KSTEPS; ++ks)
            qreg[ks] = row_valid ? *reinterpret_cast<const uint4*>(qp + ks * 32)
                                 : make_uint4(0, 0, 0, 0);
    }

    floatx16_t oacc[P::DT];
#pragma unroll
    for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
    float m = kNoMax, l = 0.f;

    // keys any row of this workgroup may see
    const int t_stop = ctx - nq + min(nq, (qt + 1) * QP);

    for (int t0 = 0; t0 < t_stop; t0 += kKeyTile) {
        // ---- K tile, natural row layout --------------------------------------
        {
            constexpr int RPI = 256 / P::CPR;    // rows per pass of the workgroup
            const int cr = tid % P::CPR;
#pragma unroll
            for (int i = 0; i < kKeyTile / RPI; ++i) {
                const int row = i * RPI + tid / P::CPR;
                const int tok = t0 + row;
                uint4 x = make_uint4(0, 0, 0, 0);
                if (tok < ctx) {
                    int pb = table[min(tok >> a.g.log2_bs, nblk - 1)];
                    pb = ((unsigned)pb < (unsigned)a.g.num_blocks) ? pb : 0;
                    x = *reinterpret_cast<const uint4*>(
                        kb + (int64_t)pb * a.g.block_stride_bytes +
                        (uint32_t)((tok & (bs - 1)) * P::RB + cr * 16));
                }
                *reinterpret_cast<uint4*>(lds_k + row * P::KPITCH + cr * 16) = x;
            }
        }
        // ---- V tile, transposed: lds_vt[d][slot(key)] -------------------------
        {
            const int kp = tid & 31;             // key pair 2kp, 2kp+1
            const int cg = tid >> 5;             // chunk group
#pragma unroll
            for (int j = 0; j < P::CPR / 8; ++j) {
                const int ch = cg + 8 * j;
                uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
                const int tk = t0 + 2 * kp;
                if (tk < ctx) {
                    int pb = table[min(tk >> a.g.log2_bs, nblk - 1)];
                    pb = ((unsigned)pb < (unsigned)a.g.num_blocks) ? pb : 0;
                    x0 = *reinterpret_cast<const uint4*>(
                        vb + (int64_t)pb * a.g.block_stride_bytes +
                        (uint32_t)((tk & (bs - 1)) * P::RB + ch * 16));
                }
                if (tk + 1 < ctx) {
                    int pb = table[min((tk + 1) >> a.g.log2_bs, nblk - 1)];
                    pb = ((unsigned)pb < (unsigned)a.g.num_blocks) ? pb : 0;
                    x1 = *reinterpret_cast<const uint4*>(
                        vb + (int64_t)pb * a.g.block_stride_bytes +
                        (uint32_t)(((tk + 1) & (bs - 1)) * P::RB + ch * 16));
                }
                const uint32_t a0[4] = {x0.x, x0.y, x0.z, x0.w};
                const uint32_t a1[4] = {x1.x, x1.y, x1.z, x1.w};
                const int col = vt_slot(2 * kp) * 2;   // byte offset in the row
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int d = ch * 8 + 2 * q;
                    *reinterpret_cast<uint32_t*>(lds_vt + d * P::VPITCH + col) = pair_lo(a0[q], a1[q]);
                    *reinterpret_cast<uint32_t*>(lds_vt + (d + 1) * P::VPITCH + col) = pair_hi(a0[q], a1[q]);
                }
            }
        }
        __syncthreads();

        // ---- S^T = K Q^T ----------------------------------------------------------
        floatx16_t sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[mt][e] = 0.f;
#pragma unroll
            for (int ks = 0; ks < P::KSTEPS; ++ks) {
                const uint4 ka = *reinterpret_cast<const uint4*>(
                    lds_k + (mt * 32 + n) * P::KPITCH + ks * 32 + half * 16);
                sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8_t, ka), __builtin_bit_cast(bf16x8_t, qreg[ks]),
                    sacc[mt], 0, 0, 0);
            }
        }

        // ---- online softmax over this row's 32 keys per lane -------------------
        float sc[2][16];
        float mloc = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = t0 + mt * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
                const bool vis = row_valid && key <= pos && key < ctx;
                sc[mt][e] = vis ? sacc[mt][e] * a.scale_log2 : -INFINITY;
                mloc = fmaxf(mloc, sc[mt][e]);
            }
        const float mn = fmaxf(m, swap32_max(mloc));
        const float alpha = fast_exp2(m - mn);
        m = mn;
        float psum = 0.f;
        uint4 pk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int mt = u >> 1, e0 = (u & 1) * 8;
            float p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                p[j] = fast_exp2(sc[mt][e0 + j] - mn);
                psum += p[j];
            }
            pk[u] = make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]),
                               pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7]));
        }
        l = l * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;

        // ---- O^T += V^T P^T ---------------------------------------------------------
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint4 va = *reinterpret_cast<const uint4*>(
                    lds_vt + (dt * 32 + n) * P::VPITCH + (u * 16 + half * 8) * 2);
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8_t, va), __builtin_bit_cast(bf16x8_t, pk[u]),
                    oacc[dt], 0, 0, 0);
            }
        __syncthreads();
    }

    // ---- normalise and store: lane holds d = 32dt + 8(e/4) + 4half + e%4 ----------
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
    const dim3 grid((max_q_len + QP - 1) / QP, a.g.num_kv_heads, num_chunks);
    hipLaunchKernelGGL((prefill_kernel<D, G>), grid, dim3(256), 0, st, a);
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
