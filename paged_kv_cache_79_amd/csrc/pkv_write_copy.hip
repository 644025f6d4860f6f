// Slot-mapped cache write and copy-on-write block copy.
//
// Cache write ("2.1 PagedAttention", section 3): the new token of a request
// fills the next free slot of its current block; the scheduler names that
// slot as physical_block * block_size + offset.  One lane moves one 16-byte
// chunk of one (token, kv head) row, so a wave stores 1 KiB of contiguous
// pool memory per instruction for block_size * head_dim * elem >= 1 KiB.
//
// Block copy ("2.1 PagedAttention", section 6, copy-on-write): a shared block
// about to be written is duplicated into a private block.  One workgroup
// copies the K (or V) block of one (src, dst) pair with 16-byte loads/stores.
#include "pkv_internal.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_write_kernel(WriteArgs a) {
    const int cpr = a.g.row_bytes >> 4;
    const int per_tok = a.g.num_kv_heads * cpr;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)a.num_tokens * per_tok) return;
    const int tok = (int)(idx / per_tok);
    const int rem = (int)(idx - (int64_t)tok * per_tok);
    const int h = rem / cpr;
    const int c = rem - h * cpr;
    const int64_t slot = a.slot_mapping[tok];
    if (slot < 0) return;
    const int64_t pb = slot >> a.g.log2_bs;
    if (pb >= a.g.num_blocks) return;  // out-of-range slot: skipped, never dereferenced
    const int off = (int)(slot & (a.g.block_size - 1));
    const int64_t dst = pb * a.g.block_stride_bytes + (int64_t)h * a.g.head_stride_bytes +
                        (int64_t)off * a.g.row_bytes + c * 16;
    const int64_t src = ((int64_t)tok * a.g.num_kv_heads + h) * a.g.row_bytes + c * 16;
    const uint4 kv = *reinterpret_cast<const uint4*>(a.k_new + src);
    const uint4 vv = *reinterpret_cast<const uint4*>(a.v_new + src);
    *reinterpret_cast<uint4*>(a.k_pool + dst) = kv;
    *reinterpret_cast<uint4*>(a.v_pool + dst) = vv;
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
    const int p = blockIdx.x;
    const int64_t src = a.block_mapping[2 * p];
    const int64_t dst = a.block_mapping[2 * p + 1];
    if ((uint64_t)src >= (uint64_t)a.g.num_blocks || (uint64_t)dst >= (uint64_t)a.g.num_blocks)
        return;
    char* pool = blockIdx.y ? a.v_pool : a.k_pool;
    const uint4* s = reinterpret_cast<const uint4*>(pool + src * a.g.block_stride_bytes);
    uint4* d = reinterpret_cast<uint4*>(pool + dst * a.g.block_stride_bytes);
    const int n16 = (int)(a.g.block_stride_bytes >> 4);
    int i = threadIdx.x;
    // four 16-byte chunks in flight per lane
    for (; i + 3 * 256 < n16; i += 4 * 256) {
        const uint4 x0 = s[i], x1 = s[i + 256], x2 = s[i + 512], x3 = s[i + 768];
        d[i] = x0;
        d[i + 256] = x1;
        d[i + 512] = x2;
        d[i + 768] = x3;
    }
    for (; i < n16; i += 256) d[i] = s[i];
}

// One workgroup per (pair, K or V): a whole block between two pools, either of which
// may be pinned host memory seen through its device mapping (PCIe / xGMI traffic).
__global__ __launch_bounds__(256) void swap_kernel(SwapArgs a) {
    const int p = blockIdx.x;
    const int64_t src = a.src[p], dst = a.dst[p];
    const char* sp = (blockIdx.y ? a.src_v : a.src_k) + src * a.block_bytes;
    char* dp = (blockIdx.y ? a.dst_v : a.dst_k) + dst * a.block_bytes;
    const uint4* s = reinterpret_cast<const uint4*>(sp);
    uint4* d = reinterpret_cast<uint4*>(dp);
    const int n16 = (int)(a.block_bytes >> 4);
    int i = threadIdx.x;
    for (; i + 3 * 256 < n16; i += 4 * 256) {
        const uint4 x0 = s[i], x1 = s[i + 256], x2 = s[i + 512], x3 = s[i + 768];
        d[i] = x0;
        d[i + 256] = x1;
        d[i + 512] = x2;
        d[i + 768] = x3;
    }
    for (; i < n16; i += 256) d[i] = s[i];
}

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t st) {
    const int64_t work = (int64_t)a.num_tokens * a.g.num_kv_heads * (a.g.row_bytes >> 4);
    if (work == 0) return hipSuccess;
    const unsigned grid = (unsigned)((work + 255) / 256);
    hipLaunchKernelGGL(kv_write_kernel, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t st) {
    if (a.num_pairs == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.num_pairs, 2), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_swap(const SwapArgs& a, hipStream_t st) {
    if (a.num_pairs <= 0) return hipSuccess;
    hipLaunchKernelGGL(swap_kernel, dim3(a.num_pairs, 2), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace pkv
