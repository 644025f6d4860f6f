// Device-side check of the preconditions the release kernels trust.
//
// What is checked ("2.1 PagedAttention", section 3: token t of a sequence lives in
// block block_tables[s][t / block_size] at offset t % block_size, and a write puts
// token i at slot block * block_size + offset; section 6: copy-on-write copies whole
// blocks):
//   counts[0]  table entries a context reaches (j < min(ceil(ctx / bs), max_blocks))
//              that name no block of the pool;
//   counts[1]  sequences whose context is negative or longer than the table holds;
//   counts[2]  tokens whose slot lies past the pool or repeats an earlier token's slot
//              (negative slots are padding);
//   counts[3]  copy pairs with an id outside the pool, a destination written by an
//              earlier pair, or a destination that some pair reads.
// Each offending entry, sequence, token or pair is counted once.  Duplicates are
// found by comparing against every earlier element, 256 at a time through LDS.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kValidateThreads = 256;

__global__ __launch_bounds__(64) void validate_zero_kernel(int32_t* counts, int n) {
    if ((int)threadIdx.x < n) counts[threadIdx.x] = 0;
}

// Adds this thread's `bad` into counts[which], one global atomic per workgroup.
__device__ __forceinline__ void add_count(int bad, int32_t* counts, int which) {
    __shared__ int total;
    if (threadIdx.x == 0) total = 0;
    __syncthreads();
    if (bad) atomicAdd(&total, bad);
    __syncthreads();
    if (threadIdx.x == 0 && total) atomicAdd(counts + which, total);
}

// one workgroup per sequence
__global__ __launch_bounds__(kValidateThreads) void validate_tables_kernel(
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
    int32_t num_blocks, int32_t block_size, int32_t* counts) {
    const int s = blockIdx.x;
    const int c = context_lens[s];
    const int64_t cap = (int64_t)max_blocks * block_size;
    const int reach = (int)min(((int64_t)max(c, 0) + block_size - 1) / block_size,
                               (int64_t)max_blocks);
    int bad = 0;
    for (int j = threadIdx.x; j < reach; j += kValidateThreads)
        bad += (unsigned)block_tables[(int64_t)s * max_blocks + j] >= (unsigned)num_blocks;
    if (threadIdx.x == 0 && (c < 0 || (int64_t)c > cap)) atomicAdd(counts + 1, 1);
    add_count(bad, counts, 0);
}

// one thread per token: range, then every earlier token's slot
__global__ __launch_bounds__(kValidateThreads) void validate_slots_kernel(
    const int64_t* slots, int32_t n, int64_t num_slots, int32_t* counts) {
    __shared__ int64_t chunk[kValidateThreads];
    const int i = blockIdx.x * kValidateThreads + threadIdx.x;
    const int64_t x = i < n ? slots[i] : -1;
    bool bad = x >= num_slots;
    bool dup = false;
    const int end = min((int)(blockIdx.x + 1) * kValidateThreads, n);   // uniform
    for (int base = 0; base < end; base += kValidateThreads) {
        __syncthreads();
        const int j = base + threadIdx.x;
        chunk[threadIdx.x] = j < n ? slots[j] : -1;
        __syncthreads();
        const int lim = min(kValidateThreads, i - base);   // earlier tokens only
        for (int k = 0; k < lim; ++k) dup |= chunk[k] == x;
    }
    bad |= x >= 0 && dup;
    add_count(bad ? 1 : 0, counts, 2);
}

// one thread per pair: ids, earlier destinations, every source
__global__ __launch_bounds__(kValidateThreads) void validate_pairs_kernel(
    const int64_t* mapping, int32_t n, int32_t num_blocks, int32_t* counts) {
    __shared__ int64_t src_chunk[kValidateThreads], dst_chunk[kValidateThreads];
    const int k = blockIdx.x * kValidateThreads + threadIdx.x;
    const int64_t src = k < n ? mapping[2 * (int64_t)k] : 0;
    const int64_t dst = k < n ? mapping[2 * (int64_t)k + 1] : 0;
    bool bad = k < n && (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks);
    for (int base = 0; base < n; base += kValidateThreads) {
        __syncthreads();
        const int j = base + threadIdx.x;
        src_chunk[threadIdx.x] = j < n ? mapping[2 * (int64_t)j] : -1;
        dst_chunk[threadIdx.x] = j < n ? mapping[2 * (int64_t)j + 1] : -1;
        __syncthreads();
        const int cnt = min(kValidateThreads, n - base);
        for (int q = 0; q < cnt; ++q) {
            bad |= k < n && src_chunk[q] == dst;                  // a destination that is read
            bad |= k < n && base + q < k && dst_chunk[q] == dst;  // written twice
        }
    }
    add_count(bad ? 1 : 0, counts, 3);
}

// one thread per chunk: cu_q_lens[0] must be 0, each chunk's queries must not run
// backwards, outnumber its context or end past total_q rows (total_q < 0: unknown)
__global__ __launch_bounds__(kValidateThreads) void validate_chunks_kernel(
    const int32_t* cu_q_lens, const int32_t* context_lens, int32_t num_chunks, int32_t total_q,
    int32_t* count) {
    const int c = blockIdx.x * kValidateThreads + threadIdx.x;
    int bad = 0;
    if (c < num_chunks) {
        const int q0 = cu_q_lens[c], q1 = cu_q_lens[c + 1], ctx = context_lens[c];
        bad = (c == 0 && q0 != 0) || q1 < q0 || ctx < 0 || q1 - q0 > ctx ||
              (total_q >= 0 && q1 > total_q);
    }
    add_count(bad, count, 0);
}

hipError_t launch_validate_chunks(const int32_t* cu_q_lens, const int32_t* context_lens,
                                  int32_t num_chunks, int32_t total_q, int32_t* count,
                                  hipStream_t st) {
    hipLaunchKernelGGL(validate_zero_kernel, dim3(1), dim3(64), 0, st, count, 1);
    hipLaunchKernelGGL(validate_chunks_kernel,
                       dim3((num_chunks + kValidateThreads - 1) / kValidateThreads),
                       dim3(kValidateThreads), 0, st, cu_q_lens, context_lens, num_chunks, total_q,
                       count);
    return hipGetLastError();
}

hipError_t launch_validate(const ValidateArgs& v, hipStream_t st) {
    hipLaunchKernelGGL(validate_zero_kernel, dim3(1), dim3(64), 0, st, v.counts, 4);
    if (v.num_seqs > 0)
        hipLaunchKernelGGL(validate_tables_kernel, dim3(v.num_seqs), dim3(kValidateThreads), 0, st,
                           v.block_tables, v.max_blocks_per_seq, v.context_lens, v.num_blocks,
                           v.block_size, v.counts);
    if (v.num_tokens > 0)
        hipLaunchKernelGGL(validate_slots_kernel,
                           dim3((v.num_tokens + kValidateThreads - 1) / kValidateThreads),
                           dim3(kValidateThreads), 0, st, v.slot_mapping, v.num_tokens,
                           (int64_t)v.num_blocks * v.block_size, v.counts);
    if (v.num_pairs > 0)
        hipLaunchKernelGGL(validate_pairs_kernel,
                           dim3((v.num_pairs + kValidateThreads - 1) / kValidateThreads),
                           dim3(kValidateThreads), 0, st, v.block_mapping, v.num_pairs,
                           v.num_blocks, v.counts);
    return hipGetLastError();
}

}  // namespace pkv
