// Streaming-read ceiling of the device, for the benchmark only (libpkvbench.so, not
// part of libpagedkv's interface): the rate at which plain contiguous 16-byte reads
// of a buffer far larger than the 256 MB Infinity Cache come back from HBM.  Decode's
// bandwidth is reported against this as well as against the 8 TB/s peak.
//
// Every wave reads one contiguous range in runs of 16 KiB (16 nontemporal 16-byte
// loads in flight per lane, the pattern decode's tiles use) and folds what it read
// into one word per lane, stored to `sink` so that no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kLoads = 16;          // loads in flight per lane
constexpr int kRun = 64 * kLoads;   // 16-byte elements per wave-wide run (16 KiB)

__global__ __launch_bounds__(64) void read_ceiling_kernel(const u32x4* buf, int64_t n16,
                                                          int64_t per_wave, uint32_t* sink) {
    const int lane = threadIdx.x;
    const int64_t b = (int64_t)blockIdx.x * per_wave;
    const int64_t e = b + per_wave < n16 ? b + per_wave : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = b; i < e; i += kRun) {
        u32x4 r[kLoads];
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            int64_t idx = i + j * 64 + lane;
            idx = idx < e ? idx : e - 1;            // the last run re-reads its end
            r[j] = __builtin_nontemporal_load(buf + idx);
        }
#pragma unroll
        for (int j = 0; j < kLoads; ++j) acc ^= r[j];
    }
    sink[(int64_t)blockIdx.x * 64 + lane] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) of device memory `buf` with `waves` single-wave
// workgroups; `sink` is device memory of waves * 64 words.  Returns 0, or -1 for bad
// arguments, or the HIP error of the launch.
int pkv_bench_read(const void* buf, size_t bytes, uint32_t* sink, int32_t waves,
                   hipStream_t stream) {
    if (!buf || !sink || waves <= 0 || bytes < 16 || bytes % 16) return -1;
    const int64_t n16 = (int64_t)(bytes / 16);
    int64_t per_wave = (n16 + waves - 1) / waves;
    per_wave = (per_wave + kRun - 1) / kRun * kRun;
    const int64_t grid = (n16 + per_wave - 1) / per_wave;
    hipLaunchKernelGGL(read_ceiling_kernel, dim3((uint32_t)grid), dim3(64), 0, stream,
                       static_cast<const u32x4*>(buf), n16, per_wave, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
