// C ABI of libpagedkv: argument validation, geometry, partition choice, launches.
// Every entry point validates what the host can see before enqueuing anything,
// never allocates, and never synchronises.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "pagedkv.h"
#include "pkv_internal.h"

using namespace pkv;

namespace {

int elem_bytes(pkv_dtype dt) { return dt == PKV_BF16 ? 2 : 4; }

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

// Shared checks of the pool geometry.  The matrix-core kernels need a (block, kv
// head) run to span at least one wave-wide 16-byte load (64 lanes x 16 B = 1 KiB) so
// that every such load stays inside one block (small_runs = false); the cache write,
// the block copy and the decode also take shorter runs.
pkv_status check_geom(pkv_dtype dt, int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                      int32_t head_dim, PoolGeom* g, bool small_runs = true) {
    if (dt != PKV_F32 && dt != PKV_BF16) return PKV_ERR_DTYPE;
    if (num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 || head_dim <= 0)
        return PKV_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (!pow2(block_size) || block_size < 4 || block_size > 32) return PKV_ERR_UNSUPPORTED;
    const int eb = elem_bytes(dt);
    if (!small_runs && block_size * head_dim * eb < 1024) return PKV_ERR_UNSUPPORTED;
    // slots are int64, block offsets int64; a single (block, head) run is < 2^31 bytes
    g->row_bytes = head_dim * eb;
    g->head_stride_bytes = block_size * head_dim * eb;
    g->block_stride_bytes = (int64_t)num_kv_heads * g->head_stride_bytes;
    // kernels form block offsets as 32 x 32 -> 64-bit products
    if (g->block_stride_bytes >= ((int64_t)1 << 31)) return PKV_ERR_UNSUPPORTED;
    g->num_blocks = num_blocks;
    g->num_kv_heads = num_kv_heads;
    g->block_size = block_size;
    g->log2_bs = ilog2(block_size);
    return PKV_OK;
}

pkv_status launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH; }

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// a * b for non-negative a, b, or limit + 1 when the product exceeds limit (no overflow)
int64_t product_exceeds(int64_t a, int64_t b, int64_t limit) {
    if (a > 0 && b > limit / a) return limit + 1;
    return a * b;
}

int32_t num_partitions(int32_t max_context_len, int32_t pt) {
    return max_context_len <= 0 ? 1 : (int32_t)cdiv64(max_context_len, pt);
}

// Upper bound of the persistent waves of the balanced split on the current device:
// 8 single-wave workgroups per CU (the register and LDS budget of the bf16 kernels;
// the fp32 ones keep fewer resident).
int64_t balanced_wave_bound() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return (int64_t)cus * 8;
}

// The balanced split's record of each (sequence, kv head) unit for the merge: the wave
// holding its first tile and the number of waves it spans.
size_t unit_desc_bytes(int32_t num_seqs, int32_t num_kv_heads) {
    return (size_t)num_seqs * num_kv_heads * 2 * sizeof(int32_t);
}

size_t decode_workspace(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t max_context_len, int32_t partition_tokens) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        num_q_heads % num_kv_heads)
        return 0;
    if (partition_tokens > 0) {
        const int32_t np = num_partitions(max_context_len, partition_tokens);
        if (np <= 1) return 0;
        return (size_t)num_seqs * num_q_heads * np * (size_t)(head_dim + 2) * sizeof(float);
    }
    const int64_t group = num_q_heads / num_kv_heads;
    return (size_t)balanced_wave_bound() * 2 * group * (size_t)(head_dim + 2) * sizeof(float) +
           unit_desc_bytes(num_seqs, num_kv_heads);
}

// Shared-prefix pass: the prefix keys are cut into at most kMaxPreSplits splits of a
// multiple of 64 tokens (chosen from the host bound alone, so both the workspace size
// and the launch agree on it).
int32_t prefix_split_tokens(int32_t max_prefix_len) {
    const int64_t per = cdiv64(std::max(max_prefix_len, 1), kMaxPreSplits);
    return (int32_t)std::max<int64_t>(64, cdiv64(per, 64) * 64);
}
int32_t prefix_splits(int32_t max_prefix_len) {
    return max_prefix_len <= 0 ? 0
                               : (int32_t)cdiv64(max_prefix_len, prefix_split_tokens(max_prefix_len));
}
size_t prefix_state_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                          int32_t max_prefix_len) {
    // one slot per split, plus the decode's own-token state of the row
    const int32_t ns = prefix_splits(max_prefix_len);
    if (ns == 0) return 0;
    return (size_t)num_seqs * num_q_heads * (ns + 1) * (size_t)(head_dim + 2) * sizeof(float);
}

// Balanced split over the resident waves (`resident`, from the kernel's occupancy):
// grid size, lead share and the partial-state layout in the workspace.
pkv_status setup_balanced(DecodeArgs& a, int64_t resident, int32_t num_seqs, int32_t num_kv_heads,
                          int32_t head_dim, int32_t max_context_len, int group, void* workspace) {
    // one wave per resident slot, but no more than there are tiles to share out
    const int64_t tiles_bound = (int64_t)num_seqs * num_kv_heads * cdiv64(max_context_len, 64);
    if (resident <= 0) return PKV_ERR_LAUNCH;
    int64_t waves = std::min(resident, balanced_wave_bound());
    // two waves per SIMD (the bf16 kernels fill every slot): lead waves get more tiles
    a.lead_share_q10 = waves == balanced_wave_bound() ? kLeadShareQ10 : 512;
    waves = std::max<int64_t>(1, std::min(waves, tiles_bound));
    a.num_waves = (int32_t)waves;
    a.part_o = static_cast<float*>(workspace);
    a.part_ml = a.part_o + (size_t)waves * 2 * group * head_dim;
    a.unit_desc = reinterpret_cast<int32_t*>(a.part_ml + (size_t)waves * 2 * group * 2);
    return PKV_OK;
}

// Scratch of paged_attention_decode_noalloc: one copy per device, kept for the
// process's lifetime.  Host code never uses the array's name as an address (on the
// host it is only a stand-in for the symbol); the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kNoallocScratchBytes = (size_t)20 << 20;
__device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// Device address of the current device's scratch, or nullptr if it cannot be had.
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

// Whether the matrix-core kernels serve this pool: bf16 with block runs of at least one
// wave-wide load (1 KiB).
bool mfma_geometry(pkv_dtype dt, int32_t block_size, int32_t head_dim) {
    return dt == PKV_BF16 && block_size * head_dim * 2 >= 1024;
}

// Causal query chunks on the vector units (fp32, or shapes no matrix-core kernel serves):
// one wave per (query slot, kv head), each streaming the keys its query sees with the
// decode's arithmetic.  cu_q_lens == nullptr: chunk c's queries are rows c * q_per_chunk..
pkv_status launch_chunked(pkv_dtype dtype, void* out, const void* q, const int32_t* cu_q_lens,
                          int32_t num_chunks, int32_t q_per_chunk, int32_t num_q_rows,
                          const void* k_pool, const void* v_pool, const PoolGeom& g,
                          int32_t head_dim, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t max_context_len, int32_t num_q_heads, float scale,
                          hipStream_t stream) {
    const int64_t units = (int64_t)num_chunks * q_per_chunk;
    if (product_exceeds(units, g.num_kv_heads, (int64_t)1 << 30) > ((int64_t)1 << 30) ||
        product_exceeds(units, num_q_heads, (int64_t)1 << 30) > ((int64_t)1 << 30))
        return PKV_ERR_UNSUPPORTED;
    DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_pool = static_cast<const char*>(k_pool);
    a.v_pool = static_cast<const char*>(v_pool);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.g = g;
    a.num_seqs = num_chunks;
    a.num_q_heads = num_q_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.part_tokens = std::max(max_context_len, 1);   // one partition: rows are written directly
    a.num_parts = 1;
    a.cu_q_lens = cu_q_lens;
    a.q_per_chunk = q_per_chunk;
    a.num_q_rows = num_q_rows;
    return launch_status(launch_decode_chunked(a, dtype == PKV_BF16, head_dim,
                                               num_q_heads / g.num_kv_heads, units, stream));
}

}  // namespace

extern "C" {

const char* pkv_status_string(pkv_status s) {
    switch (s) {
        case PKV_OK: return "PKV_OK";
        case PKV_ERR_NULL: return "PKV_ERR_NULL: a required pointer is NULL";
        case PKV_ERR_SHAPE: return "PKV_ERR_SHAPE: invalid or inconsistent size";
        case PKV_ERR_DTYPE: return "PKV_ERR_DTYPE: unknown element type";
        case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED: configuration not implemented";
        case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE: workspace missing or too small";
        case PKV_ERR_LAUNCH: return "PKV_ERR_LAUNCH: kernel launch or copy failed";
        case PKV_ERR_NO_BLOCKS: return "PKV_ERR_NO_BLOCKS: not enough free blocks in the pool";
        case PKV_ERR_VALIDATION: return "PKV_ERR_VALIDATION: device contents violate a precondition";
        default: break;
    }
    return "PKV_ERR_UNKNOWN";
}

pkv_status paged_kv_write(pkv_dtype dtype, void* k_pool, void* v_pool, int32_t num_blocks,
                          int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                          const void* k_new, const void* v_new, const int64_t* slot_mapping,
                          int32_t num_tokens, hipStream_t stream) {
    PoolGeom g;
    const pkv_status st = check_geom(dtype, num_blocks, num_kv_heads, block_size, head_dim, &g);
    if (st != PKV_OK) return st;
    if (num_tokens < 0) return PKV_ERR_SHAPE;
    if (num_tokens == 0) return PKV_OK;
    if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return PKV_ERR_NULL;
    WriteArgs a;
    a.k_pool = static_cast<char*>(k_pool);
    a.v_pool = static_cast<char*>(v_pool);
    a.k_new = static_cast<const char*>(k_new);
    a.v_new = static_cast<const char*>(v_new);
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.g = g;
    return launch_status(launch_kv_write(a, stream));
}

pkv_status copy_blocks(pkv_dtype dtype, void* k_pool, void* v_pool, int32_t num_blocks,
                       int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                       const int64_t* block_mapping, int32_t num_pairs, hipStream_t stream) {
    PoolGeom g;
    const pkv_status st = check_geom(dtype, num_blocks, num_kv_heads, block_size, head_dim, &g);
    if (st != PKV_OK) return st;
    if (num_pairs < 0) return PKV_ERR_SHAPE;
    if (num_pairs == 0) return PKV_OK;
    if (!k_pool || !v_pool || !block_mapping) return PKV_ERR_NULL;
    CopyArgs a;
    a.k_pool = static_cast<char*>(k_pool);
    a.v_pool = static_cast<char*>(v_pool);
    a.block_mapping = block_mapping;
    a.num_pairs = num_pairs;
    a.g = g;
    return launch_status(launch_copy_blocks(a, stream));
}

pkv_status pkv_validate(int32_t num_blocks, int32_t block_size, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                        const int64_t* slot_mapping, int32_t num_tokens,
                        const int64_t* block_mapping, int32_t num_pairs, int32_t* counts,
                        hipStream_t stream) {
    if (num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq < 0 || num_seqs < 0 ||
        num_tokens < 0 || num_pairs < 0)
        return PKV_ERR_SHAPE;
    if (!counts) return PKV_ERR_NULL;
    if (num_seqs > 0 && (!block_tables || !context_lens)) return PKV_ERR_NULL;
    if (num_tokens > 0 && !slot_mapping) return PKV_ERR_NULL;
    if (num_pairs > 0 && !block_mapping) return PKV_ERR_NULL;
    ValidateArgs v;
    v.block_tables = block_tables;
    v.context_lens = context_lens;
    v.slot_mapping = slot_mapping;
    v.block_mapping = block_mapping;
    v.counts = counts;
    v.num_blocks = num_blocks;
    v.block_size = block_size;
    v.max_blocks_per_seq = max_blocks_per_seq;
    v.num_seqs = num_seqs;
    v.num_tokens = num_tokens;
    v.num_pairs = num_pairs;
    return launch_status(launch_validate(v, stream));
}

pkv_status pkv_validate_chunks(const int32_t* cu_q_lens, const int32_t* context_lens,
                               int32_t num_chunks, int32_t total_q, int32_t* count,
                               hipStream_t stream) {
    if (num_chunks < 0) return PKV_ERR_SHAPE;
    if (!count) return PKV_ERR_NULL;
    if (num_chunks > 0 && (!cu_q_lens || !context_lens)) return PKV_ERR_NULL;
    if (num_chunks == 0) return PKV_OK;
    return launch_status(
        launch_validate_chunks(cu_q_lens, context_lens, num_chunks, total_q, count, stream));
}

size_t paged_attention_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t max_context_len, int32_t partition_tokens) {
    return decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                            partition_tokens);
}

pkv_status swap_blocks(pkv_dtype dtype, void* dst_k, void* dst_v, int32_t dst_num_blocks,
                       const void* src_k, const void* src_v, int32_t src_num_blocks,
                       int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                       const int64_t* block_mapping, int32_t num_pairs, hipStream_t stream) {
    PoolGeom g;
    const int32_t nb = std::max(dst_num_blocks, src_num_blocks);
    const pkv_status st = check_geom(dtype, nb, num_kv_heads, block_size, head_dim, &g);
    if (st != PKV_OK) return st;
    if (dst_num_blocks <= 0 || src_num_blocks <= 0 || num_pairs < 0) return PKV_ERR_SHAPE;
    if (num_pairs == 0) return PKV_OK;
    if (!dst_k || !dst_v || !src_k || !src_v || !block_mapping) return PKV_ERR_NULL;
    for (int32_t i = 0; i < num_pairs; ++i) {
        const int64_t s = block_mapping[2 * i], d = block_mapping[2 * i + 1];
        if (s < 0 || s >= src_num_blocks || d < 0 || d >= dst_num_blocks) return PKV_ERR_SHAPE;
    }
    const size_t blk = (size_t)g.block_stride_bytes;
    // runs of pairs whose sources and destinations both advance by one block
    int32_t runs = 0;
    for (int32_t i = 0; i < num_pairs; ++i)
        if (i == 0 || block_mapping[2 * i] != block_mapping[2 * i - 2] + 1 ||
            block_mapping[2 * i + 1] != block_mapping[2 * i - 1] + 1)
            ++runs;
    // Scattered blocks: one copy kernel over device pointers, if every pool is device
    // memory or pinned host memory with a device mapping (a DMA copy per block costs
    // ~10 us of engine overhead).  Long runs: DMA copies.
    void* dev_ptr[4] = {dst_k, dst_v, const_cast<void*>(src_k), const_cast<void*>(src_v)};
    bool kernel_ok = runs * 4 > num_pairs;
    for (int i = 0; i < 4 && kernel_ok; ++i) {
        hipPointerAttribute_t at;
        if (hipPointerGetAttributes(&at, dev_ptr[i]) != hipSuccess) {
            (void)hipGetLastError();
            kernel_ok = false;
            break;
        }
        if (at.type == hipMemoryTypeHost) {
            void* d = nullptr;
            if (hipHostGetDevicePointer(&d, dev_ptr[i], 0) != hipSuccess || !d) {
                (void)hipGetLastError();
                kernel_ok = false;
                break;
            }
            dev_ptr[i] = d;
        } else if (at.type != hipMemoryTypeDevice) {
            kernel_ok = false;
        }
    }
    if (kernel_ok) {
        SwapArgs a;
        a.dst_k = static_cast<char*>(dev_ptr[0]);
        a.dst_v = static_cast<char*>(dev_ptr[1]);
        a.src_k = static_cast<const char*>(dev_ptr[2]);
        a.src_v = static_cast<const char*>(dev_ptr[3]);
        a.block_bytes = (int64_t)blk;
        for (int32_t i0 = 0; i0 < num_pairs; i0 += kSwapPairsPerLaunch) {
            a.num_pairs = std::min(kSwapPairsPerLaunch, num_pairs - i0);
            for (int32_t k = 0; k < a.num_pairs; ++k) {
                a.src[k] = (int32_t)block_mapping[2 * (i0 + k)];
                a.dst[k] = (int32_t)block_mapping[2 * (i0 + k) + 1];
            }
            if (launch_swap(a, stream) != hipSuccess) return PKV_ERR_LAUNCH;
        }
        return PKV_OK;
    }
    for (int32_t i = 0; i < num_pairs;) {
        int32_t j = i + 1;
        while (j < num_pairs && block_mapping[2 * j] == block_mapping[2 * j - 2] + 1 &&
               block_mapping[2 * j + 1] == block_mapping[2 * j - 1] + 1)
            ++j;
        const size_t off_s = (size_t)block_mapping[2 * i] * blk;
        const size_t off_d = (size_t)block_mapping[2 * i + 1] * blk;
        const size_t bytes = (size_t)(j - i) * blk;
        if (hipMemcpyAsync(static_cast<char*>(dst_k) + off_d,
                           static_cast<const char*>(src_k) + off_s, bytes, hipMemcpyDefault,
                           stream) != hipSuccess ||
            hipMemcpyAsync(static_cast<char*>(dst_v) + off_d,
                           static_cast<const char*>(src_v) + off_s, bytes, hipMemcpyDefault,
                           stream) != hipSuccess)
            return PKV_ERR_LAUNCH;
        i = j;
    }
    return PKV_OK;
}

pkv_status paged_attention_decode(pkv_dtype dtype, void* out, const void* q, const void* k_pool,
                                  const void* v_pool, int32_t num_blocks, int32_t num_kv_heads,
                                  int32_t block_size, int32_t head_dim,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t max_context_len, int32_t num_q_heads, float scale,
                                  int32_t partition_tokens, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    PoolGeom g;
    const pkv_status st = check_geom(dtype, num_blocks, num_kv_heads, block_size, head_dim, &g);
    if (st != PKV_OK) return st;
    if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq <= 0 || num_q_heads <= 0)
        return PKV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads) return PKV_ERR_SHAPE;
    const int group = num_q_heads / num_kv_heads;
    if (group > 8) return PKV_ERR_UNSUPPORTED;
    if (partition_tokens < 0 || (partition_tokens % block_size) != 0) return PKV_ERR_SHAPE;
    if (!isfinite(scale)) return PKV_ERR_SHAPE;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PKV_ERR_NULL;
    // output rows and (sequence, kv head) units are counted in 32-bit integers
    if ((int64_t)num_seqs * num_q_heads > ((int64_t)1 << 30)) return PKV_ERR_UNSUPPORTED;
    // fixed partitions: one grid row per partition (grid.y)
    if (partition_tokens > 0 && num_partitions(max_context_len, partition_tokens) > 65535)
        return PKV_ERR_UNSUPPORTED;

    const size_t need = decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                         max_context_len, partition_tokens);
    if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;

    DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_pool = static_cast<const char*>(k_pool);
    a.v_pool = static_cast<const char*>(v_pool);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.g = g;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.part_tokens = partition_tokens;
    a.num_parts = 1;
    a.num_waves = 0;
    a.lead_share_q10 = 512;
    a.contig_seq_stride = 0;
    a.contig_row_stride = 0;
    a.seq_prefix = nullptr;
    a.pre_o = a.pre_ml = nullptr;
    a.pre_splits = 0;
    a.pre_split_tokens = 64;
    a.part_o = static_cast<float*>(workspace);
    a.part_ml = nullptr;
    a.unit_desc = nullptr;
    if (partition_tokens > 0) {
        a.num_parts = num_partitions(max_context_len, partition_tokens);
        if (a.num_parts > 1)
            a.part_ml = a.part_o + (size_t)num_seqs * num_q_heads * a.num_parts * head_dim;
    } else {
        const pkv_status sb =
            setup_balanced(a, decode_balanced_waves(dtype == PKV_BF16, head_dim, group), num_seqs,
                           num_kv_heads, head_dim, max_context_len, group, workspace);
        if (sb != PKV_OK) return sb;
    }
    return launch_status(launch_decode(a, dtype == PKV_BF16, head_dim, group, num_seqs, stream));
}

size_t paged_attention_decode_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

pkv_status paged_attention_decode_noalloc(pkv_dtype dtype, void* out, const void* q,
                                          const void* k_pool, const void* v_pool,
                                          int32_t num_blocks, int32_t num_kv_heads,
                                          int32_t block_size, int32_t head_dim,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t max_context_len, int32_t num_q_heads, float scale,
                                          int32_t partition_tokens, hipStream_t stream) {
    const size_t need = decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                         max_context_len, partition_tokens);
    if (need > kNoallocScratchBytes) {
        // more than the fixed scratch holds: run the usual argument checks with no
        // workspace; they end in PKV_ERR_WORKSPACE at the latest, and nothing is launched
        return paged_attention_decode(dtype, out, q, k_pool, v_pool, num_blocks, num_kv_heads,
                                      block_size, head_dim, block_tables, max_blocks_per_seq,
                                      context_lens, num_seqs, max_context_len, num_q_heads, scale,
                                      partition_tokens, nullptr, 0, stream);
    }
    void* ws = need > 0 ? scratch_ptr() : nullptr;
    if (need > 0 && ws == nullptr) {
        // no device address for the scratch: argument errors still come first
        const pkv_status s = paged_attention_decode(
            dtype, out, q, k_pool, v_pool, num_blocks, num_kv_heads, block_size, head_dim,
            block_tables, max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_q_heads,
            scale, partition_tokens, nullptr, 0, stream);
        return s == PKV_ERR_WORKSPACE ? PKV_ERR_LAUNCH : s;
    }
    return paged_attention_decode(dtype, out, q, k_pool, v_pool, num_blocks, num_kv_heads,
                                  block_size, head_dim, block_tables, max_blocks_per_seq,
                                  context_lens, num_seqs, max_context_len, num_q_heads, scale,
                                  partition_tokens, ws, ws ? kNoallocScratchBytes : 0, stream);
}

pkv_status contiguous_attention_decode(pkv_dtype dtype, void* out, const void* q,
                                       const void* k_cache, const void* v_cache, int32_t num_seqs,
                                       int32_t max_len, int32_t num_kv_heads, int32_t head_dim,
                                       const int32_t* context_lens, int32_t max_context_len,
                                       int32_t num_q_heads, float scale, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_DTYPE;
    if (num_seqs < 0 || max_len <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_context_len < 0 || num_q_heads <= 0)
        return PKV_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (max_len % 64) return PKV_ERR_SHAPE;                 // whole 64-token tiles per slab
    if (num_q_heads % num_kv_heads) return PKV_ERR_SHAPE;
    const int group = num_q_heads / num_kv_heads;
    if (group > 8) return PKV_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return PKV_ERR_SHAPE;
    const int eb = elem_bytes(dtype);
    const int64_t row_stride = (int64_t)num_kv_heads * head_dim * eb;
    if (row_stride * 63 >= ((int64_t)1 << 31)) return PKV_ERR_UNSUPPORTED;  // 32-bit lane offsets
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_cache || !v_cache || !context_lens) return PKV_ERR_NULL;
    if ((int64_t)num_seqs * num_q_heads > ((int64_t)1 << 30)) return PKV_ERR_UNSUPPORTED;
    const size_t need = decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                         max_context_len, 0);
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;

    DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_pool = static_cast<const char*>(k_cache);
    a.v_pool = static_cast<const char*>(v_cache);
    a.block_tables = nullptr;                                // no translation
    a.context_lens = context_lens;
    // a slab of max_len tokens seen as max_len / 64 blocks of 64 (bounds the lengths)
    a.g.row_bytes = head_dim * eb;
    a.g.head_stride_bytes = head_dim * eb;
    a.g.block_stride_bytes = 64 * row_stride;
    a.g.num_blocks = max_len / 64;
    a.g.num_kv_heads = num_kv_heads;
    a.g.block_size = 64;
    a.g.log2_bs = 6;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.max_blocks_per_seq = max_len / 64;
    a.max_context_len = max_context_len;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.part_tokens = 0;
    a.num_parts = 1;
    a.contig_seq_stride = (int64_t)max_len * row_stride;
    a.contig_row_stride = (int32_t)row_stride;
    a.seq_prefix = nullptr;
    a.pre_o = a.pre_ml = nullptr;
    a.pre_splits = 0;
    a.pre_split_tokens = 64;
    const pkv_status sb = setup_balanced(a, decode_contiguous_waves(dtype == PKV_BF16, head_dim, group),
                                         num_seqs, num_kv_heads, head_dim, max_context_len, group,
                                         workspace);
    if (sb != PKV_OK) return sb;
    return launch_status(
        launch_decode_contiguous(a, dtype == PKV_BF16, head_dim, group, num_seqs, stream));
}

size_t paged_attention_decode_multi_query_workspace_bytes(int32_t num_seqs, int32_t queries_per_seq,
                                                         int32_t num_q_heads, int32_t num_kv_heads,
                                                         int32_t head_dim) {
    if (num_seqs <= 0 || queries_per_seq <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        head_dim <= 0 || num_q_heads % num_kv_heads)
        return 0;
    const int64_t rows = (int64_t)(num_q_heads / num_kv_heads) * queries_per_seq;
    return (size_t)balanced_wave_bound() * 2 * rows * (size_t)(head_dim + 2) * sizeof(float) +
           unit_desc_bytes(num_seqs, num_kv_heads);
}

pkv_status paged_attention_decode_multi_query(
    pkv_dtype dtype, void* out, const void* q, const void* k_pool, const void* v_pool,
    int32_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t num_seqs, int32_t queries_per_seq, int32_t max_context_len, int32_t num_q_heads,
    float scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    PoolGeom g;
    const pkv_status st = check_geom(dtype, num_blocks, num_kv_heads, block_size, head_dim, &g);
    if (st != PKV_OK) return st;
    if (num_seqs < 0 || queries_per_seq <= 0 || max_context_len < 0 || max_blocks_per_seq <= 0 ||
        num_q_heads <= 0)
        return PKV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads) return PKV_ERR_SHAPE;
    const int group = num_q_heads / num_kv_heads;
    if (group > 8) return PKV_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return PKV_ERR_SHAPE;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PKV_ERR_NULL;
    if ((int64_t)num_seqs * queries_per_seq * num_q_heads > ((int64_t)1 << 30))
        return PKV_ERR_UNSUPPORTED;
    const size_t need = paged_attention_decode_multi_query_workspace_bytes(
        num_seqs, queries_per_seq, num_q_heads, num_kv_heads, head_dim);
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    // the matrix-core kernel packs the n * G rows of a (sequence, kv head) into one or two
    // groups of 16 columns of its tiles; fp32, 512-byte block runs and wider row sets go
    // query by query on the vector units
    if (!mfma_geometry(dtype, block_size, head_dim) || (int64_t)group * queries_per_seq > 32)
        return launch_chunked(dtype, out, q, nullptr, num_seqs, queries_per_seq,
                              num_seqs * queries_per_seq, k_pool, v_pool, g, head_dim, block_tables,
                              max_blocks_per_seq, context_lens, max_context_len, num_q_heads, scale,
                              stream);

    DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_pool = static_cast<const char*>(k_pool);
    a.v_pool = static_cast<const char*>(v_pool);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.g = g;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.part_tokens = 0;
    a.num_parts = 1;
    a.contig_seq_stride = 0;
    a.contig_row_stride = 0;
    a.seq_prefix = nullptr;
    a.pre_o = a.pre_ml = nullptr;
    a.pre_splits = 0;
    a.pre_split_tokens = 64;
    const pkv_status sb = setup_balanced(a, decode_mq_waves(head_dim, group, queries_per_seq), num_seqs, num_kv_heads,
                                         head_dim, max_context_len, group * queries_per_seq,
                                         workspace);
    if (sb != PKV_OK) return sb;
    return launch_status(launch_decode_mq(a, head_dim, group, queries_per_seq, num_seqs, stream));
}

size_t paged_attention_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                            int32_t num_kv_heads, int32_t head_dim,
                                                            int32_t max_context_len,
                                                            int32_t max_prefix_len) {
    const size_t dec = decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                        max_context_len, 0);
    if (dec == 0) return 0;
    return dec + prefix_state_bytes(num_seqs, num_q_heads, head_dim, std::max(max_prefix_len, 0));
}

pkv_status paged_attention_decode_shared_prefix(
    pkv_dtype dtype, void* out, const void* q, const void* k_pool, const void* v_pool,
    int32_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads, float scale,
    const int32_t* seq_prefix_lens, const int32_t* group_first_seq, const int32_t* group_num_seqs,
    const int32_t* group_prefix_lens, int32_t num_groups, int32_t max_group_seqs,
    int32_t max_prefix_len, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    PoolGeom g;
    const pkv_status st = check_geom(dtype, num_blocks, num_kv_heads, block_size, head_dim, &g);
    if (st != PKV_OK) return st;
    if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq <= 0 || num_q_heads <= 0 ||
        num_groups < 0 || max_group_seqs < 0 || max_prefix_len < 0)
        return PKV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads) return PKV_ERR_SHAPE;
    const int group = num_q_heads / num_kv_heads;
    if (group > 8) return PKV_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return PKV_ERR_SHAPE;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PKV_ERR_NULL;
    if (num_groups > 0 && (!seq_prefix_lens || !group_first_seq || !group_num_seqs ||
                           !group_prefix_lens))
        return PKV_ERR_NULL;
    if ((int64_t)num_seqs * num_q_heads > ((int64_t)1 << 30)) return PKV_ERR_UNSUPPORTED;
    const size_t need = paged_attention_decode_shared_prefix_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, max_prefix_len);
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    // nothing shared, or a pool the prefix pass (matrix cores) does not serve: plain
    // decode over the same tables gives the result this call defines
    if (num_groups == 0 || max_group_seqs == 0 || max_prefix_len == 0 ||
        !mfma_geometry(dtype, block_size, head_dim))
        return paged_attention_decode(dtype, out, q, k_pool, v_pool, num_blocks, num_kv_heads,
                                      block_size, head_dim, block_tables, max_blocks_per_seq,
                                      context_lens, num_seqs, max_context_len, num_q_heads, scale,
                                      0, workspace, workspace_bytes, stream);

    const size_t dec = decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                        max_context_len, 0);
    float* pre_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + dec);
    const int32_t nsplit = prefix_splits(max_prefix_len);
    float* pre_ml = pre_o + (size_t)num_seqs * num_q_heads * (nsplit + 1) * head_dim;

    // 1. every group's members against their shared prefix (matrix cores)
    PrefixArgs pa;
    pa.pre_o = pre_o;
    pa.pre_ml = pre_ml;
    pa.q = q;
    pa.k_pool = static_cast<const char*>(k_pool);
    pa.v_pool = static_cast<const char*>(v_pool);
    pa.block_tables = block_tables;
    pa.group_first_seq = group_first_seq;
    pa.group_num_seqs = group_num_seqs;
    pa.group_prefix_len = group_prefix_lens;
    pa.g = g;
    pa.num_seqs = num_seqs;
    pa.num_q_heads = num_q_heads;
    pa.max_blocks_per_seq = max_blocks_per_seq;
    pa.num_splits = nsplit;
    pa.state_stride = nsplit + 1;
    pa.split_tokens = prefix_split_tokens(max_prefix_len);
    pa.scale_log2 = scale * 1.4426950408889634f;
    const hipError_t e1 = launch_prefix(pa, head_dim, group, num_groups, max_group_seqs, stream);
    if (e1 != hipSuccess) return launch_status(e1);

    // 2. every sequence's own tokens after its prefix, merged with the prefix states
    DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_pool = static_cast<const char*>(k_pool);
    a.v_pool = static_cast<const char*>(v_pool);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.g = g;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.scale_log2 = pa.scale_log2;
    a.part_tokens = 0;
    a.num_parts = 1;
    a.contig_seq_stride = 0;
    a.contig_row_stride = 0;
    a.seq_prefix = seq_prefix_lens;
    a.pre_o = pre_o;
    a.pre_ml = pre_ml;
    a.pre_splits = nsplit;
    a.pre_split_tokens = pa.split_tokens;
    const pkv_status sb = setup_balanced(a, decode_prefix_waves(head_dim, group), num_seqs,
                                         num_kv_heads, head_dim, max_context_len, group, workspace);
    if (sb != PKV_OK) return sb;
    return launch_status(launch_decode_prefix(a, head_dim, group, num_seqs, stream));
}

pkv_status paged_attention_prefill_chunk(pkv_dtype dtype, void* out, const void* q,
                                         const int32_t* cu_q_lens, int32_t num_chunks,
                                         int32_t max_q_len, const void* k_pool, const void* v_pool,
                                         int32_t num_blocks, int32_t num_kv_heads,
                                         int32_t block_size, int32_t head_dim,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t max_context_len,
                                         int32_t num_q_heads, float scale, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
    PoolGeom g;
    const pkv_status st = check_geom(dtype, num_blocks, num_kv_heads, block_size, head_dim, &g);
    if (st != PKV_OK) return st;
    if (num_chunks < 0 || max_q_len < 0 || max_context_len < 0 || max_blocks_per_seq <= 0 ||
        num_q_heads <= 0)
        return PKV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads) return PKV_ERR_SHAPE;
    const int group = num_q_heads / num_kv_heads;
    if (group > 8) return PKV_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return PKV_ERR_SHAPE;
    if (num_chunks == 0 || max_q_len == 0) return PKV_OK;
    if (!out || !q || !cu_q_lens || !k_pool || !v_pool || !block_tables || !context_lens)
        return PKV_ERR_NULL;
    // work items: query tiles (128 / group query positions each) x kv heads x chunks
    if (product_exceeds(product_exceeds(cdiv64(max_q_len, 128 / group), num_kv_heads, (int64_t)1 << 30),
                        num_chunks, (int64_t)1 << 30) > ((int64_t)1 << 30))
        return PKV_ERR_UNSUPPORTED;
    if (workspace != nullptr) {
        const size_t need = paged_attention_prefill_chunk_workspace_bytes(num_q_heads, num_kv_heads,
                                                                          head_dim);
        if (need > 0 && workspace_bytes < need) return PKV_ERR_WORKSPACE;
    }
    // fp32 and 512-byte block runs: query by query on the vector units (no workspace)
    if (!mfma_geometry(dtype, block_size, head_dim))
        return launch_chunked(dtype, out, q, cu_q_lens, num_chunks, max_q_len, INT32_MAX, k_pool,
                              v_pool, g, head_dim, block_tables, max_blocks_per_seq, context_lens,
                              max_context_len, num_q_heads, scale, stream);

    PrefillArgs a;
    a.out = out;
    a.q = q;
    a.cu_q_lens = cu_q_lens;
    a.k_pool = static_cast<const char*>(k_pool);
    a.v_pool = static_cast<const char*>(v_pool);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.g = g;
    a.num_q_heads = num_q_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.part_o = nullptr;
    a.part_ml = nullptr;
    a.item_desc = nullptr;
    a.num_wgs = 0;
    if (workspace != nullptr) {
        const size_t need = paged_attention_prefill_chunk_workspace_bytes(num_q_heads, num_kv_heads,
                                                                          head_dim);
        if (need == 0) return PKV_ERR_LAUNCH;
        if (workspace_bytes < need) return PKV_ERR_WORKSPACE;
        a.num_wgs = prefill_wgs(head_dim, group);
        const size_t slots = (size_t)2 * a.num_wgs * 128;      // partial rows
        char* ws = static_cast<char*>(workspace);
        a.part_ml = reinterpret_cast<float*>(ws);
        a.item_desc = reinterpret_cast<int32_t*>(ws + slots * 2 * sizeof(float));
        a.part_o = reinterpret_cast<uint16_t*>(ws + slots * 2 * sizeof(float) +
                                               (size_t)a.num_wgs * 2 * sizeof(int32_t));
    }
    return launch_status(launch_prefill(a, head_dim, group, num_chunks, max_q_len, stream));
}

size_t paged_attention_prefill_chunk_workspace_bytes(int32_t num_q_heads, int32_t num_kv_heads,
                                                     int32_t head_dim) {
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
        num_q_heads / num_kv_heads > 8 || (head_dim != 64 && head_dim != 128))
        return 0;
    const int wgs = prefill_wgs(head_dim, num_q_heads / num_kv_heads);
    if (wgs <= 0) return 0;
    // two partial slots per workgroup, each 128 rows of (max, sum) in fp32 and head_dim
    // bf16 outputs, and a descriptor of two int32 per work item (at most one per workgroup)
    return (size_t)2 * wgs * 128 * (2 * sizeof(float) + (size_t)head_dim * 2) +
           (size_t)wgs * 2 * sizeof(int32_t);
}

}  // extern "C"
