// Internal launch interface between the C ABI (pkv_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct PoolGeom {
    int64_t block_stride_bytes;  // num_kv_heads * block_size * head_dim * elem
    int32_t head_stride_bytes;   // block_size * head_dim * elem
    int32_t row_bytes;           // head_dim * elem
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t log2_bs;
};

struct WriteArgs {
    char* k_pool;
    char* v_pool;
    const char* k_new;
    const char* v_new;
    const int64_t* slot_mapping;
    int32_t num_tokens;
    PoolGeom g;
};

struct CopyArgs {
    char* k_pool;
    char* v_pool;
    const int64_t* block_mapping;
    int32_t num_pairs;
    PoolGeom g;
};

// swap_blocks through a copy kernel: pools are device pointers (pinned host pools
// through their device mapping); up to kSwapPairsPerLaunch (src, dst) pairs travel in
// the kernel arguments.
constexpr int kSwapPairsPerLaunch = 240;
struct SwapArgs {
    char* dst_k;
    char* dst_v;
    const char* src_k;
    const char* src_v;
    int64_t block_bytes;
    int32_t num_pairs;
    int32_t src[kSwapPairsPerLaunch];
    int32_t dst[kSwapPairsPerLaunch];
};

// Most key splits of a shared prefix (the prefix pass writes one partial state per
// split; the merge reads them with all loads in flight at once).
constexpr int kMaxPreSplits = 4;

struct DecodeArgs {
    void* out;
    const void* q;
    const char* k_pool;
    const char* v_pool;
    const int32_t* block_tables;
    const int32_t* context_lens;
    // Partial softmax states.  Fixed partitions: [S][Hq][num_parts][D] and
    // [S][Hq][num_parts][2].  Balanced split: [num_waves][2 slots][G][D] and
    // [num_waves][2][G][2].  (max in log2 units, sum of exponentials)
    float* part_o;
    float* part_ml;
    // Balanced split: for unit (s, h) at [2 (s Hkv + h)], the wave holding its first
    // tile and the number of waves its tiles span (written by that wave, read by the
    // merge; units without tiles are not written).
    int32_t* unit_desc;
    PoolGeom g;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    int32_t part_tokens;   // fixed partitions (> 0), or 0 for the balanced split
    int32_t num_parts;     // fixed partitions per sequence (grid.x)
    int32_t num_waves;     // balanced split: persistent waves (grid.x)
    int32_t lead_share_q10;  // balanced split: tiles given to the first half of the waves, /1024
    // Contiguous layout (the unpaged baseline): k_pool/v_pool are [S][L][Hkv][D]; token t of
    // sequence s, head h is at s * seq_stride + t * row_stride + h * row_bytes.
    int64_t contig_seq_stride;
    int32_t contig_row_stride;
    // Shared-prefix mode: the first seq_prefix[s] tokens of sequence s were attended by
    // the prefix pass, whose partial states are pre_o [S][Hq][pre_splits + 1][D] and
    // pre_ml [S][Hq][pre_splits + 1][2] (splits of pre_split_tokens keys; the last slot
    // of a row takes the decode's state of its own tokens when one wave finishes them);
    // the merge combines them.  seq_prefix == nullptr: no prefix.
    const int32_t* seq_prefix;
    float* pre_o;
    float* pre_ml;
    int32_t pre_splits;
    int32_t pre_split_tokens;
    // Chunked mode (causal query chunks on the vector units): grid unit v is query
    // v mod q_per_chunk of chunk v / q_per_chunk; the chunk's queries start at row
    // cu_q_lens[c] (or c * q_per_chunk without cu_q_lens) of q and out, which hold
    // num_q_rows rows; context_lens and block_tables are per chunk.
    const int32_t* cu_q_lens;
    int32_t q_per_chunk;
    int32_t num_q_rows;
    float scale_log2;      // scale * log2(e)
};

// Share of the tiles (in 1/1024) that the balanced split gives the first half of its
// waves when two waves share each SIMD: the first-dispatched wave of a SIMD wins
// issue arbitration and streams faster while its partner is active, so an even
// split leaves the second half as the critical path.  Measured on MI355X with the
// matrix-core Q.K and P.V (608..688, alternated on one machine): 656 is best for both
// the long-context and the GQA decode.
constexpr int kLeadShareQ10 = 656;

// Persistent waves the balanced decode launches on the current device.
int decode_balanced_waves(bool is_bf16, int head_dim, int group);
// The same for the shared-prefix mode (bf16 only).
int decode_prefix_waves(int head_dim, int group);

// The shared-prefix pass: groups of consecutive sequences whose first
// group_prefix_len[g] tokens sit in the same physical blocks.
struct PrefixArgs {
    float* pre_o;
    float* pre_ml;
    const void* q;
    const char* k_pool;
    const char* v_pool;
    const int32_t* block_tables;
    const int32_t* group_first_seq;
    const int32_t* group_num_seqs;
    const int32_t* group_prefix_len;
    PoolGeom g;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t max_blocks_per_seq;
    int32_t num_splits;      // key splits per group prefix
    int32_t state_stride;    // state slots per row (num_splits + 1)
    int32_t split_tokens;    // keys per split (a multiple of 64)
    float scale_log2;
};
// Persistent waves of the contiguous-layout decode.
int decode_contiguous_waves(bool is_bf16, int head_dim, int group);
// Causal query chunks, one wave per (query, kv head) streaming its visible keys with
// decode's arithmetic (fp32, or shapes without a matrix-core path); units = grid slots.
hipError_t launch_decode_chunked(const DecodeArgs& a, bool is_bf16, int head_dim, int group,
                                 int64_t units, hipStream_t st);

struct PrefillArgs {
    void* out;
    const void* q;
    const int32_t* cu_q_lens;
    const char* k_pool;
    const char* v_pool;
    const int32_t* block_tables;
    const int32_t* context_lens;
    PoolGeom g;
    int32_t num_q_heads;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    float scale_log2;
    // balanced key split (null part_o: one workgroup per query tile, no split)
    uint16_t* part_o;             // [2 * num_wgs][128 rows][D] bf16 partial outputs (normalised)
    float* part_ml;               // [2 * num_wgs][128 rows][2] (max in log2 units, sum)
    int32_t* item_desc;           // [num_wgs][2]: (first workgroup, pieces; 0 = not cut) per item
    int32_t num_wgs;              // workgroups of the split: the device's resident count
};

// Device-side precondition check (pkv_validate): counts [4] in device memory.
struct ValidateArgs {
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int64_t* slot_mapping;
    const int64_t* block_mapping;
    int32_t* counts;
    int32_t num_blocks;
    int32_t block_size;
    int32_t max_blocks_per_seq;
    int32_t num_seqs;
    int32_t num_tokens;
    int32_t num_pairs;
};

hipError_t launch_validate(const ValidateArgs& v, hipStream_t st);
hipError_t launch_validate_chunks(const int32_t* cu_q_lens, const int32_t* context_lens,
                                  int32_t num_chunks, int32_t total_q, int32_t* count,
                                  hipStream_t st);
hipError_t launch_kv_write(const WriteArgs& a, hipStream_t st);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t st);
hipError_t launch_swap(const SwapArgs& a, hipStream_t st);
// is_bf16 selects the element type; group = num_q_heads / num_kv_heads (1..8).
hipError_t launch_decode(const DecodeArgs& a, bool is_bf16, int head_dim, int group,
                         int num_seqs, hipStream_t st);
// Decode over the contiguous [S][L][Hkv][D] layout (balanced split).
hipError_t launch_decode_contiguous(const DecodeArgs& a, bool is_bf16, int head_dim, int group,
                                    int num_seqs, hipStream_t st);
hipError_t launch_prefix(const PrefixArgs& a, int head_dim, int group, int num_groups,
                         int max_group_seqs, hipStream_t st);
// Decode over the tokens after each sequence's shared prefix, merging the prefix pass.
hipError_t launch_decode_prefix(const DecodeArgs& a, int head_dim, int group, int num_seqs,
                                hipStream_t st);
// Resident workgroups of the prefill kernel (the balanced split's grid), 0 if unknown.
int prefill_wgs(int head_dim, int group);
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int group, int num_chunks,
                          int max_q_len, hipStream_t st);
// Multi-query decode (bf16): nq queries per sequence, nq * group <= 32, balanced split.
int decode_mq_waves(int head_dim, int group, int nq);
hipError_t launch_decode_mq(const DecodeArgs& a, int head_dim, int group, int nq, int num_seqs,
                            hipStream_t st);
// The balanced merge for nq queries per sequence (used by the multi-query decode).
hipError_t launch_balanced_merge_mq(const DecodeArgs& a, int head_dim, int group, int nq,
                                    hipStream_t st);

}  // namespace pkv
