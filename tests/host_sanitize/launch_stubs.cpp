// Stand-ins for the kernel launchers of libpagedkv, for a host-only build of the C ABI
// under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU code is compiled).
// Each launcher checks that the arguments the ABI layer prepared are self-consistent
// and returns success without launching anything.
#include <stdio.h>
#include <stdlib.h>

#include "pkv_internal.h"

namespace pkv {

static void require(bool ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "launch stub: %s\n", what);
        abort();
    }
}

static void check_geom(const PoolGeom& g) {
    require(g.num_blocks > 0 && g.num_kv_heads > 0 && g.block_size >= 4, "pool geometry");
    require((1 << g.log2_bs) == g.block_size, "log2 of the block size");
    require(g.head_stride_bytes == g.block_size * g.row_bytes, "head stride");
    require(g.block_stride_bytes == (int64_t)g.num_kv_heads * g.head_stride_bytes, "block stride");
}

// Waves and workgroups a 256-CU device keeps resident.
int decode_balanced_waves(bool, int, int) { return 2048; }
int decode_prefix_waves(int, int) { return 2048; }
int decode_contiguous_waves(bool, int, int) { return 2048; }
int decode_mq_waves(int, int, int nq) { return nq > 0 ? 2048 : 0; }
int prefill_wgs(int, int) { return 512; }

hipError_t launch_validate(const ValidateArgs& v, hipStream_t) {
    require(v.counts != nullptr, "validate counts");
    return hipSuccess;
}
hipError_t launch_validate_chunks(const int32_t* cu_q_lens, const int32_t* context_lens,
                                  int32_t num_chunks, int32_t, int32_t* count, hipStream_t) {
    require(cu_q_lens && context_lens && count && num_chunks > 0, "validate chunks");
    return hipSuccess;
}
hipError_t launch_kv_write(const WriteArgs& a, hipStream_t) {
    check_geom(a.g);
    require(a.num_tokens > 0 && a.slot_mapping, "write");
    return hipSuccess;
}
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t) {
    check_geom(a.g);
    require(a.num_pairs > 0 && a.block_mapping, "copy");
    return hipSuccess;
}
hipError_t launch_swap(const SwapArgs& a, hipStream_t) {
    require(a.num_pairs > 0 && a.num_pairs <= kSwapPairsPerLaunch, "swap pairs");
    return hipSuccess;
}
static void check_decode(const DecodeArgs& a, bool paged = true) {
    if (paged) check_geom(a.g);
    require(a.num_seqs > 0 && a.num_q_heads > 0, "decode sizes");
    require(a.part_tokens >= 0 && a.num_parts >= 1, "decode partitions");
    require(a.part_tokens > 0 || (a.num_waves > 0 && a.part_o && a.part_ml && a.unit_desc),
            "balanced workspace");
}
hipError_t launch_decode(const DecodeArgs& a, bool, int, int group, int, hipStream_t) {
    check_decode(a);
    require(group >= 1 && group <= 8, "group");
    return hipSuccess;
}
hipError_t launch_decode_contiguous(const DecodeArgs& a, bool, int, int, int, hipStream_t) {
    check_decode(a, false);          // the slab is described as 64-token blocks of one row each
    require(a.contig_row_stride > 0 && a.contig_seq_stride > 0, "contiguous strides");
    return hipSuccess;
}
hipError_t launch_decode_chunked(const DecodeArgs& a, bool, int, int group, int64_t units,
                                 hipStream_t) {
    check_geom(a.g);
    require(units > 0 && a.q_per_chunk > 0 && a.num_parts == 1, "chunked units");
    require(units * a.g.num_kv_heads <= ((int64_t)1 << 30), "chunked grid");
    require(group >= 1 && group <= 8, "group");
    return hipSuccess;
}
hipError_t launch_prefix(const PrefixArgs& a, int, int, int, int, hipStream_t) {
    require(a.num_splits >= 1 && a.split_tokens % 64 == 0, "prefix splits");
    return hipSuccess;
}
hipError_t launch_decode_prefix(const DecodeArgs& a, int, int, int, hipStream_t) {
    check_decode(a);
    return hipSuccess;
}
hipError_t launch_prefill(const PrefillArgs& a, int, int, int, int, hipStream_t) {
    check_geom(a.g);
    return hipSuccess;
}
hipError_t launch_decode_mq(const DecodeArgs& a, int, int, int, int, hipStream_t) {
    check_decode(a);
    return hipSuccess;
}
hipError_t launch_balanced_merge_mq(const DecodeArgs& a, int, int, int, hipStream_t) {
    check_decode(a);
    return hipSuccess;
}

}  // namespace pkv
