/*
 * pagedkv.h -- C ABI of libpagedkv: PagedAttention over a block-table-indexed
 * KV cache on AMD Instinct MI355X (gfx950).
 *
 * The operations follow the "2.1 PagedAttention" chapter (vLLM tutorial):
 * a request's KV cache is cut into blocks of block_size tokens, its logical
 * blocks are mapped to physical blocks by a block table (section 3), and the
 * attention kernel reads every logical position at physical block number x
 * block stride + offset inside the block (section 5).  Blocks can be shared
 * by several tables and copied before a write (copy-on-write, section 6).
 * Chunked prefill follows "Inside vLLM, part 2" (chunked prefill section).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer owned by the caller; the
 *    library never allocates, frees, or synchronises.  Work is enqueued on
 *    the given stream in call order; the caller orders a cache write before
 *    the attention that reads it (stream order), and keeps context_lens
 *    consistent with what has been written.
 *  - KV pools: k_pool and v_pool are each
 *        [num_blocks][num_kv_heads][block_size][head_dim]
 *    contiguous, so kv_head_stride = block_size*head_dim elements and
 *    kv_block_stride = num_kv_heads*block_size*head_dim elements.
 *  - q, k/v pools, new K/V and outputs share one element type (pkv_dtype).
 *    bf16 is stored as the upper 16 bits of an IEEE float32.
 *  - Query head hq reads KV head hq / (num_q_heads / num_kv_heads).
 *  - block_tables is int32 [rows][max_blocks_per_seq], row-major; entries
 *    beyond ceil(context_len / block_size) are never read.
 *  - A context length counts every token visible to the step's queries,
 *    including the ones written in this step.
 *  - Supported by every entry point: bf16 and fp32; head_dim in {64, 128};
 *    block_size in {4, 8, 16, 32}; one pool block (all kv heads) smaller than 2 GiB;
 *    num_q_heads / num_kv_heads in 1..8.  The matrix-core kernels (chunked prefill,
 *    multi-query decode, the shared-prefix pass) serve bf16 pools whose
 *    (block, kv head) runs hold at least 1 KiB; other pools (fp32, and bf16 with
 *    head_dim 64 and block_size 4) go through the decode's vector-unit arithmetic,
 *    with the same results within the tolerance of their element type.
 *  - Host-checkable arguments are validated before anything is enqueued; a
 *    non-zero status means nothing was launched.  Device-resident contents
 *    (block ids, slots, lengths) are not validated; out-of-range block ids
 *    and slots are skipped by the kernels (never dereferenced), which keeps
 *    a bad table from faulting the GPU but yields unspecified output.
 *  - No entry point blocks or aborts; errors are status codes.
 *  - Apart from swap_blocks (host memory) every entry point only launches
 *    kernels on the given stream -- no memset, copy or host wait -- so a
 *    sequence of calls can be captured into a HIP graph and replayed.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_dtype {
    PKV_F32 = 0,
    PKV_BF16 = 1,
    /* not a type: widens the enum so that any non-negative int a foreign caller passes
       is a value of it (the library then rejects it with PKV_ERR_DTYPE) */
    PKV_DTYPE_INT32_ = 0x7fffffff
} pkv_dtype;

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_ERR_NULL = 1,          /* a required pointer is NULL */
    PKV_ERR_SHAPE = 2,         /* a size is negative/zero where it must be positive, or inconsistent */
    PKV_ERR_DTYPE = 3,         /* unknown pkv_dtype */
    PKV_ERR_UNSUPPORTED = 4,   /* valid but not implemented (head_dim, block_size, group size, dtype) */
    PKV_ERR_WORKSPACE = 5,     /* workspace missing or smaller than required */
    PKV_ERR_LAUNCH = 6,        /* the HIP runtime refused a launch or copy */
    PKV_ERR_VALIDATION = 7,    /* device contents violate a precondition (reported by the
                                  binding after pkv_validate's counts come back) */
    PKV_ERR_NO_BLOCKS = 8,     /* block pool: not enough free blocks (nothing was taken) */
    /* not a status: widens the enum so that any non-negative int is a value of it
       (pkv_status_string answers such values with "PKV_ERR_UNKNOWN") */
    PKV_STATUS_INT32_ = 0x7fffffff
} pkv_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* pkv_status_string(pkv_status status);

/*
 * paged_kv_write -- slot-mapped write of the current step's new K/V.
 * ("2.1 PagedAttention", section 3: each new token fills the next free slot of
 * its request's current block, the scheduler naming the slot.)
 *
 *   k_new, v_new   [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping   int64 [num_tokens]; slot = physical_block*block_size + offset.
 *                  slot < 0 marks padding and writes nothing.  Slots of one call
 *                  must be distinct (two tokens on one slot: unspecified winner).
 * For every token i with a valid slot, K_pool[slot/bs][h][slot%bs][:] = k_new[i][h][:]
 * for all heads h (bit copy), and likewise for V.  num_tokens == 0 is a no-op.
 */
pkv_status paged_kv_write(pkv_dtype dtype, void* k_pool, void* v_pool, int32_t num_blocks,
                          int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                          const void* k_new, const void* v_new, const int64_t* slot_mapping,
                          int32_t num_tokens, hipStream_t stream);

/*
 * copy_blocks -- block copies for copy-on-write ("2.1 PagedAttention", section 6:
 * before writing into a shared block, the block is copied to a private block and
 * the writer's table is re-pointed to the copy; re-pointing is the caller's).
 *
 *   block_mapping  int64 [num_pairs][2] = (src, dst) physical block ids.
 * Each pair copies the whole block (every KV head and slot) of K and of V.  All
 * destinations must be distinct and none may be a source of the same call.
 * num_pairs == 0 is a no-op.
 */
pkv_status copy_blocks(pkv_dtype dtype, void* k_pool, void* v_pool, int32_t num_blocks,
                       int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                       const int64_t* block_mapping, int32_t num_pairs, hipStream_t stream);

/*
 * Decode attention.  Each query head of sequence s attends to the
 * context_lens[s] tokens of the sequence, read through its block table row
 * ("2.1 PagedAttention", sections 3 and 5):
 *     out[s][hq][:] = sum_t softmax_t(scale * q[s][hq] . K_t) * V_t
 * with K_t, V_t at (block_tables[s][t / bs], kv head, t % bs).  Long contexts are
 * split into pieces whose partial softmax states are merged by log-sum-exp; the
 * result does not depend on the split beyond float rounding.  context_len 0
 * gives a zero row.
 *
 * Split: partition_tokens == 0 (default) divides all 64-token tiles of the batch
 * evenly over the waves the device keeps resident, whatever the mix of lengths
 * (the split, hence the rounding, depends on the device's compute-unit count);
 * partition_tokens > 0 cuts every context into pieces of that many positions
 * instead (device independent).
 *
 * paged_attention_decode_workspace_bytes: bytes of device workspace the call
 * needs for that choice of split (for the default split it depends on the
 * current device; for fixed partitions it is 0 when every context fits one).
 */
size_t paged_attention_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t max_context_len, int32_t partition_tokens);

/*
 *   out           [num_seqs][num_q_heads][head_dim]   (written)
 *   q             [num_seqs][num_q_heads][head_dim]
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]
 *   context_lens  int32 [num_seqs], each in [0, max_blocks_per_seq*block_size]
 *   max_context_len  host-known upper bound of context_lens (sizes the grid;
 *                    a larger context is truncated to it)
 *   partition_tokens 0 = balanced split (default), else a positive multiple of
 *                 block_size (at most 65535 partitions of max_context_len)
 *   workspace     device scratch of at least paged_attention_decode_workspace_bytes
 *                 (may be NULL when that is 0); its contents need no initialisation
 *                 and are garbage afterwards; calls sharing a workspace must not
 *                 overlap in time.
 */
pkv_status paged_attention_decode(pkv_dtype dtype, void* out, const void* q,
                                  const void* k_pool, const void* v_pool, int32_t num_blocks,
                                  int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t max_context_len, int32_t num_q_heads, float scale,
                                  int32_t partition_tokens, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_noalloc -- paged_attention_decode for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, semantics and
 * results (identical bits) as paged_attention_decode without the workspace: the call
 * uses a fixed scratch array in device memory that the library holds for the whole
 * process (one per device, paged_attention_decode_noalloc_scratch_bytes() bytes,
 * 20 MiB), and allocates nothing.
 *   - PKV_ERR_WORKSPACE (nothing launched) when the call would need more workspace
 *     than that (paged_attention_decode_workspace_bytes() > the scratch size): the
 *     default split needs at most 2 * 8 * num_compute_units * G * (head_dim + 2) * 4
 *     bytes (17 MB at G = 8, head_dim 128 on 256 compute units) plus 8 bytes per
 *     (sequence, kv head); fixed partitions need
 *     num_seqs * num_q_heads * partitions * (head_dim + 2) * 4.
 *   - Every call on a device shares that device's scratch: calls that overlap in
 *     time on one device (other streams, other threads) race and give unspecified
 *     output.  Calls ordered on one stream are fine.  The scratch keeps the last
 *     call's contents; nothing in it needs initialisation.
 *   - PKV_ERR_LAUNCH if the scratch's device address cannot be obtained.
 */
size_t paged_attention_decode_noalloc_scratch_bytes(void);
pkv_status paged_attention_decode_noalloc(pkv_dtype dtype, void* out, const void* q,
                                          const void* k_pool, const void* v_pool,
                                          int32_t num_blocks, int32_t num_kv_heads,
                                          int32_t block_size, int32_t head_dim,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t max_context_len, int32_t num_q_heads, float scale,
                                          int32_t partition_tokens, hipStream_t stream);

/*
 * contiguous_attention_decode -- the unpaged baseline of paged_attention_decode:
 * the same attention over K/V stored contiguously per sequence, as a system that
 * reserves each request's whole maximum length up front would ("vAttention",
 * the KV cache of a request as one contiguous virtual range).  No block table is
 * read; token t of sequence s, kv head h is at ((s * max_len + t) * Hkv + h) * D.
 * It exists to measure what the block-table translation costs; the split, the
 * tile order and the arithmetic are those of the balanced paged decode, so on
 * the same K/V values the two return identical bits.
 *
 *   out, q        [num_seqs][num_q_heads][head_dim] bf16
 *   k_cache, v_cache  [num_seqs][max_len][num_kv_heads][head_dim] bf16
 *   max_len       slab length, a positive multiple of 64; context_lens[s] <= max_len
 *   workspace     as for paged_attention_decode with partition_tokens 0 (size from
 *                 paged_attention_decode_workspace_bytes(..., 0)); its contents need
 *                 no initialisation.
 * bf16 or fp32.  Errors: PKV_ERR_UNSUPPORTED for head_dim not in {64, 128};
 * PKV_ERR_SHAPE for max_len not a multiple of 64; otherwise as paged_attention_decode.
 */
pkv_status contiguous_attention_decode(pkv_dtype dtype, void* out, const void* q,
                                       const void* k_cache, const void* v_cache, int32_t num_seqs,
                                       int32_t max_len, int32_t num_kv_heads, int32_t head_dim,
                                       const int32_t* context_lens, int32_t max_context_len,
                                       int32_t num_q_heads, float scale, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_multi_query -- decode with n = queries_per_seq query
 * positions per sequence, for verifying speculative tokens ("Inside vLLM, part 2",
 * speculative decoding: the k proposed tokens and the last accepted one are scored
 * in one step).  Query i of sequence s sits at position context_lens[s] - n + i and
 * attends causally: keys t <= that position, read through the block table.  The K/V
 * of all n positions must already be in the cache (paged_kv_write earlier on the
 * stream), and n must not exceed a sequence's context.
 *
 *   out, q        [num_seqs * n][num_q_heads][head_dim] (query i of sequence s is
 *                 token s * n + i: the packed layout of paged_attention_prefill_chunk
 *                 with every chunk of length n)
 *   other arguments as paged_attention_decode.
 *
 * The result equals paged_attention_prefill_chunk with cu_q_lens = 0, n, 2n, ...
 * bf16 pools with (num_q_heads / num_kv_heads) * n <= 16 (the 16 columns of one
 * matrix-core tile) run on the matrix cores; fp32, 512-byte block runs and wider row
 * sets run query by query on the vector units (each query streams the keys it sees).
 * Workspace: paged_attention_decode_multi_query_workspace_bytes(); its contents need
 * no initialisation.
 */
size_t paged_attention_decode_multi_query_workspace_bytes(int32_t num_seqs, int32_t queries_per_seq,
                                                         int32_t num_q_heads, int32_t num_kv_heads,
                                                         int32_t head_dim);
pkv_status paged_attention_decode_multi_query(
    pkv_dtype dtype, void* out, const void* q, const void* k_pool, const void* v_pool,
    int32_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t num_seqs, int32_t queries_per_seq, int32_t max_context_len, int32_t num_q_heads,
    float scale, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_shared_prefix -- decode attention for batches in which
 * groups of sequences share the physical blocks of a common prefix ("2.1
 * PagedAttention", section 6: several block tables point at the same blocks, read
 * only, e.g. one system prompt).  The result is that of paged_attention_decode on
 * the same tables; what changes is the traffic: each group's prefix K/V is read once
 * per kv head for up to 128/G members at a time (a dense product on the matrix
 * cores) instead of once per member, and each member's own tokens after the prefix
 * go through the balanced decode, which merges both by log-sum-exp.
 *
 * Groups (device arrays, num_groups entries): members are the consecutive sequences
 * group_first_seq[g] .. group_first_seq[g] + group_num_seqs[g] - 1 (groups do not
 * overlap), whose first group_prefix_lens[g] tokens (rounded down to whole blocks)
 * sit in the same physical blocks, read through the table of the first member.
 * seq_prefix_lens[s] (device, [num_seqs]) is the prefix length of the group of s,
 * 0 for a sequence in no group; a member's context must not end before its
 * prefix (it may end at it: the result is then the prefix's alone).
 * max_group_seqs >= every group_num_seqs[g] and max_prefix_len >= every
 * group_prefix_lens[g] are host bounds (they size the prefix pass).  These device
 * contents are preconditions; violating them gives unspecified output but never an
 * out-of-range access.  With num_groups == 0, or a pool the matrix-core prefix pass
 * does not serve (fp32, 512-byte block runs), this is paged_attention_decode.
 *
 * Workspace: paged_attention_decode_shared_prefix_workspace_bytes(); its contents
 * need no initialisation.
 */
size_t paged_attention_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                            int32_t num_kv_heads, int32_t head_dim,
                                                            int32_t max_context_len,
                                                            int32_t max_prefix_len);
pkv_status paged_attention_decode_shared_prefix(
    pkv_dtype dtype, void* out, const void* q, const void* k_pool, const void* v_pool,
    int32_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads, float scale,
    const int32_t* seq_prefix_lens, const int32_t* group_first_seq, const int32_t* group_num_seqs,
    const int32_t* group_prefix_lens, int32_t num_groups, int32_t max_group_seqs,
    int32_t max_prefix_len, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_validate -- device-side check of the device-content preconditions that the other
 * calls trust and do not check ("2.1 PagedAttention", section 3: token t of sequence s
 * lives in block block_tables[s][t / block_size], and a write puts token i at slot
 * block * block_size + offset; section 6: copy-on-write copies whole blocks).
 * Enqueues kernels that write counts[4] (int32, device memory owned by the caller):
 *   counts[0]  table entries a context reaches (j < min(ceil(ctx / block_size),
 *              max_blocks_per_seq)) outside [0, num_blocks)
 *   counts[1]  sequences with context_lens[s] < 0 or > max_blocks_per_seq * block_size
 *   counts[2]  tokens whose slot is >= num_blocks * block_size, or equals an earlier
 *              token's slot (negative slots are padding)
 *   counts[3]  copy pairs with an id outside [0, num_blocks), a destination written by
 *              an earlier pair, or a destination that some pair reads
 * Each part is skipped when its count (num_seqs, num_tokens, num_pairs) is 0.  The
 * call does not wait: synchronise the stream, then read counts (all zero = valid).
 * Cost is O(n^2) in num_tokens and num_pairs: a debugging aid, not for every step.
 * Errors: PKV_ERR_NULL / PKV_ERR_SHAPE for missing pointers or negative sizes (nothing
 * enqueued); PKV_ERR_LAUNCH if a launch fails.
 */
pkv_status pkv_validate(int32_t num_blocks, int32_t block_size, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                        const int64_t* slot_mapping, int32_t num_tokens,
                        const int64_t* block_mapping, int32_t num_pairs, int32_t* counts,
                        hipStream_t stream);

/*
 * pkv_validate_chunks -- device-side check of the chunk descriptors that
 * paged_attention_prefill_chunk trusts ("Inside vLLM, part 2", chunked prefill: a chunk's
 * queries are the last positions of its context, packed chunk after chunk).  Enqueues
 * kernels that set *count (int32, device memory owned by the caller) to the number of
 * chunks c in [0, num_chunks) with cu_q_lens[c + 1] < cu_q_lens[c], a negative context,
 * more queries than context (cu_q_lens[c + 1] - cu_q_lens[c] > context_lens[c]), or queries
 * ending past total_q rows (when total_q >= 0), counting chunk 0 also when cu_q_lens[0]
 * != 0.  The call does not wait.  Errors: PKV_ERR_NULL / PKV_ERR_SHAPE (nothing
 * enqueued); num_chunks == 0 enqueues nothing and leaves *count as it is.
 */
pkv_status pkv_validate_chunks(const int32_t* cu_q_lens, const int32_t* context_lens,
                               int32_t num_chunks, int32_t total_q, int32_t* count,
                               hipStream_t stream);

/*
 * paged_attention_prefill_chunk -- causal attention of prefill query chunks over
 * their paged contexts ("Inside vLLM, part 2", chunked prefill: a long prompt is
 * processed a bounded number of tokens per step, each chunk attending to the
 * already-cached prefix and to itself).
 *
 *   out, q        [total_q][num_q_heads][head_dim], total_q = cu_q_lens[num_chunks]
 *   cu_q_lens     int32 [num_chunks + 1], cu_q_lens[0] = 0, non-decreasing
 *   max_q_len     host-known max of cu_q_lens[c+1] - cu_q_lens[c]
 *   block_tables  int32 [num_chunks][max_blocks_per_seq]
 *   context_lens  int32 [num_chunks], including the chunk; chunk c's queries are the
 *                 last n_q positions, query i at p = ctx - n_q + i, seeing keys t <= p.
 *                 n_q must not exceed ctx.
 *   workspace     NULL, or device scratch of at least
 *                 paged_attention_prefill_chunk_workspace_bytes() (no initialisation
 *                 needed; garbage afterwards; calls sharing it must not overlap).
 *                 With it, a batch whose query tiles fit in one round of resident
 *                 workgroups but whose chunks differ in length is split over keys into
 *                 equal ranges and merged by log-sum-exp (the result is the same up to
 *                 rounding); without it every query tile is one workgroup.
 * The chunk's own K/V must already be in the cache (paged_kv_write earlier on the
 * stream).  bf16 pools with block runs of at least 1 KiB run on the matrix cores; fp32
 * (and 512-byte runs) run query by query on the vector units with the decode's fp32
 * arithmetic, one wave per (query, kv head), and use no workspace.
 * PKV_ERR_WORKSPACE if a workspace is given and is too small.
 */
pkv_status paged_attention_prefill_chunk(pkv_dtype dtype, void* out, const void* q,
                                         const int32_t* cu_q_lens, int32_t num_chunks,
                                         int32_t max_q_len, const void* k_pool,
                                         const void* v_pool, int32_t num_blocks,
                                         int32_t num_kv_heads, int32_t block_size,
                                         int32_t head_dim, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                                         int32_t max_context_len, int32_t num_q_heads, float scale,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * paged_attention_prefill_chunk_workspace_bytes: bytes of the optional workspace of
 * paged_attention_prefill_chunk for this head layout on the current device (two
 * partial states of 128 rows per resident workgroup); 0 for an unsupported layout.
 */
size_t paged_attention_prefill_chunk_workspace_bytes(int32_t num_q_heads, int32_t num_kv_heads,
                                                     int32_t head_dim);

/*
 * swap_blocks -- preemption by swapping ("2.1 PagedAttention", section 7: a
 * request's KV blocks are copied from GPU memory to CPU memory and back when it
 * resumes).  For each pair (src, dst) of block_mapping, the whole block (all kv
 * heads, K and V) src of the source pools is copied to block dst of the
 * destination pools.  Either side may be device memory or pinned host memory
 * (hipHostMalloc, torch's pin_memory); the copies are DMA transfers enqueued on
 * the stream (runs of consecutive pairs become one transfer).
 *   dst_k, dst_v      [dst_num_blocks][num_kv_heads][block_size][head_dim]
 *   src_k, src_v      [src_num_blocks][num_kv_heads][block_size][head_dim]
 *   block_mapping     int64 [num_pairs][2] (src, dst) in HOST memory, read before
 *                     the call returns; destinations distinct.
 * Errors: PKV_ERR_SHAPE for an id out of range (nothing enqueued); PKV_ERR_LAUNCH if
 * the runtime refuses a copy (earlier copies of the call may have been enqueued).
 */
pkv_status swap_blocks(pkv_dtype dtype, void* dst_k, void* dst_v, int32_t dst_num_blocks,
                       const void* src_k, const void* src_v, int32_t src_num_blocks,
                       int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                       const int64_t* block_mapping, int32_t num_pairs, hipStream_t stream);

/*
 * Host block manager ("2.1 PagedAttention", the V1 engine walk-through: the block
 * pool with per-block reference counts and a doubly linked free queue; "Inside
 * vLLM, part 2": prefix caching by chained block hashes).  Pure host code; one pool
 * per KV cache; not thread-safe (one caller at a time).
 *
 * Free queue: initially blocks 0..n-1 in order.  allocate takes blocks from its
 * head (a block that still carried a prefix hash loses it: its contents will be
 * overwritten).  free decrements counts in the order given -- a request passes
 * its blocks tail first -- and a block reaching zero goes to the queue's tail if
 * it carries a hash (kept longer, reusable) or to its head otherwise (reused
 * first).  touch revives blocks on a prefix-cache hit: a block at zero leaves the
 * queue (wherever it is) and every count goes up by one.
 */
typedef struct pkv_block_pool pkv_block_pool;

/* A pool of num_blocks blocks, all free; NULL if num_blocks <= 0 or out of memory. */
pkv_block_pool* pkv_pool_create(int32_t num_blocks);
void pkv_pool_destroy(pkv_block_pool* pool);
/* Free blocks (-1 for a NULL pool). */
int32_t pkv_pool_num_free(const pkv_block_pool* pool);
/* Reference count of block id (-1 if out of range). */
int32_t pkv_pool_ref_count(const pkv_block_pool* pool, int32_t id);
/* n blocks from the head of the free queue into ids[n], each with count 1;
 * PKV_ERR_NO_BLOCKS (and nothing taken) when fewer than n are free. */
pkv_status pkv_pool_allocate(pkv_block_pool* pool, int32_t n, int32_t* ids);
/* Drop one reference per listed id (PKV_ERR_SHAPE, nothing changed, if an id is out
 * of range or listed more often than it is referenced). */
pkv_status pkv_pool_free(pkv_block_pool* pool, const int32_t* ids, int32_t n);
/* Add one reference per listed id; blocks at zero leave the free queue. */
pkv_status pkv_pool_touch(pkv_block_pool* pool, const int32_t* ids, int32_t n);
/* Index full blocks under their hashes.  A block that already has a hash, or a hash
 * already held by another block, is left as it is. */
pkv_status pkv_pool_cache_blocks(pkv_block_pool* pool, const int32_t* ids,
                                 const uint64_t* hashes, int32_t n);
/* Longest cached prefix: the number k of leading hashes[] found (stopping at the
 * first miss), their blocks in ids[0..k); -1 on a bad argument. */
int32_t pkv_pool_longest_hit(const pkv_block_pool* pool, const uint64_t* hashes, int32_t n,
                             int32_t* ids);
/* Copy-on-write trigger ("2.1 PagedAttention", section 6) before writing into block
 * id: sole owner (count 1) -> *out_id = id, *copy_needed = 0; shared -> a fresh
 * block is allocated, id loses the writer's reference, *out_id = the fresh block and
 * *copy_needed = 1 (the caller copies with copy_blocks and re-points its table).
 * PKV_ERR_NO_BLOCKS when no block is free (nothing changed). */
pkv_status pkv_pool_cow(pkv_block_pool* pool, int32_t id, int32_t* out_id, int32_t* copy_needed);
/* The free queue from head to tail into ids[0..capacity); returns its length. */
int32_t pkv_pool_free_queue(const pkv_block_pool* pool, int32_t* ids, int32_t capacity);
/* Chained block hash: 64-bit FNV-1a over the parent hash (8 bytes, little endian)
 * followed by the block's token ids (4 bytes each, little endian). */
uint64_t pkv_block_hash(uint64_t parent, const int32_t* tokens, int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
