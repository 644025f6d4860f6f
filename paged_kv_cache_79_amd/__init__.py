"""paged_kv_cache_79_amd -- PagedAttention over a block-table KV cache on MI355X (gfx950).

Thin Python binding of ``libpagedkv.so`` (C ABI declared in ``include/pagedkv.h``).
The functions here only marshal torch device tensors into pointers, sizes and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  There is no fallback: if the library is not built, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

# every symbol include/pagedkv.h declares
EXPORTS = (
    "pkv_status_string",
    "pkv_validate",
    "pkv_validate_chunks",
    "paged_kv_write",
    "copy_blocks",
    "paged_attention_decode_workspace_bytes",
    "paged_attention_decode",
    "paged_attention_decode_noalloc_scratch_bytes",
    "paged_attention_decode_noalloc",
    "contiguous_attention_decode",
    "paged_attention_decode_shared_prefix_workspace_bytes",
    "paged_attention_decode_shared_prefix",
    "paged_attention_decode_multi_query_workspace_bytes",
    "paged_attention_decode_multi_query",
    "paged_attention_prefill_chunk_workspace_bytes",
    "paged_attention_prefill_chunk",
    "swap_blocks",
    "pkv_pool_create",
    "pkv_pool_destroy",
    "pkv_pool_num_free",
    "pkv_pool_ref_count",
    "pkv_pool_allocate",
    "pkv_pool_free",
    "pkv_pool_touch",
    "pkv_pool_cache_blocks",
    "pkv_pool_longest_hit",
    "pkv_pool_cow",
    "pkv_pool_free_queue",
    "pkv_block_hash",
)

PKV_F32, PKV_BF16 = 0, 1
PKV_ERR_VALIDATION = 7
PKV_ERR_NO_BLOCKS = 8

_lib = None


class PagedKVError(RuntimeError):
    """A non-zero pkv_status returned by the library."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def load_library(path: Optional[str] = None):
    """Load libpagedkv.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with paged_kv_cache_79_amd.build.build_library()")
    lib = ctypes.CDLL(p)
    I32, I64, SZ, VP, F = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.paged_kv_write.argtypes = [ctypes.c_int, VP, VP, I32, I32, I32, I32, VP, VP, VP, I32, VP]
    lib.paged_kv_write.restype = ctypes.c_int
    lib.copy_blocks.argtypes = [ctypes.c_int, VP, VP, I32, I32, I32, I32, VP, I32, VP]
    lib.copy_blocks.restype = ctypes.c_int
    lib.paged_attention_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.paged_attention_decode_workspace_bytes.restype = SZ
    lib.paged_attention_decode.argtypes = [ctypes.c_int, VP, VP, VP, VP, I32, I32, I32, I32, VP, I32,
                                           VP, I32, I32, I32, F, I32, VP, SZ, VP]
    lib.paged_attention_decode.restype = ctypes.c_int
    lib.paged_attention_decode_noalloc_scratch_bytes.argtypes = []
    lib.paged_attention_decode_noalloc_scratch_bytes.restype = SZ
    lib.paged_attention_decode_noalloc.argtypes = [ctypes.c_int, VP, VP, VP, VP, I32, I32, I32, I32,
                                                   VP, I32, VP, I32, I32, I32, F, I32, VP]
    lib.paged_attention_decode_noalloc.restype = ctypes.c_int
    lib.contiguous_attention_decode.argtypes = [ctypes.c_int, VP, VP, VP, VP, I32, I32, I32, I32, VP,
                                                I32, I32, F, VP, SZ, VP]
    lib.contiguous_attention_decode.restype = ctypes.c_int
    lib.paged_attention_decode_shared_prefix_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.paged_attention_decode_shared_prefix_workspace_bytes.restype = SZ
    lib.paged_attention_decode_shared_prefix.argtypes = [
        ctypes.c_int, VP, VP, VP, VP, I32, I32, I32, I32, VP, I32, VP, I32, I32, I32, F,
        VP, VP, VP, VP, I32, I32, I32, VP, SZ, VP]
    lib.paged_attention_decode_shared_prefix.restype = ctypes.c_int
    lib.paged_attention_decode_multi_query_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.paged_attention_decode_multi_query_workspace_bytes.restype = SZ
    lib.paged_attention_decode_multi_query.argtypes = [
        ctypes.c_int, VP, VP, VP, VP, I32, I32, I32, I32, VP, I32, VP, I32, I32, I32, I32, F, VP,
        SZ, VP]
    lib.paged_attention_decode_multi_query.restype = ctypes.c_int
    lib.paged_attention_prefill_chunk_workspace_bytes.argtypes = [I32, I32, I32]
    lib.paged_attention_prefill_chunk_workspace_bytes.restype = SZ
    lib.paged_attention_prefill_chunk.argtypes = [ctypes.c_int, VP, VP, VP, I32, I32, VP, VP, I32, I32,
                                                  I32, I32, VP, I32, VP, I32, I32, F, VP, SZ, VP]
    lib.paged_attention_prefill_chunk.restype = ctypes.c_int
    U64 = ctypes.c_uint64
    lib.swap_blocks.argtypes = [ctypes.c_int, VP, VP, I32, VP, VP, I32, I32, I32, I32, VP, I32, VP]
    lib.swap_blocks.restype = ctypes.c_int
    lib.pkv_validate.argtypes = [I32, I32, VP, I32, VP, I32, VP, I32, VP, I32, VP, VP]
    lib.pkv_validate.restype = ctypes.c_int
    lib.pkv_validate_chunks.argtypes = [VP, VP, I32, I32, VP, VP]
    lib.pkv_validate_chunks.restype = ctypes.c_int
    lib.pkv_pool_create.argtypes = [I32]
    lib.pkv_pool_create.restype = VP
    lib.pkv_pool_destroy.argtypes = [VP]
    lib.pkv_pool_destroy.restype = None
    for fn in ("pkv_pool_num_free",):
        getattr(lib, fn).argtypes = [VP]
        getattr(lib, fn).restype = I32
    lib.pkv_pool_ref_count.argtypes = [VP, I32]
    lib.pkv_pool_ref_count.restype = I32
    lib.pkv_pool_allocate.argtypes = [VP, I32, VP]
    lib.pkv_pool_allocate.restype = ctypes.c_int
    lib.pkv_pool_free.argtypes = [VP, VP, I32]
    lib.pkv_pool_free.restype = ctypes.c_int
    lib.pkv_pool_touch.argtypes = [VP, VP, I32]
    lib.pkv_pool_touch.restype = ctypes.c_int
    lib.pkv_pool_cache_blocks.argtypes = [VP, VP, VP, I32]
    lib.pkv_pool_cache_blocks.restype = ctypes.c_int
    lib.pkv_pool_longest_hit.argtypes = [VP, VP, I32, VP]
    lib.pkv_pool_longest_hit.restype = I32
    lib.pkv_pool_cow.argtypes = [VP, I32, VP, VP]
    lib.pkv_pool_cow.restype = ctypes.c_int
    lib.pkv_pool_free_queue.argtypes = [VP, VP, I32]
    lib.pkv_pool_free_queue.restype = I32
    lib.pkv_block_hash.argtypes = [U64, VP, I32]
    lib.pkv_block_hash.restype = U64
    del I64
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().pkv_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PagedKVError(fn, status, status_string(status))


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float32:
        return PKV_F32
    raise TypeError(f"unsupported element type {t.dtype} (bfloat16 or float32)")


def _dev(t, name, dtype=None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _ptr(t) -> Optional[int]:
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _pool_geom(k_pool, v_pool):
    if k_pool.shape != v_pool.shape or k_pool.dtype != v_pool.dtype or k_pool.dim() != 4:
        raise ValueError("k_pool and v_pool must both be [num_blocks][num_kv_heads][block_size][head_dim]")
    nb, hkv, bs, d = (int(x) for x in k_pool.shape)
    return nb, hkv, bs, d


# ----------------------------------------------------------------------------
# the four operations (same names as the C entry points)
# ----------------------------------------------------------------------------
def paged_kv_write(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None) -> None:
    """k_pool/v_pool[slot // bs][:, slot % bs, :] = k_new/v_new[i] for every slot >= 0."""
    import torch
    for n, t in (("k_pool", k_pool), ("v_pool", v_pool), ("k_new", k_new), ("v_new", v_new)):
        _dev(t, n)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    T = int(slot_mapping.shape[0])
    if tuple(k_new.shape) != (T, hkv, d) or k_new.shape != v_new.shape or k_new.dtype != k_pool.dtype:
        raise ValueError("k_new/v_new must be [num_tokens][num_kv_heads][head_dim] of the pool dtype")
    lib = load_library()
    _check("paged_kv_write", lib.paged_kv_write(
        _dtype_code(k_pool), _ptr(k_pool), _ptr(v_pool), nb, hkv, bs, d, _ptr(k_new), _ptr(v_new),
        _ptr(slot_mapping), T, _stream(stream)))


def copy_blocks(k_pool, v_pool, block_mapping, stream=None) -> None:
    """Copy whole blocks (src -> dst pairs, int64 [n][2]) of both pools."""
    import torch
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool")
    _dev(block_mapping, "block_mapping", torch.int64)
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    n = int(block_mapping.shape[0]) if block_mapping.numel() else 0
    if block_mapping.numel() and (block_mapping.dim() != 2 or block_mapping.shape[1] != 2):
        raise ValueError("block_mapping must be int64 [n][2]")
    lib = load_library()
    _check("copy_blocks", lib.copy_blocks(
        _dtype_code(k_pool), _ptr(k_pool), _ptr(v_pool), nb, hkv, bs, d, _ptr(block_mapping), n,
        _stream(stream)))


def decode_workspace(num_bytes: int, device, stream=None):
    """Device scratch for a call (its contents need no initialisation).

    The caching allocator ties a block to the stream it was allocated on and hands it
    out again only in that stream's order, so a workspace for a call on ``stream`` is
    allocated on ``stream``: when the binding drops it after enqueuing, no allocation
    on another stream can reuse the memory while the kernels still write to it."""
    import torch
    if stream is None:
        return torch.empty(max(int(num_bytes), 1), dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(max(int(num_bytes), 1), dtype=torch.uint8, device=device)


def paged_attention_decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                           head_dim: int, max_context_len: int,
                                           partition_tokens: int = 0) -> int:
    return int(load_library().paged_attention_decode_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_tokens))


def paged_attention_decode(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
                           scale: float, partition_tokens: int = 0, workspace=None, stream=None) -> None:
    """Decode attention of q [S][Hq][D] over each sequence's paged context into out."""
    import torch
    for n, t in (("out", out), ("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(t, n)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    S, hq = int(q.shape[0]), int(q.shape[1])
    if q.dim() != 3 or q.shape[2] != d or out.shape != q.shape or q.dtype != k_pool.dtype or out.dtype != q.dtype:
        raise ValueError("q/out must be [num_seqs][num_q_heads][head_dim] of the pool dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs][max_blocks], context_lens [num_seqs]")
    need = paged_attention_decode_workspace_bytes(S, hq, hkv, d, max_context_len, partition_tokens)
    if workspace is None and need > 0:
        workspace = decode_workspace(need, q.device, stream)
    if workspace is not None:
        _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    _check("paged_attention_decode", lib.paged_attention_decode(
        _dtype_code(q), _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), nb, hkv, bs, d,
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), S, int(max_context_len),
        hq, float(scale), int(partition_tokens), _ptr(workspace), wbytes, _stream(stream)))


def paged_attention_decode_noalloc_scratch_bytes() -> int:
    return int(load_library().paged_attention_decode_noalloc_scratch_bytes())


def paged_attention_decode_noalloc(out, q, k_pool, v_pool, block_tables, context_lens,
                                   max_context_len: int, scale: float, partition_tokens: int = 0,
                                   stream=None) -> None:
    """paged_attention_decode through the library's fixed per-device scratch: nothing is
    allocated (for graph capture and callers that cannot allocate).  Calls that overlap
    in time on one device share that scratch and race."""
    import torch
    for n, t in (("out", out), ("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(t, n)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    S, hq = int(q.shape[0]), int(q.shape[1])
    if q.dim() != 3 or q.shape[2] != d or out.shape != q.shape or q.dtype != k_pool.dtype or out.dtype != q.dtype:
        raise ValueError("q/out must be [num_seqs][num_q_heads][head_dim] of the pool dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs][max_blocks], context_lens [num_seqs]")
    lib = load_library()
    _check("paged_attention_decode_noalloc", lib.paged_attention_decode_noalloc(
        _dtype_code(q), _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), nb, hkv, bs, d,
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), S, int(max_context_len),
        hq, float(scale), int(partition_tokens), _stream(stream)))


def contiguous_attention_decode(out, q, k_cache, v_cache, context_lens, max_context_len: int,
                                scale: float, workspace=None, stream=None) -> None:
    """The unpaged baseline: decode attention over K/V stored contiguously per sequence,
    k_cache/v_cache [S][max_len][Hkv][D] bf16 (max_len a multiple of 64)."""
    import torch
    for n, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, n)
    _dev(context_lens, "context_lens", torch.int32)
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or not k_cache.is_contiguous() or \
            not v_cache.is_contiguous():
        raise ValueError("k_cache/v_cache must be contiguous [num_seqs][max_len][num_kv_heads][head_dim]")
    S, L, hkv, d = (int(x) for x in k_cache.shape)
    hq = int(q.shape[1])
    if q.dim() != 3 or q.shape[0] != S or q.shape[2] != d or out.shape != q.shape or \
            q.dtype != k_cache.dtype or out.dtype != q.dtype or context_lens.shape != (S,):
        raise ValueError("q/out must be [num_seqs][num_q_heads][head_dim] of the cache dtype")
    need = paged_attention_decode_workspace_bytes(S, hq, hkv, d, max_context_len, 0)
    if workspace is None and need > 0:
        workspace = decode_workspace(need, q.device, stream)
    if workspace is not None:
        _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    _check("contiguous_attention_decode", lib.contiguous_attention_decode(
        _dtype_code(q), _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), S, L, hkv, d,
        _ptr(context_lens), int(max_context_len), hq, float(scale), _ptr(workspace), wbytes,
        _stream(stream)))


def paged_attention_decode_shared_prefix_workspace_bytes(num_seqs: int, num_q_heads: int,
                                                         num_kv_heads: int, head_dim: int,
                                                         max_context_len: int,
                                                         max_prefix_len: int) -> int:
    return int(load_library().paged_attention_decode_shared_prefix_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, max_prefix_len))


def paged_attention_decode_shared_prefix(out, q, k_pool, v_pool, block_tables, context_lens,
                                         max_context_len: int, scale: float, seq_prefix_lens,
                                         group_first_seq, group_num_seqs, group_prefix_lens,
                                         max_group_seqs: int, max_prefix_len: int, workspace=None,
                                         stream=None) -> None:
    """paged_attention_decode for batches whose groups of consecutive sequences share the
    physical blocks of a prefix: the prefix K/V is read once per group and kv head.
    Group arrays are int32 device tensors of one length; max_group_seqs and
    max_prefix_len are host bounds over them."""
    import torch
    for n, t in (("out", out), ("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(t, n)
    for n, t in (("block_tables", block_tables), ("context_lens", context_lens),
                 ("seq_prefix_lens", seq_prefix_lens), ("group_first_seq", group_first_seq),
                 ("group_num_seqs", group_num_seqs), ("group_prefix_lens", group_prefix_lens)):
        _dev(t, n, torch.int32)
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    S, hq = int(q.shape[0]), int(q.shape[1])
    if q.dim() != 3 or q.shape[2] != d or out.shape != q.shape or q.dtype != k_pool.dtype or \
            out.dtype != q.dtype:
        raise ValueError("q/out must be [num_seqs][num_q_heads][head_dim] of the pool dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,) or \
            seq_prefix_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs][max_blocks], context_lens and "
                         "seq_prefix_lens [num_seqs]")
    G = int(group_first_seq.numel())
    if group_num_seqs.numel() != G or group_prefix_lens.numel() != G:
        raise ValueError("group_first_seq, group_num_seqs, group_prefix_lens differ in length")
    need = paged_attention_decode_shared_prefix_workspace_bytes(S, hq, hkv, d, max_context_len,
                                                                max_prefix_len)
    if workspace is None and need > 0:
        workspace = decode_workspace(need, q.device, stream)
    if workspace is not None:
        _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    _check("paged_attention_decode_shared_prefix", lib.paged_attention_decode_shared_prefix(
        _dtype_code(q), _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), nb, hkv, bs, d,
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), S,
        int(max_context_len), hq, float(scale), _ptr(seq_prefix_lens), _ptr(group_first_seq),
        _ptr(group_num_seqs), _ptr(group_prefix_lens), G, int(max_group_seqs),
        int(max_prefix_len), _ptr(workspace), wbytes, _stream(stream)))


def paged_attention_decode_multi_query_workspace_bytes(num_seqs: int, queries_per_seq: int,
                                                       num_q_heads: int, num_kv_heads: int,
                                                       head_dim: int) -> int:
    return int(load_library().paged_attention_decode_multi_query_workspace_bytes(
        num_seqs, queries_per_seq, num_q_heads, num_kv_heads, head_dim))


def paged_attention_decode_multi_query(out, q, k_pool, v_pool, block_tables, context_lens,
                                       queries_per_seq: int, max_context_len: int, scale: float,
                                       workspace=None, stream=None) -> None:
    """Decode with n = queries_per_seq causal queries per sequence (speculative
    verification): q/out [num_seqs * n][Hq][D] bf16, query i of sequence s at position
    context_lens[s] - n + i."""
    import torch
    for nm, t in (("out", out), ("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(t, nm)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    n = int(queries_per_seq)
    S = int(context_lens.shape[0])
    hq = int(q.shape[1])
    if q.dim() != 3 or q.shape[0] != S * n or q.shape[2] != d or out.shape != q.shape or \
            q.dtype != k_pool.dtype or out.dtype != q.dtype:
        raise ValueError("q/out must be [num_seqs * queries_per_seq][num_q_heads][head_dim] of the "
                         "pool dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [num_seqs][max_blocks]")
    need = paged_attention_decode_multi_query_workspace_bytes(S, n, hq, hkv, d)
    if workspace is None and need > 0:
        workspace = decode_workspace(need, q.device, stream)
    if workspace is not None:
        _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    _check("paged_attention_decode_multi_query", lib.paged_attention_decode_multi_query(
        _dtype_code(q), _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), nb, hkv, bs, d,
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), S, n,
        int(max_context_len), hq, float(scale), _ptr(workspace), wbytes, _stream(stream)))


def paged_attention_prefill_chunk_workspace_bytes(num_q_heads: int, num_kv_heads: int,
                                                  head_dim: int) -> int:
    return int(load_library().paged_attention_prefill_chunk_workspace_bytes(
        num_q_heads, num_kv_heads, head_dim))


def paged_attention_prefill_chunk(out, q, cu_q_lens, k_pool, v_pool, block_tables, context_lens,
                                  max_q_len: int, max_context_len: int, scale: float,
                                  workspace=None, split: bool = True, stream=None) -> None:
    """Causal attention of prefill chunks (the last n_q positions of each context).

    With ``split`` (the default) the call gets a workspace (``workspace``, or a fresh
    one), so the library may balance uneven chunks by splitting their keys; with
    ``split=False`` it passes none and every query tile is one workgroup."""
    import torch
    for n, t in (("out", out), ("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(t, n)
    _dev(cu_q_lens, "cu_q_lens", torch.int32)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    nc = int(context_lens.shape[0])
    if q.dim() != 3 or q.shape[2] != d or out.shape != q.shape or q.dtype != k_pool.dtype or out.dtype != q.dtype:
        raise ValueError("q/out must be [total_q][num_q_heads][head_dim] of the pool dtype")
    if cu_q_lens.shape != (nc + 1,) or block_tables.dim() != 2 or block_tables.shape[0] != nc:
        raise ValueError("cu_q_lens must be [chunks + 1], block_tables [chunks][max_blocks]")
    lib = load_library()
    if not split:
        workspace = None
    elif workspace is None:
        need = paged_attention_prefill_chunk_workspace_bytes(int(q.shape[1]), hkv, d)
        if need > 0:
            workspace = decode_workspace(need, q.device, stream)
    if workspace is not None:
        _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("paged_attention_prefill_chunk", lib.paged_attention_prefill_chunk(
        _dtype_code(q), _ptr(out), _ptr(q), _ptr(cu_q_lens), nc, int(max_q_len), _ptr(k_pool),
        _ptr(v_pool), nb, hkv, bs, d, _ptr(block_tables), int(block_tables.shape[1]),
        _ptr(context_lens), int(max_context_len), int(q.shape[1]), float(scale), _ptr(workspace),
        wbytes, _stream(stream)))


# ----------------------------------------------------------------------------
# swapping and the host block manager
# ----------------------------------------------------------------------------
def swap_blocks(dst_k, dst_v, src_k, src_v, block_mapping, stream=None) -> None:
    """Copy whole blocks src -> dst (pairs of block_mapping, a host int64 [n][2] array)
    between pools in device memory or pinned host memory, as DMA copies on the stream."""
    import numpy as np
    for n, t in (("dst_k", dst_k), ("dst_v", dst_v), ("src_k", src_k), ("src_v", src_v)):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
        if not t.is_cuda and not t.is_pinned():
            raise ValueError(f"{n} must be device memory or pinned host memory")
    if dst_k.dim() != 4 or src_k.dim() != 4 or dst_k.shape[1:] != src_k.shape[1:] or \
            dst_v.shape != dst_k.shape or src_v.shape != src_k.shape or dst_k.dtype != src_k.dtype:
        raise ValueError("pools must be [num_blocks][num_kv_heads][block_size][head_dim] of one dtype")
    m = np.ascontiguousarray(np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2))
    _, hkv, bs, d = (int(x) for x in src_k.shape)
    lib = load_library()
    _check("swap_blocks", lib.swap_blocks(
        _dtype_code(src_k), _ptr(dst_k), _ptr(dst_v), int(dst_k.shape[0]), _ptr(src_k), _ptr(src_v),
        int(src_k.shape[0]), hkv, bs, d, m.ctypes.data if m.size else None, int(m.shape[0]),
        _stream(stream)))


def validate(num_blocks: int, block_size: int, block_tables=None, context_lens=None,
             slot_mapping=None, block_mapping=None, stream=None) -> dict:
    """Device-side check of the preconditions the other calls trust (pkv_validate):
    returns the violation counts after synchronising the stream."""
    import torch
    dev_t = None
    for n, t, dt in (("block_tables", block_tables, torch.int32),
                     ("context_lens", context_lens, torch.int32),
                     ("slot_mapping", slot_mapping, torch.int64),
                     ("block_mapping", block_mapping, torch.int64)):
        if t is not None:
            _dev(t, n, dt)
            dev_t = t
    if dev_t is None:
        raise ValueError("nothing to validate")
    S = 0 if context_lens is None else int(context_lens.numel())
    if S and (block_tables is None or block_tables.dim() != 2 or block_tables.shape[0] != S):
        raise ValueError("block_tables must be [num_seqs][max_blocks] with context_lens [num_seqs]")
    mb = int(block_tables.shape[1]) if block_tables is not None and block_tables.dim() == 2 else 0
    T = 0 if slot_mapping is None else int(slot_mapping.numel())
    n = 0 if block_mapping is None else int(block_mapping.numel()) // 2
    if stream is None:
        counts = torch.empty(4, dtype=torch.int32, device=dev_t.device)
    else:
        with torch.cuda.stream(stream):
            counts = torch.empty(4, dtype=torch.int32, device=dev_t.device)
    _check("pkv_validate", load_library().pkv_validate(
        int(num_blocks), int(block_size), _ptr(block_tables), mb, _ptr(context_lens), S,
        _ptr(slot_mapping), T, _ptr(block_mapping), n, _ptr(counts), _stream(stream)))
    if stream is None:
        torch.cuda.current_stream(dev_t.device).synchronize()
    else:
        stream.synchronize()
    c = counts.cpu().tolist()
    return {"bad_table_entries": c[0], "bad_context_lens": c[1], "bad_slots": c[2],
            "bad_copy_pairs": c[3]}


def validate_chunks(cu_q_lens, context_lens, total_q: int = -1, stream=None) -> int:
    """Device-side check of prefill chunk descriptors (pkv_validate_chunks): the number
    of malformed chunks, after synchronising the stream."""
    import torch
    _dev(cu_q_lens, "cu_q_lens", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    n = int(context_lens.numel())
    if cu_q_lens.numel() != n + 1:
        raise ValueError("cu_q_lens must hold num_chunks + 1 entries")
    if stream is None:
        count = torch.zeros(1, dtype=torch.int32, device=context_lens.device)
    else:
        with torch.cuda.stream(stream):
            count = torch.zeros(1, dtype=torch.int32, device=context_lens.device)
    _check("pkv_validate_chunks", load_library().pkv_validate_chunks(
        _ptr(cu_q_lens), _ptr(context_lens), n, int(total_q), _ptr(count), _stream(stream)))
    (torch.cuda.current_stream(context_lens.device) if stream is None else stream).synchronize()
    return int(count.item())


def check_preconditions(num_blocks: int, block_size: int, **kw) -> None:
    """validate(), raising PagedKVError (PKV_ERR_VALIDATION) if anything is violated."""
    c = validate(num_blocks, block_size, **kw)
    if any(c.values()):
        raise PagedKVError("pkv_validate", PKV_ERR_VALIDATION, str(c))


def block_hash(parent: int, tokens) -> int:
    """Chained hash of a full block: FNV-1a 64 over the parent hash and the token ids."""
    import numpy as np
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    return int(load_library().pkv_block_hash(ctypes.c_uint64(parent & (2**64 - 1)),
                                             t.ctypes.data if t.size else None, int(t.size)))


class BlockPool:
    """The library's host block manager (pkv_pool_*): reference counts, the doubly
    linked free queue, prefix-hash index and the copy-on-write trigger."""

    def __init__(self, num_blocks: int):
        self._lib = load_library()
        self._h = self._lib.pkv_pool_create(int(num_blocks))
        if not self._h:
            raise ValueError("pkv_pool_create failed (num_blocks must be positive)")

    def close(self):
        if self._h:
            self._lib.pkv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _ids(ids):
        import numpy as np
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).reshape(-1))
        return a, (a.ctypes.data if a.size else None), int(a.size)

    @property
    def num_free(self) -> int:
        return int(self._lib.pkv_pool_num_free(self._h))

    def ref_count(self, block_id: int) -> int:
        return int(self._lib.pkv_pool_ref_count(self._h, int(block_id)))

    def allocate(self, n: int):
        """n blocks from the head of the free queue, or None when fewer are free."""
        import numpy as np
        out = np.zeros(max(int(n), 1), dtype=np.int32)
        st = self._lib.pkv_pool_allocate(self._h, int(n), out.ctypes.data)
        if st == PKV_ERR_NO_BLOCKS:
            return None
        _check("pkv_pool_allocate", st)
        return out[:int(n)].tolist()

    def free(self, ids) -> None:
        a, p, n = self._ids(ids)
        _check("pkv_pool_free", self._lib.pkv_pool_free(self._h, p, n))

    def touch(self, ids) -> None:
        a, p, n = self._ids(ids)
        _check("pkv_pool_touch", self._lib.pkv_pool_touch(self._h, p, n))

    def cache_blocks(self, ids, hashes) -> None:
        import numpy as np
        a, p, n = self._ids(ids)
        h = np.ascontiguousarray(np.asarray([x & (2**64 - 1) for x in hashes], dtype=np.uint64))
        if h.size != n:
            raise ValueError("one hash per block")
        _check("pkv_pool_cache_blocks", self._lib.pkv_pool_cache_blocks(
            self._h, p, h.ctypes.data if h.size else None, n))

    def longest_hit(self, hashes):
        """Blocks of the longest prefix of hashes that is cached."""
        import numpy as np
        h = np.ascontiguousarray(np.asarray([x & (2**64 - 1) for x in hashes], dtype=np.uint64))
        out = np.zeros(max(h.size, 1), dtype=np.int32)
        k = self._lib.pkv_pool_longest_hit(self._h, h.ctypes.data if h.size else None, int(h.size),
                                           out.ctypes.data)
        if k < 0:
            raise ValueError("pkv_pool_longest_hit: bad argument")
        return out[:k].tolist()

    def cow(self, block_id: int):
        """(block to write, copy needed) before writing into block_id; None if no block
        is free for the private copy."""
        a = ctypes.c_int32(0)
        c = ctypes.c_int32(0)
        st = self._lib.pkv_pool_cow(self._h, int(block_id), ctypes.byref(a), ctypes.byref(c))
        if st == PKV_ERR_NO_BLOCKS:
            return None
        _check("pkv_pool_cow", st)
        return int(a.value), bool(c.value)

    def free_queue(self):
        import numpy as np
        n = self._lib.pkv_pool_free_queue(self._h, None, 0)
        out = np.zeros(max(n, 1), dtype=np.int32)
        self._lib.pkv_pool_free_queue(self._h, out.ctypes.data, n)
        return out[:n].tolist()
