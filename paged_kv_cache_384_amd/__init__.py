"""Paged KV-cache attention (decode and prefill) for AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libpa.so`` (declared in ``include/pa.h``). The
functions keep the C names and only marshal arguments: torch tensors become device pointers,
the current torch stream becomes the HIP stream. Every step of the computation runs in the HIP
kernels; there is no fallback. If the library is not built, the first call raises.

    pa_reshape_and_cache(key_cache, value_cache, key, value, block_tables, token_seq, token_pos)
    pa_decode(out, query, key_cache, value_cache, block_tables, context_lens, scale,
              max_context_len, partition_size=0, workspace=None)
    pa_decode_static(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                     max_context_len, partition_size=0)        # allocates nothing
    pa_prefill(out, query, key_cache, value_cache, block_tables, query_start, context_lens,
               scale, max_query_len, max_context_len)
    pa_copy_blocks(key_cache, value_cache, src_dst)

Pools are tensors of shape [num_blocks, num_kv_heads, block_size * head_dim] in the element
dtype; the order of elements inside each (block, head) tile is the library's (see pa.h). The
block size (8, 16 or 32) is read off the pool shape unless passed as ``block_size``.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "PaError", "lib", "library_path", "pa_reshape_and_cache", "pa_decode", "pa_decode_static",
    "pa_decode_attention", "STATIC_WORKSPACE_BYTES",
    "pa_decode_reduce", "pa_decode_contiguous", "pa_prefill", "pa_swap_blocks",
    "pa_decode_workspace_bytes", "pa_copy_blocks", "pa_validate_tables", "pa_validate_writes",
    "pa_measure_tile_read",
    "pa_status_string",
    "pa_abi_version", "ABI_VERSION", "CACHE_SHARED_BLOCKS", "DTYPE_CODES", "EXPORTED_SYMBOLS",
]

ABI_VERSION = 7
STATIC_WORKSPACE_BYTES = 32 * 1024 * 1024  # PA_STATIC_WORKSPACE_BYTES
CACHE_SHARED_BLOCKS = 1  # pa_cache_desc.flags bit: blocks may be shared by several sequences
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY selects another build of the same library (e.g. one with host-side sanitizers)
library_path = os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpa.so")

EXPORTED_SYMBOLS = ["pa_reshape_and_cache", "pa_decode_workspace_bytes", "pa_decode",
                    "pa_decode_static",
                    "pa_decode_attention", "pa_decode_reduce", "pa_decode_contiguous",
                    "pa_prefill", "pa_copy_blocks", "pa_swap_blocks", "pa_validate_tables",
                    "pa_validate_writes", "pa_measure_tile_read", "pa_status_string",
                    "pa_abi_version"]


class CacheDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({pa_status_string(status)})")


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_desc_p = ctypes.POINTER(CacheDesc)
_DECODE_ARGS = [_desc_p, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, ctypes.c_float, _i32,
                _i32, _vp, ctypes.c_size_t, _vp]


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is missing: build it first (python -m paged_kv_cache_384_amd._build"
                " or __graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(library_path)
        L.pa_reshape_and_cache.argtypes = [_desc_p, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp,
                                           _i32, _vp]
        L.pa_reshape_and_cache.restype = ctypes.c_int
        L.pa_decode_workspace_bytes.argtypes = [_desc_p, _i32, _i32, _i32, _i32]
        L.pa_decode_workspace_bytes.restype = ctypes.c_size_t
        for name in ("pa_decode", "pa_decode_attention", "pa_decode_reduce"):
            getattr(L, name).argtypes = _DECODE_ARGS
            getattr(L, name).restype = ctypes.c_int
        L.pa_decode_static.argtypes = _DECODE_ARGS[:13] + [_vp]
        L.pa_decode_static.restype = ctypes.c_int
        L.pa_decode_contiguous.argtypes = [_desc_p, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                           ctypes.c_float, _i32, _i32, _vp, ctypes.c_size_t, _vp]
        L.pa_decode_contiguous.restype = ctypes.c_int
        L.pa_prefill.argtypes = [_desc_p, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                 ctypes.c_float, _i32, _i32, _vp]
        L.pa_prefill.restype = ctypes.c_int
        L.pa_swap_blocks.argtypes = [_desc_p, _vp, _vp, _desc_p, _vp, _vp, _vp, _i32, _vp]
        L.pa_swap_blocks.restype = ctypes.c_int
        L.pa_copy_blocks.argtypes = [_desc_p, _vp, _vp, _vp, _i32, _vp]
        L.pa_copy_blocks.restype = ctypes.c_int
        L.pa_validate_tables.argtypes = [_desc_p, _vp, _i32, _i32, _vp, _vp, _i32, _vp, _vp]
        L.pa_validate_tables.restype = ctypes.c_int
        L.pa_validate_writes.argtypes = [_desc_p, _vp, _i32, _i32, _vp, _vp, _i32, _vp, _i32, _vp,
                                         _vp]
        L.pa_validate_writes.restype = ctypes.c_int
        L.pa_measure_tile_read.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp, _vp]
        L.pa_measure_tile_read.restype = ctypes.c_int
        L.pa_status_string.argtypes = [ctypes.c_int]
        L.pa_status_string.restype = ctypes.c_char_p
        L.pa_abi_version.argtypes = []
        L.pa_abi_version.restype = ctypes.c_int32
        if L.pa_abi_version() != ABI_VERSION:
            raise RuntimeError(f"libpa ABI {L.pa_abi_version()} != binding ABI {ABI_VERSION}")
        _lib = L
    return _lib


def pa_status_string(status: int) -> str:
    return lib().pa_status_string(int(status)).decode()


def pa_abi_version() -> int:
    return int(lib().pa_abi_version())


# ---- marshalling helpers ------------------------------------------------------------------

def _dtype_name(t) -> str:
    import torch
    names = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}
    if t.dtype not in names:
        raise TypeError(f"unsupported element dtype {t.dtype}")
    return names[t.dtype]


def _dev(t, what, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    return _vp(t.data_ptr()) if t.numel() else _vp(0)


def _stream(t, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return _vp(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _desc(key_cache, head_dim, block_size=None, shared_blocks=False) -> CacheDesc:
    """The pools' descriptor; the block size is read off the pool shape unless given."""
    if key_cache.dim() != 3 or key_cache.shape[2] % head_dim:
        raise ValueError("pools must be [num_blocks, num_kv_heads, block_size * head_dim]")
    if block_size is None:
        block_size = key_cache.shape[2] // head_dim
    if key_cache.shape[2] != block_size * head_dim:
        raise ValueError("pools must be [num_blocks, num_kv_heads, block_size * head_dim]")
    return CacheDesc(DTYPE_CODES[_dtype_name(key_cache)], key_cache.shape[0], key_cache.shape[1],
                     head_dim, block_size, CACHE_SHARED_BLOCKS if shared_blocks else 0)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise PaError(status, where)


# ---- the calls ----------------------------------------------------------------------------

def pa_reshape_and_cache(key_cache, value_cache, key, value, block_tables, token_seq, token_pos,
                         *, block_size: int | None = None, stream=None) -> None:
    """Write key[n] / value[n] ([T, Hkv, d]) into the slot of (token_seq[n], token_pos[n])."""
    import torch
    head_dim = key.shape[-1]
    d = _desc(key_cache, head_dim, block_size)
    if value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("key and value pools differ in shape or dtype")
    T = token_seq.numel()
    if tuple(key.shape) != (T, d.num_kv_heads, head_dim) or value.shape != key.shape:
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_dim]")
    if token_pos.numel() != T or block_tables.dim() != 2:
        raise ValueError("token_pos must match token_seq; block_tables must be 2-D")
    args = (ctypes.byref(d), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
            _dev(key, "key", key_cache.dtype), _dev(value, "value", key_cache.dtype),
            _dev(block_tables, "block_tables", torch.int32), block_tables.shape[0],
            block_tables.shape[1], _dev(token_seq, "token_seq", torch.int32),
            _dev(token_pos, "token_pos", torch.int32), token_seq.numel(),
            _stream(key_cache, stream))
    _check(lib().pa_reshape_and_cache(*args), "pa_reshape_and_cache")


def pa_decode_workspace_bytes(key_cache, num_seqs: int, num_q_heads: int, head_dim: int,
                              max_context_len: int, partition_size: int = 0,
                              block_size: int | None = None, shared_blocks: bool = False) -> int:
    d = _desc(key_cache, head_dim, block_size, shared_blocks)
    n = lib().pa_decode_workspace_bytes(ctypes.byref(d), num_seqs, num_q_heads, max_context_len,
                                        partition_size)
    if n == ctypes.c_size_t(-1).value:
        raise PaError(2, "pa_decode_workspace_bytes")
    return int(n)


def _decode_call(fn_name, out, query, key_cache, value_cache, block_tables, context_lens, scale,
                 max_context_len, partition_size, workspace, block_size, shared_blocks, stream):
    import torch
    S, Hq, head_dim = query.shape
    d = _desc(key_cache, head_dim, block_size, shared_blocks)
    if out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("out must match query in shape and dtype")
    if value_cache.shape != key_cache.shape:
        raise ValueError("key and value pools differ in shape")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [num_seqs, max_blocks]; context_lens [num_seqs]")
    need = pa_decode_workspace_bytes(key_cache, S, Hq, head_dim, max_context_len, partition_size,
                                     block_size, shared_blocks)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else _vp(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (ctypes.byref(d), _dev(key_cache, "key_cache", query.dtype),
            _dev(value_cache, "value_cache", query.dtype), _dev(out, "out"),
            _dev(query, "query"), _dev(block_tables, "block_tables", torch.int32),
            block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32), S, Hq,
            float(scale), int(max_context_len), int(partition_size), ws_ptr, ws_bytes,
            _stream(query, stream))
    _check(getattr(lib(), fn_name)(*args), fn_name)
    return workspace


def pa_decode(out, query, key_cache, value_cache, block_tables, context_lens, scale,
              max_context_len, partition_size: int = 0, workspace=None, *,
              block_size: int | None = None, shared_blocks: bool = False, stream=None):
    """out[s, h] = attention of query[s, h] over sequence s's paged cache (both stages).

    shared_blocks: some physical blocks are referenced by several sequences in this call, so the
    key/value tiles are read through the caches instead of as a stream, and (16-bit pools,
    head_dim 128) a partition that consecutive sequences share is computed once for up to 8 of
    them; the workspace then also holds the map of those groups.
    Returns the workspace used (allocated with torch when none is given and one is needed).
    """
    return _decode_call("pa_decode", out, query, key_cache, value_cache, block_tables,
                        context_lens, scale, max_context_len, partition_size, workspace,
                        block_size, shared_blocks, stream)


def pa_decode_static(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                     max_context_len, partition_size: int = 0, *, block_size: int | None = None,
                     shared_blocks: bool = False, stream=None) -> None:
    """pa_decode with the partition states in the library's own fixed device array
    (STATIC_WORKSPACE_BYTES per GPU) instead of a workspace: allocates nothing. Calls that
    overlap on one GPU share that array and must be ordered by the caller."""
    import torch
    S, Hq, head_dim = query.shape
    d = _desc(key_cache, head_dim, block_size, shared_blocks)
    if out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("out must match query in shape and dtype")
    if value_cache.shape != key_cache.shape:
        raise ValueError("key and value pools differ in shape")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [num_seqs, max_blocks]; context_lens [num_seqs]")
    args = (ctypes.byref(d), _dev(key_cache, "key_cache", query.dtype),
            _dev(value_cache, "value_cache", query.dtype), _dev(out, "out"),
            _dev(query, "query"), _dev(block_tables, "block_tables", torch.int32),
            block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32), S, Hq,
            float(scale), int(max_context_len), int(partition_size), _stream(query, stream))
    with torch.cuda.device(query.device):  # the library uses the current device's array
        _check(lib().pa_decode_static(*args), "pa_decode_static")


def pa_decode_attention(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                        max_context_len, partition_size: int = 0, workspace=None, *,
                        block_size: int | None = None, shared_blocks: bool = False, stream=None):
    """First stage of pa_decode only (per-partition attention)."""
    return _decode_call("pa_decode_attention", out, query, key_cache, value_cache, block_tables,
                        context_lens, scale, max_context_len, partition_size, workspace,
                        block_size, shared_blocks, stream)


def pa_decode_reduce(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                     max_context_len, partition_size: int = 0, workspace=None, *,
                     block_size: int | None = None, shared_blocks: bool = False, stream=None):
    """Second stage of pa_decode only (merge of partition states)."""
    return _decode_call("pa_decode_reduce", out, query, key_cache, value_cache, block_tables,
                        context_lens, scale, max_context_len, partition_size, workspace,
                        block_size, shared_blocks, stream)


def pa_decode_contiguous(out, query, key_cache, value_cache, context_lens, scale, max_context_len,
                         max_blocks_per_seq, partition_size: int = 0, workspace=None, *,
                         block_size: int | None = None, stream=None):
    """The contiguous twin of pa_decode: sequence s's block j is physical block
    s * max_blocks_per_seq + j (no block table). Returns the workspace used."""
    import torch
    S, Hq, head_dim = query.shape
    d = _desc(key_cache, head_dim, block_size)
    if out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("out must match query in shape and dtype")
    if value_cache.shape != key_cache.shape or context_lens.numel() != S:
        raise ValueError("pools differ in shape, or context_lens is not [num_seqs]")
    need = pa_decode_workspace_bytes(key_cache, S, Hq, head_dim, max_context_len, partition_size,
                                     block_size)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else _vp(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (ctypes.byref(d), _dev(key_cache, "key_cache", query.dtype),
            _dev(value_cache, "value_cache", query.dtype), _dev(out, "out"),
            _dev(query, "query"), int(max_blocks_per_seq),
            _dev(context_lens, "context_lens", torch.int32), S, Hq, float(scale),
            int(max_context_len), int(partition_size), ws_ptr, ws_bytes, _stream(query, stream))
    _check(lib().pa_decode_contiguous(*args), "pa_decode_contiguous")
    return workspace


def pa_prefill(out, query, key_cache, value_cache, block_tables, query_start, context_lens, scale,
               max_query_len, max_context_len, *, block_size: int | None = None,
               shared_blocks: bool = False, stream=None) -> None:
    """Causal attention of every new query row over its sequence's paged cache.

    query/out are [T, Hq, d]; sequence s owns rows query_start[s] .. query_start[s+1]-1, its
    newest tokens, so its query j sits at position context_lens[s] - q_len + j.
    """
    import torch
    T, Hq, head_dim = query.shape
    d = _desc(key_cache, head_dim, block_size, shared_blocks)
    if out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("out must match query in shape and dtype")
    if value_cache.shape != key_cache.shape:
        raise ValueError("key and value pools differ in shape")
    S = context_lens.numel()
    if block_tables.dim() != 2 or block_tables.shape[0] != S or query_start.numel() != S + 1:
        raise ValueError("block_tables must be [num_seqs, max_blocks]; query_start [num_seqs + 1]")
    args = (ctypes.byref(d), _dev(key_cache, "key_cache", query.dtype),
            _dev(value_cache, "value_cache", query.dtype), _dev(out, "out"),
            _dev(query, "query"), _dev(block_tables, "block_tables", torch.int32),
            block_tables.shape[1], _dev(query_start, "query_start", torch.int32),
            _dev(context_lens, "context_lens", torch.int32), S, Hq, float(scale),
            int(max_query_len), int(max_context_len), _stream(query, stream))
    _check(lib().pa_prefill(*args), "pa_prefill")


def pa_copy_blocks(key_cache, value_cache, src_dst, *, head_dim: int, block_size: int | None = None,
                   stream=None) -> None:
    """Copy block src_dst[k, 0] onto block src_dst[k, 1] in both pools."""
    import torch
    d = _desc(key_cache, head_dim, block_size)
    if value_cache.shape != key_cache.shape:
        raise ValueError("key and value pools differ in shape")
    if src_dst.numel() % 2:
        raise ValueError("src_dst must hold (src, dst) pairs")
    pairs = src_dst.reshape(-1, 2) if src_dst.numel() else src_dst
    args = (ctypes.byref(d), _dev(key_cache, "key_cache"),
            _dev(value_cache, "value_cache", key_cache.dtype),
            _dev(src_dst, "src_dst", torch.int32), pairs.shape[0] if src_dst.numel() else 0,
            _stream(key_cache, stream))
    _check(lib().pa_copy_blocks(*args), "pa_copy_blocks")


def pa_validate_tables(key_cache, block_tables, context_lens, max_context_len: int,
                       violations=None, *, head_dim: int, query_start=None,
                       block_size: int | None = None, stream=None):
    """Count violations of the device-side contract (context lengths, the table entries the
    attention calls read, and query ranges if ``query_start`` is given) into ``violations``
    (a GPU int32 tensor of one element, allocated if None), which is returned."""
    import torch
    d = _desc(key_cache, head_dim, block_size)
    if block_tables.dim() != 2 or context_lens.shape != (block_tables.shape[0],):
        raise ValueError("block_tables must be [num_seqs, max_blocks] and context_lens [num_seqs]")
    num_seqs = block_tables.shape[0]
    if query_start is not None and query_start.shape != (num_seqs + 1,):
        raise ValueError("query_start must be [num_seqs + 1]")
    if violations is None:
        violations = torch.empty(1, dtype=torch.int32, device=key_cache.device)
    if violations.numel() != 1:
        raise ValueError("violations must hold one int32")
    args = (ctypes.byref(d), _dev(block_tables, "block_tables", torch.int32), num_seqs,
            block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
            _vp(0) if query_start is None else _dev(query_start, "query_start", torch.int32),
            int(max_context_len), _dev(violations, "violations", torch.int32),
            _stream(key_cache, stream))
    _check(lib().pa_validate_tables(*args), "pa_validate_tables")
    return violations


def pa_validate_writes(key_cache, violations=None, *, head_dim: int, block_tables=None,
                       token_seq=None, token_pos=None, src_dst=None, block_size: int | None = None,
                       stream=None):
    """Count violations of the write-race contract of one step's pa_reshape_and_cache (tokens
    given by block_tables, token_seq, token_pos) and pa_copy_blocks (src_dst pairs) into
    ``violations`` (a GPU int32 tensor of one element, allocated if None), which is returned:
    table entries outside the pool, slots written twice, destinations written twice or read
    by a pair of the same call."""
    import torch
    d = _desc(key_cache, head_dim, block_size)
    none = _vp(0)
    T = 0 if token_seq is None else token_seq.numel()
    if T:
        if block_tables is None or block_tables.dim() != 2 or token_pos is None or \
                token_pos.numel() != T:
            raise ValueError("tokens need block_tables [num_seqs, max_blocks] and token_pos")
    npairs = 0 if src_dst is None else src_dst.numel() // 2
    if src_dst is not None and src_dst.numel() % 2:
        raise ValueError("src_dst must hold (src, dst) pairs")
    if violations is None:
        violations = torch.empty(1, dtype=torch.int32, device=key_cache.device)
    if violations.numel() != 1:
        raise ValueError("violations must hold one int32")
    args = (ctypes.byref(d),
            _dev(block_tables, "block_tables", torch.int32) if T else none,
            block_tables.shape[0] if T else 0, block_tables.shape[1] if T else 0,
            _dev(token_seq, "token_seq", torch.int32) if T else none,
            _dev(token_pos, "token_pos", torch.int32) if T else none, T,
            _dev(src_dst, "src_dst", torch.int32) if npairs else none, npairs,
            _dev(violations, "violations", torch.int32), _stream(key_cache, stream))
    _check(lib().pa_validate_writes(*args), "pa_validate_writes")
    return violations


def pa_swap_blocks(dst_key, dst_value, src_key, src_value, src_dst, *, head_dim: int,
                   block_size: int | None = None, stream=None) -> None:
    """Copy block src_dst[k, 0] of the source pools onto block src_dst[k, 1] of the destination
    pools. Pools are GPU tensors or pinned CPU tensors (``pin_memory=True``) of the same shape
    apart from the number of blocks; ``src_dst`` holds int32 pairs (a GPU tensor, or any array,
    which is then copied to the GPU)."""
    import numpy as np
    import torch

    def ptr(t, what):
        if not isinstance(t, torch.Tensor) or not t.is_contiguous():
            raise ValueError(f"{what} must be a contiguous torch tensor")
        if t.device.type != "cuda" and not t.is_pinned():
            raise ValueError(f"{what} must be on the GPU or in pinned host memory")
        return _vp(t.data_ptr())

    dd = _desc(dst_key, head_dim, block_size)
    sd = _desc(src_key, head_dim, block_size)
    if dst_value.shape != dst_key.shape or src_value.shape != src_key.shape:
        raise ValueError("key and value pools differ in shape")
    gpu = dst_key if dst_key.device.type == "cuda" else src_key
    if not (isinstance(src_dst, torch.Tensor) and src_dst.device.type == "cuda"):
        src_dst = torch.as_tensor(np.ascontiguousarray(src_dst, dtype=np.int32)).to(gpu.device)
    if src_dst.dtype != torch.int32 or src_dst.numel() % 2 or not src_dst.is_contiguous():
        raise ValueError("src_dst must hold contiguous int32 (src, dst) pairs")
    args = (ctypes.byref(dd), ptr(dst_key, "dst_key"), ptr(dst_value, "dst_value"),
            ctypes.byref(sd), ptr(src_key, "src_key"), ptr(src_value, "src_value"),
            _vp(src_dst.data_ptr()), src_dst.numel() // 2, _stream(gpu, stream))
    _check(lib().pa_swap_blocks(*args), "pa_swap_blocks")


def pa_measure_tile_read(pool_a, pool_b, tiles, tile_bytes: int, sink=None, *, stream=None):
    """Measurement only: read tiles ``tiles`` (int32, GPU) of ``tile_bytes`` from both GPU
    tensors with the attention kernel's loads; returns ``sink`` (uint32 per 32 tiles, the XOR of
    the words each wavefront read; allocated if None)."""
    import torch
    n = tiles.numel()
    if sink is None:
        sink = torch.empty((n + 31) // 32, dtype=torch.int32, device=tiles.device)
    if sink.numel() < (n + 31) // 32:
        raise ValueError("sink must hold one word per 32 tiles")
    args = (_dev(pool_a, "pool_a"), _dev(pool_b, "pool_b"), _dev(tiles, "tiles", torch.int32),
            n, int(tile_bytes), _dev(sink, "sink"), _stream(tiles, stream))
    _check(lib().pa_measure_tile_read(*args), "pa_measure_tile_read")
    return sink
