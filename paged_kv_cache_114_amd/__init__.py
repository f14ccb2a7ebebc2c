"""Python binding of the paged KV-cache attention library (libpa.so, gfx950).

Argument marshalling only: every function here takes PyTorch device tensors,
reads their pointers, sizes and strides, and calls the C entry point of the
same name on the current HIP stream.  All computation happens in the HIP
kernels of ``libpa.so``; there is no fallback.  The library is loaded on
first use, and every entry point raises ``ImportError`` if it is not built
(build it with ``python -m paged_kv_cache_114_amd._build`` or
``__graft_entry__.build()``).
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_WORKSPACE = -3
PA_ERR_LAUNCH = -4
PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1
PA_CACHE_BSHD = 0   # [num_blocks, block_size, num_kv_heads, head_dim]
PA_CACHE_BHSD = 1   # [num_blocks, num_kv_heads, block_size, head_dim]
LAYOUTS = {"bshd": PA_CACHE_BSHD, "bhsd": PA_CACHE_BHSD}

EXPORTS = (
    "pa_version",
    "pa_strerror",
    "pa_store_kv",
    "pa_qk_norm_rope_store",
    "pa_decode_workspace_size",
    "pa_decode",
    "pa_store_decode",
    "pa_store_decode_noalloc",
    "pa_decode_shared_prefix",
    "pa_decode_reduce",
    "pa_prefill_workspace_size",
    "pa_prefill_varlen",
    "pa_store_prefill_varlen",
    "pa_prefill_plan",
    "pa_prefill_varlen_planned",
    "pa_store_prefill_varlen_planned",
)


class PAError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({strerror(status)})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m paged_kv_cache_114_amd._build")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, f32, sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float,
                             ctypes.c_size_t)
    lib.pa_version.restype = ctypes.c_int
    lib.pa_version.argtypes = []
    lib.pa_strerror.restype = ctypes.c_char_p
    lib.pa_strerror.argtypes = [ctypes.c_int]
    lib.pa_store_kv.restype = ctypes.c_int
    lib.pa_store_kv.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp, i32, i32, i32, i32, i64,
                                i32, i32, vp]
    lib.pa_qk_norm_rope_store.restype = ctypes.c_int
    lib.pa_qk_norm_rope_store.argtypes = [vp, i64, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                          ctypes.c_double, vp, i64, vp, vp, i32, i64, i32, i32,
                                          vp]
    lib.pa_decode_workspace_size.restype = ctypes.c_int
    lib.pa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz),
                                             ctypes.POINTER(i32)]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode.argtypes = [vp, i64, i64, vp, vp, vp, i64, vp, i32, i32, i32, i32, i32, i64,
                              i32, i32, i32, f32, vp, sz, i32, vp]
    lib.pa_store_decode.restype = ctypes.c_int
    lib.pa_store_decode.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, i64, i64, vp, vp, vp, i64,
                                    vp, i32, i32, i32, i32, i32, i64, i32, i32, i32, f32, vp, sz,
                                    i32, vp]
    lib.pa_store_decode_noalloc.restype = ctypes.c_int
    lib.pa_store_decode_noalloc.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, i64, i64, vp, vp,
                                            vp, i64, vp, i32, i32, i32, i32, i32, i64, i32, i32,
                                            i32, f32, vp, i64, i64, i32, vp]
    lib.pa_decode_shared_prefix.restype = ctypes.c_int
    lib.pa_decode_shared_prefix.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, i64, i64, vp, vp,
                                            vp, i64, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                            i32, i64, i32, i32, i32, f32, vp, sz, i32, vp]
    lib.pa_decode_reduce.restype = ctypes.c_int
    lib.pa_decode_reduce.argtypes = [vp, sz, vp, i32, i32, i32, i32, i32, vp, i64, i64, i32, vp]
    lib.pa_prefill_workspace_size.restype = ctypes.c_int
    lib.pa_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32,
                                              ctypes.POINTER(sz), ctypes.POINTER(i32)]
    lib.pa_prefill_varlen.restype = ctypes.c_int
    lib.pa_prefill_varlen.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32,
                                      i32, i32, i64, i32, i32, i32, f32, i32, vp, sz, vp, i64,
                                      i64, i32, vp]
    lib.pa_store_prefill_varlen.restype = ctypes.c_int
    lib.pa_store_prefill_varlen.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, i64, i64, vp, vp,
                                            vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, i64,
                                            i32, i32, i32, f32, i32, vp, sz, vp, i64, i64, i32,
                                            vp]
    lib.pa_prefill_plan.restype = ctypes.c_int
    lib.pa_prefill_plan.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.pa_prefill_varlen_planned.restype = ctypes.c_int
    lib.pa_prefill_varlen_planned.argtypes = lib.pa_prefill_varlen.argtypes
    lib.pa_store_prefill_varlen_planned.restype = ctypes.c_int
    lib.pa_store_prefill_varlen_planned.argtypes = lib.pa_store_prefill_varlen.argtypes
    return lib


_LIB = None


def library():
    """The loaded ``libpa.so`` (ctypes handle); raises ImportError if it is not built."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def version() -> int:
    return library().pa_version()


def strerror(status: int) -> str:
    return library().pa_strerror(status).decode()


def _check(fn, status):
    if status != PA_OK:
        raise PAError(fn, status)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return PA_DTYPE_BF16
    if t.dtype == torch.float32:
        return PA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _cache_shape(cache, layout):
    """``(num_blocks, block_size, num_kv_heads, head_dim, layout code)`` of a cache tensor:
    ``[NB, bs, Hkv, d]`` for layout "bshd", ``[NB, Hkv, bs, d]`` for "bhsd"."""
    code = LAYOUTS[layout]
    if code == PA_CACHE_BHSD:
        nb, hkv, bs, d = cache.shape
    else:
        nb, bs, hkv, d = cache.shape
    return nb, bs, hkv, d, code


def _check_pool(k_cache, v_cache, *same_dtype):
    """The library derives a cache's strides from its shape, so both caches must be
    contiguous, of one shape and of the dtype of every other float tensor passed."""
    assert k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous"
    assert k_cache.shape == v_cache.shape, "k_cache and v_cache shapes differ"
    for t in (v_cache, *same_dtype):
        if t is not None:
            assert t.dtype == k_cache.dtype, f"dtype {t.dtype} differs from the cache's {k_cache.dtype}"


def _check_table(block_table, block_size, max_len):
    """Every row must have a column for each block a sequence of max_len tokens uses."""
    assert block_table.dim() == 2 and block_table.stride(1) == 1, "block_table must be [B, W]"
    assert block_table.shape[1] * block_size >= max_len, (
        f"block_table has {block_table.shape[1]} columns, fewer than "
        f"ceil({max_len} / {block_size})")


def pa_store_kv(k, v, k_cache, v_cache, slot_mapping, stream=None, layout="bshd") -> None:
    """Store this step's K/V rows ``[T, Hkv, d]`` into the paged caches."""
    nb, bs, hkv, d, lay = _cache_shape(k_cache, layout)
    _check_pool(k_cache, v_cache, k, v)
    assert k.stride(-1) == 1 and v.stride(-1) == 1, "innermost stride must be 1"
    _check("pa_store_kv", library().pa_store_kv(
        _ptr(k), _ptr(v), k.stride(0), k.stride(1), v.stride(0), v.stride(1), _ptr(k_cache),
        _ptr(v_cache), _ptr(slot_mapping), slot_mapping.shape[0], hkv, d, bs, nb, lay,
        _dtype_code(k_cache), _stream(stream)))


def pa_qk_norm_rope_store(qkv, q_norm_weight, k_norm_weight, positions, slot_mapping,
                          num_q_heads, num_kv_heads, eps, rope_theta, q_out, k_cache, v_cache,
                          stream=None, layout="bshd") -> None:
    """Per-head q/k RMSNorm + RoPE of ``qkv [T, (Hq + 2 Hkv) d]``; writes ``q_out [T, Hq, d]``
    and stores rotated K and raw V at ``slot_mapping`` in the paged caches.
    Both norm weights ``None``: rotation only."""
    nb, bs, hkv, d, lay = _cache_shape(k_cache, layout)
    assert hkv == num_kv_heads, "cache head count differs from num_kv_heads"
    _check_pool(k_cache, v_cache, qkv, q_out, q_norm_weight, k_norm_weight)
    assert qkv.stride(-1) == 1 and q_out.stride(-1) == 1, "innermost stride must be 1"
    assert q_out.dim() == 3 and q_out.stride(1) == d, "q_out must be [T, Hq, d] with head stride d"
    _check("pa_qk_norm_rope_store", library().pa_qk_norm_rope_store(
        _ptr(qkv), qkv.stride(0), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(positions),
        _ptr(slot_mapping), qkv.shape[0], num_q_heads, num_kv_heads, d, eps, rope_theta,
        _ptr(q_out), q_out.stride(0), _ptr(k_cache), _ptr(v_cache), bs, nb, lay,
        _dtype_code(qkv), _stream(stream)))


def pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                             partition_tokens):
    """Returns ``(bytes, num_splits)`` of the decode workspace."""
    nbytes = ctypes.c_size_t(0)
    splits = ctypes.c_int32(0)
    _check("pa_decode_workspace_size", library().pa_decode_workspace_size(
        num_seqs, num_q_heads, head_dim, max_context_len, partition_tokens,
        ctypes.byref(nbytes), ctypes.byref(splits)))
    return nbytes.value, splits.value


def pa_decode(q, k_cache, v_cache, block_table, context_lens, max_context_len, partition_tokens,
              scale, workspace, stream=None, layout="bshd") -> None:
    """Partition pass: ``q [B, Hq, d]``; fills ``workspace`` (a float32 device tensor)."""
    nb, bs, hkv, d, lay = _cache_shape(k_cache, layout)
    _check_pool(k_cache, v_cache, q)
    _check_table(block_table, bs, max_context_len)
    b, hq, _ = q.shape
    _check("pa_decode", library().pa_decode(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        block_table.stride(0), _ptr(context_lens), b, hq, hkv, d, bs, nb, lay, max_context_len,
        partition_tokens, scale, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _dtype_code(k_cache), _stream(stream)))


def pa_store_decode(k_new, v_new, slot_mapping, q, k_cache, v_cache, block_table, context_lens,
                    max_context_len, partition_tokens, scale, workspace, stream=None,
                    layout="bshd") -> None:
    """Store each sequence's new K/V row (``[B, Hkv, d]``, at position ``context_lens - 1``)
    through ``slot_mapping`` and run the partition pass, in one launch."""
    nb, bs, hkv, d, lay = _cache_shape(k_cache, layout)
    _check_pool(k_cache, v_cache, q, k_new, v_new)
    _check_table(block_table, bs, max_context_len)
    b, hq, _ = q.shape
    assert k_new.stride(-1) == 1 and v_new.stride(-1) == 1, "innermost stride must be 1"
    _check("pa_store_decode", library().pa_store_decode(
        _ptr(k_new), _ptr(v_new), k_new.stride(0), k_new.stride(1), v_new.stride(0),
        v_new.stride(1), _ptr(slot_mapping), _ptr(q), q.stride(0), q.stride(1), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_table), block_table.stride(0), _ptr(context_lens), b, hq, hkv,
        d, bs, nb, lay, max_context_len, partition_tokens, scale, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _dtype_code(k_cache), _stream(stream)))


def pa_store_decode_noalloc(k_new, v_new, slot_mapping, q, k_cache, v_cache, block_table,
                            context_lens, max_context_len, partition_tokens, scale, out,
                            stream=None, layout="bshd") -> None:
    """pa_store_decode then pa_decode_reduce into ``out [B, Hq, d]``, with the split
    workspace in the library's own fixed device array (nothing is allocated)."""
    nb, bs, hkv, d, lay = _cache_shape(k_cache, layout)
    _check_pool(k_cache, v_cache, q, k_new, v_new, out)
    _check_table(block_table, bs, max_context_len)
    b, hq, _ = q.shape
    assert k_new.stride(-1) == 1 and v_new.stride(-1) == 1, "innermost stride must be 1"
    _check("pa_store_decode_noalloc", library().pa_store_decode_noalloc(
        _ptr(k_new), _ptr(v_new), k_new.stride(0), k_new.stride(1), v_new.stride(0),
        v_new.stride(1), _ptr(slot_mapping), _ptr(q), q.stride(0), q.stride(1), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_table), block_table.stride(0), _ptr(context_lens), b, hq, hkv,
        d, bs, nb, lay, max_context_len, partition_tokens, scale, _ptr(out), out.stride(0),
        out.stride(1), _dtype_code(k_cache), _stream(stream)))


def pa_decode_shared_prefix(q, k_cache, v_cache, block_table, context_lens, prefix_group,
                            prefix_tokens, max_prefix_tokens, max_context_len, partition_tokens,
                            scale, workspace, k_new=None, v_new=None, slot_mapping=None,
                            stream=None, layout="bshd") -> None:
    """The partition pass for a batch whose groups share prefix blocks: ``prefix_group
    [B]`` (-1: none) and ``prefix_tokens [num_groups]`` (int32, on the device); the
    splits inside a group's prefix are computed once for all its members.  With
    ``k_new, v_new, slot_mapping`` the step's rows are stored as by pa_store_decode."""
    nb, bs, hkv, d, lay = _cache_shape(k_cache, layout)
    store = k_new is not None
    assert store == (v_new is not None) == (slot_mapping is not None), "store all or nothing"
    _check_pool(k_cache, v_cache, q, *((k_new, v_new) if store else ()))
    _check_table(block_table, bs, max_context_len)
    b, hq, _ = q.shape
    assert prefix_group.dtype == prefix_tokens.dtype == context_lens.dtype, "int32 metadata"
    assert prefix_group.numel() >= b, "prefix_group needs one entry per sequence"
    if store:
        assert k_new.stride(-1) == 1 and v_new.stride(-1) == 1, "innermost stride must be 1"
    _check("pa_decode_shared_prefix", library().pa_decode_shared_prefix(
        _ptr(k_new) if store else None, _ptr(v_new) if store else None,
        k_new.stride(0) if store else 0, k_new.stride(1) if store else 0,
        v_new.stride(0) if store else 0, v_new.stride(1) if store else 0,
        _ptr(slot_mapping) if store else None, _ptr(q), q.stride(0), q.stride(1), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_table), block_table.stride(0), _ptr(context_lens),
        _ptr(prefix_group), _ptr(prefix_tokens), prefix_tokens.numel(), max_prefix_tokens, b,
        hq, hkv, d, bs, nb, lay, max_context_len, partition_tokens, scale, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _dtype_code(k_cache), _stream(stream)))


def pa_decode_reduce(workspace, context_lens, num_splits, partition_tokens, out,
                     stream=None) -> None:
    """Merge the splits into ``out [B, Hq, d]``."""
    b, hq, d = out.shape
    _check("pa_decode_reduce", library().pa_decode_reduce(
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(context_lens), b, hq,
        d, num_splits, partition_tokens, _ptr(out), out.stride(0), out.stride(1),
        _dtype_code(out), _stream(stream)))


def pa_prefill_workspace_size(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                              max_seqlen_k, split_keys=0):
    """Returns ``(bytes, num_splits)`` of the prefill workspace for ``split_keys``."""
    nbytes = ctypes.c_size_t(0)
    splits = ctypes.c_int32(0)
    _check("pa_prefill_workspace_size", library().pa_prefill_workspace_size(
        num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, max_seqlen_k, split_keys,
        ctypes.byref(nbytes), ctypes.byref(splits)))
    return nbytes.value, splits.value


def pa_prefill_varlen(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_table,
                      max_seqlen_q, max_seqlen_k, scale, out, workspace, split_keys=0,
                      stream=None, layout="bshd", _planned=False) -> None:
    """Causal varlen prefill: ``q, out [Tq, Hq, d]``; K/V read from the paged caches.
    ``workspace``: a device tensor of at least pa_prefill_workspace_size bytes for the
    same sizes and ``split_keys`` (> 0 cuts long query tiles' key loops)."""
    nb, bs, hkv, d, lay = _cache_shape(k_cache, layout)
    _check_pool(k_cache, v_cache, q, out)
    _check_table(block_table, bs, max_seqlen_k)
    tq, hq, _ = q.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    fn = "pa_prefill_varlen_planned" if _planned else "pa_prefill_varlen"
    _check(fn, getattr(library(), fn)(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), _ptr(block_table), block_table.stride(0), cu_seqlens_q.shape[0] - 1,
        tq, hq, hkv, d, bs, nb, lay, max_seqlen_q, max_seqlen_k, scale, split_keys,
        _ptr(workspace), ws_bytes, _ptr(out), out.stride(0), out.stride(1), _dtype_code(q),
        _stream(stream)))


def pa_store_prefill_varlen(k_new, v_new, slot_mapping, q, k_cache, v_cache, cu_seqlens_q,
                            cu_seqlens_k, block_table, max_seqlen_q, max_seqlen_k, scale, out,
                            workspace, split_keys=0, stream=None, layout="bshd",
                            _planned=False) -> None:
    """Store the query rows' K/V (``[Tq, Hkv, d]``, any token and head strides) through
    ``slot_mapping`` and run the causal varlen prefill; the tile kernel reads these rows
    from ``k_new`` / ``v_new`` and writes them to the cache itself."""
    nb, bs, hkv, d, lay = _cache_shape(k_cache, layout)
    _check_pool(k_cache, v_cache, q, out, k_new, v_new)
    _check_table(block_table, bs, max_seqlen_k)
    tq, hq, _ = q.shape
    assert k_new.stride(-1) == 1 and v_new.stride(-1) == 1, "innermost stride must be 1"
    ws_bytes = workspace.numel() * workspace.element_size()
    fn = "pa_store_prefill_varlen_planned" if _planned else "pa_store_prefill_varlen"
    _check(fn, getattr(library(), fn)(
        _ptr(k_new), _ptr(v_new), k_new.stride(0), k_new.stride(1), v_new.stride(0),
        v_new.stride(1), _ptr(slot_mapping), _ptr(q), q.stride(0), q.stride(1), _ptr(k_cache),
        _ptr(v_cache), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(block_table),
        block_table.stride(0), cu_seqlens_q.shape[0] - 1, tq, hq, hkv, d, bs, nb, lay,
        max_seqlen_q, max_seqlen_k, scale, split_keys, _ptr(workspace), ws_bytes, _ptr(out),
        out.stride(0), out.stride(1), _dtype_code(q), _stream(stream)))


def pa_prefill_plan(cu_seqlens_q, cu_seqlens_k, total_q, num_q_heads, num_kv_heads, head_dim,
                    max_seqlen_q, max_seqlen_k, workspace, split_keys=0, stream=None) -> None:
    """Build the prefill work list for this metadata into ``workspace`` once; the
    ``*_planned`` calls then reuse it (every layer of a step)."""
    _check("pa_prefill_plan", library().pa_prefill_plan(
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), cu_seqlens_q.shape[0] - 1, total_q, num_q_heads,
        num_kv_heads, head_dim, max_seqlen_q, max_seqlen_k, split_keys, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def pa_prefill_varlen_planned(*args, **kwargs) -> None:
    """pa_prefill_varlen on the work list pa_prefill_plan built in ``workspace``."""
    pa_prefill_varlen(*args, _planned=True, **kwargs)


def pa_store_prefill_varlen_planned(*args, **kwargs) -> None:
    """pa_store_prefill_varlen on the work list pa_prefill_plan built in ``workspace``."""
    pa_store_prefill_varlen(*args, _planned=True, **kwargs)
