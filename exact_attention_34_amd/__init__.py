"""Exact attention for AMD MI355X (gfx950): Python binding of libattn.so.

The binding only marshals arguments: it checks tensor shapes and dtypes,
passes device pointers, strides and the current HIP stream to the C ABI
declared in ``include/attn.h``, and turns error codes into exceptions.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  If ``libattn.so`` has not been built, every call raises.

PyTorch provides device memory and streams only.
"""

import ctypes
import math
import os

import torch

from . import build as _build

__all__ = [
    "AttnError", "lib", "abi_version", "attn_fwd", "attn_bwd", "attn_bwd_workspace_size",
    "paged_attn_decode", "paged_attn_decode_noalloc", "DECODE_SCRATCH_BYTES",
    "paged_attn_decode_workspace_size", "paged_attn_decode_shared",
    "paged_attn_decode_shared_workspace_size", "paged_kv_write", "paged_kv_copy_blocks",
    "attn_fwd_paged", "validate_paged_tables",
    "BlockManager", "LIB_PATH",
]

LIB_PATH = _build.LIB_PATH

ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}
ERROR_NAMES = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
               4: "ATTN_ERR_WORKSPACE", 5: "ATTN_ERR_ALIGN", 6: "ATTN_ERR_HIP",
               7: "ATTN_ERR_NO_BLOCKS"}


class AttnError(RuntimeError):
    """A non-OK status from libattn.so (``code`` is the ATTN_ERR_* value)."""

    def __init__(self, code, message):
        super().__init__("%s: %s" % (ERROR_NAMES.get(code, code), message))
        self.code = code


_LIB = None
_I64x3 = ctypes.c_int64 * 3


def lib():
    """The loaded library (ctypes.CDLL) with argument types declared."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libattn.so is not built (%s); run "
                           "`python -m exact_attention_34_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    i64p = ctypes.POINTER(ctypes.c_int64)
    L.attn_abi_version.restype = i32
    L.attn_abi_version.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_last_error.argtypes = []
    L.attn_fwd.restype = i32
    L.attn_fwd.argtypes = [i32, vp, vp, vp, vp, vp,
                           i32, i32, i32, i32, i32, i32,
                           i64p, i64p, i64p, i64p, f32, i32, vp]
    L.attn_bwd_workspace_size.restype = ctypes.c_size_t
    L.attn_bwd_workspace_size.argtypes = [i32, i32, i32]
    L.attn_bwd.restype = i32
    L.attn_bwd.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                           i32, i32, i32, i32, i32, i32,
                           i64p, i64p, i64p, i64p, i64p, i64p, i64p, i64p,
                           f32, i32, vp, ctypes.c_size_t, vp]
    L.paged_attn_decode_workspace_size.restype = ctypes.c_size_t
    L.paged_attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.paged_attn_decode.restype = i32
    L.paged_attn_decode.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp,
                                    i32, i32, i32, i32, i32, i32, i32, i32,
                                    f32, vp, ctypes.c_size_t, vp]
    L.paged_attn_decode_noalloc.restype = i32
    L.paged_attn_decode_noalloc.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp,
                                            i32, i32, i32, i32, i32, i32, i32, i32, f32, vp]
    L.paged_attn_decode_shared_workspace_size.restype = ctypes.c_size_t
    L.paged_attn_decode_shared_workspace_size.argtypes = [i32] * 8
    L.paged_attn_decode_shared.restype = i32
    L.paged_attn_decode_shared.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                           i32, f32, vp, ctypes.c_size_t, vp]
    i64, i32p, i64p_ = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    L.attn_fwd_paged.restype = i32
    L.attn_fwd_paged.argtypes = [i32, vp, i64p, vp, vp, vp, vp, vp, i64p, vp,
                                 i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    L.paged_kv_write.restype = i32
    L.paged_kv_write.argtypes = [i32, vp, vp, i64p, i64p, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    L.paged_kv_copy_blocks.restype = i32
    L.paged_kv_copy_blocks.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    L.attn_validate_paged_tables.restype = i32
    L.attn_validate_paged_tables.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, i32]
    L.attn_bm_create.restype = i32
    L.attn_bm_create.argtypes = [i32, i32, ctypes.POINTER(vp)]
    L.attn_bm_destroy.restype = None
    L.attn_bm_destroy.argtypes = [vp]
    L.attn_bm_num_free.restype = i32
    L.attn_bm_num_free.argtypes = [vp]
    L.attn_bm_ref_count.restype = i32
    L.attn_bm_ref_count.argtypes = [vp, i32]
    L.attn_bm_length.restype = i64
    L.attn_bm_length.argtypes = [vp, i64]
    L.attn_bm_add_sequence.restype = i32
    L.attn_bm_add_sequence.argtypes = [vp, i64]
    L.attn_bm_fork.restype = i32
    L.attn_bm_fork.argtypes = [vp, i64, i64]
    L.attn_bm_append.restype = i32
    L.attn_bm_append.argtypes = [vp, i64, i32, i32p, i32p, i32p, ctypes.POINTER(i32)]
    L.attn_bm_free_sequence.restype = i32
    L.attn_bm_free_sequence.argtypes = [vp, i64]
    L.attn_bm_block_table.restype = i32
    L.attn_bm_block_table.argtypes = [vp, i64p_, i32, i32, i32p, i32p]
    _LIB = L
    return L


def abi_version():
    return lib().attn_abi_version()


def _check(code):
    if code != 0:
        raise AttnError(code, lib().attn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _strides3(t):
    if t.stride(-1) != 1:
        raise ValueError("the head_dim axis must have stride 1")
    return _I64x3(t.stride(0), t.stride(1), t.stride(2))


def attn_fwd(q, k, v, causal=False, scale=None, out=None, lse=None, return_lse=False):
    """Exact attention O = softmax(Q K^T * scale) V on the GPU.

    ``q``: ``[B][Nq][Hq][d]``; ``k``, ``v``: ``[B][Nk][Hkv][d]`` (any strides
    with the last axis contiguous), one dtype among float32/float16/bfloat16,
    on one GPU.  ``scale`` defaults to ``1/sqrt(d)``.  ``causal`` applies the
    bottom-right aligned mask.  ``out`` (same shape as ``q``) and ``lse``
    (``[B][Hq][Nq]`` float32, contiguous) are optional preallocated outputs;
    with ``return_lse`` the log-sum-exp is computed and returned too.
    The call is asynchronous on the current stream.
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B][N][H][d]")
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype among float32, float16, bfloat16")
    B, Nq, Hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must be [B][Nk][Hkv][d] matching q")
    Nk, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must have q's shape and dtype")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, Hq, Nq) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B][Hq][Nq] tensor")
    for t in (q, k, v, out):
        if not t.is_cuda or t.device != q.device:
            raise ValueError("all tensors must be on the same GPU")
    code = lib().attn_fwd(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                          B, Nq, Nk, Hq, Hkv, d,
                          _strides3(q), _strides3(k), _strides3(v), _strides3(out),
                          float(scale), int(bool(causal)), _stream(q.device))
    _check(code)
    if return_lse:
        return out, lse
    return out


def attn_bwd_workspace_size(batch, n_q, h_q):
    """Bytes of workspace :func:`attn_bwd` needs (0 if none)."""
    return int(lib().attn_bwd_workspace_size(batch, n_q, h_q))


def attn_bwd(q, k, v, o, do, lse, causal=False, scale=None, dq=None, dk=None, dv=None,
             workspace=None):
    """Gradients (dq, dk, dv) of :func:`attn_fwd` for the upstream gradient ``do``.

    ``q``, ``o``, ``do``: ``[B][Nq][Hq][d]``; ``k``, ``v``: ``[B][Nk][Hkv][d]``
    (any strides with the last axis contiguous), float16 or bfloat16; ``o`` and
    ``lse`` (``[B][Hq][Nq]`` float32, contiguous) as returned by
    ``attn_fwd(..., return_lse=True)`` for the same inputs.  The outputs
    default to new contiguous tensors.  Asynchronous on the current stream.
    """
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("attn_bwd takes float16 or bfloat16 tensors")
    for t in (k, v, o, do):
        if t.dtype != q.dtype:
            raise ValueError("all tensors must share one dtype")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if o.shape != q.shape or do.shape != q.shape or v.shape != k.shape or k.shape[0] != B \
            or k.shape[3] != d:
        raise ValueError("q, o, do must be [B][Nq][Hq][d] and k, v [B][Nk][Hkv][d]")
    if lse.shape != (B, Hq, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B][Hq][Nq] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("dq, dk, dv must have the shapes of q, k, v")
    for t in (q, k, v, o, do, lse, dq, dk, dv):
        if not t.is_cuda or t.device != q.device:
            raise ValueError("all tensors must be on the same GPU")
    need = attn_bwd_workspace_size(B, Nq, Hq)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = lib().attn_bwd(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                          _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, Nq, Nk, Hq, Hkv, d,
                          _strides3(q), _strides3(k), _strides3(v), _strides3(o), _strides3(do),
                          _strides3(dq), _strides3(dk), _strides3(dv), float(scale),
                          int(bool(causal)), _ptr(workspace), ws_bytes, _stream(q.device))
    _check(code)
    return dq, dk, dv


def paged_attn_decode_workspace_size(num_seqs, h_q, h_kv, head_dim, max_context_len):
    """Bytes of workspace :func:`paged_attn_decode` needs (0 if none)."""
    return int(lib().paged_attn_decode_workspace_size(num_seqs, h_q, h_kv, head_dim,
                                                       max_context_len))


def _decode_common(q, k_cache, v_cache, block_table, context_lens, scale, out, lse,
                   return_lse):
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [S][Hq][d] and the caches [blocks][Hkv][bs][d]")
    if q.dtype not in (torch.float16, torch.bfloat16) or k_cache.dtype != q.dtype \
            or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must share float16 or bfloat16")
    if block_table.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_table and context_lens must be int32")
    for t in (q, k_cache, v_cache, block_table, context_lens):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
        if not t.is_cuda or t.device != q.device:
            raise ValueError("all tensors must be on the same GPU")
    S, Hq, d = q.shape
    if k_cache.shape[3] != d:
        raise ValueError("head_dim mismatch")
    if block_table.dim() != 2 or block_table.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_table must be [S][max_blocks] and context_lens [S]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None and return_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (S, Hq) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [S][Hq] tensor")
    return scale, out, lse


def paged_attn_decode(q, k_cache, v_cache, block_table, context_lens, max_context_len,
                      scale=None, out=None, lse=None, workspace=None, return_lse=False):
    """Single-token decode over a paged KV cache.

    ``q``: ``[S][Hq][d]``; ``k_cache``, ``v_cache``:
    ``[num_blocks][Hkv][16][d]`` (contiguous, float16 or bfloat16);
    ``block_table``: ``[S][max_blocks_per_seq]`` int32; ``context_lens``:
    ``[S]`` int32, each at most ``max_context_len`` (a host int).  The
    workspace is allocated from torch's caching allocator when not given.
    Asynchronous on the current stream.
    """
    scale, out, lse = _decode_common(q, k_cache, v_cache, block_table, context_lens, scale,
                                     out, lse, return_lse)
    S, Hq, d = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    need = paged_attn_decode_workspace_size(S, Hq, Hkv, d, int(max_context_len))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = lib().paged_attn_decode(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(block_table), _ptr(context_lens), _ptr(out), _ptr(lse),
                                   S, Hq, Hkv, d, bs, block_table.shape[1], int(max_context_len),
                                   NB, float(scale), _ptr(workspace), ws_bytes,
                                   _stream(q.device))
    _check(code)
    if return_lse:
        return out, lse
    return out


# ATTN_DECODE_SCRATCH_BYTES of include/attn.h: the scratch the library holds
# per GPU for paged_attn_decode_noalloc
DECODE_SCRATCH_BYTES = 40 << 20


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_table, context_lens, max_context_len,
                              scale=None, out=None, lse=None, return_lse=False):
    """:func:`paged_attn_decode` on the library's own device scratch (the C
    ABI's paged_attn_decode_noalloc): the library call allocates nothing.
    Pass ``out`` (and ``lse`` with ``return_lse``) preallocated to keep the
    whole call free of allocation.  Calls that overlap on one GPU race (one
    scratch per GPU); calls ordered on one stream are safe."""
    scale, out, lse = _decode_common(q, k_cache, v_cache, block_table, context_lens, scale,
                                     out, lse, return_lse)
    S, Hq, d = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    code = lib().paged_attn_decode_noalloc(
        _DTYPE_CODE[q.dtype], _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(context_lens), _ptr(out), _ptr(lse), S, Hq, Hkv, d, bs, block_table.shape[1],
        int(max_context_len), NB, float(scale), _stream(q.device))
    _check(code)
    if return_lse:
        return out, lse
    return out


def paged_attn_decode_shared_workspace_size(num_seqs, num_groups, max_group_size, h_q, h_kv,
                                            head_dim, max_context_len, max_prefix_len):
    """Bytes of workspace :func:`paged_attn_decode_shared` needs (0 if invalid)."""
    return int(lib().paged_attn_decode_shared_workspace_size(
        num_seqs, num_groups, max_group_size, h_q, h_kv, head_dim, max_context_len,
        max_prefix_len))


def paged_attn_decode_shared(q, k_cache, v_cache, block_table, context_lens, group_starts,
                             prefix_lens, max_context_len, max_group_size, max_prefix_len,
                             scale=None, out=None, lse=None, workspace=None,
                             return_lse=False):
    """Single-token decode for groups of sequences that share a prefix.

    Arguments as :func:`paged_attn_decode`, plus ``group_starts``
    (``[G + 1]`` int32 on the GPU: group ``g`` is sequences
    ``group_starts[g] .. group_starts[g+1]-1``) and ``prefix_lens`` (``[G]``
    int32 on the GPU: tokens of each group's common prefix, whose block ids
    are the same in every member's table row), with host-side bounds
    ``max_group_size`` and ``max_prefix_len``.  Each shared prefix block is
    read once per group.  Asynchronous on the current stream.
    """
    scale, out, lse = _decode_common(q, k_cache, v_cache, block_table, context_lens, scale,
                                     out, lse, return_lse)
    for t in (group_starts, prefix_lens):
        if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda \
                or t.device != q.device:
            raise ValueError("group_starts and prefix_lens must be contiguous int32 GPU tensors")
    G = prefix_lens.shape[0]
    if group_starts.shape != (G + 1,):
        raise ValueError("group_starts must have one more entry than prefix_lens")
    S, Hq, d = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    need = paged_attn_decode_shared_workspace_size(S, G, int(max_group_size), Hq, Hkv, d,
                                                   int(max_context_len), int(max_prefix_len))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = lib().paged_attn_decode_shared(
        _DTYPE_CODE[q.dtype], _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(context_lens), _ptr(group_starts), _ptr(prefix_lens), _ptr(out), _ptr(lse),
        S, G, int(max_group_size), Hq, Hkv, d, bs, block_table.shape[1], int(max_context_len),
        int(max_prefix_len), NB, float(scale), _ptr(workspace), ws_bytes, _stream(q.device))
    _check(code)
    if return_lse:
        return out, lse
    return out


def _kv_strides(t):
    if t.dim() != 3 or t.stride(-1) != 1:
        raise ValueError("new K/V must be [tokens][h_kv][d] views with d contiguous")
    return (ctypes.c_int64 * 2)(t.stride(0), t.stride(1))


def paged_kv_write(k_new, v_new, slot_mapping, k_cache, v_cache):
    """Write new tokens' K/V rows (``[T][Hkv][d]``, any token/head strides)
    into the paged caches at ``slot_mapping`` (``[T]`` int32 on the GPU;
    slots outside the pool are skipped).  Asynchronous."""
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [num_blocks][Hkv][block_size][d]")
    NB, Hkv, bs, d = k_cache.shape
    if k_new.shape != v_new.shape or k_new.shape[1:] != (Hkv, d):
        raise ValueError("k_new and v_new must be [T][Hkv][d] matching the cache")
    for t in (k_new, v_new):
        if t.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
            raise ValueError("new K/V and caches must share one dtype")
    if slot_mapping.dtype != torch.int32 or slot_mapping.shape != (k_new.shape[0],) \
            or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int32 [T] tensor")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    code = lib().paged_kv_write(_DTYPE_CODE[k_cache.dtype], _ptr(k_new), _ptr(v_new),
                                _kv_strides(k_new), _kv_strides(v_new), _ptr(slot_mapping),
                                _ptr(k_cache), _ptr(v_cache), k_new.shape[0], Hkv, d, bs, NB,
                                _stream(k_cache.device))
    _check(code)


def paged_kv_copy_blocks(k_cache, v_cache, src, dst):
    """Copy whole blocks ``src[i] -> dst[i]`` (int32 GPU tensors) in both
    caches.  Asynchronous."""
    NB, Hkv, bs, d = k_cache.shape
    if src.dtype != torch.int32 or dst.dtype != torch.int32 or src.shape != dst.shape \
            or src.dim() != 1:
        raise ValueError("src and dst must be int32 [n] tensors")
    code = lib().paged_kv_copy_blocks(_DTYPE_CODE[k_cache.dtype], _ptr(k_cache), _ptr(v_cache),
                                      _ptr(src), _ptr(dst), src.shape[0], Hkv, d, bs, NB,
                                      _stream(k_cache.device))
    _check(code)


class BlockManager:
    """Host bookkeeping of a paged KV cache (the C ABI's attn_bm_* calls).

    ``append`` returns the slots of the new tokens and the copy-on-write block
    copies (a list of ``(src, dst)``) to run before writing them."""

    def __init__(self, num_blocks, block_size=16):
        h = ctypes.c_void_p()
        _check(lib().attn_bm_create(int(num_blocks), int(block_size), ctypes.byref(h)))
        self._h = h
        self.block_size = int(block_size)

    def close(self):
        if getattr(self, "_h", None):
            lib().attn_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def num_free(self):
        return lib().attn_bm_num_free(self._h)

    def ref_count(self, block):
        return lib().attn_bm_ref_count(self._h, int(block))

    def length(self, seq_id):
        return lib().attn_bm_length(self._h, int(seq_id))

    def add_sequence(self, seq_id):
        _check(lib().attn_bm_add_sequence(self._h, int(seq_id)))

    def fork(self, parent, child):
        _check(lib().attn_bm_fork(self._h, int(parent), int(child)))

    def append(self, seq_id, n_tokens):
        import numpy as np
        slots = np.zeros(max(1, n_tokens), dtype=np.int32)
        cs, cd = ctypes.c_int32(), ctypes.c_int32()
        n = ctypes.c_int32()
        p32 = ctypes.POINTER(ctypes.c_int32)
        _check(lib().attn_bm_append(self._h, int(seq_id), int(n_tokens),
                                    slots.ctypes.data_as(p32), ctypes.byref(cs), ctypes.byref(cd),
                                    ctypes.byref(n)))
        return slots[:n_tokens], ([(cs.value, cd.value)] if n.value else [])

    def free_sequence(self, seq_id):
        _check(lib().attn_bm_free_sequence(self._h, int(seq_id)))

    def block_table(self, seq_ids, max_blocks):
        import numpy as np
        ids = np.asarray(seq_ids, dtype=np.int64)
        table = np.zeros((len(ids), max(1, max_blocks)), dtype=np.int32)
        ctx = np.zeros(max(1, len(ids)), dtype=np.int32)
        _check(lib().attn_bm_block_table(
            self._h, ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(ids),
            int(max_blocks), table.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            ctx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        return table[:, :max_blocks] if max_blocks else table[:, :0], ctx[:len(ids)]


def attn_fwd_paged(q, k_cache, v_cache, block_table, context_lens, max_context_len, causal=True,
                   scale=None, out=None, lse=None, return_lse=False):
    """Prefill over a paged KV cache: ``q`` ``[B][Nq][Hq][d]`` are the last
    ``Nq`` tokens of each sequence, whose K/V (``context_lens[b]`` tokens, int32
    on the GPU) are read through ``block_table`` (``[B][max_blocks]`` int32).
    Asynchronous on the current stream."""
    if q.dim() != 4 or q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q must be a float16/bfloat16 [B][Nq][Hq][d] tensor")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or k_cache.dtype != q.dtype \
            or v_cache.dtype != q.dtype:
        raise ValueError("caches must be [blocks][Hkv][bs][d] of q's dtype")
    B, Nq, Hq, d = q.shape
    NB, Hkv, bs, dk = k_cache.shape
    if dk != d:
        raise ValueError("head_dim mismatch")
    if block_table.dtype != torch.int32 or context_lens.dtype != torch.int32 \
            or block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table must be int32 [B][max_blocks], context_lens int32 [B]")
    for t in (k_cache, v_cache, block_table, context_lens):
        if not t.is_contiguous():
            raise ValueError("caches, block_table and context_lens must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    code = lib().attn_fwd_paged(_DTYPE_CODE[q.dtype], _ptr(q), _strides3(q), _ptr(k_cache),
                                _ptr(v_cache), _ptr(block_table), _ptr(context_lens), _ptr(out),
                                _strides3(out), _ptr(lse), B, Nq, Hq, Hkv, d, bs,
                                block_table.shape[1], int(max_context_len), NB, float(scale),
                                int(bool(causal)), _stream(q.device))
    _check(code)
    if return_lse:
        return out, lse
    return out


def validate_paged_tables(block_table, context_lens, max_context_len, num_blocks, block_size=16,
                          group_starts=None, prefix_lens=None):
    """Host range check of a paged call's metadata (the C ABI's
    attn_validate_paged_tables): ``block_table`` ``[S][max_blocks]`` and
    ``context_lens`` ``[S]``, optionally ``group_starts`` ``[G + 1]`` and
    ``prefix_lens`` ``[G]``, as int32 host arrays (numpy or CPU tensors).
    Raises :class:`AttnError` naming the first violation."""
    import numpy as np

    def host(x):
        if x is None:
            return None
        if torch.is_tensor(x):
            x = x.cpu().numpy()
        return np.ascontiguousarray(x, dtype=np.int32)

    tab, ctx = host(block_table), host(context_lens)
    gs, pl = host(group_starts), host(prefix_lens)
    if tab.ndim != 2 or ctx.shape != (tab.shape[0],):
        raise ValueError("block_table must be [S][max_blocks] and context_lens [S]")
    G = 0 if pl is None else pl.shape[0]
    if gs is not None and gs.shape != (G + 1,):
        raise ValueError("group_starts must have one more entry than prefix_lens")
    p = lambda a: None if a is None else ctypes.c_void_p(a.ctypes.data)
    _check(lib().attn_validate_paged_tables(p(tab), p(ctx), tab.shape[0], tab.shape[1],
                                            int(max_context_len), int(num_blocks),
                                            int(block_size), p(gs), p(pl), G))
