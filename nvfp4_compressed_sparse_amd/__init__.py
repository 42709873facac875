"""Python binding of libmla_nvfp4 (include/mla_nvfp4.h): NVFP4 compressed-latent sparse-MLA decode on
MI355X (gfx950).

The functions keep the C names and only marshal arguments: torch tensors supply device pointers,
strides and the current HIP stream; every step of the computation runs in the library's kernels.
There is no fallback: if the library cannot be loaded, or a call returns an error status, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB as LIB_PATH
from .build import TIMELINE_LIB as TIMELINE_LIB_PATH
from .build import build

LATENT_DIM, ROPE_DIM, QK_DIM, PAGE_TOKENS = 512, 64, 576, 64
NVFP4_ROW_BYTES, FP8_ROW_BYTES, MAX_TOPK = 352, 576, 2048

STATUS = {0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_STRIDE_ALIGN", 4: "MLA_ERR_WORKSPACE",
          5: "MLA_ERR_DEVICE", 6: "MLA_ERR_HIP"}

EXPORTS = [
    "mla_abi_version", "mla_status_string", "mla_kv_quant_nvfp4", "mla_kv_quant_fp8", "mla_sparse_decode_splits",
    "mla_dense_decode_splits", "mla_sparse_decode_workspace_bytes", "mla_dense_decode_workspace_bytes",
    "mla_sparse_decode", "mla_sparse_decode_append", "mla_sparse_decode_fp8_splits", "mla_sparse_decode_fp8_workspace_bytes",
    "mla_sparse_decode_fp8", "mla_noalloc_scratch_bytes", "mla_sparse_decode_noalloc", "mla_dense_decode_fp8", "mla_stage_nvfp4_fp8", "mla_kv_quant_pth",
    "mla_sparse_decode_pth_workspace_bytes", "mla_sparse_decode_pth", "mla_index_key_quant", "mla_index_logits",
    "mla_index_topk_workspace_bytes", "mla_index_topk",
]


class MlaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (built in-tree on first use if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    _lib = _load(LIB_PATH)
    return _lib


def use_timeline_library() -> None:
    """Bind every function to the instrumented build of the library instead (the same kernels with the
    decode kernel's phase timestamps compiled in; see timeline()).  For bench.py --timeline: call it
    before any other function of this module."""
    global _lib
    if _lib is not None:
        raise RuntimeError("use_timeline_library() must come before the library is first used")
    if not os.path.exists(TIMELINE_LIB_PATH):
        build()
    _lib = _load(TIMELINE_LIB_PATH, timeline=True)


def timeline(workgroups: int):
    """The instrumented library's phase stamps of the last decode launch: int64 [workgroups, 16]
    (slots described beside MLA_STAMP in csrc/mla_decode.hip; stamps in 10 ns ticks)."""
    import numpy as np
    if _lib is None or not hasattr(_lib, "mla_debug_timeline"):
        raise RuntimeError("timeline() needs use_timeline_library()")
    out = np.zeros((workgroups, 16), np.uint64)
    if _lib.mla_debug_timeline(out.ctypes.data, workgroups) != 0:
        raise RuntimeError("mla_debug_timeline failed")
    return out.astype(np.int64)


def _load(path, timeline=False) -> ctypes.CDLL:
    L = ctypes.CDLL(path)
    P, i64, i32, sz, f = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    sig = {
        "mla_abi_version": (ctypes.c_int, []),
        "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "mla_kv_quant_nvfp4": (ctypes.c_int, [P, i64, P, i64, P, i64, P, i64, i64, P]),
        "mla_kv_quant_fp8": (ctypes.c_int, [P, i64, P, i64, P, i64, P, i64, i64, P]),
        "mla_sparse_decode_splits": (ctypes.c_int, [i32, i32, i32, i32]),
        "mla_dense_decode_splits": (ctypes.c_int, [i32, i32, i32, i32]),
        "mla_sparse_decode_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "mla_dense_decode_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "mla_sparse_decode": (ctypes.c_int, [P, P, i64, i64, P, i64, P, P, i32, i32, i32, i32, f, i32, i32, P, P, P,
                                             sz, P]),
        "mla_sparse_decode_append": (ctypes.c_int, [P, P, i64, i64, P, i64, P, P, P, i64, P, i64, i32, i32, i32, i32,
                                                    f, i32, i32, P, P, P, sz, P]),
        "mla_dense_decode_fp8": (ctypes.c_int, [P, P, i64, i64, P, i64, P, i32, i32, i32, i32, f, i32, i32, P, P, P,
                                                sz, P]),
        "mla_sparse_decode_fp8_splits": (ctypes.c_int, [i32, i32, i32, i32]),
        "mla_noalloc_scratch_bytes": (sz, []),
        "mla_sparse_decode_noalloc": (ctypes.c_int, [P, P, i64, i64, P, i64, P, P, i32, i32, i32, i32, f, i32, i32, P,
                                                     P, P]),
        "mla_sparse_decode_fp8_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "mla_sparse_decode_fp8": (ctypes.c_int, [P, P, i64, i64, P, i64, P, P, i32, i32, i32, i32, f, i32, i32, P, P,
                                                 P, sz, P]),
        "mla_stage_nvfp4_fp8": (ctypes.c_int, [P, i64, i64, P, i64, P, P, i32, i32, i32, i32, P, P, P, P]),
        "mla_kv_quant_pth": (ctypes.c_int, [P, i64, P, i64, P, i64, P, P, P, i64, P]),
        "mla_sparse_decode_pth_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "mla_sparse_decode_pth": (ctypes.c_int, [P, P, P, P, i64, P, i64, P, P, i32, i32, i32, i32, f, i32, i32, P, P,
                                                 P, sz, P]),
        "mla_index_key_quant": (ctypes.c_int, [P, i64, P, i64, P, i64, i64, P]),
        "mla_index_logits": (ctypes.c_int, [P, P, i32, P, i64, i64, P, i64, P, i32, i32, i32, i32, P, i64, P]),
        "mla_index_topk_workspace_bytes": (sz, [i64, i64]),
        "mla_index_topk": (ctypes.c_int, [P, i64, P, i64, i32, P, P, sz, P]),
    }
    if timeline:
        sig["mla_debug_timeline"] = (ctypes.c_int, [P, i64])
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


# While `prepare` runs a binding function, its C-ABI calls are recorded instead of made.
_recording = None


def _call(name, *args):
    if _recording is not None:
        _recording.append((getattr(lib(), name), name, args))
        return 0
    return getattr(lib(), name)(*args)


class Prepared:
    """C-ABI call(s) of one binding call with their arguments checked and converted once (see prepare)."""

    def __init__(self, calls, keep):
        self._calls = calls
        self._keep = keep  # the tensors whose addresses the calls hold

    def __call__(self):
        for fn, name, args in self._calls:
            st = fn(*args)
            if st != 0:
                raise MlaError(name, st)


def prepare(fn, *args, **kwargs):
    """Check and convert the arguments of a binding call once, e.g. prepare(mla_sparse_decode, q, ...,
    out=out, workspace=ws, stream=s); the returned callable enqueues the same C-ABI call(s) again on the same
    stream, with no per-call validation.  Its tensors must stay alive, in place and of the same shape."""
    global _recording
    _recording = []
    try:
        result = fn(*args, **kwargs)
    finally:
        calls, _recording = _recording, None
    return Prepared(calls, (args, kwargs, result))


def _check(fn, status):
    if status != 0:
        raise MlaError(fn, status)


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


# --------------------------------------------------------------------------- quantize-on-write

def _quant(fn_name, k_nope, k_rope, slot_mapping, pool, page_stride_bytes, num_pages, stream):
    import torch
    _dev(k_nope, torch.bfloat16, "k_nope")
    _dev(k_rope, torch.bfloat16, "k_rope")
    _dev(slot_mapping, torch.int64, "slot_mapping")
    _dev(pool, torch.uint8, "pool")
    n = slot_mapping.numel()
    if k_nope.dim() != 2 or k_nope.shape[1] != LATENT_DIM or k_nope.stride(1) != 1 or k_nope.shape[0] != n:
        raise ValueError("k_nope must be [n, 512] with unit inner stride")
    if k_rope.dim() != 2 or k_rope.shape[1] != ROPE_DIM or k_rope.stride(1) != 1 or k_rope.shape[0] != n:
        raise ValueError("k_rope must be [n, 64] with unit inner stride")
    if not slot_mapping.is_contiguous() or not pool.is_contiguous():
        raise ValueError("slot_mapping and pool must be contiguous")
    row_bytes = NVFP4_ROW_BYTES if fn_name == "mla_kv_quant_nvfp4" else FP8_ROW_BYTES
    # the last page's 64 rows must lie inside the pool (which may be one layer of a block-major cache)
    if num_pages < 1 or pool.numel() < page_stride_bytes * (num_pages - 1) + PAGE_TOKENS * row_bytes:
        raise ValueError("pool too small for num_pages pages of page_stride_bytes")
    st = _call(fn_name, k_nope.data_ptr(), k_nope.stride(0), k_rope.data_ptr(), k_rope.stride(0),
                                 slot_mapping.data_ptr(), n, pool.data_ptr(), int(page_stride_bytes), int(num_pages),
                                 _stream(stream))
    _check(fn_name, st)


def mla_kv_quant_nvfp4(k_nope, k_rope, slot_mapping, pool, page_stride_bytes, num_pages, stream=None):
    """Write n tokens as 352-byte NVFP4 rows into the page pool (see include/mla_nvfp4.h)."""
    _quant("mla_kv_quant_nvfp4", k_nope, k_rope, slot_mapping, pool, page_stride_bytes, num_pages, stream)


def mla_kv_quant_fp8(k_nope, k_rope, slot_mapping, pool, page_stride_bytes, num_pages, stream=None):
    """Write n tokens as 576-byte FP8 rows into the page pool (see include/mla_nvfp4.h)."""
    _quant("mla_kv_quant_fp8", k_nope, k_rope, slot_mapping, pool, page_stride_bytes, num_pages, stream)


# --------------------------------------------------------------------------- decode

def mla_sparse_decode_splits(B, T, H, topk):
    return lib().mla_sparse_decode_splits(B, T, H, topk)


def mla_dense_decode_splits(B, T, H, max_context):
    return lib().mla_dense_decode_splits(B, T, H, max_context)


def mla_sparse_decode_workspace_bytes(B, T, H, topk, num_splits=0):
    return lib().mla_sparse_decode_workspace_bytes(B, T, H, topk, num_splits)


def mla_dense_decode_workspace_bytes(B, T, H, max_context, num_splits=0):
    return lib().mla_dense_decode_workspace_bytes(B, T, H, max_context, num_splits)


def _decode_io(q, out, lse, workspace, ws_bytes):
    import torch
    B, T, H, _ = q.shape
    if out is None:
        out = torch.empty((B, T, H, LATENT_DIM), dtype=torch.bfloat16, device=q.device)
    _dev(out, torch.bfloat16, "out")
    if tuple(out.shape) != (B, T, H, LATENT_DIM) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, T, H, 512] bf16 tensor")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
        if tuple(lse.shape) != (B, T, H) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous [B, T, H] fp32 tensor")
    if ws_bytes and workspace is None:
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=q.device)  # counters start at zero
    if workspace is not None:
        _dev(workspace, torch.uint8, "workspace")
    return out, lse, workspace


def _common(q, pool, block_table, context_lens):
    import torch
    _dev(q, torch.bfloat16, "q")
    _dev(pool, torch.uint8, "pool")
    _dev(block_table, torch.int32, "block_table")
    _dev(context_lens, torch.int32, "context_lens")
    if q.dim() != 4 or q.shape[3] != QK_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, T, H, 576] bf16 tensor")
    if block_table.dim() != 2 or not block_table.is_contiguous() or block_table.shape[0] != q.shape[0]:
        raise ValueError("block_table must be a contiguous [B, pages] int32 tensor")
    if context_lens.numel() != q.shape[0] or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [B] int32 tensor")


def _sparse(fn, ws_fn, q, pool, page_stride_bytes, num_pages, block_table, context_lens, indices, sm_scale, causal,
            num_splits, out, lse, workspace, stream):
    import torch
    _common(q, pool, block_table, context_lens)
    _dev(indices, torch.int32, "indices")
    B, T, H, _ = q.shape
    if indices.dim() != 3 or tuple(indices.shape[:2]) != (B, T) or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous [B, T, topk] int32 tensor")
    topk = indices.shape[2]
    ws = getattr(lib(), ws_fn)(B, T, H, topk, int(num_splits))
    out, lse, workspace = _decode_io(q, out, lse, workspace, ws)
    st = _call(fn, q.data_ptr(), pool.data_ptr(), int(page_stride_bytes), int(num_pages),
                            block_table.data_ptr(), block_table.stride(0), context_lens.data_ptr(), indices.data_ptr(),
                            B, T, H, topk, float(sm_scale), int(bool(causal)), int(num_splits), out.data_ptr(),
                            None if lse is None else lse.data_ptr(), None if workspace is None else workspace.data_ptr(),
                            0 if workspace is None else workspace.numel(), _stream(stream))
    _check(fn, st)
    return out, lse


def mla_sparse_decode(q, pool, page_stride_bytes, num_pages, block_table, context_lens, indices, sm_scale,
                      causal=False, num_splits=0, out=None, lse=None, workspace=None, stream=None):
    """Sparse MLA decode over NVFP4 rows; returns (out [B,T,H,512] bf16, lse or None)."""
    return _sparse("mla_sparse_decode", "mla_sparse_decode_workspace_bytes", q, pool, page_stride_bytes, num_pages,
                   block_table, context_lens, indices, sm_scale, causal, num_splits, out, lse, workspace, stream)


def mla_sparse_decode_append(q, pool, page_stride_bytes, num_pages, block_table, context_lens, indices, k_nope, k_rope,
                             sm_scale, causal=False, num_splits=0, out=None, lse=None, workspace=None, stream=None):
    """One decode step in one launch: each query token's new row (k_nope [B*T, 512], k_rope [B*T, 64] bf16,
    row b*T + t) written at position context_lens[b] - T + t, then mla_sparse_decode over the cache with
    those rows in it; returns (out, lse).  The pool is written."""
    import torch
    _common(q, pool, block_table, context_lens)
    _dev(indices, torch.int32, "indices")
    _dev(k_nope, torch.bfloat16, "k_nope")
    _dev(k_rope, torch.bfloat16, "k_rope")
    B, T, H, _ = q.shape
    if indices.dim() != 3 or tuple(indices.shape[:2]) != (B, T) or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous [B, T, topk] int32 tensor")
    if k_nope.dim() != 2 or tuple(k_nope.shape) != (B * T, LATENT_DIM) or k_nope.stride(1) != 1:
        raise ValueError("k_nope must be [B*T, 512] with unit inner stride")
    if k_rope.dim() != 2 or tuple(k_rope.shape) != (B * T, ROPE_DIM) or k_rope.stride(1) != 1:
        raise ValueError("k_rope must be [B*T, 64] with unit inner stride")
    topk = indices.shape[2]
    ws = lib().mla_sparse_decode_workspace_bytes(B, T, H, topk, int(num_splits))
    out, lse, workspace = _decode_io(q, out, lse, workspace, ws)
    st = _call("mla_sparse_decode_append", q.data_ptr(), pool.data_ptr(), int(page_stride_bytes), int(num_pages),
               block_table.data_ptr(), block_table.stride(0), context_lens.data_ptr(), indices.data_ptr(),
               k_nope.data_ptr(), k_nope.stride(0), k_rope.data_ptr(), k_rope.stride(0), B, T, H, topk,
               float(sm_scale), int(bool(causal)), int(num_splits), out.data_ptr(),
               None if lse is None else lse.data_ptr(), None if workspace is None else workspace.data_ptr(),
               0 if workspace is None else workspace.numel(), _stream(stream))
    _check("mla_sparse_decode_append", st)
    return out, lse


def mla_sparse_decode_fp8(q, pool, page_stride_bytes, num_pages, block_table, context_lens, indices, sm_scale,
                          causal=False, num_splits=0, out=None, lse=None, workspace=None, stream=None):
    """Sparse MLA decode over 576-byte FP8 rows (the FP8-cache arm of the pages' comparison); returns
    (out [B,T,H,512] bf16, lse or None)."""
    return _sparse("mla_sparse_decode_fp8", "mla_sparse_decode_fp8_workspace_bytes", q, pool, page_stride_bytes,
                   num_pages, block_table, context_lens, indices, sm_scale, causal, num_splits, out, lse, workspace,
                   stream)


def mla_sparse_decode_noalloc(q, pool, page_stride_bytes, num_pages, block_table, context_lens, indices, sm_scale,
                              causal=False, num_splits=0, out=None, lse=None, stream=None):
    """mla_sparse_decode with the library's own scratch array instead of a workspace (the call allocates
    nothing; out and lse must then be given): returns (out, lse)."""
    import torch
    _common(q, pool, block_table, context_lens)
    _dev(indices, torch.int32, "indices")
    B, T, H, _ = q.shape
    if indices.dim() != 3 or tuple(indices.shape[:2]) != (B, T) or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous [B, T, topk] int32 tensor")
    if out is None:
        raise ValueError("out must be given (the call allocates nothing)")
    out, lse, _ = _decode_io(q, out, lse, None, 0)
    st = _call("mla_sparse_decode_noalloc", q.data_ptr(), pool.data_ptr(), int(page_stride_bytes), int(num_pages),
                                         block_table.data_ptr(), block_table.stride(0), context_lens.data_ptr(),
                                         indices.data_ptr(), B, T, H, indices.shape[2], float(sm_scale),
                                         int(bool(causal)), int(num_splits), out.data_ptr(),
                                         None if lse is None else lse.data_ptr(), _stream(stream))
    _check("mla_sparse_decode_noalloc", st)
    return out, lse


def mla_sparse_decode_fp8_splits(B, T, H, topk):
    return lib().mla_sparse_decode_fp8_splits(B, T, H, topk)


def mla_sparse_decode_fp8_workspace_bytes(B, T, H, topk, num_splits=0):
    return lib().mla_sparse_decode_fp8_workspace_bytes(B, T, H, topk, num_splits)


def mla_dense_decode_fp8(q, pool, page_stride_bytes, num_pages, block_table, context_lens, max_context, sm_scale,
                         causal=False, num_splits=0, out=None, lse=None, workspace=None, stream=None):
    """Dense MLA decode over 576-byte FP8 rows; returns (out [B,T,H,512] bf16, lse or None)."""
    _common(q, pool, block_table, context_lens)
    B, T, H, _ = q.shape
    ws = lib().mla_dense_decode_workspace_bytes(B, T, H, int(max_context), int(num_splits))
    out, lse, workspace = _decode_io(q, out, lse, workspace, ws)
    st = _call("mla_dense_decode_fp8", q.data_ptr(), pool.data_ptr(), int(page_stride_bytes), int(num_pages),
                                    block_table.data_ptr(), block_table.stride(0), context_lens.data_ptr(), B, T, H,
                                    int(max_context), float(sm_scale), int(bool(causal)), int(num_splits),
                                    out.data_ptr(), None if lse is None else lse.data_ptr(),
                                    None if workspace is None else workspace.data_ptr(),
                                    0 if workspace is None else workspace.numel(), _stream(stream))
    _check("mla_dense_decode_fp8", st)
    return out, lse


def mla_stage_nvfp4_fp8(pool, page_stride_bytes, num_pages, block_table, context_lens, indices, causal=False,
                        staged=None, staged_block_table=None, staged_lens=None, stream=None):
    """The staged path's unpack: each query token's selected NVFP4 rows as 576-byte FP8 rows of a paged
    copy.  Returns (staged uint8 [B*T*P*64*576], staged_block_table int32 [B*T, P], staged_lens int32
    [B*T]), P = ceil(topk/64); mla_dense_decode_fp8 reads the copy (see include/mla_nvfp4.h)."""
    import torch
    _dev(pool, torch.uint8, "pool")
    _dev(indices, torch.int32, "indices")
    if indices.dim() != 3 or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous [B, T, topk] int32 tensor")
    B, T, topk = indices.shape
    if block_table.dim() != 2 or not block_table.is_contiguous() or block_table.shape[0] != B:
        raise ValueError("block_table must be a contiguous [B, pages] int32 tensor")
    if context_lens.numel() != B or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [B] int32 tensor")
    P = (topk + PAGE_TOKENS - 1) // PAGE_TOKENS
    dev = indices.device
    if staged is None:
        staged = torch.empty(B * T * P * PAGE_TOKENS * FP8_ROW_BYTES, dtype=torch.uint8, device=dev)
    if staged_block_table is None:
        staged_block_table = torch.empty((B * T, P), dtype=torch.int32, device=dev)
    if staged_lens is None:
        staged_lens = torch.empty(B * T, dtype=torch.int32, device=dev)
    if staged.numel() < B * T * P * PAGE_TOKENS * FP8_ROW_BYTES or tuple(staged_block_table.shape) != (B * T, P) \
            or staged_lens.numel() != B * T:
        raise ValueError("staged buffers have the wrong size")
    st = _call("mla_stage_nvfp4_fp8", pool.data_ptr(), int(page_stride_bytes), int(num_pages), block_table.data_ptr(),
                                   block_table.stride(0), context_lens.data_ptr(), indices.data_ptr(), B, T, topk,
                                   int(bool(causal)), staged.data_ptr(), staged_block_table.data_ptr(),
                                   staged_lens.data_ptr(), _stream(stream))
    _check("mla_stage_nvfp4_fp8", st)
    return staged, staged_block_table, staged_lens


# --------------------------------------------------------------------------- per-token-head FP8 layout

def mla_kv_quant_pth(k_nope, k_rope, slot_mapping, lat, scale, rope, stream=None):
    """Write n tokens in TokenSpeed's per-token-head FP8 layout (see include/mla_nvfp4.h): lat uint8
    [slots, 512], scale float32 [slots], rope bfloat16 [slots, 64]."""
    import torch
    _dev(k_nope, torch.bfloat16, "k_nope")
    _dev(k_rope, torch.bfloat16, "k_rope")
    _dev(slot_mapping, torch.int64, "slot_mapping")
    _dev(lat, torch.uint8, "lat")
    _dev(scale, torch.float32, "scale")
    _dev(rope, torch.bfloat16, "rope")
    n = slot_mapping.numel()
    if k_nope.dim() != 2 or k_nope.shape != (n, LATENT_DIM) or k_nope.stride(1) != 1:
        raise ValueError("k_nope must be [n, 512] with unit inner stride")
    if k_rope.dim() != 2 or k_rope.shape != (n, ROPE_DIM) or k_rope.stride(1) != 1:
        raise ValueError("k_rope must be [n, 64] with unit inner stride")
    slots = scale.numel()
    if (lat.shape != (slots, LATENT_DIM) or rope.shape != (slots, ROPE_DIM) or not lat.is_contiguous()
            or not rope.is_contiguous() or not scale.is_contiguous() or not slot_mapping.is_contiguous()):
        raise ValueError("lat [slots, 512], scale [slots] and rope [slots, 64] must be contiguous")
    st = _call("mla_kv_quant_pth", k_nope.data_ptr(), k_nope.stride(0), k_rope.data_ptr(), k_rope.stride(0),
                                slot_mapping.data_ptr(), n, lat.data_ptr(), scale.data_ptr(), rope.data_ptr(), slots,
                                _stream(stream))
    _check("mla_kv_quant_pth", st)


def mla_sparse_decode_pth(q, lat, scale, rope, block_table, context_lens, indices, sm_scale, causal=False,
                          num_splits=0, out=None, lse=None, stream=None):
    """Sparse decode over the per-token-head layout (see include/mla_nvfp4.h).  Returns (out, lse)."""
    import torch
    _dev(q, torch.bfloat16, "q")
    for t, dt, name in ((lat, torch.uint8, "lat"), (scale, torch.float32, "scale"), (rope, torch.bfloat16, "rope"),
                        (block_table, torch.int32, "block_table"), (context_lens, torch.int32, "context_lens"),
                        (indices, torch.int32, "indices")):
        _dev(t, dt, name)
    if q.dim() != 4 or q.shape[3] != QK_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, T, H, 576] tensor")
    B, T, H, _ = q.shape
    if indices.dim() != 3 or indices.shape[:2] != (B, T) or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous [B, T, topk] tensor")
    if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [B, pages] tensor")
    topk = indices.shape[2]
    ws_bytes = lib().mla_sparse_decode_pth_workspace_bytes(B, T, H, topk, int(num_splits))
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device) if ws_bytes else None
    if out is None:
        out = torch.empty((B, T, H, LATENT_DIM), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    st = _call("mla_sparse_decode_pth", q.data_ptr(), lat.data_ptr(), scale.data_ptr(), rope.data_ptr(), scale.numel(),
                                     block_table.data_ptr(), block_table.shape[1], context_lens.data_ptr(),
                                     indices.data_ptr(), B, T, H, topk, float(sm_scale), int(bool(causal)),
                                     int(num_splits), out.data_ptr(), lse.data_ptr(),
                                     None if workspace is None else workspace.data_ptr(),
                                     0 if workspace is None else workspace.numel(), _stream(stream))
    _check("mla_sparse_decode_pth", st)
    return out, lse


# --------------------------------------------------------------------------- sparse-indexer keys and logits
INDEX_DIM, INDEX_PAGE_BYTES = 128, 64 * 128 + 64 * 4


def mla_index_key_quant(keys, slot_mapping, pool, page_stride_bytes, num_pages, stream=None):
    """Write n indexer keys (bf16 [n, 128], unit inner stride) as 128 E4M3 codes + an fp32 scale each into
    the paged indexer pool (see include/mla_nvfp4.h)."""
    import torch
    _dev(keys, torch.bfloat16, "keys")
    _dev(slot_mapping, torch.int64, "slot_mapping")
    _dev(pool, torch.uint8, "pool")
    n = slot_mapping.numel()
    if keys.dim() != 2 or keys.shape[1] != INDEX_DIM or keys.stride(1) != 1 or keys.shape[0] != n:
        raise ValueError("keys must be [n, 128] with unit inner stride")
    if not slot_mapping.is_contiguous() or not pool.is_contiguous():
        raise ValueError("slot_mapping and pool must be contiguous")
    if num_pages < 1 or pool.numel() < page_stride_bytes * (num_pages - 1) + INDEX_PAGE_BYTES:
        raise ValueError("pool too small for num_pages pages of page_stride_bytes")
    st = _call("mla_index_key_quant", keys.data_ptr(), keys.stride(0), slot_mapping.data_ptr(), n, pool.data_ptr(),
                                   int(page_stride_bytes), int(num_pages), _stream(stream))
    _check("mla_index_key_quant", st)


def mla_index_logits(q, w, pool, page_stride_bytes, num_pages, block_table, context_lens, max_context, causal=False,
                     out=None, stream=None):
    """Indexer logits (a DeepSeek-style reading; see include/mla_nvfp4.h): q bf16 [B, T, HI, 128], w fp32
    [B, T, HI].  Returns fp32 [B*T, ld] (ld = max_context rounded up to 4; positions past each query
    token's limit are left as allocated)."""
    import torch
    _dev(q, torch.bfloat16, "q")
    _dev(w, torch.float32, "w")
    _dev(pool, torch.uint8, "pool")
    _dev(block_table, torch.int32, "block_table")
    _dev(context_lens, torch.int32, "context_lens")
    if q.dim() != 4 or q.shape[3] != INDEX_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, T, HI, 128] tensor")
    B, T, HI, _ = q.shape
    if tuple(w.shape) != (B, T, HI) or not w.is_contiguous():
        raise ValueError("w must be a contiguous [B, T, HI] tensor")
    if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [B, pages] tensor")
    if context_lens.numel() != B or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [B] tensor")
    ld = (int(max_context) + 3) // 4 * 4
    if out is None:
        out = torch.empty((B * T, ld), dtype=torch.float32, device=q.device)
    _dev(out, torch.float32, "out")
    if out.dim() != 2 or out.shape[0] != B * T or out.shape[1] < max_context or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B*T, >= max_context] tensor")
    st = _call("mla_index_logits", q.data_ptr(), w.data_ptr(), HI, pool.data_ptr(), int(page_stride_bytes),
                                int(num_pages), block_table.data_ptr(), block_table.shape[1], context_lens.data_ptr(),
                                B, T, int(max_context), int(bool(causal)), out.data_ptr(), out.shape[1],
                                _stream(stream))
    _check("mla_index_logits", st)
    return out


# --------------------------------------------------------------------------- index top-k

def mla_index_topk_workspace_bytes(n, ld):
    return lib().mla_index_topk_workspace_bytes(int(n), int(ld))


def mla_index_topk(logits, lengths, k, out=None, workspace=None, stream=None):
    """Per row of fp32 logits [n, ld] (contiguous, ld a multiple of 4), the positions below
    lengths[r] of the k largest values, lower positions first among ties, in ascending order and padded
    with -1 (see include/mla_nvfp4.h).  Returns int32 [n, k].  A workspace passed in must be a uint8
    device tensor zero-filled before its first use; one is allocated (zero-filled) when none is."""
    import torch
    _dev(logits, torch.float32, "logits")
    _dev(lengths, torch.int32, "lengths")
    if logits.dim() != 2 or not logits.is_contiguous():
        # contiguous, so that the device-side clamp of lengths to ld keeps every read inside the tensor
        raise ValueError("logits must be a contiguous [n, ld] tensor")
    n, ld = logits.shape
    if lengths.numel() != n or not lengths.is_contiguous():
        raise ValueError("lengths must be a contiguous [n] tensor")
    if out is None:
        out = torch.empty((n, int(k)), dtype=torch.int32, device=logits.device)
    _dev(out, torch.int32, "out")
    if tuple(out.shape) != (n, int(k)) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [n, k] int32 tensor")
    if n == 0:
        return out
    ws = lib().mla_index_topk_workspace_bytes(n, ld)
    if workspace is None:
        workspace = torch.zeros(ws, dtype=torch.uint8, device=logits.device)  # counters start at zero
    _dev(workspace, torch.uint8, "workspace")
    st = _call("mla_index_topk", logits.data_ptr(), ld, lengths.data_ptr(), n, int(k), out.data_ptr(),
                              workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check("mla_index_topk", st)
    return out
