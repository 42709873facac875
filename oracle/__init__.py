"""FP64 CPU oracle for NVFP4 compressed-latent sparse-MLA decode (ctypes binding of mla_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline leg of the benchmark
are the only callers.  Nothing in the GPU path imports this package, and this package imports
nothing from the GPU path.

Each function documents the passage it follows; mla_oracle.c's header lists the pages and the
readings taken where they are silent.  Arrays cross the boundary as numpy arrays on the host:
bf16 values travel as their uint16 bit patterns.  The index selection (topk_positions) is plain numpy
here; the pages fix only its size (2,048) and the -1 padding, and its tie rule and list order are
readings stated in its docstring.  index_logits is PARITY UNPINNED: the pages do not define the
indexer's logits, and the function computes the DeepSeek-style form named in its docstring.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")

LATENT, ROPE, QK, PAGE = 512, 64, 576, 64
NVFP4_ROW_BYTES, FP8_ROW_BYTES = 352, 576

_lib = None


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"],
                   check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64, i32, d = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    sig = {
        "mlo_bf16_value": (d, [ctypes.c_uint16]),
        "mlo_e4m3_value": (d, [ctypes.c_uint32]),
        "mlo_e2m1_value": (d, [ctypes.c_uint32]),
        "mlo_e4m3_encode_bf16": (ctypes.c_uint32, [ctypes.c_uint16]),
        "mlo_scale_code": (ctypes.c_uint32, [d]),
        "mlo_e2m1_encode": (ctypes.c_uint32, [ctypes.c_uint16, ctypes.c_uint32]),
        "mlo_e2m1_encode_bulk": (None, [P, i64, ctypes.c_uint32, P]),
        "mlo_e4m3_encode_bulk": (None, [P, i64, P]),
        "mlo_scale_code_bulk": (None, [P, i64, P]),
        "mlo_quant_row_nvfp4": (None, [P, P, P]),
        "mlo_index_key_quant_row": (None, [P, P, P]),
        "mlo_pth_quant_row": (None, [P, P, P, P, P]),
        "mlo_kv_quant_pth": (i64, [P, i64, P, i64, P, i64, P, P, P, i64]),
        "mlo_dequant_row_pth": (None, [P, ctypes.c_float, P, P]),
        "mlo_sparse_decode_pth": (i32, [P, P, P, P, i64, P, i64, P, P, i32, i32, i32, i32, d, i32, P, i64, P, P, i32]),
        "mlo_index_key_quant": (i64, [P, i64, P, i64, P, i64, i64]),
        "mlo_index_logits": (i32, [P, P, i32, P, i64, i64, P, i64, P, i32, i32, i32, P, i64, i32]),
        "mlo_quant_row_fp8": (None, [P, P, P]),
        "mlo_dequant_row_nvfp4": (None, [P, P]),
        "mlo_dequant_row_fp8": (None, [P, P]),
        "mlo_kv_quant_nvfp4": (i64, [P, i64, P, i64, P, i64, P, i64, i64]),
        "mlo_kv_quant_fp8": (i64, [P, i64, P, i64, P, i64, P, i64, i64]),
        "mlo_sparse_decode": (i32, [P, P, i64, i64, P, i64, P, P, i32, i32, i32, i32, d, i32, P, i64, P, P, i32]),
        "mlo_sparse_decode_fp8": (i32, [P, P, i64, i64, P, i64, P, P, i32, i32, i32, i32, d, i32, P, i64, P, P,
                                        i32]),
        "mlo_dense_decode_fp8": (i32, [P, P, i64, i64, P, i64, P, i32, i32, i32, d, i32, P, i64, P, P, i32]),
        "mlo_merge_partials": (None, [P, P, i32, i32, P, P]),
        "mlo_stage_nvfp4_fp8": (None, [P, i64, i64, P, i64, P, P, i32, i32, i32, i32, i64, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


# --------------------------------------------------------------------------- value definitions

def bf16_value(bits) -> float:
    return _load().mlo_bf16_value(int(bits))


def e4m3_value(code) -> float:
    """E4M3FN byte -> value (TokenSpeed write-up, MLA KV layout: torch.float8_e4m3fn, max 448)."""
    return _load().mlo_e4m3_value(int(code))


def e2m1_value(code) -> float:
    """e2m1 nibble -> value (launch post, making room for low-latency decode: four bits per value)."""
    return _load().mlo_e2m1_value(int(code))


def e4m3_encode(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> E4M3FN bytes, nearest finite, ties to even, saturating at +-448."""
    x = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(x.shape, np.uint8)
    _load().mlo_e4m3_encode_bulk(_ptr(x), x.size, _ptr(out))
    return out


def scale_code(amax_bits: np.ndarray) -> np.ndarray:
    """Block amax (bf16 bits, sign ignored) -> E4M3 scale byte nearest to amax/6."""
    x = np.ascontiguousarray(amax_bits, dtype=np.uint16)
    out = np.empty(x.shape, np.uint8)
    _load().mlo_scale_code_bulk(_ptr(x), x.size, _ptr(out))
    return out


def e2m1_encode(bits: np.ndarray, scale: int) -> np.ndarray:
    """bf16 bits -> e2m1 nibbles under one scale byte (nearest grid point of |x|/s, ties even)."""
    x = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(x.shape, np.uint8)
    _load().mlo_e2m1_encode_bulk(_ptr(x), x.size, int(scale), _ptr(out))
    return out


# --------------------------------------------------------------------------- rows

def quant_row_nvfp4(latent_bits: np.ndarray, rope_bits: np.ndarray) -> np.ndarray:
    """One token -> 352-byte row (launch post, making room for low-latency decode; analysis, row table)."""
    lat = np.ascontiguousarray(latent_bits, dtype=np.uint16).reshape(LATENT)
    rope = np.ascontiguousarray(rope_bits, dtype=np.uint16).reshape(ROPE)
    row = np.zeros(NVFP4_ROW_BYTES, np.uint8)
    _load().mlo_quant_row_nvfp4(_ptr(lat), _ptr(rope), _ptr(row))
    return row


def quant_row_fp8(latent_bits: np.ndarray, rope_bits: np.ndarray) -> np.ndarray:
    """One token -> 576-byte FP8 row (analysis, row table: no per-row scale)."""
    lat = np.ascontiguousarray(latent_bits, dtype=np.uint16).reshape(LATENT)
    rope = np.ascontiguousarray(rope_bits, dtype=np.uint16).reshape(ROPE)
    row = np.zeros(FP8_ROW_BYTES, np.uint8)
    _load().mlo_quant_row_fp8(_ptr(lat), _ptr(rope), _ptr(row))
    return row


def dequant_row_nvfp4(row: np.ndarray) -> np.ndarray:
    r = np.ascontiguousarray(row, dtype=np.uint8).reshape(NVFP4_ROW_BYTES)
    K = np.empty(QK, np.float64)
    _load().mlo_dequant_row_nvfp4(_ptr(r), _ptr(K))
    return K


def dequant_row_fp8(row: np.ndarray) -> np.ndarray:
    r = np.ascontiguousarray(row, dtype=np.uint8).reshape(FP8_ROW_BYTES)
    K = np.empty(QK, np.float64)
    _load().mlo_dequant_row_fp8(_ptr(r), _ptr(K))
    return K


# --------------------------------------------------------------------------- pool writers

def kv_quant(fmt: str, k_nope: np.ndarray, k_rope: np.ndarray, slot_mapping: np.ndarray, pool: np.ndarray,
             page_stride: int, num_pages: int) -> int:
    """Quantize-on-write into a paged pool (TokenSpeed write-up, MLA KV layout: rows written at slot
    indices).  k_nope bf16 bits [N,512], k_rope [N,64], slot_mapping int64 [N]; pool uint8 flat array
    modified in place.  Returns the number of rows written."""
    kn = np.ascontiguousarray(k_nope, dtype=np.uint16)
    kr = np.ascontiguousarray(k_rope, dtype=np.uint16)
    sl = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    n = sl.shape[0]
    assert kn.shape == (n, LATENT) and kr.shape == (n, ROPE)
    row_bytes = NVFP4_ROW_BYTES if fmt == "nvfp4" else FP8_ROW_BYTES
    # the last page's rows end PAGE rows into it (a pool may be one layer of a block-major cache, whose
    # page stride spans every layer's rows)
    assert page_stride >= PAGE * row_bytes and pool.size >= (num_pages - 1) * page_stride + PAGE * row_bytes
    f = _load().mlo_kv_quant_nvfp4 if fmt == "nvfp4" else _load().mlo_kv_quant_fp8
    return f(_ptr(kn), LATENT, _ptr(kr), ROPE, _ptr(sl), n, _ptr(pool), page_stride, num_pages)


# --------------------------------------------------------------------------- attention

def sparse_decode(q, pool, page_stride, num_pages, block_table, ctx, indices, sm_scale, causal=False, units=None,
                  nthreads=0, fmt="nvfp4"):
    """Sparse decode (launch post, native NVFP4 sparse MLA decode kernel): q bf16 bits [B,T,H,576];
    indices int32 [B,T,k] of logical positions (-1 = unused).  Returns (out [n,H,512], lse [n,H], threads)
    in float64, n = B*T or len(units).  fmt "nvfp4" reads 352-byte rows; "fp8" reads 576-byte FP8 rows
    with the same selection rule (the FP8-cache arm of the launch post's native / staged / FP8
    comparison)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    B, T, H, D = q.shape
    assert D == QK
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    k = idx.shape[2]
    assert idx.shape[:2] == (B, T)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cx = np.ascontiguousarray(ctx, dtype=np.int32)
    un = None if units is None else np.ascontiguousarray(units, dtype=np.int64)
    n = B * T if un is None else un.size
    out = np.empty((n, H, LATENT), np.float64)
    lse = np.empty((n, H), np.float64)
    assert fmt in ("nvfp4", "fp8")
    f = _load().mlo_sparse_decode if fmt == "nvfp4" else _load().mlo_sparse_decode_fp8
    used = f(_ptr(q), _ptr(pool), page_stride, num_pages, _ptr(bt), bt.shape[1], _ptr(cx), _ptr(idx), B, T, H, k,
             float(sm_scale), int(bool(causal)), _ptr(un), 0 if un is None else un.size, _ptr(out), _ptr(lse),
             int(nthreads))
    return out, lse, used


def dense_decode_fp8(q, pool, page_stride, num_pages, block_table, ctx, sm_scale, causal=False, units=None,
                     nthreads=0):
    """Dense decode over a 576-byte FP8 row cache (the FP8 attention the launch post compares with):
    every position up to the limit is attended."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    B, T, H, D = q.shape
    assert D == QK
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cx = np.ascontiguousarray(ctx, dtype=np.int32)
    un = None if units is None else np.ascontiguousarray(units, dtype=np.int64)
    n = B * T if un is None else un.size
    out = np.empty((n, H, LATENT), np.float64)
    lse = np.empty((n, H), np.float64)
    used = _load().mlo_dense_decode_fp8(_ptr(q), _ptr(pool), page_stride, num_pages, _ptr(bt), bt.shape[1],
                                        _ptr(cx), B, T, H, float(sm_scale), int(bool(causal)), _ptr(un),
                                        0 if un is None else un.size, _ptr(out), _ptr(lse), int(nthreads))
    return out, lse, used


def merge_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """LSE-weighted merge of S partial results of one query token (launch post: the blocks of a
    cluster merge their partial results).  o_parts [S,H,512], lse_parts [S,H] -> (out [H,512], lse [H])."""
    o = np.ascontiguousarray(o_parts, dtype=np.float64)
    l = np.ascontiguousarray(lse_parts, dtype=np.float64)
    S, H, _ = o.shape
    out = np.empty((H, LATENT), np.float64)
    lse = np.empty(H, np.float64)
    _load().mlo_merge_partials(_ptr(o), _ptr(l), S, H, _ptr(out), _ptr(lse))
    return out, lse


# --------------------------------------------------------------------------- staged path

def stage_nvfp4_fp8(pool, page_stride, num_pages, block_table, ctx, indices, causal=False, rows_per_token=None):
    """The staged path (launch post, native NVFP4 sparse MLA decode section; analysis page, "A kernel
    that reads four bits directly"): each query token's selected NVFP4 rows unpacked into 576-byte FP8
    rows of a temporary buffer.  indices int32 [B,T,k].  Returns (staged uint8 [B*T, R, 576] with R =
    rows_per_token (default k rounded up to whole 64-row pages), counts int32 [B*T]); row id*R + j for
    j < counts[id] is the j-th selected row of query token id, later rows are zero."""
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    B, T, k = idx.shape
    R = ((k + PAGE - 1) // PAGE) * PAGE if rows_per_token is None else int(rows_per_token)
    assert R >= k
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cx = np.ascontiguousarray(ctx, dtype=np.int32)
    staged = np.zeros((B * T, R, FP8_ROW_BYTES), np.uint8)
    counts = np.zeros(B * T, np.int32)
    _load().mlo_stage_nvfp4_fp8(_ptr(pool), page_stride, num_pages, _ptr(bt), bt.shape[1], _ptr(cx), _ptr(idx), B, T,
                                k, int(bool(causal)), R, _ptr(staged), _ptr(counts))
    return staged, counts


# --------------------------------------------------------------------------- per-token-head FP8 layout

def kv_quant_pth(k_nope, k_rope, slot_mapping, lat_buf, scale_buf, rope_buf):
    """TokenSpeed's per-token-head FP8 write (its MLA KV layout section): latent codes uint8 [slots, 512],
    fp32 scales [slots], bf16-bit rope [slots, 64], modified in place.  Returns the number written."""
    kn = np.ascontiguousarray(k_nope, dtype=np.uint16)
    kr = np.ascontiguousarray(k_rope, dtype=np.uint16)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    n = sm.size
    assert kn.shape == (n, LATENT) and kr.shape == (n, ROPE)
    slots = scale_buf.size
    assert lat_buf.dtype == np.uint8 and lat_buf.shape == (slots, LATENT) and lat_buf.flags.c_contiguous
    assert scale_buf.dtype == np.float32 and rope_buf.dtype == np.uint16 and rope_buf.shape == (slots, ROPE)
    return _load().mlo_kv_quant_pth(_ptr(kn), LATENT, _ptr(kr), ROPE, _ptr(sm), n, _ptr(lat_buf), _ptr(scale_buf),
                                    _ptr(rope_buf), slots)


def pth_quant_row(lat, rope):
    """One token: (codes uint8 [512], scale float, rope bf16 bits [64])."""
    lv = np.ascontiguousarray(lat, dtype=np.uint16)
    rv = np.ascontiguousarray(rope, dtype=np.uint16)
    codes = np.zeros(LATENT, np.uint8)
    sc = np.zeros(1, np.float32)
    rq = np.zeros(ROPE, np.uint16)
    _load().mlo_pth_quant_row(_ptr(lv), _ptr(rv), _ptr(codes), _ptr(sc), _ptr(rq))
    return codes, float(sc[0]), rq


def dequant_row_pth(codes, scale, rq):
    """K[576] (float64) of one per-token-head slot: code values x scale, stored rope x scale."""
    K = np.zeros(QK, np.float64)
    _load().mlo_dequant_row_pth(_ptr(np.ascontiguousarray(codes, np.uint8)), ctypes.c_float(scale),
                                _ptr(np.ascontiguousarray(rq, np.uint16)), _ptr(K))
    return K


def sparse_decode_pth(q, lat_buf, scale_buf, rope_buf, block_table, ctx, indices, sm_scale, causal=False, units=None,
                      nthreads=0):
    """Sparse decode over the per-token-head layout (same selection rule as sparse_decode; slot =
    page*64 + position%64).  Returns (out float64 [B,T,H,512] or [n_units,H,512], lse, threads used)."""
    qv = np.ascontiguousarray(q, dtype=np.uint16)
    B, T, H, _ = qv.shape
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    k = idx.shape[2]
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cx = np.ascontiguousarray(ctx, dtype=np.int32)
    un = None if units is None else np.ascontiguousarray(units, dtype=np.int64)
    nq = B * T if un is None else un.size
    out = np.zeros((nq, H, LATENT), np.float64)
    lse = np.zeros((nq, H), np.float64)
    used = _load().mlo_sparse_decode_pth(_ptr(qv), _ptr(lat_buf), _ptr(scale_buf), _ptr(rope_buf), scale_buf.size,
                                         _ptr(bt), bt.shape[1], _ptr(cx), _ptr(idx), B, T, H, k, float(sm_scale),
                                         int(bool(causal)), None if un is None else _ptr(un), nq, _ptr(out),
                                         _ptr(lse), nthreads)
    if un is None:
        out = out.reshape(B, T, H, LATENT)
        lse = lse.reshape(B, T, H)
    return out, lse, used


# --------------------------------------------------------------------------- sparse indexer keys and logits
INDEX_DIM = 128
INDEX_PAGE_BYTES = PAGE * INDEX_DIM + PAGE * 4  # 64 rows of 128 codes, then 64 fp32 scales


def index_key_quant(keys, slot_mapping, pool, page_stride, num_pages):
    """Indexer keys (analysis page, "Four bits per latent value: where 352 comes from": 128 FP8 values
    plus a scale per token; the quantization is the TokenSpeed write-up's per-token FP8 rule, a reading):
    keys bf16 bits [n, 128] into the paged indexer pool (uint8, modified in place).  Returns the number
    of keys written."""
    k = np.ascontiguousarray(keys, dtype=np.uint16)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    assert k.ndim == 2 and k.shape[1] == INDEX_DIM and sm.shape == (k.shape[0],)
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    assert page_stride >= INDEX_PAGE_BYTES and pool.size >= page_stride * (num_pages - 1) + INDEX_PAGE_BYTES
    return _load().mlo_index_key_quant(_ptr(k), INDEX_DIM, _ptr(sm), k.shape[0], _ptr(pool), page_stride, num_pages)


def index_key_quant_row(x):
    """One key: bf16 bits [128] -> (codes uint8 [128], fp32 scale)."""
    xv = np.ascontiguousarray(x, dtype=np.uint16)
    codes = np.zeros(INDEX_DIM, np.uint8)
    sc = np.zeros(1, np.float32)
    _load().mlo_index_key_quant_row(_ptr(xv), _ptr(codes), _ptr(sc))
    return codes, float(sc[0])


def index_logits(q, w, pool, page_stride, num_pages, block_table, ctx, causal=False, ld=None, nthreads=0):
    """Indexer logits, PARITY UNPINNED: the pages do not define them; this is the DeepSeek-style form
    the analysis page points to.  logits[b*T+t, p] = s_p * sum_j w[b,t,j] * max(0, <q[b,t,j], k_p>)
    for p up to the query token's limit (k_p: the key's E4M3 values, s_p its scale), -inf on page
    entries outside the pool, NaN past the limit.  q bf16 bits [B,T,HI,128], w float32 [B,T,HI].
    Returns float64 [B*T, ld]."""
    qv = np.ascontiguousarray(q, dtype=np.uint16)
    wv = np.ascontiguousarray(w, dtype=np.float32)
    B, T, HI, D = qv.shape
    assert D == INDEX_DIM and wv.shape == (B, T, HI)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cx = np.ascontiguousarray(ctx, dtype=np.int32)
    if ld is None:
        ld = int(cx.max()) if cx.size else 0
    out = np.full((B * T, ld), np.nan, np.float64)
    _load().mlo_index_logits(_ptr(qv), _ptr(wv), HI, _ptr(pool), page_stride, num_pages, _ptr(bt), bt.shape[1],
                             _ptr(cx), B, T, int(bool(causal)), _ptr(out), ld, nthreads)
    return out


# --------------------------------------------------------------------------- index selection (top-k)

def topk_positions(logits, lengths, k):
    """The sparse indexer's last step (launch post, native NVFP4 sparse MLA decode section: each query
    token attends to at most 2,048 positions the indexer selects, -1 marking unused list entries; the
    analysis page, section "Decode: TP4, and the copies it keeps": index_topk 2048): for each row, the
    positions i < lengths[r] of the k largest logits[r, i], compared as numbers (-0 equals +0).
    Readings where the pages are silent: ties at the k-th value go to the lower positions, and the list
    is in ascending position order (the decode reads it as a set); a row with at most k positions lists
    them all, then -1.  logits float32 [n, ld] (no NaN), lengths int [n] (0 <= lengths <= ld).
    Returns int32 [n, k]."""
    x = np.asarray(logits, dtype=np.float32)
    n = x.shape[0]
    out = np.full((n, k), -1, np.int32)
    for r in range(n):
        m = int(lengths[r])
        if m <= 0:
            continue
        v = x[r, :m].astype(np.float64)
        pos = np.arange(m)
        order = np.lexsort((pos, -v))  # by value descending, then by position ascending
        chosen = np.sort(order[:min(k, m)])
        out[r, :chosen.size] = chosen
    return out
