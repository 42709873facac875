"""C-ABI library checks that need no GPU: it loads, exports every symbol include/mla_nvfp4.h declares,
and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

import nvfp4_compressed_sparse_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header="mla_nvfp4.h"):
    with open(os.path.join(ROOT, "include", header)) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 10
    L = M.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(M.EXPORTS)


def test_timeline_library_exports_the_decode_abi_and_its_reader():
    from nvfp4_compressed_sparse_amd.build import TIMELINE_LIB
    T = ctypes.CDLL(TIMELINE_LIB)
    for n in _declared_functions() + _declared_functions("mla_timeline.h"):
        assert hasattr(T, n), n
    assert _declared_functions("mla_timeline.h") == ["mla_debug_timeline"]
    assert not hasattr(M.lib(), "mla_debug_timeline")  # the product library has no instrumentation
    T.mla_debug_timeline.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    assert T.mla_debug_timeline(None, 1) == 1 and T.mla_debug_timeline(FAKE, 4097) == 1  # rejected on the host


def test_probe_library_exports_every_declared_symbol():
    from nvfp4_compressed_sparse_amd import probe
    names = _declared_functions("mla_probe.h")
    assert set(names) == set(probe.EXPORTS)
    for n in names:
        assert hasattr(probe.lib(), n), n
    assert probe.lib().mla_probe_stream_read(None, 1 << 20, FAKE, 1, None) == 1  # bad argument: nothing launched
    assert probe.lib().mla_probe_row_gather(FAKE, FAKE, 1000, 352, FAKE, 1, None) == 2  # grid too small
    assert probe.mfma_flops(10, 2) == 2 * 4 * 10 * 8 * 16 * 16 * 32 * 2


def test_version_and_status_strings():
    L = M.lib()
    assert L.mla_abi_version() == 1
    for s in range(7):
        assert L.mla_status_string(s)
    assert L.mla_status_string(0) == b"ok"


FAKE = 1 << 20  # a 16/256-byte aligned fake device address; never dereferenced (checks fail first)


def _sparse(**kw):
    a = dict(q=FAKE, pool=FAKE, ps=64 * 352, npg=10, bt=FAKE, bts=4, ctx=FAKE, idx=FAKE, B=2, T=1, H=16, k=256,
             sc=0.07, causal=0, S=0, out=FAKE, lse=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    return M.lib().mla_sparse_decode(a["q"], a["pool"], a["ps"], a["npg"], a["bt"], a["bts"], a["ctx"], a["idx"],
                                     a["B"], a["T"], a["H"], a["k"], a["sc"], a["causal"], a["S"], a["out"],
                                     a["lse"], a["ws"], a["wsb"], a["stream"])


def test_sparse_decode_argument_errors():
    assert _sparse(q=None) == 1
    assert _sparse(idx=None) == 1
    assert _sparse(out=None) == 1
    assert _sparse(B=0) == 2
    assert _sparse(T=0) == 2
    assert _sparse(H=48) == 2
    assert _sparse(k=0) == 2
    assert _sparse(k=2049) == 2
    assert _sparse(causal=2) == 2
    assert _sparse(S=65) == 2
    assert _sparse(npg=0) == 2
    assert _sparse(ps=64 * 352 - 16) == 3
    assert _sparse(ps=64 * 352 + 8) == 3
    assert _sparse(q=FAKE + 8) == 3
    assert _sparse(out=FAKE + 2) == 3
    assert _sparse(sc=float("nan")) == 2
    assert _sparse(sc=0.0) == 2
    assert _sparse(sc=-0.07) == 2
    assert _sparse(sc=float("inf")) == 2
    # split path needs a workspace of the advertised size
    need = M.lib().mla_sparse_decode_workspace_bytes(2, 1, 16, 256, 4)
    assert need > 0
    assert _sparse(S=4) == 1
    assert _sparse(S=4, ws=FAKE, wsb=need - 1) == 4
    assert _sparse(S=4, ws=FAKE + 16, wsb=need) == 3
    # valid arguments reach the device check: no gfx950 device here
    import torch
    if not torch.cuda.is_available():
        assert _sparse(S=4, ws=FAKE, wsb=need) == 5
        assert _sparse(S=1) == 5


def test_launch_size_limits():
    """Grids past 2^32 - 1 threads, and split launches with more than 65,536 counters, are refused on the
    host (sizes whose 32-bit grid product would wrap)."""
    big = dict(ws=FAKE, wsb=1 << 62)
    # 16 heads: B*T*S workgroups of 512 threads; 2^23 of them is 2^32 threads
    assert _sparse(B=1 << 20, T=8, S=1) == 2
    assert _sparse(B=(1 << 20) - 1, T=8, S=1, **big) in (5, 0)  # fits; reaches the device check
    assert _sparse(B=1 << 16, T=2, S=64, **big) == 2
    # split launches: at most 65,536 query tokens x head groups
    assert _sparse(B=65537, T=1, S=2, **big) == 2
    assert _sparse(B=65536, T=1, S=2, **big) in (5, 0)
    # writers: one 64-lane wave per token, fewer than 2^26 tokens
    assert _quant(n=1 << 26) == 2
    assert _quant(n=(1 << 26) - 1) in (5, 0)
    # top-k: n * ceil(ld / 8192) workgroups of 512 threads
    assert _topk(n=1 << 23, ld=4096, wsb=1 << 62) == 2
    assert _topk(n=(1 << 23) - 1, ld=4096, wsb=1 << 62) in (5, 0)
    # stage: up to 16 workgroups of 256 threads per query token
    assert _stage(B=1 << 20) == 2


def test_sparse_fp8_decode_argument_errors():
    def call(**kw):
        a = dict(q=FAKE, pool=FAKE, ps=64 * 576, npg=10, bt=FAKE, bts=4, ctx=FAKE, idx=FAKE, B=2, T=1, H=16, k=256,
                 sc=0.07, causal=0, S=0, out=FAKE, lse=None, ws=None, wsb=0, stream=None)
        a.update(kw)
        return M.lib().mla_sparse_decode_fp8(a["q"], a["pool"], a["ps"], a["npg"], a["bt"], a["bts"], a["ctx"],
                                             a["idx"], a["B"], a["T"], a["H"], a["k"], a["sc"], a["causal"], a["S"],
                                             a["out"], a["lse"], a["ws"], a["wsb"], a["stream"])
    assert call(idx=None) == 1
    assert call(ps=64 * 352) == 3  # an NVFP4-sized page is too small for 576-byte rows
    assert call(k=2049) == 2
    assert call(sc=3e38) == 2  # sm_scale * log2(e) overflows fp32
    need = M.lib().mla_sparse_decode_fp8_workspace_bytes(2, 1, 16, 256, 2)
    assert call(S=2, ws=FAKE, wsb=need - 1) == 4
    import torch
    if not torch.cuda.is_available():
        assert call() == 5


def test_noalloc_decode_argument_errors():
    L = M.lib()
    cap = L.mla_noalloc_scratch_bytes()
    assert cap == 32 << 20

    def call(**kw):
        a = dict(q=FAKE, pool=FAKE, ps=64 * 352, npg=10, bt=FAKE, bts=4, ctx=FAKE, idx=FAKE, B=2, T=1, H=16, k=256,
                 sc=0.07, causal=0, S=0, out=FAKE, lse=None, stream=None)
        a.update(kw)
        return L.mla_sparse_decode_noalloc(a["q"], a["pool"], a["ps"], a["npg"], a["bt"], a["bts"], a["ctx"], a["idx"],
                                           a["B"], a["T"], a["H"], a["k"], a["sc"], a["causal"], a["S"], a["out"],
                                           a["lse"], a["stream"])
    assert call(idx=None) == 1 and call(q=None) == 1
    assert call(H=48) == 2 and call(k=0) == 2 and call(S=65) == 2
    # splits whose partial results exceed the scratch array: refused before any device call
    assert L.mla_sparse_decode_workspace_bytes(256, 1, 32, 2048, 64) > cap
    assert call(B=256, H=32, k=2048, S=64) == 4
    import torch
    if not torch.cuda.is_available():
        assert call(S=4) == 5  # fits: reaches the device check


def _dense(**kw):
    a = dict(q=FAKE, pool=FAKE, ps=64 * 576, npg=10, bt=FAKE, bts=4, ctx=FAKE, B=2, T=1, H=128, L=8192,
             sc=0.07, causal=0, S=0, out=FAKE, lse=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return M.lib().mla_dense_decode_fp8(a["q"], a["pool"], a["ps"], a["npg"], a["bt"], a["bts"], a["ctx"], a["B"],
                                        a["T"], a["H"], a["L"], a["sc"], a["causal"], a["S"], a["out"], a["lse"],
                                        a["ws"], a["wsb"], a["stream"])


def test_dense_decode_argument_errors():
    assert _dense(pool=None) == 1
    assert _dense(L=0) == 2
    assert _dense(H=8) == 2
    assert _dense(ps=64 * 352) == 3  # an NVFP4-sized page is too small for 576-byte rows
    assert _dense(S=2) == 2  # 8192 positions in 2 splits exceeds the 2048 entries one workgroup holds


def _quant(fn="mla_kv_quant_nvfp4", **kw):
    a = dict(kn=FAKE, ns=512, kr=FAKE, rs=64, sl=FAKE, n=4, pool=FAKE, ps=64 * 352, npg=4, stream=None)
    a.update(kw)
    return getattr(M.lib(), fn)(a["kn"], a["ns"], a["kr"], a["rs"], a["sl"], a["n"], a["pool"], a["ps"], a["npg"],
                                a["stream"])


def test_quant_argument_errors():
    assert _quant(n=0, kn=None) == 0  # nothing to do
    assert _quant(n=-1) == 2
    assert _quant(kn=None) == 1
    assert _quant(sl=None) == 1
    assert _quant(ns=511) == 3
    assert _quant(rs=60) == 3
    assert _quant(ns=516) == 3
    assert _quant(kn=FAKE + 2) == 3
    assert _quant(npg=0) == 2
    assert _quant("mla_kv_quant_fp8", ps=64 * 352) == 3


def test_split_choice_and_workspace_sizes():
    L = M.lib()
    # one resident workgroup per compute unit: 64 query tokens x 1 head group -> 4 splits
    assert L.mla_sparse_decode_splits(64, 1, 32, 2048) == 4
    assert L.mla_sparse_decode_splits(128, 4, 32, 2048) == 1
    assert L.mla_sparse_decode_splits(256, 1, 128, 2048) == 1
    assert L.mla_sparse_decode_splits(2, 1, 16, 256) == 1  # at least 256 list entries per split
    # small launches: at most one workgroup per compute unit, at least 256 entries per split
    assert L.mla_sparse_decode_splits(15, 1, 16, 2048) == 8
    assert L.mla_sparse_decode_splits(20, 1, 16, 2048) == 8
    assert L.mla_sparse_decode_splits(35, 1, 16, 2048) == 7
    assert L.mla_dense_decode_splits(16, 1, 128, 8192) == 4
    assert L.mla_dense_decode_splits(4, 1, 128, 8192) == 16
    assert L.mla_sparse_decode_splits(0, 1, 32, 2048) == 0
    assert L.mla_sparse_decode_workspace_bytes(64, 1, 32, 2048, 1) == 0
    rows = 64 * 32
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # the fixed region of 65,536 split counters (the same for every shape) + FP16 partial outputs + fp32
    # partial lse
    cnt = 65536 * 4
    assert L.mla_sparse_decode_workspace_bytes(64, 1, 32, 2048, 4) == cnt + r256(rows * 4 * 512 * 2) + r256(rows * 4 * 4)
    assert L.mla_sparse_decode_workspace_bytes(8, 1, 128, 2048, 2) == (cnt + r256(8 * 128 * 2 * 512 * 2) +
                                                                       r256(8 * 128 * 2 * 4))
    assert L.mla_sparse_decode_fp8_workspace_bytes(64, 1, 32, 2048, 4) == L.mla_sparse_decode_workspace_bytes(
        64, 1, 32, 2048, 4)
    assert L.mla_sparse_decode_fp8_splits(64, 1, 32, 2048) == 4
    assert L.mla_sparse_decode_fp8_splits(2, 1, 128, 2048) == 8  # 16/32-head groups at every H (4 x 2 units)


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        M.mla_kv_quant_nvfp4(torch.zeros(1, 512, dtype=torch.bfloat16), torch.zeros(1, 64, dtype=torch.bfloat16),
                             torch.zeros(1, dtype=torch.int64), torch.zeros(22528, dtype=torch.uint8), 22528, 1)


def _stage(**kw):
    a = dict(pool=FAKE, ps=64 * 352, npg=10, bt=FAKE, bts=4, ctx=FAKE, idx=FAKE, B=2, T=1, k=256, causal=0,
             staged=FAKE, sbt=FAKE, slen=FAKE, stream=None)
    a.update(kw)
    return M.lib().mla_stage_nvfp4_fp8(a["pool"], a["ps"], a["npg"], a["bt"], a["bts"], a["ctx"], a["idx"], a["B"],
                                       a["T"], a["k"], a["causal"], a["staged"], a["sbt"], a["slen"], a["stream"])


def test_stage_argument_errors():
    for name in ("pool", "bt", "ctx", "idx", "staged", "sbt", "slen"):
        assert _stage(**{name: None}) == 1, name
    assert _stage(B=0) == 2
    assert _stage(T=0) == 2
    assert _stage(k=0) == 2
    assert _stage(k=2049) == 2
    assert _stage(causal=2) == 2
    assert _stage(npg=0) == 2
    assert _stage(ps=64 * 352 - 16) == 3
    assert _stage(ps=64 * 352 + 8) == 3
    assert _stage(staged=FAKE + 8) == 3
    assert _stage(slen=FAKE + 2) == 3
    import torch
    if not torch.cuda.is_available():
        assert _stage() == 5  # valid arguments reach the device check


def _topk(**kw):
    a = dict(x=FAKE, ld=4096, lens=FAKE, n=4, k=2048, out=FAKE, ws=FAKE, wsb=None, stream=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = M.lib().mla_index_topk_workspace_bytes(a["n"], a["ld"])
    return M.lib().mla_index_topk(a["x"], a["ld"], a["lens"], a["n"], a["k"], a["out"], a["ws"], a["wsb"],
                                  a["stream"])


def test_index_topk_argument_errors():
    for name in ("x", "lens", "out", "ws"):
        assert _topk(**{name: None}) == 1, name
    assert _topk(n=-1) == 2
    assert _topk(k=0) == 2
    assert _topk(k=2049) == 2
    assert _topk(ld=(1 << 31) + 4) == 2
    assert _topk(ld=4094) == 3
    assert _topk(ld=0) == 3
    assert _topk(x=FAKE + 4) == 3
    assert _topk(out=FAKE + 2) == 3
    assert _topk(ws=FAKE + 16) == 3
    assert _topk(wsb=M.lib().mla_index_topk_workspace_bytes(4, 4096) - 1) == 4
    assert _topk(n=0, x=None, lens=None, out=None, ws=None) == 0  # nothing to do
    import torch
    if not torch.cuda.is_available():
        assert _topk() == 5  # valid arguments reach the device check


def test_index_topk_workspace_size():
    # per row: 2^12 histogram bins and 8 counters (int32), a segment per 8192 positions (2 x int32) and
    # 8192 candidates (2 x int32), each region rounded up to 256 bytes
    r256 = lambda x: (x + 255) // 256 * 256
    for n, ld in [(1, 4), (64, 140000), (3, 8192), (3, 8196)]:
        chunks = -(-ld // 8192)
        want = r256(n * 4096 * 4) + r256(n * 32) + r256(n * chunks * 8) + r256(n * 8192 * 8)
        assert M.lib().mla_index_topk_workspace_bytes(n, ld) == want, (n, ld)
    assert M.lib().mla_index_topk_workspace_bytes(0, 4096) == 0


def test_index_key_quant_argument_errors():
    def call(**kw):
        a = dict(keys=FAKE, ks=128, sm=FAKE, n=10, pool=FAKE, ps=8448, npg=4)
        a.update(kw)
        return M.lib().mla_index_key_quant(a["keys"], a["ks"], a["sm"], a["n"], a["pool"], a["ps"], a["npg"], None)
    for name in ("keys", "sm", "pool"):
        assert call(**{name: None}) == 1, name
    assert call(n=-1) == 2
    assert call(n=0, keys=None, sm=None, pool=None) == 0
    assert call(npg=0) == 2
    assert call(ks=127) == 3 and call(ks=129) == 3
    assert call(ps=8448 - 16) == 3 and call(ps=8448 + 8) == 3
    assert call(keys=FAKE + 2) == 3 and call(sm=FAKE + 4) == 3 and call(pool=FAKE + 8) == 3
    import torch
    if not torch.cuda.is_available():
        assert call() == 5


def test_index_logits_argument_errors():
    def call(**kw):
        a = dict(q=FAKE, w=FAKE, HI=64, pool=FAKE, ps=8448, npg=4, bt=FAKE, bts=4, ctx=FAKE, B=2, T=1, maxc=256,
                 causal=0, out=FAKE, ld=256)
        a.update(kw)
        return M.lib().mla_index_logits(a["q"], a["w"], a["HI"], a["pool"], a["ps"], a["npg"], a["bt"], a["bts"],
                                        a["ctx"], a["B"], a["T"], a["maxc"], a["causal"], a["out"], a["ld"], None)
    for name in ("q", "w", "pool", "bt", "ctx", "out"):
        assert call(**{name: None}) == 1, name
    for HI in (0, 8, 48, 128):
        assert call(HI=HI) == 2
    assert call(B=0) == 2 and call(T=0) == 2 and call(maxc=0) == 2 and call(npg=0) == 2 and call(bts=0) == 2
    assert call(causal=2) == 2
    assert call(ld=255) == 2
    assert call(ps=8432) == 3 and call(ps=8456) == 3
    assert call(q=FAKE + 8) == 3 and call(w=FAKE + 4) == 3 and call(out=FAKE + 2) == 3
    import torch
    if not torch.cuda.is_available():
        assert call() == 5


def test_pth_argument_errors():
    def quant(**kw):
        a = dict(kn=FAKE, ns=512, kr=FAKE, rs=64, sm=FAKE, n=8, lat=FAKE, sc=FAKE, rope=FAKE, slots=128)
        a.update(kw)
        return M.lib().mla_kv_quant_pth(a["kn"], a["ns"], a["kr"], a["rs"], a["sm"], a["n"], a["lat"], a["sc"],
                                        a["rope"], a["slots"], None)
    for name in ("kn", "kr", "sm", "lat", "sc", "rope"):
        assert quant(**{name: None}) == 1, name
    assert quant(n=-1) == 2 and quant(slots=0) == 2
    assert quant(n=0, kn=None) == 0
    assert quant(ns=511) == 3 and quant(ns=516) == 3 and quant(rs=63) == 3
    assert quant(kn=FAKE + 8) == 3 and quant(lat=FAKE + 4) == 3

    def dec(**kw):
        a = dict(q=FAKE, lat=FAKE, sc=FAKE, rope=FAKE, slots=4096, bt=FAKE, bts=4, ctx=FAKE, idx=FAKE, B=2, T=1, H=32,
                 k=256, scale=0.07, causal=0, S=0, out=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 20)
        a.update(kw)
        return M.lib().mla_sparse_decode_pth(a["q"], a["lat"], a["sc"], a["rope"], a["slots"], a["bt"], a["bts"],
                                             a["ctx"], a["idx"], a["B"], a["T"], a["H"], a["k"], a["scale"],
                                             a["causal"], a["S"], a["out"], a["lse"], a["ws"], a["wsb"], None)
    for name in ("q", "lat", "sc", "rope", "bt", "ctx", "idx", "out"):
        assert dec(**{name: None}) == 1, name
    assert dec(H=48) == 2 and dec(H=8) == 2 and dec(k=0) == 2 and dec(k=2049) == 2 and dec(S=65) == 2
    assert dec(scale=0.0) == 2 and dec(scale=float("inf")) == 2 and dec(causal=3) == 2 and dec(slots=63) == 2
    # a requested split count sets the chunk (rounded up to whole 64-entry steps): fewer splits may run,
    # and the workspace query sizes for the same effective count
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert M.lib().mla_sparse_decode_pth_workspace_bytes(2, 1, 32, 256, 8) == r256(64 * 4 * 512 * 4) + r256(64 * 4 * 4)
    assert M.lib().mla_sparse_decode_pth_workspace_bytes(2, 1, 32, 300, 4) == r256(64 * 3 * 512 * 4) + r256(64 * 3 * 4)
    assert dec(S=8, k=256, wsb=M.lib().mla_sparse_decode_pth_workspace_bytes(2, 1, 32, 256, 8) - 1) == 4
    assert dec(q=FAKE + 8) == 3 and dec(rope=FAKE + 8) == 3 and dec(out=FAKE + 2) == 3
    need = M.lib().mla_sparse_decode_pth_workspace_bytes(2, 1, 32, 256, 2)
    assert need > 0 and M.lib().mla_sparse_decode_pth_workspace_bytes(2, 1, 32, 256, 1) == 0
    assert dec(S=2, wsb=need - 1) == 4 and dec(S=2, ws=None) == 1
    import torch
    if not torch.cuda.is_available():
        assert quant() == 5 and dec(S=2, wsb=need) == 5


def test_sparse_decode_append_argument_errors():
    def call(**kw):
        a = dict(q=FAKE, pool=FAKE, ps=64 * 352, npg=10, bt=FAKE, bts=4, ctx=FAKE, idx=FAKE, kn=FAKE, kns=512,
                 kr=FAKE, krs=64, B=2, T=1, H=16, k=256, sc=0.07, causal=0, S=0, out=FAKE, lse=None, ws=None, wsb=0,
                 stream=None)
        a.update(kw)
        return M.lib().mla_sparse_decode_append(a["q"], a["pool"], a["ps"], a["npg"], a["bt"], a["bts"], a["ctx"],
                                                a["idx"], a["kn"], a["kns"], a["kr"], a["krs"], a["B"], a["T"],
                                                a["H"], a["k"], a["sc"], a["causal"], a["S"], a["out"], a["lse"],
                                                a["ws"], a["wsb"], a["stream"])
    assert call(q=None) == 1
    assert call(pool=None) == 1
    assert call(idx=None) == 1
    assert call(kn=None) == 1
    assert call(kr=None) == 1
    assert call(B=0) == 2
    assert call(H=48) == 2
    assert call(k=2049) == 2
    assert call(S=65) == 2
    assert call(causal=2) == 2
    assert call(sc=float("nan")) == 2
    assert call(ps=64 * 576 + 8) == 3
    assert call(kns=504) == 3  # rows shorter than 512 values
    assert call(krs=60) == 3
    assert call(kns=520 + 4) == 3  # not a multiple of 16 bytes
    assert call(kn=FAKE + 8) == 3
    assert call(kr=FAKE + 2) == 3
    need = M.lib().mla_sparse_decode_workspace_bytes(2, 1, 16, 256, 4)
    assert call(S=4) == 1
    assert call(S=4, ws=FAKE, wsb=need - 1) == 4
    import torch
    if not torch.cuda.is_available():
        assert call() == 5
        need4 = M.lib().mla_sparse_decode_workspace_bytes(2, 4, 16, 256, 4)
        assert call(S=4, ws=FAKE, wsb=need4 - 1, T=4, causal=1) == 4
        assert call(S=4, ws=FAKE, wsb=need4, T=4, causal=1) == 5
