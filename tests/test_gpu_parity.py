"""GPU parity: the HIP path (through the C ABI) against the FP64 oracle on the same seeded inputs.

Quantized bytes must match bit for bit; attention outputs must meet the tolerances in cases.py."""
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from cases import Case, bf16_to_np, compare_outputs, sampled_oracle, v_abs_of_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import nvfp4_compressed_sparse_amd as M  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name="t", B=2, T=1, H=16, topk=256, L=4096, fmt="nvfp4", causal=False, seed=7):
    return W.DecodeConfig(name, B=B, T=T, H=H, topk=topk, fmt=fmt, ctx=L, causal=causal, seed=seed)


def gpu_pool(case, d):
    c = case.cfg
    fn = M.mla_kv_quant_nvfp4 if c.fmt == "nvfp4" else M.mla_kv_quant_fp8
    fn(d["lat"], d["rope"], d["slots"], d["pool"], c.page_stride, case.lay.num_pages)
    torch.cuda.synchronize()
    return d["pool"]


def gpu_decode(case, d, num_splits=0, idx=None, q=None, sm_scale=None):
    c = case.cfg
    lse = torch.empty((c.B, c.T, c.H), dtype=torch.float32, device="cuda")
    qq = d["q"] if q is None else q
    if c.topk:
        fn = M.mla_sparse_decode if c.fmt == "nvfp4" else M.mla_sparse_decode_fp8
        out, _ = fn(qq, d["pool"], c.page_stride, case.lay.num_pages, d["bt"], d["ctx"], d["idx"] if idx is None else idx,
                    c.sm_scale if sm_scale is None else sm_scale, causal=c.causal, num_splits=num_splits, lse=lse)
    else:
        out, _ = M.mla_dense_decode_fp8(qq, d["pool"], c.page_stride, case.lay.num_pages, d["bt"], d["ctx"],
                                        int(case.lay.ctx.max()), c.sm_scale if sm_scale is None else sm_scale,
                                        causal=c.causal, num_splits=num_splits, lse=lse)
    torch.cuda.synchronize()
    return bf16_to_np(out).reshape(c.B * c.T, c.H, 512), lse.cpu().numpy().astype(np.float64).reshape(c.B * c.T, c.H)


# --------------------------------------------------------------------------- quantize-on-write: bit exact
@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_quant_pool_bit_exact(fmt):
    case = Case(small(fmt=fmt, topk=256 if fmt == "nvfp4" else 0, L=3000, seed=11))
    say(f"quant pool {fmt}: {case.slots.size} rows")
    d = case.to_device()
    g = gpu_pool(case, d).cpu().numpy()
    ref = case.oracle_pool()
    bad = np.nonzero(g != ref)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def _adversarial_rows():
    """Rows that cover every finite bf16 value as latent and rope entries, every scale tie, zero /
    negative-zero / subnormal-scale / saturating blocks."""
    fin = np.array([b for b in range(65536) if ((b >> 7) & 0xFF) != 0xFF], dtype=np.uint16)
    rows = []
    # every finite bf16 value inside blocks of its own neighbourhood (sorted by magnitude), and shuffled
    srt = fin[np.argsort(np.abs(W.bf16_to_f32(fin)), kind="stable")]
    n = (srt.size // 512) * 512
    rows.append(srt[:n].reshape(-1, 512))
    rng = np.random.default_rng(3)
    rows.append(rng.permutation(fin)[:n].reshape(-1, 512))
    # scale ties: amax exactly 6 x the midpoint of two neighbouring E4M3 values (plus neighbours)
    ties = []
    for c in range(0x7E):
        m6 = 3.0 * (oracle.e4m3_value(c) + oracle.e4m3_value(c + 1))
        b = W.bf16_bits(np.array([m6], np.float32))[0]
        if W.bf16_to_f32(np.array([b]))[0] == m6:
            ties.append(b)
    ties = np.array(ties, np.uint16)
    blk = rng.choice(fin[(fin >> 15) == 0][:20000], size=(ties.size, 16))  # small magnitudes
    blk[:, 0] = ties
    blk[:, 5] = ties | 0x8000
    pad = (-blk.shape[0]) % 32
    blk = np.concatenate([blk, np.zeros((pad, 16), np.uint16)])
    rows.append(blk.reshape(-1, 512))
    special = np.zeros((4, 512), np.uint16)
    special[0, 16:32] = 0x8000  # negative zeros
    special[1] = W.bf16_bits(rng.standard_normal(512).astype(np.float32) * 1e-3)  # subnormal scales
    special[2] = W.bf16_bits(rng.standard_normal(512).astype(np.float32) * 1e4)  # saturating blocks
    special[3] = W.bf16_bits(np.where(rng.random(512) < 0.5, 1e30, -1e-30).astype(np.float32))
    rows.append(special)
    lat = np.concatenate(rows)
    rope_src = np.concatenate([fin, fin[: (-fin.size) % 64]])
    rope = np.resize(rng.permutation(rope_src), (lat.shape[0], 64)).astype(np.uint16)
    return lat, rope


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_quant_adversarial_rows_bit_exact(fmt):
    lat, rope = _adversarial_rows()
    n = lat.shape[0]
    rb = 352 if fmt == "nvfp4" else 576
    page_stride = 64 * rb + 48  # a padded page stride
    num_pages = (n + 63) // 64 + 2
    rng = np.random.default_rng(9)
    slots = rng.permutation(num_pages * 64)[:n].astype(np.int64)
    slots[::97] = -1  # skipped tokens
    slots[5] = num_pages * 64 + 3  # on a page outside the pool: skipped
    say(f"adversarial quant {fmt}: {n} rows")
    ref = np.zeros(num_pages * page_stride, np.uint8)
    oracle.kv_quant(fmt, lat, rope, slots, ref, page_stride, num_pages)
    pool = torch.zeros(num_pages * page_stride, dtype=torch.uint8, device="cuda")
    kn = torch.from_numpy(lat.view(np.int16)).cuda().view(torch.bfloat16)
    kr = torch.from_numpy(rope.view(np.int16)).cuda().view(torch.bfloat16)
    fn = M.mla_kv_quant_nvfp4 if fmt == "nvfp4" else M.mla_kv_quant_fp8
    fn(kn, kr, torch.from_numpy(slots).cuda(), pool, page_stride, num_pages)
    g = pool.cpu().numpy()
    bad = np.nonzero(g != ref)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def test_quant_every_block_amax_bit_exact():
    """Every non-negative finite bf16 value as the largest magnitude of a 16-value block (the block scale
    is the E4M3 code nearest to amax / 6), with the block's other values below it and of either sign:
    the NVFP4 writer's bytes against the oracle's, and the same rows through the fused step's writes."""
    vals = np.arange(0, 0x7F80, dtype=np.uint16)  # bit patterns of 0 .. largest finite bf16
    nblk = vals.size
    rng = np.random.default_rng(31)
    amax = W.bf16_to_f32(vals).astype(np.float64)
    frac = rng.random((nblk, 16))
    blk = W.bf16_bits((amax[:, None] * frac).astype(np.float32))  # magnitudes at most amax
    blk = np.where(rng.random((nblk, 16)) < 0.5, blk | 0x8000, blk).astype(np.uint16)
    blk[np.arange(nblk), rng.integers(0, 16, nblk)] = vals | (rng.integers(0, 2, nblk) << 15).astype(np.uint16)
    pad = (-nblk) % 32
    blk = np.concatenate([blk, np.zeros((pad, 16), np.uint16)])
    lat = blk.reshape(-1, 512)
    n = lat.shape[0]
    rope = W.bf16_bits(rng.standard_normal((n, 64)).astype(np.float32))
    num_pages = (n + 63) // 64 + 1
    slots = np.arange(n, dtype=np.int64) + 64
    say(f"every block amax: {nblk} blocks in {n} rows")
    ref = np.zeros(num_pages * 64 * 352, np.uint8)
    oracle.kv_quant("nvfp4", lat, rope, slots, ref, 64 * 352, num_pages)
    pool = torch.zeros(ref.size, dtype=torch.uint8, device="cuda")
    kn = torch.from_numpy(lat.view(np.int16)).cuda().view(torch.bfloat16)
    kr = torch.from_numpy(rope.view(np.int16)).cuda().view(torch.bfloat16)
    M.mla_kv_quant_nvfp4(kn, kr, torch.from_numpy(slots).cuda(), pool, 64 * 352, num_pages)
    bad = np.nonzero(pool.cpu().numpy() != ref)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"
    # the fused step writes the same rows: one request per row, each row its request's newest position
    # request b has one page-table entry, page 1 + b // 64, and its new row is position b % 64 (context
    # b % 64 + 1): slot 64 + b, as above
    B = n
    ctx = (np.arange(B) % 64 + 1).astype(np.int32)
    bt = (1 + np.arange(B) // 64).astype(np.int32).reshape(B, 1)
    q = torch.zeros((B, 1, 16, 576), dtype=torch.bfloat16, device="cuda")
    idx = torch.full((B, 1, 1), -1, dtype=torch.int32, device="cuda")
    pool2 = torch.zeros(ref.size, dtype=torch.uint8, device="cuda")
    M.mla_sparse_decode_append(q, pool2, 64 * 352, num_pages, torch.from_numpy(bt).cuda(), torch.from_numpy(ctx).cuda(),
                               idx, kn, kr, 0.07)
    torch.cuda.synchronize()
    bad = np.nonzero(pool2.cpu().numpy() != ref)[0]
    assert bad.size == 0, f"fused step: {bad.size} bytes differ, first at {bad[:8]}"


def test_quant_strided_inputs_from_one_kv_tensor():
    # nope and rope as views of one [n, 576] tensor (stride 576), written through a pool of 2 layers
    rng = np.random.default_rng(21)
    lat, rope = W.gen_latent_rope(rng, 700)
    kv = np.concatenate([lat, rope], axis=1)
    kvd = torch.from_numpy(kv.view(np.int16)).cuda().view(torch.bfloat16)
    layers, pages = 2, 12
    page_stride = layers * 64 * 352  # block-major: pages hold both layers' rows
    pool = torch.zeros(pages * page_stride, dtype=torch.uint8, device="cuda")
    slots = rng.permutation(pages * 64)[:700].astype(np.int64)
    layer1 = pool[64 * 352:]  # layer 1 rows start 64*352 bytes into each page
    M.mla_kv_quant_nvfp4(kvd[:, :512], kvd[:, 512:], torch.from_numpy(slots).cuda(), layer1, page_stride, pages - 1)
    ref = np.zeros(pages * page_stride, np.uint8)
    oracle.kv_quant("nvfp4", lat, rope, slots, ref[64 * 352:], page_stride, pages - 1)
    assert np.array_equal(pool.cpu().numpy(), ref)


# --------------------------------------------------------------------------- sparse decode
def test_sparse_decode_tiny_config():
    case = Case(W.CONFIGS["tiny"])
    say("tiny config decode")
    d = case.to_device()
    gpu_pool(case, d)
    assert np.array_equal(d["pool"].cpu().numpy(), case.oracle_pool())
    out, lse = gpu_decode(case, d)
    ro, rl = case.oracle_decode()
    say(compare_outputs(out, ro, lse, rl, "tiny", vmax=case.vmax()))


@pytest.mark.parametrize("H", [32, 128])
@pytest.mark.parametrize("S", [1, 2, 3, 4, 8, 64])
def test_sparse_decode_split_counts(S, H):
    # 300 entries: 4 full 64-row steps + a ragged 44
    case = Case(small(H=H, topk=300, L=5000, seed=13))
    say(f"split count {S} H={H}")
    d = case.to_device()
    gpu_pool(case, d)
    out, lse = gpu_decode(case, d, num_splits=S)
    ro, rl = case.oracle_decode()
    say(compare_outputs(out, ro, lse, rl, f"S={S} H={H}", vmax=case.vmax()))


def test_workspace_zero_filled_once_serves_calls_of_any_shape():
    """The workspace rule of the header: zero-filled before its first use, then reused without clearing
    by calls of different sizes, head counts, split counts and row formats.  Each call's output and lse
    are bit-identical to the same call with a freshly zeroed workspace (and so within the oracle's
    tolerance, which the other tests check)."""
    shapes = [dict(B=4, H=32, topk=300, S=4), dict(B=2, H=16, topk=700, S=8), dict(B=3, H=128, topk=300, S=2),
              dict(B=1, H=64, topk=513, S=3), dict(B=4, H=32, topk=300, S=4, fmt="fp8"), dict(B=4, H=32, topk=300, S=4)]
    need = max((M.mla_sparse_decode_fp8_workspace_bytes if s.get("fmt") == "fp8" else
                M.mla_sparse_decode_workspace_bytes)(s["B"], 1, s["H"], s["topk"], s["S"]) for s in shapes)
    shared = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, s in enumerate(shapes):
        fmt = s.get("fmt", "nvfp4")
        case = Case(small(B=s["B"], H=s["H"], topk=s["topk"], L=5000, fmt=fmt, seed=60 + i))
        say(f"shared workspace call {i}: {s}")
        d = case.to_device()
        gpu_pool(case, d)
        c = case.cfg
        fn = M.mla_sparse_decode if fmt == "nvfp4" else M.mla_sparse_decode_fp8
        res = []
        for ws in (shared, None):
            lse = torch.empty((c.B, 1, c.H), dtype=torch.float32, device="cuda")
            out, _ = fn(d["q"], d["pool"], c.page_stride, case.lay.num_pages, d["bt"], d["ctx"], d["idx"], c.sm_scale,
                        num_splits=s["S"], lse=lse, workspace=ws)
            torch.cuda.synchronize()
            res.append((out.view(torch.int16).cpu().numpy(), lse.cpu().numpy()))
        assert np.array_equal(res[0][0], res[1][0]), f"call {i}: output differs with the reused workspace"
        assert np.array_equal(res[0][1], res[1][1]), f"call {i}: lse differs with the reused workspace"


def _bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("H", [32, 128])
@pytest.mark.parametrize("pattern", ["rising", "steep", "late_jump", "huge_jump"])
@pytest.mark.parametrize("S", [1, 2])
def test_softmax_reference_rises(H, pattern, S):
    """Scores that grow along the index list make the running softmax reference rise step after step
    ('rising': about 10 in log2 units per 32 rows; 'steep': about 33) or once at the very end
    ('late_jump': by about 66, 'huge_jump': by about 266), so the accumulated output is rescaled
    inside the kernel (its reference rises by more than 15 log2 units at a time).
    The query's latent part is zero and its rope part one, so a row's score is sm_scale times the sum
    of its rope values, which the test sets."""
    cfg = small(B=2, H=H, topk=256, L=3000, seed=41)
    case = Case(cfg)
    off = np.concatenate([[0], np.cumsum(case.lay.ctx)[:-1]])
    for b in range(cfg.B):
        pos = case.idx[b, 0]
        if pattern in ("rising", "steep"):
            r = np.arange(pos.size) * ((1.5 if pattern == "rising" else 5.0) / 32)
        else:
            r = np.zeros(pos.size)
            r[-5:] = 10.0 if pattern == "late_jump" else 40.0
        case.rope[off[b] + pos] = _bf16_bits(r)[:, None]
    case.q[..., :512] = 0
    case.q[..., 512:] = _bf16_bits(1.0)
    say(f"reference rises: {pattern} H={H} S={S}")
    d = case.to_device()
    gpu_pool(case, d)
    out, lse = gpu_decode(case, d, num_splits=S)
    ro, rl = case.oracle_decode()
    say(compare_outputs(out, ro, lse, rl, f"{pattern} H={H} S={S}", vmax=case.vmax()))


@pytest.mark.parametrize("H", [16, 32, 64, 128])
@pytest.mark.parametrize("topk", [1, 77, 2048])
def test_sparse_decode_heads_and_topk(H, topk):
    case = Case(small(B=3, H=H, topk=topk, L=9000, seed=100 + H + topk))
    say(f"H={H} topk={topk}")
    d = case.to_device()
    gpu_pool(case, d)
    out, lse = gpu_decode(case, d)
    ro, rl = case.oracle_decode()
    say(compare_outputs(out, ro, lse, rl, f"H={H} topk={topk}", vmax=case.vmax()))


def test_sparse_decode_padding_and_invalid_entries():
    cfg = small(B=4, H=32, topk=512, L=2000, seed=17)
    rng = np.random.default_rng(5)
    case = Case(cfg)
    idx = case.idx.copy()
    # -1 runs, entries past the context, far out of range, negative garbage
    idx[0, 0, :200] = -1
    idx[1, 0, rng.choice(512, 100, replace=False)] = -1
    idx[2, 0, :10] = 2000
    idx[2, 0, 10:20] = 10 ** 8
    idx[2, 0, 20:30] = -5
    idx[3, 0, :] = -1  # empty selection
    case.idx = idx
    # a page-table entry outside the pool drops the positions on that page
    bt = case.lay.block_table
    bt[1, 3] = case.lay.num_pages + 5
    say("padding / invalid entries")
    d = case.to_device()
    gpu_pool(case, d)
    for S in (1, 4):
        out, lse = gpu_decode(case, d, num_splits=S)
        ro, rl = case.oracle_decode()
        say(compare_outputs(out, ro, lse, rl, f"invalid entries S={S}", vmax=case.vmax()))
        assert not out[3].any() and np.all(lse[3] == -np.inf)


def test_sparse_decode_causal_speculative_verify():
    cfg = small(B=3, T=4, H=32, topk=256, L=3000, causal=True, seed=19)
    case = Case(cfg, ctx=[3000, 700, 260])
    # some entries beyond each token's own limit (inside the context) must be ignored
    for b in range(3):
        L = int(case.lay.ctx[b])
        case.idx[b, 0, :3] = [L - 1, L - 2, L - 3]
    say("causal T=4")
    d = case.to_device()
    gpu_pool(case, d)
    for S in (0, 1, 2):
        out, lse = gpu_decode(case, d, num_splits=S)
        ro, rl = case.oracle_decode()
        say(compare_outputs(out, ro, lse, rl, f"causal S={S}", vmax=case.vmax()))


def test_single_index_returns_that_row_exactly():
    cfg = small(B=2, H=32, topk=64, L=1000, seed=23)
    case = Case(cfg)
    idx = np.full_like(case.idx, -1)
    idx[:, :, 17] = case.idx[:, :, 0]
    case.idx = idx
    d = case.to_device()
    gpu_pool(case, d)
    out, lse = gpu_decode(case, d, num_splits=1)
    ro, rl = case.oracle_decode()
    # P = 1: the output is the dequantized V row itself, which is exact in bf16
    assert np.array_equal(out, ro)
    assert np.abs(lse - rl).max() <= 1e-3


def test_zero_query_gives_mean_of_v():
    cfg = small(B=2, H=16, topk=200, L=1500, seed=29)
    case = Case(cfg)
    case.q[:] = 0
    d = case.to_device()
    gpu_pool(case, d)
    out, lse = gpu_decode(case, d, num_splits=1)
    ro, rl = case.oracle_decode()
    say(compare_outputs(out, ro, lse, rl, "q=0", vmax=case.vmax()))
    # all heads see the same uniform weights
    assert np.array_equal(out[:, 0:1, :].repeat(16, 1), out)


def test_permuted_index_list_gives_same_result():
    cfg = small(B=2, H=32, topk=512, L=4000, seed=31)
    case = Case(cfg)
    d = case.to_device()
    gpu_pool(case, d)
    out0, lse0 = gpu_decode(case, d, num_splits=1)
    perm = torch.from_numpy(case.idx[:, :, np.random.default_rng(1).permutation(512)].copy()).cuda()
    out1, lse1 = gpu_decode(case, d, num_splits=1, idx=perm)
    ro, rl = case.oracle_decode()
    compare_outputs(out1, ro, lse1, rl, "permuted", vmax=case.vmax())
    compare_outputs(out0, ro, lse0, rl, "original", vmax=case.vmax())


# --------------------------------------------------------------------------- sparse decode over FP8 rows
@pytest.mark.parametrize("H,topk,S", [(16, 2048, 0), (32, 300, 1), (32, 300, 3), (64, 77, 0), (128, 512, 2), (16, 1, 0)])
def test_sparse_fp8_decode(H, topk, S):
    """The FP8-cache arm of the pages' comparison: the same selection over 576-byte FP8 rows."""
    case = Case(small(H=H, topk=topk, L=5000, fmt="fp8", seed=140 + H + topk))
    say(f"sparse fp8 H={H} topk={topk} S={S}")
    d = case.to_device()
    gpu_pool(case, d)
    assert np.array_equal(d["pool"].cpu().numpy(), case.oracle_pool())
    out, lse = gpu_decode(case, d, num_splits=S)
    ro, rl = case.oracle_decode()
    say(compare_outputs(out, ro, lse, rl, f"sparse fp8 H={H} topk={topk} S={S}", vmax=case.vmax()))


def test_sparse_fp8_decode_causal_padding_and_invalid_entries():
    cfg = small(B=4, T=2, H=32, topk=400, L=2500, fmt="fp8", causal=True, seed=151)
    case = Case(cfg, ctx=[2500, 900, 130, 2000])
    idx = case.idx.copy()
    idx[0, 0, :150] = -1
    idx[1, 1, 10:30] = 10 ** 7
    idx[2, 0, :] = -1  # empty selection
    idx[3, 1, :5] = [1999, 1998, 1997, 1996, 1995]  # past token 1's causal limit (2000 - 2 + 1) except 1999
    case.idx = idx
    case.lay.block_table[0, 7] = case.lay.num_pages + 2  # positions on this page select nothing
    say("sparse fp8 causal / padding / invalid")
    d = case.to_device()
    d["pool"].fill_(0xFF)  # unwritten rows read as NaN if they ever reached the output
    gpu_pool(case, d)
    for S in (1, 2, 0):
        out, lse = gpu_decode(case, d, num_splits=S)
        assert np.isfinite(out).all()
        ro, rl = case.oracle_decode()
        say(compare_outputs(out, ro, lse, rl, f"sparse fp8 invalid entries S={S}", vmax=case.vmax()))
        assert not out[4].any() and np.all(lse[4] == -np.inf)


# --------------------------------------------------------------------------- the query's range
def _q_times_pow2(qbits, k):
    """bf16 bits of q * 2^k per element (k scalar or broadcastable); asserts the product is exact in bf16."""
    x = W.bf16_to_f32(qbits).astype(np.float64) * np.exp2(np.asarray(k, np.float64))
    bits = W.bf16_bits(x.astype(np.float32))
    assert np.array_equal(W.bf16_to_f32(bits).astype(np.float64), x), "scaled query not exact in bf16"
    return bits


def _q_device(qbits):
    return torch.from_numpy(qbits.view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("fmt,H,topk", [("nvfp4", 16, 300), ("nvfp4", 32, 300), ("nvfp4", 64, 300),
                                        ("nvfp4", 128, 300), ("fp8", 32, 300), ("fp8", 128, 0)])
def test_query_times_power_of_two_gives_identical_results(fmt, H, topk):
    """q * 2^k with sm_scale * 2^-k leaves every score unchanged.  Each head's query is normalised by a power
    of two before its FP16 conversion, so the results are bit-identical for k far outside FP16's range
    (|q| up to about 2^102 and down to about 2^-110), and they match the oracle."""
    case = Case(small(B=2, H=H, topk=topk, L=1200, fmt=fmt, seed=160 + H))
    d = case.to_device()
    gpu_pool(case, d)
    sm = case.cfg.sm_scale
    for S in (1, 2):
        base_out, base_lse = gpu_decode(case, d, num_splits=S)
        ro, rl = case.oracle_decode()
        say(compare_outputs(base_out, ro, base_lse, rl, f"{fmt} H={H} S={S} unscaled", vmax=case.vmax()))
        for k in (-100, -30, 30, 100):
            qk = _q_times_pow2(case.q, k)
            out, lse = gpu_decode(case, d, num_splits=S, q=_q_device(qk), sm_scale=sm * 2.0 ** -k)
            assert np.array_equal(out, base_out), f"k={k}: output differs from the unscaled query's"
            assert np.array_equal(lse, base_lse), f"k={k}: lse differs from the unscaled query's"
        say(f"{fmt} H={H} S={S}: bit-identical for q * 2^k, k = -100, -30, 30, 100")


@pytest.mark.parametrize("fmt,H,topk", [("nvfp4", 16, 256), ("nvfp4", 32, 256), ("nvfp4", 128, 256),
                                        ("fp8", 32, 256), ("fp8", 128, 0)])
def test_query_outside_fp16_range_matches_oracle(fmt, H, topk):
    """Finite bf16 queries outside FP16's range (elements up to 1e5 and 1e30, tiny ones down to 1e-38, bf16
    subnormals included), each head on its own scale, with sm_scale set so that the scores are of order one:
    the softmax weights then depend on every large element, and the outputs must match the oracle."""
    cfg = small(B=2, H=H, topk=topk, L=1000, fmt=fmt, seed=170 + H)
    case = Case(cfg)
    rng = np.random.default_rng(171)
    q = W.bf16_to_f32(case.q).astype(np.float64)
    # heads in four groups: a 1e5-sized spike in each head among N(0,1) values; whole heads at 1e30; whole
    # heads at 1e-30 with bf16 subnormals (~1e-39) mixed in; heads whose values span 1e-20 .. 1e20
    g = np.arange(H) % 4
    spike = rng.integers(0, 576, size=(cfg.B, cfg.T, H))
    for b in range(cfg.B):
        for h in np.nonzero(g == 0)[0]:
            q[b, 0, h, spike[b, 0, h]] = 1.0e5 * np.sign(q[b, 0, h, spike[b, 0, h]] + 0.5)
    q[:, :, g == 1, :] *= 1.0e30
    q[:, :, g == 2, :] *= 1.0e-30
    q[:, :, g == 2, ::7] *= 1.0e-9  # ~1e-39: bf16 subnormals
    span = 10.0 ** rng.uniform(-20, 20, size=(cfg.B, cfg.T, int((g == 3).sum()), 576))
    q[:, :, g == 3, :] *= span
    qbits = W.bf16_bits(q.astype(np.float32))
    assert np.isfinite(W.bf16_to_f32(qbits)).all()
    assert (np.abs(W.bf16_to_f32(qbits)) > 65504).any() and ((qbits & 0x7F80) == 0).sum() > 100
    # one sm_scale for all heads cannot make every head's scores of order one: run one head group at a
    # time, each with its own scale, against the oracle with that scale
    d = case.to_device()
    gpu_pool(case, d)
    case.q = qbits
    dq = _q_device(qbits)
    vm = case.vmax()
    # scores of order one: the 1e5 spike times |K| ~ 1; 24 ~ sqrt(576) N(0,1) products for whole heads
    for grp, sm in ((0, 1.0e-5), (1, 1.0 / 2.4e31), (2, 1.0 / 2.4e-29), (3, 1.0e-21)):
        for S in (1, 2):
            out, lse = gpu_decode(case, d, num_splits=S, q=dq, sm_scale=sm)
            pool = case.oracle_pool()
            if topk:
                ro, rl, _ = oracle.sparse_decode(qbits, pool, cfg.page_stride, case.lay.num_pages, case.lay.block_table,
                                                 case.lay.ctx, case.idx, sm, fmt=fmt)
            else:
                ro, rl, _ = oracle.dense_decode_fp8(qbits, pool, cfg.page_stride, case.lay.num_pages,
                                                    case.lay.block_table, case.lay.ctx, sm)
            sel = g == grp
            # (the other groups' scores may leave fp32's range at this sm_scale: outside the contract)
            assert np.isfinite(out[:, sel]).all() and np.isfinite(lse[:, sel]).all()
            say(compare_outputs(out[:, sel], ro[:, sel], lse[:, sel], rl[:, sel], f"{fmt} H={H} group {grp} S={S}",
                                vmax=vm))


# --------------------------------------------------------------------------- 64-head workgroups
# Unsplit NVFP4 launches at 64 or 128 heads with at least 256 workgroups of 64 heads run the 64-head
# workgroup (each score wave takes two 16-row tiles for half of the heads; the 64 heads' queries are
# staged in LDS once per workgroup).  Its results match the oracle on sampled query tokens, and the
# 32-head workgroup bit for bit: a smaller batch of the same requests (unsplit, too few tokens for
# 64-head workgroups) runs that one, and a token's results do not depend on the rest of the batch.
@pytest.mark.parametrize("H,B,T,topk,L,causal", [(128, 32, 4, 300, 1000, True), (64, 256, 1, 77, 400, False),
                                                 (128, 128, 1, 2048, 2100, False)])
def test_sparse_decode_64_head_groups(H, B, T, topk, L, causal):
    cfg = small(B=B, T=T, H=H, topk=topk, L=L, causal=causal, seed=180 + H + topk)
    case = Case(cfg)
    rng = np.random.default_rng(181)
    idx = case.idx
    idx[0, :, : topk // 3] = -1            # a run of unused entries
    idx[1, 0, rng.choice(topk, topk // 4, replace=False)] = -1
    idx[2, 0, :5] = 10 ** 8                # beyond the context
    idx[3, :, :] = -1                      # an empty selection
    case.lay.block_table[4, 1] = case.lay.num_pages + 3  # a page outside the pool
    assert M.mla_sparse_decode_splits(B, T, H, topk) == 1 and B * T * (H // 64) >= 256
    say(f"64-head workgroups: H={H} B={B} T={T} topk={topk}")
    d = case.to_device()
    gpu_pool(case, d)
    out, lse = gpu_decode(case, d)
    n = B * T
    units = np.unique(np.concatenate([[0, 1, 2, 3 * T, 4 * T, n - 1], rng.choice(n, 10, replace=False)]))
    ro, rl = case.oracle_decode(units=units)
    say(compare_outputs(out[units], ro, lse[units], rl, f"64-head H={H} sampled", vmax=case.vmax()[units]))
    assert not out[3 * T:4 * T].any() and np.all(lse[3 * T:4 * T] == -np.inf)
    # the 32-head workgroup on the first nb requests
    nb = max(1, (255 // (T * (H // 64))))
    lse2 = torch.empty((nb, T, H), dtype=torch.float32, device="cuda")
    out2, _ = M.mla_sparse_decode(d["q"][:nb], d["pool"], cfg.page_stride, case.lay.num_pages, d["bt"][:nb],
                                  d["ctx"][:nb], d["idx"][:nb], cfg.sm_scale, causal=causal, num_splits=1, lse=lse2)
    torch.cuda.synchronize()
    out2 = bf16_to_np(out2).reshape(nb * T, H, 512)
    assert np.array_equal(out2, out[:nb * T]), "64-head and 32-head workgroups differ"
    assert np.array_equal(lse2.cpu().numpy().reshape(nb * T, H), lse[:nb * T])
    # a query scaled by 2^k with sm_scale * 2^-k: bit-identical (each head's own power-of-two shift)
    for k in (-100, 100):
        o3, l3 = gpu_decode(case, d, q=_q_device(_q_times_pow2(case.q, k)), sm_scale=cfg.sm_scale * 2.0 ** -k)
        assert np.array_equal(o3, out) and np.array_equal(l3, lse), f"q * 2^{k} differs"
    say(f"64-head H={H}: bit-identical to the 32-head workgroup on {nb * T} tokens and for q * 2^k")


def test_sparse_decode_64_head_groups_extreme_queries():
    """Queries far outside FP16's range in the 64-head workgroup (its score waves convert their own
    query rows): whole heads at 1e30 and at 1e-30 with bf16 subnormals, against the oracle."""
    cfg = small(B=32, T=4, H=128, topk=256, L=800, seed=190)
    case = Case(cfg)
    q = W.bf16_to_f32(case.q).astype(np.float64)
    g = np.arange(cfg.H) % 2
    q[:, :, g == 0, :] *= 1.0e30
    q[:, :, g == 1, :] *= 1.0e-30
    q[:, :, g == 1, ::7] *= 1.0e-9
    qbits = W.bf16_bits(q.astype(np.float32))
    assert np.isfinite(W.bf16_to_f32(qbits)).all()
    d = case.to_device()
    gpu_pool(case, d)
    case.q = qbits
    dq = _q_device(qbits)
    units = np.array([0, 5, 17, 64, 127])
    vm = case.vmax()[units]
    for grp, sm in ((0, 1.0 / 2.4e31), (1, 1.0 / 2.4e-29)):
        out, lse = gpu_decode(case, d, q=dq, sm_scale=sm)
        ro, rl, _ = oracle.sparse_decode(qbits, case.oracle_pool(), cfg.page_stride, case.lay.num_pages,
                                         case.lay.block_table, case.lay.ctx, case.idx, sm, units=units)
        sel = g == grp
        assert np.isfinite(out[units][:, sel]).all() and np.isfinite(lse[units][:, sel]).all()
        say(compare_outputs(out[units][:, sel], ro[:, sel], lse[units][:, sel], rl[:, sel], f"64-head group {grp}",
                            vmax=vm))


# --------------------------------------------------------------------------- dense FP8 decode
@pytest.mark.parametrize("T,causal,S", [(1, False, 0), (1, False, 1), (2, True, 0), (1, False, 7)])
def test_dense_fp8_decode(T, causal, S):
    cfg = small(B=2, T=T, H=128, topk=0, fmt="fp8", L=1100, causal=causal, seed=37)
    case = Case(cfg, ctx=[1100, 333])
    say(f"dense fp8 T={T} causal={causal} S={S}")
    d = case.to_device()
    gpu_pool(case, d)
    assert np.array_equal(d["pool"].cpu().numpy(), case.oracle_pool())
    out, lse = gpu_decode(case, d, num_splits=S)
    ro, rl = case.oracle_decode()
    say(compare_outputs(out, ro, lse, rl, f"dense T={T} S={S}", vmax=case.vmax()))


@pytest.mark.parametrize("H,S", [(64, 0), (64, 3), (32, 0), (16, 2)])
def test_dense_fp8_decode_heads(H, S):
    """Dense FP8 decode at 64, 32 and 16 heads (two 32-head groups, one group), unsplit and split."""
    cfg = small(B=3, T=1, H=H, topk=0, fmt="fp8", L=1300, seed=43 + H)
    case = Case(cfg, ctx=[1300, 700, 65])
    say(f"dense fp8 H={H} S={S}")
    d = case.to_device()
    gpu_pool(case, d)
    out, lse = gpu_decode(case, d, num_splits=S)
    ro, rl = case.oracle_decode()
    say(compare_outputs(out, ro, lse, rl, f"dense H={H} S={S}", vmax=case.vmax()))


def test_dense_fp8_pages_outside_the_pool():
    """Page-table entries outside [0, num_pages) select nothing: in the middle of a context, on its
    last (partial) page, and for a split that holds only such pages."""
    cfg = small(B=3, T=1, H=128, topk=0, fmt="fp8", L=1500, seed=41)
    case = Case(cfg, ctx=[1500, 900, 70])
    bt = case.lay.block_table
    bt[0, 2] = -1
    bt[0, 5] = case.lay.num_pages + 3
    bt[1, 14] = -2  # request 1's last page (900 = 14 * 64 + 4)
    bt[2, 0] = case.lay.num_pages  # request 2 keeps only positions 64..69
    say("dense fp8 pages outside the pool")
    d = case.to_device()
    gpu_pool(case, d)
    for S in (1, 3, 0):
        out, lse = gpu_decode(case, d, num_splits=S)
        ro, rl = case.oracle_decode()
        say(compare_outputs(out, ro, lse, rl, f"dense invalid pages S={S}", vmax=case.vmax()))


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_unwritten_pool_bytes_do_not_leak(fmt):
    """Pool bytes no row was written to hold 0xFF (NaN as E4M3): the rows a decode gathers but masks
    (past the list in the last step, past the context on a last page, pages outside the pool) must not
    reach the output."""
    H = 32 if fmt == "nvfp4" else 128
    cfg = small(B=3, T=1, H=H, topk=300 if fmt == "nvfp4" else 0, L=1000, fmt=fmt, seed=45)
    case = Case(cfg, ctx=[1000, 333, 70])
    if fmt == "fp8":
        case.lay.block_table[0, 4] = -1
    say(f"unwritten pool bytes {fmt}")
    d = case.to_device()
    d["pool"].fill_(0xFF)
    gpu_pool(case, d)
    for S in (1, 3):
        out, lse = gpu_decode(case, d, num_splits=S)
        assert np.isfinite(out).all() and np.isfinite(lse).all()
        ro, rl = case.oracle_decode()
        say(compare_outputs(out, ro, lse, rl, f"0xFF pool {fmt} S={S}", vmax=case.vmax()))


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_block_major_multi_layer_pool(fmt):
    """Block-major pages (the analysis page's KV layout section: all layers of a block adjacent): page p
    holds layer 0's 64 rows, then layer 1's, ...; layer l is the pool shifted by l x 64 rows with a page
    stride of n_layers x 64 rows.  Each layer's writes and decodes touch only its own rows."""
    n_layers = 3
    H = 32 if fmt == "nvfp4" else 128
    cfg = small(B=2, T=1, H=H, topk=384 if fmt == "nvfp4" else 0, L=1500, fmt=fmt, seed=46)
    rb = cfg.row_bytes
    stride = n_layers * 64 * rb
    cases = [Case(cfg, seed_offset=l) for l in range(n_layers)]
    lay = cases[0].lay
    for c in cases[1:]:  # one page table for every layer, as in a block-major cache
        c.lay = lay
        c.slots = np.concatenate([W.slots_for_request(lay, b, np.arange(int(lay.ctx[b]))) for b in range(cfg.B)])
    say(f"block-major {n_layers} layers {fmt}")
    pool = torch.full((lay.num_pages * stride,), 0xFF, dtype=torch.uint8, device="cuda")
    ref_pool = np.zeros(lay.num_pages * stride, np.uint8)
    quant = M.mla_kv_quant_nvfp4 if fmt == "nvfp4" else M.mla_kv_quant_fp8
    for l, c in enumerate(cases):
        d = c.to_device()
        quant(d["lat"], d["rope"], d["slots"], pool[l * 64 * rb:], stride, lay.num_pages)
        oracle.kv_quant(fmt, c.lat, c.rope, c.slots, ref_pool[l * 64 * rb:], stride, lay.num_pages)
    torch.cuda.synchronize()
    host = pool.cpu().numpy()
    written = ref_pool != 0
    assert np.array_equal(host[written], ref_pool[written])
    for l, c in enumerate(cases):
        d = c.to_device()
        lse = torch.empty((cfg.B, 1, H), dtype=torch.float32, device="cuda")
        if fmt == "nvfp4":
            out, _ = M.mla_sparse_decode(d["q"], pool[l * 64 * rb:], stride, lay.num_pages, d["bt"], d["ctx"], d["idx"],
                                         cfg.sm_scale, lse=lse)
            ro, rl, _ = oracle.sparse_decode(c.q, ref_pool[l * 64 * rb:], stride, lay.num_pages, lay.block_table,
                                             lay.ctx, c.idx, cfg.sm_scale)
        else:
            out, _ = M.mla_dense_decode_fp8(d["q"], pool[l * 64 * rb:], stride, lay.num_pages, d["bt"], d["ctx"],
                                            int(lay.ctx.max()), cfg.sm_scale, lse=lse)
            ro, rl, _ = oracle.dense_decode_fp8(c.q, ref_pool[l * 64 * rb:], stride, lay.num_pages, lay.block_table,
                                                lay.ctx, cfg.sm_scale)
        torch.cuda.synchronize()
        say(compare_outputs(bf16_to_np(out).reshape(cfg.B, H, 512), ro,
                            lse.cpu().numpy().astype(np.float64).reshape(cfg.B, H), rl, f"layer {l}", vmax=c.vmax()))


# --------------------------------------------------------------------------- staged path (NVFP4 -> FP8 copy)
def _gpu_stage(pool_d, page_stride, num_pages, bt_d, ctx_d, idx_d, causal=False):
    staged, sbt, slen = M.mla_stage_nvfp4_fp8(pool_d, page_stride, num_pages, bt_d, ctx_d, idx_d, causal=causal)
    torch.cuda.synchronize()
    nq, P = sbt.shape
    return staged.cpu().numpy().reshape(nq, P * 64, 576), sbt.cpu().numpy(), slen.cpu().numpy()


def _check_staged(staged, sbt, slen, ref_staged, ref_counts):
    nq, P = sbt.shape
    assert np.array_equal(slen, ref_counts)
    assert np.array_equal(sbt, np.arange(nq)[:, None] * P + np.arange(P)[None, :])
    for i in range(nq):
        n = int(ref_counts[i])
        if not np.array_equal(staged[i, :n], ref_staged[i, :n]):
            bad = np.argwhere(staged[i, :n] != ref_staged[i, :n])[:5]
            raise AssertionError(f"token {i}: staged bytes differ at {bad.tolist()}: "
                                 f"{[(int(staged[i][tuple(x)]), int(ref_staged[i][tuple(x)])) for x in bad]}")


def test_stage_every_scale_and_nibble_bit_exact():
    """Every (scale byte, nibble) pair the format can hold, NaN scale bytes aside, unpacked to FP8 bit
    for bit as the oracle does it (including products above 448, -0 and E4M3 subnormals)."""
    rows = []
    for r in range(8):
        row = np.zeros(352, np.uint8)
        for j in range(32):
            sc = 32 * r + j
            row[256 + j] = 0 if sc in (0x7F, 0xFF) else sc
            nib = np.arange(16, dtype=np.uint8)
            row[8 * j:8 * j + 8] = nib[0::2] | (nib[1::2] << 4)
        row[288:352] = (np.arange(64) * 7 + r).astype(np.uint8)
        rows.append(row)
    pool = np.zeros(2 * 64 * 352, np.uint8)
    pool[64 * 352:64 * 352 + 8 * 352] = np.concatenate(rows)
    bt = np.array([[1]], np.int32)
    ctx = np.array([8], np.int32)
    idx = np.array([[[7, 0, 3, 5, 1, 6, 2, 4]]], np.int32)
    ref, cnt = oracle.stage_nvfp4_fp8(pool, 64 * 352, 2, bt, ctx, idx)
    say("stage every scale x nibble")
    got = _gpu_stage(torch.from_numpy(pool).cuda(), 64 * 352, 2, torch.from_numpy(bt).cuda(),
                     torch.from_numpy(ctx).cuda(), torch.from_numpy(idx).cuda())
    _check_staged(*got, ref, cnt)


@pytest.mark.parametrize("T,causal", [(1, False), (2, True)])
def test_stage_selection_bit_exact(T, causal):
    """Selection (padding, entries past the context, pages outside the pool), order and bytes of the
    staged copy, several tokens, topk not a multiple of 64."""
    cfg = small(B=3, T=T, H=16, topk=300, L=2000, causal=causal, seed=43)
    case = Case(cfg, ctx=[2000, 650, 90])
    idx = case.idx.copy()
    idx[0, 0, :37] = -1
    idx[1, -1, 10:20] = 10 ** 7
    case.idx = idx
    case.lay.block_table[0, 5] = -3
    say(f"stage selection T={T} causal={causal}")
    d = case.to_device()
    gpu_pool(case, d)
    ref, cnt = oracle.stage_nvfp4_fp8(case.oracle_pool(), cfg.page_stride, case.lay.num_pages, case.lay.block_table,
                                      case.lay.ctx, idx, causal=causal)
    got = _gpu_stage(d["pool"], cfg.page_stride, case.lay.num_pages, d["bt"], d["ctx"], d["idx"], causal=causal)
    _check_staged(*got, ref, cnt)


@pytest.mark.parametrize("H", [16, 32, 128])
def test_staged_decode_matches_oracle(H):
    """The staged path end to end: the GPU copy read by the GPU FP8 decoder against the oracle's FP8
    attention over the oracle's copy."""
    cfg = small(B=4, T=1, H=H, topk=512, L=5000, seed=44)
    case = Case(cfg, ctx=[5000, 3000, 900, 400])
    say(f"staged decode H={H}")
    d = case.to_device()
    gpu_pool(case, d)
    staged, sbt, slen = M.mla_stage_nvfp4_fp8(d["pool"], cfg.page_stride, case.lay.num_pages, d["bt"], d["ctx"],
                                              d["idx"])
    nq, P = sbt.shape
    q1 = d["q"].view(nq, 1, H, 576)
    lse = torch.empty((nq, 1, H), dtype=torch.float32, device="cuda")
    out, _ = M.mla_dense_decode_fp8(q1, staged, 64 * 576, nq * P, sbt, slen, P * 64, cfg.sm_scale, lse=lse)
    torch.cuda.synchronize()
    ref_st, cnt = oracle.stage_nvfp4_fp8(case.oracle_pool(), cfg.page_stride, case.lay.num_pages,
                                         case.lay.block_table, case.lay.ctx, case.idx)
    bt = (np.arange(nq)[:, None] * P + np.arange(P)[None, :]).astype(np.int32)
    ro, rl, _ = oracle.dense_decode_fp8(case.q.reshape(nq, 1, H, 576), ref_st.reshape(-1), 64 * 576, nq * P, bt, cnt,
                                        cfg.sm_scale)
    vm = np.zeros((nq, 1, 512))
    for u in range(nq):
        if cnt[u]:
            vm[u, 0] = v_abs_of_rows(ref_st[u, :cnt[u]], "fp8").max(0)
    say(compare_outputs(bf16_to_np(out).reshape(nq, H, 512), ro,
                        lse.cpu().numpy().astype(np.float64).reshape(nq, H), rl, f"staged decode H={H}", vmax=vm))


# --------------------------------------------------------------------------- full-size configs, sampled
@pytest.mark.parametrize("name", ["sparse", "spec", "mixed", "dense_b4", "dense_b8", "dense_b16", "pages15", "pages20",
                                  "short35", "pages15_fp8"])
def test_full_size_config_sampled(name):
    cfg = W.CONFIGS[name]
    say(f"full-size {name}: generating inputs")
    inp = W.device_inputs(cfg, "cuda", n_sets=1)
    lay = inp["layout"]
    pool = torch.zeros(lay.num_pages * cfg.page_stride, dtype=torch.uint8, device="cuda")
    inp["pool"] = pool
    fn = M.mla_kv_quant_nvfp4 if cfg.fmt == "nvfp4" else M.mla_kv_quant_fp8
    fn(inp["lat"], inp["rope"], inp["slots"], pool, cfg.page_stride, lay.num_pages)
    if cfg.quant_chunk:
        fn(inp["chunk_lat"], inp["chunk_rope"], inp["chunk_slots"], pool, cfg.page_stride, lay.num_pages)
    q = inp["q_sets"][0]
    lse = torch.empty((cfg.B, cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    say(f"full-size {name}: decode")
    if cfg.topk:
        idx = inp["idx_sets"][0]
        fn = M.mla_sparse_decode if cfg.fmt == "nvfp4" else M.mla_sparse_decode_fp8
        out, _ = fn(q, pool, cfg.page_stride, lay.num_pages, inp["bt"], inp["ctx"], idx, cfg.sm_scale,
                    causal=cfg.causal, lse=lse)
    else:
        idx = None
        out, _ = M.mla_dense_decode_fp8(q, pool, cfg.page_stride, lay.num_pages, inp["bt"], inp["ctx"],
                                        int(lay.ctx.max()), cfg.sm_scale, causal=cfg.causal, lse=lse)
    torch.cuda.synchronize()
    nq = cfg.B * cfg.T
    qtoks = sorted(set([0, nq - 1] + list(np.random.default_rng(cfg.seed).choice(nq, min(6, nq), replace=False))))
    say(f"full-size {name}: oracle on query tokens {qtoks}")
    ro, rl, vm, pools_ok = sampled_oracle(cfg, inp, qtoks, idx, q)
    assert pools_ok, "pool rows differ from the oracle's quantization"
    g = bf16_to_np(out).reshape(nq, cfg.H, 512)[qtoks]
    gl = lse.cpu().numpy().astype(np.float64).reshape(nq, cfg.H)[qtoks]
    say(compare_outputs(g, ro, gl, rl, f"full-size {name}", vmax=vm))
    # the write chunk of the mixed step: bit exact on every row
    if cfg.quant_chunk:
        cl = inp["chunk_lat"].view(torch.int16).cpu().numpy().view(np.uint16)
        cr = inp["chunk_rope"].view(torch.int16).cpu().numpy().view(np.uint16)
        cs = inp["chunk_slots"].cpu().numpy()
        rb = cfg.row_bytes
        offs = (cs // 64) * cfg.page_stride + (cs % 64) * rb
        gidx = torch.from_numpy((offs[:, None] + np.arange(rb)[None, :]).reshape(-1)).cuda()
        grows = pool[gidx].cpu().numpy().reshape(-1, rb)
        for r in range(0, cs.size, 37):
            assert np.array_equal(grows[r], oracle.quant_row_nvfp4(cl[r], cr[r]))
    del inp, pool
    torch.cuda.empty_cache()


def test_full_size_staged_path_sampled():
    """The staged path at the primary config's full size, as bench.py --path staged times it: for sampled
    query tokens, the FP8 copy is bit-exact against the oracle's unpack of the token's selected rows (the
    oracle quantizes the source rows itself), and the FP8 decode over the GPU copy matches the oracle's
    FP8 attention over its own copy."""
    cfg = W.CONFIGS["sparse"]
    say("full-size staged: generating inputs")
    inp = W.device_inputs(cfg, "cuda", n_sets=1)
    lay = inp["layout"]
    pool = torch.zeros(lay.num_pages * cfg.page_stride, dtype=torch.uint8, device="cuda")
    M.mla_kv_quant_nvfp4(inp["lat"], inp["rope"], inp["slots"], pool, cfg.page_stride, lay.num_pages)
    idx = inp["idx_sets"][0]
    q = inp["q_sets"][0]
    nq = cfg.B * cfg.T
    say("full-size staged: stage + FP8 decode")
    staged, sbt, slen = M.mla_stage_nvfp4_fp8(pool, cfg.page_stride, lay.num_pages, inp["bt"], inp["ctx"], idx)
    P = sbt.shape[1]
    lse = torch.empty((nq, 1, cfg.H), dtype=torch.float32, device="cuda")
    out, _ = M.mla_dense_decode_fp8(q.view(nq, 1, cfg.H, 576), staged, 64 * 576, nq * P, sbt, slen, P * 64,
                                    cfg.sm_scale, lse=lse)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    q_h = q.view(torch.int16).cpu().numpy().view(np.uint16)
    lens = slen.cpu().numpy()
    g_out = bf16_to_np(out).reshape(nq, cfg.H, 512)
    g_lse = lse.cpu().numpy().astype(np.float64).reshape(nq, cfg.H)
    qtoks = sorted(set([0, nq - 1] + list(np.random.default_rng(cfg.seed + 1).choice(nq, 4, replace=False))))
    say(f"full-size staged: oracle on query tokens {qtoks}")
    for qt in qtoks:
        b, t = divmod(int(qt), cfg.T)
        lim = W.position_limit(int(lay.ctx[b]), cfg.T, t, cfg.causal)
        ids = idx_h[b, t]
        pos = ids[(ids >= 0) & (ids <= lim)]  # list order, as staged
        n = pos.size
        assert lens[qt] == n
        rows = torch.from_numpy(inp["row_off"][b] + pos).cuda()
        lat = inp["lat"][rows].view(torch.int16).cpu().numpy().view(np.uint16)
        rope = inp["rope"][rows].view(torch.int16).cpu().numpy().view(np.uint16)
        npg = (n + 63) // 64
        mini = np.zeros(npg * 64 * 352, np.uint8)
        oracle.kv_quant("nvfp4", lat, rope, np.arange(n, dtype=np.int64), mini, 64 * 352, npg)
        ref, cnt = oracle.stage_nvfp4_fp8(mini, 64 * 352, npg, np.arange(npg, dtype=np.int32)[None, :],
                                          np.array([n], np.int32), np.arange(n, dtype=np.int32).reshape(1, 1, n))
        got = staged[qt * P * 64 * 576:(qt * P * 64 + n) * 576].cpu().numpy().reshape(n, 576)
        assert cnt[0] == n and np.array_equal(got, ref[0, :n]), f"staged rows of query token {qt}"
        ro, rl, _ = oracle.dense_decode_fp8(q_h[b:b + 1, t:t + 1], ref[0].reshape(-1), 64 * 576, ref.shape[1] // 64,
                                            np.arange(ref.shape[1] // 64, dtype=np.int32)[None, :],
                                            np.array([n], np.int32), cfg.sm_scale)
        vm = v_abs_of_rows(ref[0, :n], "fp8").max(0)[None, None, :]
        say(compare_outputs(g_out[qt:qt + 1], ro, g_lse[qt:qt + 1], rl, f"staged token {qt}", vmax=vm))
