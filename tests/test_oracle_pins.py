"""Pins of the FP64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a figure printed on the pages (tests/golden/, cited
there), a library routine (torch's float8 decoders and casts), exact rational arithmetic, a second
independent algorithm, or a mathematical invariant of softmax attention.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

FINITE_BF16 = np.array([b for b in range(65536) if ((b >> 7) & 0xFF) != 0xFF], dtype=np.uint16)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_f64(bits):
    return W.bf16_to_f32(bits).astype(np.float64)


# --------------------------------------------------------------------------- generic minifloat decoder
def minifloat(code, ebits, mbits, bias):
    """Sign / exponent / mantissa decoding with subnormals (no special values)."""
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    v = (m / (1 << mbits)) * 2.0 ** (1 - bias) if e == 0 else (1 + m / (1 << mbits)) * 2.0 ** (e - bias)
    return -v if s else v


def test_generic_minifloat_matches_torch_float8_formats():
    # Pins the generic decoder used below against two library formats.
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    e5 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).double().numpy()
    for c in range(256):
        if (c & 0x7F) != 0x7F:
            assert minifloat(c, 4, 3, 7) == e4[c]
        if ((c >> 2) & 0x1F) != 0x1F:
            assert minifloat(c, 5, 2, 15) == e5[c]


# --------------------------------------------------------------------------- row layout (pages' numbers)
def test_row_size_closed_form_from_pages():
    g = _golden("row_layout.json")
    n, r, grp = g["latent_values"], g["rope_values"], g["values_per_scale"]
    assert n * 4 // 8 == g["nvfp4"]["latent_bytes"]
    assert n // grp == g["nvfp4"]["scale_bytes"]
    assert r == g["nvfp4"]["rope_bytes"]
    assert sum(g["nvfp4"][k] for k in ("latent_bytes", "scale_bytes", "rope_bytes")) == g["nvfp4"]["row_bytes"] == 352
    assert g["fp8"]["latent_bytes"] + g["fp8"]["rope_bytes"] == g["fp8"]["row_bytes"] == 576
    assert round(576 / 352, 2) == g["row_ratio_printed"]
    rng = np.random.default_rng(0)
    lat, rope = W.gen_latent_rope(rng, 1)
    assert oracle.quant_row_nvfp4(lat[0], rope[0]).size == g["nvfp4"]["row_bytes"]
    assert oracle.quant_row_fp8(lat[0], rope[0]).size == g["fp8"]["row_bytes"]
    assert oracle.NVFP4_ROW_BYTES == 352 and oracle.FP8_ROW_BYTES == 576


def test_pool_placement_rows_at_352_byte_stride():
    # Rows of one page sit back to back; pages at page_stride; negative / out-of-pool slots skipped.
    rng = np.random.default_rng(1)
    lat, rope = W.gen_latent_rope(rng, 5)
    page_stride = 64 * 352 + 160  # a padded page stride (block-major pools have larger strides)
    pool = np.zeros(3 * page_stride, np.uint8)
    slots = np.array([0, 1, 64 + 63, -1, 3 * 64], np.int64)
    n = oracle.kv_quant("nvfp4", lat, rope, slots, pool, page_stride, 3)
    assert n == 3
    assert np.array_equal(pool[0:352], oracle.quant_row_nvfp4(lat[0], rope[0]))
    assert np.array_equal(pool[352:704], oracle.quant_row_nvfp4(lat[1], rope[1]))
    assert np.array_equal(pool[page_stride + 63 * 352: page_stride + 64 * 352], oracle.quant_row_nvfp4(lat[2], rope[2]))
    written = np.zeros_like(pool, dtype=bool)
    written[0:704] = True
    written[page_stride + 63 * 352: page_stride + 64 * 352] = True
    assert not pool[~written].any()


def test_fp8_row_bytes_are_the_e4m3_casts_latent_then_rope():
    """The 576-byte FP8 row (analysis page, row table: 512 latent + 64 rope values, no per-row scale) holds
    torch's float8_e4m3fn cast of each value, saturated to +-448, latent first and rope after it: a row
    written in another order, or with a scale, fails here.  Also its placement in a padded page."""
    rng = np.random.default_rng(71)
    mags = np.concatenate([rng.standard_normal(4000), rng.standard_normal(1000) * 600, rng.standard_normal(600) * 1e-3,
                           [0.0, -0.0, 448.0, -449.0, 464.0, 1e30, -1e-30, 2.0 ** -10, 2.0 ** -9 * 3]])
    vals = rng.permutation(np.resize(mags, 8 * 576)).astype(np.float32).reshape(8, 576)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)  # bf16 by truncation: exact bf16 inputs
    exact = (bits.astype(np.uint32) << 16).view(np.float32)
    ref = torch.from_numpy(exact).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for r in range(8):
        row = oracle.quant_row_fp8(bits[r, :512], bits[r, 512:])
        assert np.array_equal(row, ref[r]), f"row {r}: bytes {np.nonzero(row != ref[r])[0][:8]}"
    page_stride = 64 * 576 + 32
    pool = np.zeros(2 * page_stride, np.uint8)
    assert oracle.kv_quant("fp8", bits[:3, :512], bits[:3, 512:], np.array([64 + 5, 2, -1], np.int64), pool,
                           page_stride, 2) == 2
    assert np.array_equal(pool[page_stride + 5 * 576:page_stride + 6 * 576], ref[0])
    assert np.array_equal(pool[2 * 576:3 * 576], ref[1])
    written = np.zeros(pool.size, bool)
    written[page_stride + 5 * 576:page_stride + 6 * 576] = True
    written[2 * 576:3 * 576] = True
    assert not pool[~written].any()


def _one_hot_pool(fmt, num_pages, value=1.5):
    """A pool whose row in slot s has latent value `value` at column s % 512 and zeros elsewhere (rope 0).
    1.5 is exact in every layout: NVFP4 block scale 0.25 with code 6, E4M3 1.5."""
    n = num_pages * 64
    lat = np.zeros((n, 512), np.float32)
    lat[np.arange(n), np.arange(n) % 512] = value
    lat_bits = (lat.view(np.uint32) >> 16).astype(np.uint16)
    rope_bits = np.zeros((n, 64), np.uint16)
    rb = 352 if fmt == "nvfp4" else 576
    pool = np.zeros(num_pages * 64 * rb, np.uint8)
    oracle.kv_quant(fmt, lat_bits, rope_bits, np.arange(n, dtype=np.int64), pool, 64 * rb, num_pages)
    return pool, lat_bits, rope_bits


def _selected_slot_counts(bt, ctx, idx, T, causal, num_pages):
    """The selection rule restated: entry i of query token (b, t) counts iff 0 <= i <= limit and its page
    entry bt[b][i // 64] lies in [0, num_pages); it stands for slot bt[b][i // 64] * 64 + i % 64."""
    B = bt.shape[0]
    counts = np.zeros((B * T, num_pages * 64), np.int64)
    for b in range(B):
        for t in range(T):
            lim = int(ctx[b]) - T + t if causal else int(ctx[b]) - 1
            for i in idx[b, t]:
                i = int(i)
                if i < 0 or i > lim or i // 64 >= bt.shape[1]:
                    continue
                pg = int(bt[b, i // 64])
                if 0 <= pg < num_pages:
                    counts[b * T + t, pg * 64 + i % 64] += 1
    return counts


def _selection_case():
    """Two requests, shuffled multi-page tables with entries outside the pool, T = 2 causal, lists with -1
    runs, positions past the limit, positions on bad pages and a duplicate."""
    num_pages = 8
    bt = np.array([[5, 2, 7, -1, 0], [3, 6, 1, 4, 9]], np.int32)  # 9 is outside the pool
    ctx = np.array([250, 300], np.int32)
    idx = np.array([[[3, 70, 130, 200, -1, 249, 64, 3, 10 ** 6, -7],
                     [249, 248, 131, 1, -1, -1, 199, 192, 65, 100]],
                    [[0, 63, 64, 299, 260, 257, 150, -1, 298, 129],
                     [299, 298, 256, 5, 70, 140, 255, 200, 64, 63]]], np.int32)
    return num_pages, bt, ctx, idx


@pytest.mark.parametrize("decoder", ["nvfp4", "fp8", "dense_fp8", "pth"])
def test_decoders_select_rows_through_the_page_table(decoder):
    """With q = 0 every selected row weighs the same, so out = mean of the selected V rows; with one-hot
    rows per slot the mean reveals exactly which slots were read and how often.  The expected multiset is
    the selection rule applied by hand: a decoder that ignored the page table, the causal limit, the
    -1 entries or duplicates would fail here."""
    num_pages, bt, ctx, idx = _selection_case()
    B, T, H = 2, 2, 4
    q = np.zeros((B, T, H, 576), np.uint16)
    if decoder == "dense_fp8":
        idx = np.broadcast_to(np.arange(300, dtype=np.int32), (B, T, 300)).copy()
    counts = _selected_slot_counts(bt, ctx, idx, T, True, num_pages)
    expect = 1.5 * counts[:, :512] / np.maximum(counts.sum(1, keepdims=True), 1)
    if decoder == "pth":
        _, lat_bits, rope_bits = _one_hot_pool("fp8", num_pages)
        n = num_pages * 64
        lat_buf = np.zeros((n, 512), np.uint8)
        sc_buf = np.zeros(n, np.float32)
        rope_buf = np.zeros((n, 64), np.uint16)
        oracle.kv_quant_pth(lat_bits, rope_bits, np.arange(n, dtype=np.int64), lat_buf, sc_buf, rope_buf)
        out, lse, _ = oracle.sparse_decode_pth(q, lat_buf, sc_buf, rope_buf, bt, ctx, idx, 0.1, causal=True)
        out = out.reshape(B * T, H, 512)
        lse = lse.reshape(B * T, H)
        tol = 1e-6  # the per-slot fp32 scale: 448 * fl(1.5 / 448) is 1.5 to fp32 precision
    else:
        fmt = "nvfp4" if decoder == "nvfp4" else "fp8"
        pool, _, _ = _one_hot_pool(fmt, num_pages)
        rb = 352 if fmt == "nvfp4" else 576
        if decoder == "dense_fp8":
            out, lse, _ = oracle.dense_decode_fp8(q, pool, 64 * rb, num_pages, bt, ctx, 0.1, causal=True)
        else:
            out, lse, _ = oracle.sparse_decode(q, pool, 64 * rb, num_pages, bt, ctx, idx, 0.1, causal=True, fmt=fmt)
        tol = 1e-14
    for u in range(B * T):
        for h in range(H):
            np.testing.assert_allclose(out[u, h], expect[u], rtol=tol, atol=tol)
        # q = 0: every score is 0, so lse = ln |J|
        assert np.allclose(lse[u], math.log(counts[u].sum()), atol=1e-12)
    assert counts.sum(1).min() > 0
    assert decoder == "dense_fp8" or (counts > 1).any()  # the sparse lists hold a duplicate


def test_constants_from_pages():
    g = _golden("constants.json")
    # the printed softmax scale is 1/sqrt(192) (192 = 128 + 64) to the 7 digits shown
    assert abs(1 / math.sqrt(192) - g["softmax_scale_printed"]) < 5e-8
    assert W.CONFIGS["sparse"].sm_scale == pytest.approx(g["softmax_scale_printed"], abs=5e-8)
    assert oracle.e4m3_value(0x7E) == g["e4m3_max"]
    assert W.PAGE == g["page_size"] and W.CONFIGS["sparse"].topk == g["index_topk"]


# --------------------------------------------------------------------------- decoders
def test_e4m3_decode_all_codes_vs_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        v = oracle.e4m3_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(v)
        else:
            assert v == ref[c], c
    assert max(abs(oracle.e4m3_value(c)) for c in range(256) if (c & 0x7F) != 0x7F) == 448.0


def test_e2m1_decode_all_codes_vs_generic_minifloat():
    # e2m1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no special values
    vals = [oracle.e2m1_value(c) for c in range(16)]
    assert vals == [minifloat(c, 2, 1, 1) for c in range(16)]
    assert sorted(set(abs(v) for v in vals)) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_bf16_decode_vs_torch():
    ref = torch.from_numpy(FINITE_BF16.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_value(b) for b in FINITE_BF16[::97]])
    assert np.array_equal(got, ref[::97])


# --------------------------------------------------------------------------- encoders
def _threshold_e2m1(a, s):
    """Nearest e2m1 magnitude code of a/s by counting crossed midpoints (ties to even code)."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * s
    code = np.zeros(a.shape, np.int64)
    for k, t in enumerate(mids):
        code += (a > t) | ((a == t) & (k % 2 == 1))
    return code


def test_e2m1_encode_exhaustive_vs_threshold_method():
    # every finite bf16 value x every positive finite E4M3 scale (about 8.2M pairs)
    x = FINITE_BF16
    a = np.abs(_bf16_f64(x))
    sign = (x >> 15).astype(np.int64)
    for sc in range(1, 0x7F):
        s = oracle.e4m3_value(sc)
        got = oracle.e2m1_encode(x, sc).astype(np.int64)
        want = _threshold_e2m1(a, s) | (sign << 3)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (sc, x[bad[:5]], got[bad[:5]], want[bad[:5]])
    # zero scale: magnitude 0, sign kept
    got0 = oracle.e2m1_encode(x, 0).astype(np.int64)
    assert np.array_equal(got0, sign << 3)


def test_e2m1_encode_exact_rational_sample():
    rng = np.random.default_rng(5)
    grid = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    xs = rng.choice(FINITE_BF16, 4000)
    scs = rng.integers(1, 0x7F, 4000)
    for xb, sc in zip(xs, scs):
        a = abs(Fraction(oracle.bf16_value(int(xb))))
        s = Fraction(oracle.e4m3_value(int(sc)))
        r = a / s
        d = [abs(r - g) for g in grid]
        best = min(range(8), key=lambda k: (d[k], k % 2))
        got = oracle.e2m1_encode(np.array([xb], np.uint16), int(sc))[0]
        assert got & 7 == best and (got >> 3) == (int(xb) >> 15)


def test_scale_code_all_bf16_amax_vs_torch_cast():
    pos = FINITE_BF16[(FINITE_BF16 >> 15) == 0]
    amax = _bf16_f64(pos)
    got = oracle.scale_code(pos).astype(np.int64)
    r = amax / 6.0
    ref = torch.from_numpy(np.minimum(r, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    assert np.array_equal(got, ref)


def test_scale_code_exact_rational_sample_and_ties():
    rng = np.random.default_rng(6)
    pos = FINITE_BF16[(FINITE_BF16 >> 15) == 0]
    cand = [(c, Fraction(oracle.e4m3_value(c))) for c in range(0x7F)]
    # includes every amax that sits exactly on a midpoint x 6 (the tie cases)
    mids = set()
    for c in range(0x7E):
        m6 = (cand[c][1] + cand[c + 1][1]) / 2 * 6
        mids.add(float(m6))
    tie_bits = [b for b in pos if oracle.bf16_value(int(b)) in mids]
    assert len(tie_bits) > 50
    sample = list(rng.choice(pos, 3000)) + tie_bits
    for b in sample:
        r = Fraction(oracle.bf16_value(int(b))) / 6
        best = min(cand, key=lambda cv: (abs(r - cv[1]), cv[0] % 2))[0]
        assert oracle.scale_code(np.array([b], np.uint16))[0] == best, b


def test_e4m3_encode_all_bf16_vs_torch_cast_and_saturation():
    x = FINITE_BF16
    v = _bf16_f64(x)
    got = oracle.e4m3_encode(x).astype(np.int64)
    inside = np.abs(v) <= 448.0
    ref = torch.from_numpy(v[inside]).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    assert np.array_equal(got[inside], ref)
    sign = (x[~inside] >> 15).astype(np.int64)
    assert np.array_equal(got[~inside], 0x7E | (sign << 7))


def test_round_trip_of_representable_values():
    # decode(encode(decode(c))) == decode(c)
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        v = oracle.e4m3_value(c)
        bits = W.bf16_bits(np.array([v], np.float32))  # every E4M3 value is exact in bf16
        assert W.bf16_to_f32(bits)[0] == v
        assert oracle.e4m3_value(int(oracle.e4m3_encode(bits)[0])) == v
    one = 0x38  # scale 1.0
    assert oracle.e4m3_value(one) == 1.0
    for c in range(16):
        v = oracle.e2m1_value(c)
        bits = W.bf16_bits(np.array([v], np.float32))
        assert oracle.e2m1_value(int(oracle.e2m1_encode(bits, one)[0])) == v


# --------------------------------------------------------------------------- row quantization properties
def _split(row):
    nib = np.empty(512, np.int64)
    nib[0::2] = row[:256] & 15
    nib[1::2] = row[:256] >> 4
    return nib, row[256:288].astype(np.int64), row[288:352]


def test_row_error_bound_and_grid():
    rng = np.random.default_rng(7)
    lat, rope = W.gen_latent_rope(rng, 64)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for r in range(64):
        row = oracle.quant_row_nvfp4(lat[r], rope[r])
        x = _bf16_f64(lat[r])
        K = oracle.dequant_row_nvfp4(row)
        nib, sc, _ = _split(row)
        s = np.array([oracle.e4m3_value(c) for c in sc]).repeat(16)
        # dequantized value = e2m1 value x block scale
        assert np.array_equal(K[:512], np.array([oracle.e2m1_value(c) for c in nib]) * s)
        # nearest grid point: no other grid point is closer to x/s
        a = np.abs(x) / s
        assert np.all(np.abs(a - np.abs(K[:512]) / s) <= np.min(np.abs(a[:, None] - grid[None, :]), axis=1) + 0)
        # block scale is the E4M3 value nearest to amax/6
        amax = np.abs(x).reshape(32, 16).max(1)
        for j in range(32):
            d = [abs(amax[j] / 6 - oracle.e4m3_value(c)) for c in range(0x7F)]
            assert abs(amax[j] / 6 - oracle.e4m3_value(int(sc[j]))) == min(d)
        # rope: E4M3 cast without scale
        ref_rope = torch.from_numpy(_bf16_f64(rope[r])).to(torch.float8_e4m3fn).double().numpy()
        assert np.array_equal(K[512:], ref_rope)


def test_power_of_two_and_sign_equivariance():
    rng = np.random.default_rng(8)
    lat, rope = W.gen_latent_rope(rng, 16)
    tested = 0
    for r in range(16):
        x = W.bf16_to_f32(lat[r])
        base = oracle.quant_row_nvfp4(lat[r], rope[r])
        nib0, sc0, _ = _split(base)
        if sc0.min() < 0x10 or sc0.max() > 0x6E:  # scales stay normal and below 448 after the shift
            continue
        tested += 1
        for k in (-1, 1, 2):
            row = oracle.quant_row_nvfp4(W.bf16_bits(x * np.float32(2.0 ** k)), rope[r])
            nib, sc, _ = _split(row)
            assert np.array_equal(nib, nib0)
            assert np.array_equal(sc, sc0 + 8 * k)  # exponent field moves by k
        neg = oracle.quant_row_nvfp4(lat[r] ^ np.uint16(0x8000), rope[r])
        nibn, scn, _ = _split(neg)
        assert np.array_equal(scn, sc0)
        assert np.array_equal(nibn, nib0 ^ 8)
    assert tested >= 8


def test_zero_and_tiny_blocks():
    lat = np.zeros(512, np.uint16)
    lat[16:32] = 0x8000  # negative zeros keep their sign bit
    lat[32] = W.bf16_bits(np.array([6 * 2.0 ** -10], np.float32))[0]  # amax/6 = 2^-10: tie -> code 0
    lat[48] = W.bf16_bits(np.array([6 * 2.0 ** -10 * 1.0078125], np.float32))[0]  # just above the tie
    row = oracle.quant_row_nvfp4(lat, np.zeros(64, np.uint16))
    nib, sc, rope = _split(row)
    assert sc[0] == 0 and not nib[:16].any()
    assert sc[1] == 0 and np.all(nib[16:32] == 8)
    assert sc[2] == 0 and nib[32] == 0
    assert sc[3] == 1 and nib[48] == 5  # smallest subnormal scale 2^-9; |x|/s ~ 3.02 -> 3
    assert not rope.any()


def test_saturation_of_large_values():
    lat = np.zeros(512, np.uint16)
    lat[0] = W.bf16_bits(np.array([1e6], np.float32))[0]
    lat[1] = W.bf16_bits(np.array([-3e5], np.float32))[0]
    rope = W.bf16_bits(np.full(64, -1e4, np.float32))
    row = oracle.quant_row_nvfp4(lat, rope)
    nib, sc, rp = _split(row)
    assert sc[0] == 0x7E and nib[0] == 7 and nib[1] == 15
    assert np.all(rp == 0xFE)


# --------------------------------------------------------------------------- attention
def _small_case(seed, B=2, T=1, H=4, L=300, topk=64, causal=False, fmt="nvfp4"):
    rng = np.random.default_rng(seed)
    cfg = W.DecodeConfig("t", B=B, T=T, H=H, topk=topk, fmt=fmt, ctx=L, causal=causal, seed=seed)
    lay = W.gen_layout(cfg, rng)
    pool = np.zeros(lay.num_pages * cfg.page_stride, np.uint8)
    src = {}
    for b in range(B):
        pos = np.arange(int(lay.ctx[b]))
        lat, rope = W.gen_latent_rope(rng, pos.size)
        oracle.kv_quant(fmt, lat, rope, W.slots_for_request(lay, b, pos), pool, cfg.page_stride, lay.num_pages)
        src[b] = (lat, rope)
    q = W.gen_q(rng, B, T, H)
    idx = W.gen_indices(rng, lay.ctx, T, topk, causal) if topk else None
    return cfg, lay, pool, q, idx, rng


def _rows_of(cfg, lay, pool, b, positions):
    rb = cfg.row_bytes
    out = []
    for p in positions:
        page = lay.block_table[b, p // 64]
        off = page * cfg.page_stride + (p % 64) * rb
        out.append(pool[off:off + rb])
    return out


def _independent_K(row, fmt):
    """Dequantize with the test's own decoders: torch float8 for E4M3, the generic minifloat for e2m1."""
    f8 = torch.from_numpy(np.ascontiguousarray(row)).view(torch.float8_e4m3fn).double().numpy()
    if fmt == "fp8":
        return f8
    nib = np.empty(512, np.int64)
    nib[0::2] = row[:256] & 15
    nib[1::2] = row[:256] >> 4
    e2 = np.array([minifloat(int(c), 2, 1, 1) for c in nib])
    return np.concatenate([e2 * f8[256:288].repeat(16), f8[288:352]])


def _independent_attention(qbits, K, sm_scale):
    """Softmax attention via log-sum-exp in numpy."""
    from scipy.special import logsumexp
    q = _bf16_f64(qbits)  # [H,576]
    z = sm_scale * (q @ K.T)  # [H,n]
    lse = logsumexp(z, axis=1)
    P = np.exp(z - lse[:, None])
    return P @ K[:, :512], lse


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_full_selection_equals_independent_attention(fmt):
    cfg, lay, pool, q, _, _ = _small_case(11, L=200, topk=0, fmt=fmt)
    positions = np.arange(200)
    idx = np.tile(np.random.default_rng(3).permutation(positions).astype(np.int32), (cfg.B, 1, 1)).reshape(cfg.B, 1, 200)
    for b in range(cfg.B):
        K = np.stack([_independent_K(r, fmt) for r in _rows_of(cfg, lay, pool, b, positions)])
        ref_o, ref_l = _independent_attention(q[b, 0], K, cfg.sm_scale)
        if fmt == "nvfp4":
            out, lse, _ = oracle.sparse_decode(q, pool, cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx, idx,
                                               cfg.sm_scale)
        else:
            out, lse, _ = oracle.dense_decode_fp8(q, pool, cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx,
                                                  cfg.sm_scale)
        np.testing.assert_allclose(out[b], ref_o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse[b], ref_l, rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_selected_v():
    cfg, lay, pool, q, idx, _ = _small_case(12)
    q[:] = 0
    out, lse, _ = oracle.sparse_decode(q, pool, cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx, idx,
                                       cfg.sm_scale)
    for b in range(cfg.B):
        V = np.stack([_independent_K(r, "nvfp4")[:512] for r in _rows_of(cfg, lay, pool, b, idx[b, 0])])
        np.testing.assert_allclose(out[b], np.broadcast_to(V.mean(0), out[b].shape), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b], math.log(idx.shape[2]), rtol=1e-13)


def test_identical_keys_give_mean_of_v():
    # q_nope = 0 and every selected row has the same rope part: all scores equal although latents differ
    rng = np.random.default_rng(13)
    H, n = 4, 40
    lat, rope = W.gen_latent_rope(rng, n)
    rope[:] = rope[0]
    pool = np.zeros(64 * 352 * 2, np.uint8)
    bt = np.array([[1]], np.int32)
    oracle.kv_quant("nvfp4", lat, rope, 64 + np.arange(n), pool, 64 * 352, 2)
    q = W.gen_q(rng, 1, 1, H)
    q[..., :512] = 0
    idx = rng.permutation(n).astype(np.int32).reshape(1, 1, n)
    out, _, _ = oracle.sparse_decode(q, pool, 64 * 352, 2, bt, np.array([n], np.int32), idx, 0.07)
    V = np.stack([oracle.dequant_row_nvfp4(pool[(64 + i) * 352:(65 + i) * 352])[:512] for i in range(n)])
    assert np.abs(V - V[0]).max() > 0.1
    np.testing.assert_allclose(out[0], np.broadcast_to(V.mean(0), (H, 512)), rtol=1e-12, atol=1e-13)


def test_single_index_gives_that_row():
    cfg, lay, pool, q, idx, _ = _small_case(14)
    one = np.full_like(idx, -1)
    one[:, :, 7] = idx[:, :, 0]
    out, lse, _ = oracle.sparse_decode(q, pool, cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx, one,
                                       cfg.sm_scale)
    for b in range(cfg.B):
        K = _independent_K(_rows_of(cfg, lay, pool, b, [idx[b, 0, 0]])[0], "nvfp4")
        assert np.array_equal(out[b], np.broadcast_to(K[:512], out[b].shape))
        np.testing.assert_allclose(lse[b], cfg.sm_scale * (_bf16_f64(q[b, 0]) @ K), rtol=1e-13)


def test_permutation_and_padding_invariance():
    cfg, lay, pool, q, idx, rng = _small_case(15)
    args = (cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx)
    out0, lse0, _ = oracle.sparse_decode(q, pool, *args, idx, cfg.sm_scale)
    perm = idx[:, :, rng.permutation(idx.shape[2])]
    out1, lse1, _ = oracle.sparse_decode(q, pool, *args, perm, cfg.sm_scale)
    pad = np.full((cfg.B, 1, idx.shape[2] + 50), -1, np.int32)
    where = np.sort(rng.choice(pad.shape[2], idx.shape[2], replace=False))
    pad[:, :, where] = idx
    out2, lse2, _ = oracle.sparse_decode(q, pool, *args, pad, cfg.sm_scale)
    for o, l in ((out1, lse1), (out2, lse2)):
        np.testing.assert_allclose(o, out0, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l, lse0, rtol=1e-13)


def test_split_and_merge_equals_unsplit():
    cfg, lay, pool, q, idx, rng = _small_case(16, topk=100)
    args = (cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx)
    out0, lse0, _ = oracle.sparse_decode(q, pool, *args, idx, cfg.sm_scale)
    for S in (2, 3, 7):
        parts_o, parts_l = [], []
        bounds = np.linspace(0, idx.shape[2], S + 1).astype(int)
        for s in range(S):
            sub = np.full_like(idx, -1)
            sub[:, :, bounds[s]:bounds[s + 1]] = idx[:, :, bounds[s]:bounds[s + 1]]
            o, l, _ = oracle.sparse_decode(q, pool, *args, sub, cfg.sm_scale)
            parts_o.append(o)
            parts_l.append(l)
        for b in range(cfg.B):
            mo, ml = oracle.merge_partials(np.stack([p[b] for p in parts_o]), np.stack([p[b] for p in parts_l]))
            np.testing.assert_allclose(mo, out0[b], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(ml, lse0[b], rtol=1e-13)
    # an empty part (lse = -inf) carries no weight; all-empty gives 0 / -inf
    mo, ml = oracle.merge_partials(np.stack([out0[0], np.zeros_like(out0[0])]),
                                   np.stack([lse0[0], np.full_like(lse0[0], -np.inf)]))
    np.testing.assert_allclose(mo, out0[0], rtol=1e-14)
    mo, ml = oracle.merge_partials(np.zeros((2, cfg.H, 512)), np.full((2, cfg.H), -np.inf))
    assert not mo.any() and np.all(ml == -np.inf)


def test_causal_limit_and_invalid_entries_are_ignored():
    cfg, lay, pool, q, idx, rng = _small_case(17, T=4, L=257, topk=80, causal=True)
    args = (cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx)
    out0, lse0, _ = oracle.sparse_decode(q, pool, *args, idx, cfg.sm_scale, causal=True)
    # entries past each token's limit, past the context, or < -1 behave as absent
    bad = idx.copy()
    L = int(lay.ctx[0])
    extra = np.full((cfg.B, cfg.T, 5), -1, np.int32)
    for t in range(cfg.T):
        extra[:, t, :] = [L - cfg.T + t + 1 if t < cfg.T - 1 else L, L + 10, -7, 10 ** 6, -1]
    bad = np.concatenate([bad, extra], axis=2)
    out1, lse1, _ = oracle.sparse_decode(q, pool, *args, bad, cfg.sm_scale, causal=True)
    np.testing.assert_allclose(out1, out0, rtol=1e-12, atol=1e-13)
    # a page-table entry outside the pool removes the positions on that page
    bt = lay.block_table.copy()
    bt[0, 1] = lay.num_pages + 3
    keep = idx.copy()
    keep[0][(keep[0] // 64) == 1] = -1
    out2, _, _ = oracle.sparse_decode(q, pool, cfg.page_stride, lay.num_pages, bt, lay.ctx, idx, cfg.sm_scale,
                                      causal=True)
    out3, _, _ = oracle.sparse_decode(q, pool, *args, keep, cfg.sm_scale, causal=True)
    np.testing.assert_allclose(out2, out3, rtol=1e-12, atol=1e-13)


def test_empty_selection():
    cfg, lay, pool, q, idx, _ = _small_case(18)
    none = np.full_like(idx, -1)
    out, lse, _ = oracle.sparse_decode(q, pool, cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx, none,
                                       cfg.sm_scale)
    assert not out.any() and np.all(lse == -np.inf)


def test_dense_equals_sparse_over_full_list_on_same_rows():
    # dense FP8 decode and sparse decode agree in definition: same positions, same rows -> same result
    cfg, lay, pool, q, _, _ = _small_case(19, L=150, topk=0, fmt="fp8", T=2, causal=True)
    out_d, lse_d, _ = oracle.dense_decode_fp8(q, pool, cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx,
                                              cfg.sm_scale, causal=True)
    for b in range(cfg.B):
        for t in range(cfg.T):
            lim = 150 - 2 + t
            K = np.stack([_independent_K(r, "fp8") for r in _rows_of(cfg, lay, pool, b, np.arange(lim + 1))])
            ro, rl = _independent_attention(q[b, t], K, cfg.sm_scale)
            np.testing.assert_allclose(out_d[b * cfg.T + t], ro, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(lse_d[b * cfg.T + t], rl, rtol=1e-12)


def test_units_subset_matches_full_run():
    cfg, lay, pool, q, idx, _ = _small_case(20, B=3, T=2, causal=True)
    args = (cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx)
    out, lse, _ = oracle.sparse_decode(q, pool, *args, idx, cfg.sm_scale, causal=True)
    units = np.array([5, 0, 3], np.int64)
    out_u, lse_u, _ = oracle.sparse_decode(q, pool, *args, idx, cfg.sm_scale, causal=True, units=units)
    assert np.array_equal(out_u, out[units]) and np.array_equal(lse_u, lse[units])


# --------------------------------------------------------------------------- staged path (NVFP4 -> FP8 copy)
def _all_pairs_pool():
    """One page whose rows hold every (scale byte, nibble) pair: block j of row r has scale code
    sc = 32r + j (NaN codes 0x7F / 0xFF replaced by 0) and nibbles 0..15."""
    rows = []
    for r in range(8):
        row = np.zeros(352, np.uint8)
        for j in range(32):
            sc = 32 * r + j
            row[256 + j] = 0 if sc in (0x7F, 0xFF) else sc
            nib = np.arange(16, dtype=np.uint8)
            row[8 * j:8 * j + 8] = nib[0::2] | (nib[1::2] << 4)
        row[288:352] = np.arange(64, dtype=np.uint8) * 3 + r
        rows.append(row)
    pool = np.zeros(64 * 352, np.uint8)
    pool[:8 * 352] = np.concatenate(rows)
    return pool, rows


def test_stage_fp8_every_scale_and_nibble_vs_torch_cast():
    """Each staged latent byte is the E4M3 cast of the exact product e2m1 x scale: torch's float8_e4m3fn
    cast (nearest, ties to even) below 448, 448 with the product's sign at or above it."""
    pool, rows = _all_pairs_pool()
    idx = np.arange(8, dtype=np.int32).reshape(1, 1, 8)
    staged, counts = oracle.stage_nvfp4_fp8(pool, 64 * 352, 1, np.zeros((1, 1), np.int32), np.array([8], np.int32), idx)
    assert counts.tolist() == [8]
    checked = 0
    for r, row in enumerate(rows):
        got = staged[0, r, :512].astype(np.int64)
        for d in range(512):
            nib = (row[d // 2] >> (4 * (d & 1))) & 15
            sc = int(row[256 + d // 16])
            prod = minifloat(int(nib), 2, 1, 1) * minifloat(sc, 4, 3, 7)  # exact in double
            neg = bool(nib >> 3) != bool(sc >> 7)
            if abs(prod) < 448.0:
                ref = int(torch.tensor([prod], dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8)[0])
                # a zero product keeps the sign rule (nibble sign xor scale sign) where the cast of +-0 does not
                if prod == 0.0:
                    ref = 0x80 if neg else 0x00
            else:
                ref = 0x7E | (0x80 if neg else 0)
            assert got[d] == ref, (r, d, nib, sc, prod, got[d], ref)
            checked += 1
        assert np.array_equal(staged[0, r, 512:], row[288:352])  # rope bytes copied
    assert checked == 8 * 512


def test_stage_fp8_selection_order_and_counts():
    """The staged rows are the sparse decode's selection in list order (invalid entries skipped), and
    their dequantized values are the NVFP4 values rounded to E4M3 (within half an E4M3 step)."""
    cfg, lay, pool, q, idx, rng = _small_case(31, B=3, T=2, L=700, topk=128, causal=True)
    idx = idx.copy()
    idx[0, 0, :20] = -1
    idx[1, 1, 5:9] = 10 ** 6
    lay.block_table[2, 3] = lay.num_pages + 1
    staged, counts = oracle.stage_nvfp4_fp8(pool, cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx, idx,
                                            causal=True)
    assert staged.shape == (6, 128, 576)
    for b in range(3):
        for t in range(2):
            lim = W.position_limit(int(lay.ctx[b]), 2, t, True)
            sel = [p for p in idx[b, t] if 0 <= p <= lim and 0 <= lay.block_table[b, p // 64] < lay.num_pages]
            n = counts[b * 2 + t]
            assert n == len(sel)
            for j, p in enumerate(sel):
                src = _rows_of(cfg, lay, pool, b, [p])[0]
                K = _independent_K(src, "nvfp4")
                got = _independent_K(staged[b * 2 + t, j], "fp8")
                assert np.array_equal(got[512:], K[512:])
                err = np.abs(got[:512] - K[:512])
                assert np.all(err <= np.maximum(np.abs(K[:512]) * 2.0 ** -4, 2.0 ** -10)), (b, t, j)
            assert not staged[b * 2 + t, n:].any()


def test_staged_decode_close_to_native_decode():
    """FP8 attention over the staged copy (identity page table over the copy, one query token per
    request) approximates the native decode of the same selection: the copy only rounds values to E4M3."""
    cfg, lay, pool, q, idx, rng = _small_case(32, B=2, T=1, H=8, L=900, topk=256)
    staged, counts = oracle.stage_nvfp4_fp8(pool, cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx, idx)
    nq, R = staged.shape[:2]
    P = R // 64
    bt = (np.arange(nq)[:, None] * P + np.arange(P)[None, :]).astype(np.int32)
    o_st, l_st, _ = oracle.dense_decode_fp8(q.reshape(nq, 1, cfg.H, 576), staged.reshape(-1), 64 * 576, nq * P, bt,
                                            counts, cfg.sm_scale)
    o_na, l_na, _ = oracle.sparse_decode(q, pool, cfg.page_stride, lay.num_pages, lay.block_table, lay.ctx, idx,
                                         cfg.sm_scale)
    # Scores move by sm_scale * <q, K' - K> with |K' - K| <= 2^-4 |K| per value: a few hundredths
    # typically, a few tenths at the extremes of 2,048 scores.  A lost scale or sign moves both by O(1).
    rel = np.linalg.norm(o_st - o_na) / np.linalg.norm(o_na)
    assert 0 < rel < 0.05, rel
    assert np.abs(l_st - l_na).max() < 0.5


# --------------------------------------------------------------------------- index selection (top-k)
def test_topk_positions_brute_force_small():
    """Tiny rows with many ties, -0.0 next to +0.0 and infinities: the right count of positions, in
    ascending order, -1 after them, and no unchosen position beats a chosen one under the order
    (value, then lower position) -- with Python's float comparison, in which -0.0 equals 0.0."""
    rng = np.random.default_rng(50)
    for trial in range(200):
        m = int(rng.integers(0, 12))
        k = int(rng.integers(1, 8))
        # few distinct values, so that ties are common; some infinities
        vals = rng.choice(np.array([-np.inf, -1.0, -0.0, 0.0, 0.5, 2.0, np.inf], np.float32), size=max(m, 1))
        logits = np.zeros((1, 12), np.float32)
        logits[0, :m] = vals[:m]
        got = oracle.topk_positions(logits, [m], k)[0]
        chosen = [int(p) for p in got if p >= 0]
        assert len(chosen) == min(k, m)
        assert chosen == sorted(chosen)
        assert np.all(got[len(chosen):] == -1)
        rest = [p for p in range(m) if p not in chosen]
        for c in chosen:
            for o in rest:  # an unchosen position is never strictly better
                assert (vals[o], -o) < (vals[c], -c), (trial, c, o)


def test_topk_positions_properties():
    rng = np.random.default_rng(51)
    x = rng.standard_normal((3, 5000)).astype(np.float32)
    x[1, ::7] = 1.5  # a large tie block straddling the threshold
    lens = [5000, 4000, 100]
    got = oracle.topk_positions(x, lens, 2048)
    for r, m in enumerate(lens):
        sel = got[r][got[r] >= 0]
        assert sel.size == min(2048, m)
        assert np.all(np.diff(sel) > 0) and sel.max() < m
        thr = np.sort(x[r, :m])[::-1][min(2048, m) - 1]
        assert np.all(x[r, sel] >= thr)
        assert np.sum(x[r, :m] > thr) <= sel.size
        outside = np.setdiff1d(np.arange(m), sel)
        if outside.size:
            assert np.all(x[r, outside] <= thr)
            ties_in = sel[x[r, sel] == thr]
            ties_out = outside[x[r, outside] == thr]
            if ties_in.size and ties_out.size:
                assert ties_in.max() < ties_out.min()  # ties go to lower positions


# --------------------------------------------------------------------------- indexer keys and logits
def _bits(x):
    """bf16 bit patterns of values that bf16 holds exactly."""
    v = np.asarray(x, np.float32).view(np.uint32)
    assert np.all((v & 0xFFFF) == 0)
    return (v >> 16).astype(np.uint16)


def test_index_key_scale_and_codes():
    # amax 448 -> scale exactly 1: the values themselves are encoded; 1.0625 and 1.1875 sit halfway
    # between E4M3 neighbours and go to the even code (1.0 = 0x38, 1.25 = 0x3A)
    x = np.zeros(128, np.float32)
    x[:6] = [448.0, 1.0625, 1.1875, -3.0, -0.0, 0.0078125]
    codes, s = oracle.index_key_quant_row(_bits(x))
    assert s == 1.0
    # 448 = 1.75 * 2^8 (e 15, m 6); -3 = -1.5 * 2^1 (e 8, m 4); 2^-7 is the subnormal m = 4
    assert list(codes[:6]) == [0x7E, 0x38, 0x3A, 0xC4, 0x80, 0x04]
    assert all(c == 0 for c in codes[6:])
    # amax 3: scale is the fp32 quotient 3/448, the largest value maps to 448
    x = np.zeros(128, np.float32)
    x[7] = -3.0
    codes, s = oracle.index_key_quant_row(_bits(x))
    assert s == float(np.float32(3.0) / np.float32(448.0))
    assert codes[7] == 0xFE and all(c == 0 for i, c in enumerate(codes) if i != 7)
    # an all-zero key: the clamped scale, every code zero (the sign of -0 kept)
    x = np.zeros(128, np.float32)
    x[1] = -0.0
    codes, s = oracle.index_key_quant_row(_bits(x))
    assert s == float(np.float32(1e-26) / np.float32(448.0))
    assert codes[0] == 0 and codes[1] == 0x80


def test_index_key_round_trip():
    """Decoded values stay within half an E4M3 step of the quotient x / s (relative 1/16 for normal
    values, 2^-10 absolute below 2^-6), and the largest magnitude decodes to 448 * s."""
    rng = np.random.default_rng(60)
    for _ in range(50):
        x = (rng.standard_normal(128) * np.exp(rng.uniform(-8, 8))).astype(np.float32)
        xb = _bits((x.view(np.uint32) & 0xFFFF0000).view(np.float32))
        codes, s = oracle.index_key_quant_row(xb)
        xv = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        dec = np.array([oracle._load().mlo_e4m3_value(int(c)) for c in codes])
        y = xv / s
        err = np.abs(dec - y)
        assert np.all(err <= np.maximum(np.abs(y) / 16, 2.0 ** -10) * (1 + 1e-9))
        assert np.abs(dec).max() == 448.0


def _index_pool(keys_codes, scales, page_stride=oracle.INDEX_PAGE_BYTES):
    """A pool whose page i holds rows 64i.. of the given codes / scales (identity page table)."""
    n = keys_codes.shape[0]
    pages = (n + 63) // 64
    pool = np.zeros(pages * page_stride, np.uint8)
    for r in range(n):
        base = (r // 64) * page_stride
        pool[base + (r % 64) * 128: base + (r % 64) * 128 + 128] = keys_codes[r]
        pool[base + 8192 + (r % 64) * 4: base + 8192 + (r % 64) * 4 + 4] = np.frombuffer(np.float32(scales[r]).tobytes(), np.uint8)
    return pool, pages


def test_index_logits_closed_forms():
    # three keys: key 0 has code 0x38 (1.0) at dim 5, key 1 code 0xB8 (-1.0) at dim 5, key 2 code 0x40
    # (2.0) at dim 9; scales 0.5, 1, 4
    codes = np.zeros((3, 128), np.uint8)
    codes[0, 5], codes[1, 5], codes[2, 9] = 0x38, 0xB8, 0x40
    pool, pages = _index_pool(codes, [0.5, 1.0, 4.0])
    bt = np.arange(pages, dtype=np.int32)[None, :]
    q = np.zeros((1, 1, 2, 128), np.float32)
    q[0, 0, 0, 5] = 3.0   # head 0 looks at dim 5
    q[0, 0, 1, 9] = -1.0  # head 1 looks at dim 9 with a negative sign
    w = np.array([[[2.0, 5.0]]], np.float32)
    lg = oracle.index_logits(_bits(q), w, pool, oracle.INDEX_PAGE_BYTES, pages, bt, [3])
    # key 0: head 0 dot 3*1 = 3 -> 2*3 = 6, head 1 dot 0; times 0.5 -> 3
    # key 1: head 0 dot -3 -> ReLU 0; head 1 dot 0 -> 0
    # key 2: head 0 dot 0; head 1 dot -2 -> ReLU 0 -> 0
    assert list(lg[0]) == [3.0, 0.0, 0.0]
    q[0, 0, 1, 9] = 1.5   # now head 1 sees key 2: 1.5*2 = 3, weight 5 -> 15, scale 4 -> 60
    lg = oracle.index_logits(_bits(q), w, pool, oracle.INDEX_PAGE_BYTES, pages, bt, [3])
    assert list(lg[0]) == [3.0, 0.0, 60.0]
    # a negative weight can make a logit negative; the ReLU acts on the dot product, not on the sum
    w2 = np.array([[[2.0, -5.0]]], np.float32)
    lg = oracle.index_logits(_bits(q), w2, pool, oracle.INDEX_PAGE_BYTES, pages, bt, [3])
    assert list(lg[0]) == [3.0, 0.0, -60.0]


def test_index_logits_structure():
    """Linearity in the head weights, proportionality to the key scale, the causal limit and pages
    outside the pool, on random keys."""
    rng = np.random.default_rng(61)
    L, HI, T = 150, 4, 2
    keys = _bits((rng.standard_normal((L, 128)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32))
    pool = np.zeros(3 * oracle.INDEX_PAGE_BYTES, np.uint8)
    oracle.index_key_quant(keys, np.arange(L), pool, oracle.INDEX_PAGE_BYTES, 3)
    bt = np.array([[0, 1, 2]], np.int32)
    q = _bits((rng.standard_normal((1, T, HI, 128)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32))
    # multiples of 1/64 below 8 in magnitude: w1 + w2 is exact in fp32
    w1 = (np.round(rng.standard_normal((1, T, HI)) * 64) / 64).astype(np.float32)
    w2 = (np.round(rng.standard_normal((1, T, HI)) * 64) / 64).astype(np.float32)
    a = oracle.index_logits(q, w1, pool, oracle.INDEX_PAGE_BYTES, 3, bt, [L], causal=True)
    b = oracle.index_logits(q, w2, pool, oracle.INDEX_PAGE_BYTES, 3, bt, [L], causal=True)
    c = oracle.index_logits(q, w1 + w2, pool, oracle.INDEX_PAGE_BYTES, 3, bt, [L], causal=True)
    ok = ~np.isnan(c)
    assert np.allclose(c[ok], (a + b)[ok], rtol=1e-12, atol=1e-12)
    # causal: token 0 sees positions 0..L-2, token 1 sees 0..L-1
    assert np.isnan(a[0, L - 1]) and not np.isnan(a[1, L - 1]) and not np.isnan(a[0, L - 2])
    # doubling every scale doubles every logit
    pool2 = pool.copy()
    for pg in range(3):
        sc = pool2[pg * oracle.INDEX_PAGE_BYTES + 8192: pg * oracle.INDEX_PAGE_BYTES + 8448].view(np.float32)
        sc *= 2
    d = oracle.index_logits(q, w1, pool2, oracle.INDEX_PAGE_BYTES, 3, bt, [L], causal=True)
    assert np.array_equal(d[ok], 2 * a[ok])
    # a page entry outside the pool gives -inf for its 64 positions
    bt_bad = np.array([[0, 7, 2]], np.int32)
    e = oracle.index_logits(q, w1, pool, oracle.INDEX_PAGE_BYTES, 3, bt_bad, [L], causal=True)
    assert np.all(e[:, 64:128] == -np.inf) and np.array_equal(e[:, :64], a[:, :64])


# --------------------------------------------------------------------------- per-token-head FP8 layout
def _bf16_of(x):
    """bf16 bits of float32 values, nearest with ties to even, computed here independently."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_pth_write_closed_forms():
    lat = np.zeros(512, np.float32)
    lat[:3] = [448.0, -3.0, 1.0625]
    rope = np.zeros(64, np.float32)
    rope[:2] = [1.5, -2.0]
    codes, s, rq = oracle.pth_quant_row(_bits(lat), _bits(rope))
    assert s == 1.0  # amax 448
    assert list(codes[:3]) == [0x7E, 0xC4, 0x38] and not codes[3:].any()
    assert list(rq[:2]) == list(_bf16_of([1.5, -2.0])) and not rq[2:].any()
    # amax 3: the fp32 scale 3/448; the rope is the bf16 of the fp32 quotient r / s
    lat[:] = 0
    lat[9] = 3.0
    rope[:2] = [1.5, 0.1015625]
    codes, s, rq = oracle.pth_quant_row(_bits(lat), _bits(rope))
    s32 = np.float32(3.0) / np.float32(448.0)
    assert s == float(s32) and codes[9] == 0x7E
    assert list(rq[:2]) == list(_bf16_of(np.array([1.5, 0.1015625], np.float32) / s32))
    # a near-zero latent: the clamped scale, and a large rope part overflows bf16 to inf
    lat[:] = 0
    rope[:2] = [1.0, 2.0 ** 33]
    codes, s, rq = oracle.pth_quant_row(_bits(lat), _bits(rope))
    assert s == float(np.float32(1e-26) / np.float32(448.0))
    assert rq[0] == _bf16_of([np.float32(1.0) / np.float32(s)])[0] and rq[1] == 0x7F80


def test_pth_round_trip_and_single_row_decode():
    rng = np.random.default_rng(62)
    n = 3
    lat = _bits((rng.standard_normal((n, 512)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32))
    rope = _bits((rng.standard_normal((n, 64)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32))
    slots = 64
    lat_buf = np.zeros((slots, 512), np.uint8)
    sc_buf = np.zeros(slots, np.float32)
    rope_buf = np.zeros((slots, 64), np.uint16)
    assert oracle.kv_quant_pth(lat, rope, [5, 6, 7], lat_buf, sc_buf, rope_buf) == 3
    for r in range(n):
        K = oracle.dequant_row_pth(lat_buf[5 + r], sc_buf[5 + r], rope_buf[5 + r])
        x = (lat[r].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        y = (rope[r].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        s = float(sc_buf[5 + r])
        assert np.all(np.abs(K[:512] - x) <= np.maximum(np.abs(x) / 16, 2.0 ** -10 * s) * (1 + 1e-6))
        assert np.all(np.abs(K[512:] - y) <= np.abs(y) * 2.0 ** -8 * (1 + 1e-6))
    # one selected row: the output is that row's latent exactly and lse is its score; the row twice: same
    # output, lse + ln 2
    q = _bits((rng.standard_normal((1, 1, 16, 576)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32))
    bt = np.array([[0]], np.int32)
    K = oracle.dequant_row_pth(lat_buf[6], sc_buf[6], rope_buf[6])
    qv = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[0, 0]
    for idx, extra in (([6, -1], 0.0), ([6, 6], math.log(2.0))):
        out, lse, _ = oracle.sparse_decode_pth(q, lat_buf, sc_buf, rope_buf, bt, [64], np.array([[idx]], np.int32), 0.1)
        assert np.allclose(out[0, 0], np.broadcast_to(K[:512], (16, 512)), rtol=1e-14, atol=0)
        assert np.allclose(lse[0, 0], 0.1 * (qv @ K) + extra, rtol=1e-12, atol=1e-12)
