"""GPU parity of the sparse-indexer keys and logits (through the C ABI) against the oracle.

Keys must match byte for byte.  The logits' definition is a reading (parity unpinned against the pages);
the GPU must match the oracle's value of it within the fp32 accumulation bound stated below."""
import sys

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import nvfp4_compressed_sparse_amd as M  # noqa: E402

PS = M.INDEX_PAGE_BYTES


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def bf16_dev(bits):
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def build_pool(rng, ctx, layout_seed=0, extra_pages=2):
    """An indexer pool holding N(0,1) keys for every position of every request, written by the GPU and
    by the oracle; returns (gpu pool, oracle pool, block table, num_pages)."""
    cfg = W.DecodeConfig("ix", B=len(ctx), T=1, H=16, topk=64, fmt="nvfp4", ctx=0, ctx_range=(1, 2), seed=layout_seed)
    lay = W.gen_layout(cfg, rng, np.asarray(ctx, np.int32))
    num_pages = lay.num_pages + extra_pages
    slots = np.concatenate([W.slots_for_request(lay, b, np.arange(ctx[b])) for b in range(len(ctx))])
    keys = W.gen_index_keys(rng, slots.size)
    pool_o = np.zeros(num_pages * PS, np.uint8)
    oracle.index_key_quant(keys, slots, pool_o, PS, num_pages)
    pool_g = torch.zeros(num_pages * PS, dtype=torch.uint8, device="cuda")
    M.mla_index_key_quant(bf16_dev(keys), dev(slots.astype(np.int64)), pool_g, PS, num_pages)
    torch.cuda.synchronize()
    return pool_g, pool_o, lay.block_table, num_pages


def test_index_key_quant_bit_exact():
    rng = np.random.default_rng(80)
    n = 1000
    x = rng.standard_normal((n, 128)).astype(np.float32) * np.exp(rng.uniform(-30, 30, (n, 1))).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2, :] = 0.0
    x[2, 5] = 448.0
    x[3] = np.float32(1e-30)  # below the clamp: the clamped scale
    keys = W.bf16_bits(x)
    slots = rng.permutation(n + 100)[:n].astype(np.int64)
    slots[7] = -1
    num_pages = (n + 100 + 63) // 64
    pool_o = np.zeros(num_pages * PS, np.uint8)
    oracle.index_key_quant(keys, slots, pool_o, PS, num_pages)
    pool_g = torch.zeros(num_pages * PS, dtype=torch.uint8, device="cuda")
    M.mla_index_key_quant(bf16_dev(keys), dev(slots), pool_g, PS, num_pages)
    torch.cuda.synchronize()
    assert np.array_equal(pool_g.cpu().numpy(), pool_o)


def logit_bound(q, w, pool_o, bt, ctx, T, causal):
    """Per-position bound for fp32 accumulation: s_p * sum_j |w_j| * sum_d |q_jd k_pd| * 2^-16 (the
    products are exact; 128 + 64 fp32 additions stay below 2^-16 relative to the sum of magnitudes)."""
    absq = np.abs(W.bf16_to_f32(q).astype(np.float64))
    B, _, HI, _ = q.shape
    lut = np.array([abs(oracle._load().mlo_e4m3_value(c)) for c in range(256)])
    out = np.zeros((B * T, int(max(ctx))))
    for b in range(B):
        L = int(ctx[b])
        pos = np.arange(L)
        pages = bt[b, pos // 64].astype(np.int64)
        rows = pages * PS + (pos % 64) * 128
        kabs = lut[pool_o[rows[:, None] + np.arange(128)[None, :]]]  # [L, 128]
        sidx = pages * PS + 8192 + (pos % 64) * 4
        scales = np.ascontiguousarray(pool_o[sidx[:, None] + np.arange(4)[None, :]]).view(np.float32)[:, 0]
        scales = scales.astype(np.float64)
        for t in range(T):
            mag = (np.abs(w[b, t]).astype(np.float64)[:, None] * (absq[b, t] @ kabs.T)).sum(0)  # [L]
            out[b * T + t, :L] = scales * mag * 2.0 ** -16
    return out


@pytest.mark.parametrize("HI,T,causal", [(16, 1, False), (32, 2, True), (64, 1, False), (64, 3, True)])
def test_index_logits_match_oracle(HI, T, causal):
    say(f"index logits HI={HI} T={T} causal={causal}")
    rng = np.random.default_rng(81 + HI + T)
    ctx = np.array([1, 63, 64, 65, 700, 1000], np.int32)
    pool_g, pool_o, bt, num_pages = build_pool(rng, ctx)
    B = ctx.size
    q, w = W.gen_index_query(rng, B, T, HI)
    maxc = int(ctx.max())
    ref = oracle.index_logits(q, w, pool_o, PS, num_pages, bt, ctx, causal=causal, ld=maxc)
    out = torch.full((B * T, (maxc + 3) // 4 * 4), 12345.0, dtype=torch.float32, device="cuda")
    M.mla_index_logits(bf16_dev(q), dev(w), pool_g, PS, num_pages, dev(bt), dev(ctx), maxc, causal=causal, out=out)
    got = out.cpu().numpy()[:, :maxc].astype(np.float64)
    defined = ~np.isnan(ref)
    assert np.all(got[~defined] == 12345.0)  # positions past each query token's limit are not written
    bound = logit_bound(q, w, pool_o, bt, ctx, T, causal)
    err = np.abs(got[defined] - ref[defined])
    assert np.all(err <= bound[defined] + 1e-30), float((err / (bound[defined] + 1e-30)).max())


def test_index_logits_page_outside_pool():
    rng = np.random.default_rng(90)
    ctx = np.array([300, 200], np.int32)
    pool_g, pool_o, bt, num_pages = build_pool(rng, ctx)
    bt = bt.copy()
    bt[0, 1] = num_pages + 5  # positions 64..127 of request 0 on a page outside the pool
    bt[1, 2] = -3
    q, w = W.gen_index_query(rng, 2, 1, 32)
    ref = oracle.index_logits(q, w, pool_o, PS, num_pages, bt, ctx, ld=300)
    out = M.mla_index_logits(bf16_dev(q), dev(w), pool_g, PS, num_pages, dev(bt), dev(ctx), 300)
    got = out.cpu().numpy()
    assert np.all(got[0, 64:128] == -np.inf) and np.all(ref[0, 64:128] == -np.inf)
    assert np.all(got[1, 128:192] == -np.inf)
    ok = np.isfinite(ref)
    assert np.allclose(got[ok], ref[ok], rtol=1e-4, atol=1e-6)


def test_indexer_logits_then_topk():
    """Logits into the top-k: the GPU's 2,048 positions are those of the oracle's ranking up to values
    within the logits' accuracy (each chosen position's oracle logit is at least the oracle's k-th
    largest minus the bound, and each position left out is at most it plus the bound)."""
    rng = np.random.default_rng(91)
    ctx = np.array([1500, 5000, 9000], np.int32)
    pool_g, pool_o, bt, num_pages = build_pool(rng, ctx)
    q, w = W.gen_index_query(rng, 3, 1, 64)
    maxc = int(ctx.max())
    ref = oracle.index_logits(q, w, pool_o, PS, num_pages, bt, ctx, ld=maxc)
    lg = M.mla_index_logits(bf16_dev(q), dev(w), pool_g, PS, num_pages, dev(bt), dev(ctx), maxc)
    sel = M.mla_index_topk(lg, dev(ctx), 2048).cpu().numpy()
    bound = logit_bound(q, w, pool_o, bt, ctx, 1, False)
    for r in range(3):
        L = int(ctx[r])
        chosen = sel[r][sel[r] >= 0]
        assert chosen.size == min(L, 2048) and np.all(np.diff(chosen) > 0)
        if L <= 2048:
            assert np.array_equal(chosen, np.arange(L))
            continue
        kth = np.sort(ref[r, :L])[::-1][2047]
        tol = 2 * bound[r, :L].max()
        assert np.all(ref[r, chosen] >= kth - tol)
        out_pos = np.setdiff1d(np.arange(L), chosen)
        assert np.all(ref[r, out_pos] <= kth + tol)


def test_index_logits_full_size_sampled():
    """The decode workload's shape (64 requests x 140,000 positions, 64 index heads), in the launch the
    bench times; query tokens 0 and 37 checked against the oracle over their whole contexts."""
    cfg = W.CONFIGS["sparse"]
    say("index logits full size 64 x 140000")
    rng = np.random.default_rng(cfg.seed)
    lay = W.gen_layout(cfg, rng)
    pool = torch.zeros(lay.num_pages * PS, dtype=torch.uint8, device="cuda")
    keys_host = {}
    for b in range(cfg.B):
        L = int(lay.ctx[b])
        keys = W.gen_index_keys(rng, L) if b in (0, 37) else None
        if keys is None:
            kd = torch.randn((L, 128), device="cuda").to(torch.bfloat16)
        else:
            kd = bf16_dev(keys)
            keys_host[b] = keys
        M.mla_index_key_quant(kd, dev(W.slots_for_request(lay, b, np.arange(L)).astype(np.int64)), pool, PS,
                              lay.num_pages)
    q, w = W.gen_index_query(rng, cfg.B, 1, 64)
    maxc = int(lay.ctx.max())
    out = M.mla_index_logits(bf16_dev(q), dev(w), pool, PS, lay.num_pages, dev(lay.block_table), dev(lay.ctx), maxc)
    got = out.cpu().numpy()
    for b in (0, 37):
        L = int(lay.ctx[b])
        pool_o = np.zeros(((L + 63) // 64) * PS, np.uint8)
        oracle.index_key_quant(keys_host[b], np.arange(L), pool_o, PS, (L + 63) // 64)
        bt1 = np.arange((L + 63) // 64, dtype=np.int32)[None, :]
        ref = oracle.index_logits(q[b:b + 1], w[b:b + 1], pool_o, PS, (L + 63) // 64, bt1, [L], ld=L)
        bound = logit_bound(q[b:b + 1], w[b:b + 1], pool_o, bt1, [L], 1, False)
        err = np.abs(got[b, :L] - ref[0])
        assert np.all(err <= bound[0] + 1e-30), (b, float((err / (bound[0] + 1e-30)).max()))
