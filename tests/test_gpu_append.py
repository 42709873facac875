"""GPU parity of the fused decode step (mla_sparse_decode_append): each request's T new rows written into
the cache and the sparse decode over the cache with them, in one launch.

Against the two-launch path (mla_kv_quant_nvfp4 of the new rows, then mla_sparse_decode) the pool bytes,
the outputs and the lse must match bit for bit (the same kernels' arithmetic on the same bytes); against
the FP64 oracle the outputs meet the tolerances in cases.py."""
import sys

import numpy as np
import pytest

import workloads as W
from cases import Case, bf16_to_np, compare_outputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import nvfp4_compressed_sparse_amd as M  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cfg(B=2, T=1, H=16, topk=256, L=4096, causal=False, seed=31):
    return W.DecodeConfig("append", B=B, T=T, H=H, topk=topk, fmt="nvfp4", ctx=L, causal=causal, seed=seed)


def split_rows(case, ctx, bt):
    """The rows of positions ctx[b] - T + t as the new-row inputs [B*T, 512] / [B*T, 64] (random rows for
    positions before 0, which are not written), and the slots of every source row under table bt, with
    the new rows' slots set to -1 (the cache as it stands before the step)."""
    c = case.cfg
    knope = np.zeros((c.B * c.T, 512), np.uint16)
    krope = np.zeros((c.B * c.T, 64), np.uint16)
    rng = np.random.default_rng(c.seed + 99)
    fill_n, fill_r = W.gen_latent_rope(rng, c.B * c.T)
    full_slots = np.empty(case.slots.size, np.int64)
    old_slots = np.empty(case.slots.size, np.int64)
    start = 0
    for b in range(c.B):
        n = int(case.lay.ctx[b])
        pos = np.arange(n)
        col = pos // 64
        pg = np.where(col < bt.shape[1], bt[b, np.minimum(col, bt.shape[1] - 1)], -1).astype(np.int64)
        sl = np.where(pg >= 0, pg * 64 + pos % 64, -1)
        full_slots[start:start + n] = sl
        keep = pos < int(ctx[b]) - c.T
        old_slots[start:start + n] = np.where(keep, sl, -1)
        for t in range(c.T):
            p = int(ctx[b]) - c.T + t
            r = b * c.T + t
            if 0 <= p < n:
                knope[r], krope[r] = case.lat[start + p], case.rope[start + p]
            else:
                knope[r], krope[r] = fill_n[r], fill_r[r]
        start += n
    return knope, krope, full_slots, old_slots


def dev_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def quant(d, slots, pool, case):
    s = torch.from_numpy(slots).cuda()
    M.mla_kv_quant_nvfp4(d["lat"], d["rope"], s, pool, case.cfg.page_stride, case.lay.num_pages)


def two_launch(case, d, bt_dev, ctx_dev, idx_dev, full_slots, num_splits):
    c = case.cfg
    pool = torch.zeros(case.pool_bytes, dtype=torch.uint8, device="cuda")
    quant(d, full_slots, pool, case)
    lse = torch.empty((c.B, c.T, c.H), dtype=torch.float32, device="cuda")
    out, _ = M.mla_sparse_decode(d["q"], pool, c.page_stride, case.lay.num_pages, bt_dev, ctx_dev, idx_dev,
                                 c.sm_scale, causal=c.causal, num_splits=num_splits, lse=lse)
    torch.cuda.synchronize()
    return pool, out, lse


def poison_new_rows(case, pool, ctx, bt):
    """Fill the bytes where the step's new rows go with 0xFF (an E4M3 NaN in every scale and rope byte),
    so that a read of a new row that does not see the step's own row shows up in the outputs."""
    c = case.cfg
    offs = []
    for b in range(c.B):
        for t in range(c.T):
            p = int(ctx[b]) - c.T + t
            if p < 0 or p // 64 >= bt.shape[1] or bt[b, p // 64] < 0:
                continue
            offs.append(int(bt[b, p // 64]) * c.page_stride + (p % 64) * c.row_bytes)
    if offs:
        o = torch.tensor(offs, dtype=torch.int64, device="cuda")
        pool[(o[:, None] + torch.arange(c.row_bytes, device="cuda")[None, :]).reshape(-1)] = 255


def fused(case, d, bt_dev, ctx_dev, idx_dev, old_slots, knope, krope, num_splits, pool=None, poison=None):
    c = case.cfg
    if pool is None:
        pool = torch.zeros(case.pool_bytes, dtype=torch.uint8, device="cuda")
        quant(d, old_slots, pool, case)
    if poison is not None:
        poison_new_rows(case, pool, *poison)
    lse = torch.empty((c.B, c.T, c.H), dtype=torch.float32, device="cuda")
    out, _ = M.mla_sparse_decode_append(d["q"], pool, c.page_stride, case.lay.num_pages, bt_dev, ctx_dev, idx_dev,
                                        dev_bf16(knope), dev_bf16(krope), c.sm_scale, causal=c.causal,
                                        num_splits=num_splits, lse=lse)
    torch.cuda.synchronize()
    return pool, out, lse


def with_new_rows_selected(case):
    """Indices where every query token selects the request's T newest positions (the rows the step
    writes), the rest as generated."""
    c = case.cfg
    idx = case.idx.copy()
    for b in range(c.B):
        L = int(case.lay.ctx[b])
        newest = np.arange(max(L - c.T, 0), L, dtype=np.int32)
        for t in range(c.T):
            row = idx[b, t]
            row = row[~np.isin(row, newest)]
            keep = np.concatenate([newest, row])[: c.topk]
            idx[b, t, :] = -1
            idx[b, t, : keep.size] = keep
    return idx


def check_equal(name, a, b):
    a = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32 if a.dtype == torch.float32 else a.dtype)
    b = b.view(a.dtype)
    bad = (a != b).nonzero()
    assert bad.numel() == 0, f"{name}: {bad.shape[0]} elements differ, first at {bad[:4].tolist()}"


CASES = [
    # (B, T, H, topk, causal, splits)
    (2, 1, 16, 256, False, 0),
    (2, 1, 16, 200, False, 3),  # partial last steps: their padding rows read a new row
    (2, 2, 32, 200, True, 0),
    (3, 1, 16, 2048, False, 3),
    (2, 4, 16, 256, True, 0),
    (2, 4, 32, 512, True, 2),
    (2, 10, 16, 256, True, 0),  # more new rows than the workgroup has waves
    (2, 1, 64, 256, False, 0),
    (2, 4, 128, 256, True, 2),
    (1, 6, 128, 512, True, 0),  # 128 heads: four head groups of one token write the same rows
    (32, 4, 128, 256, True, 1),  # 256 workgroups of 64 heads: the 64-head workgroup writes and decodes
]


@pytest.mark.parametrize("B,T,H,topk,causal,splits", CASES)
def test_append_matches_two_launches_and_oracle(B, T, H, topk, causal, splits):
    case = Case(cfg(B=B, T=T, H=H, topk=topk, L=3000, causal=causal, seed=40 + T + H))
    case.idx = with_new_rows_selected(case)
    bt = case.lay.block_table
    knope, krope, full_slots, old_slots = split_rows(case, case.lay.ctx, bt)
    say(f"append B={B} T={T} H={H} topk={topk} causal={causal} splits={splits}")
    d = case.to_device()
    p2, o2, l2 = two_launch(case, d, d["bt"], d["ctx"], d["idx"], full_slots, splits)
    p1, o1, l1 = fused(case, d, d["bt"], d["ctx"], d["idx"], old_slots, knope, krope, splits,
                       poison=(case.lay.ctx, bt))
    check_equal("pool", p1, p2)
    check_equal("out", o1, o2)
    check_equal("lse", l1, l2)
    assert np.array_equal(p1.cpu().numpy(), case.oracle_pool()), "pool differs from the oracle's writer"
    ref_o, ref_l = case.oracle_decode()
    say(compare_outputs(bf16_to_np(o1).reshape(B * T, H, 512), ref_o, l1.cpu().numpy().astype(np.float64)
                        .reshape(B * T, H), ref_l, f"append H={H} T={T}", vmax=case.vmax()))


@pytest.mark.parametrize("H", [16, 128])
def test_append_edges(H):
    """A context shorter than T (positions before 0 are not written), new positions on a page whose table
    entry is -1 and on a page beyond the table width (both skipped, as the writer skips such slots)."""
    import oracle
    T = 4
    ctx = np.array([2, 400, 450], np.int32)
    case = Case(cfg(B=3, T=T, H=H, topk=256, causal=True, seed=51), ctx=ctx)
    bt = case.lay.block_table.copy()  # 8 columns: request 2 needs them all
    bt[1, (400 - 1) // 64] = -1  # request 1's newest rows land on an unmapped page
    narrow = np.ascontiguousarray(bt[:, :7])  # request 2's positions 448, 449 lie beyond the table width
    case.idx = with_new_rows_selected(case)
    knope, krope, full_slots, old_slots = split_rows(case, ctx, narrow)
    say(f"append edges H={H}: ctx={ctx.tolist()} table {narrow.shape}")
    d = case.to_device()
    bt_dev = torch.from_numpy(narrow).cuda()
    p2, o2, l2 = two_launch(case, d, bt_dev, d["ctx"], d["idx"], full_slots, 0)
    p1, o1, l1 = fused(case, d, bt_dev, d["ctx"], d["idx"], old_slots, knope, krope, 0, poison=(ctx, narrow))
    check_equal("pool", p1, p2)
    check_equal("out", o1, o2)
    check_equal("lse", l1, l2)
    ref = np.zeros(case.pool_bytes, np.uint8)
    oracle.kv_quant("nvfp4", case.lat, case.rope, full_slots, ref, case.cfg.page_stride, case.lay.num_pages)
    assert np.array_equal(p1.cpu().numpy(), ref), "pool differs from the oracle's writer"
    assert not np.isfinite(l1.cpu().numpy()[0, :2]).any(), "positions before 0 selected"


def test_append_two_steps():
    """Two decode steps in a row on one pool (the context grows by T between them): after both, the pool
    equals the oracle's writer over the whole context, and the second step's outputs match the oracle."""
    T, H = 2, 32
    case = Case(cfg(B=3, T=T, H=H, topk=512, L=2000, causal=True, seed=61))
    c = case.cfg
    ctx = case.lay.ctx
    bt = case.lay.block_table
    d = case.to_device()
    # step 1: context ctx - T, its new rows are positions ctx - 2T .. ctx - T - 1
    ctx1 = ctx - T
    kn1, kr1, _, slots0 = split_rows(case, ctx1, bt)
    rng = np.random.default_rng(5)
    idx1 = W.gen_indices(rng, ctx1, T, c.topk, True)
    pool = torch.zeros(case.pool_bytes, dtype=torch.uint8, device="cuda")
    quant(d, slots0, pool, case)
    say("append two steps: step 1")
    _, o1, _ = fused(case, d, d["bt"], torch.from_numpy(ctx1).cuda(), torch.from_numpy(idx1).cuda(), None, kn1, kr1,
                     0, pool=pool)
    ref1, _ = case_oracle_at(case, ctx1, idx1)
    say(compare_outputs(bf16_to_np(o1).reshape(c.B * T, H, 512), ref1, what="step 1", vmax=case.vmax(idx1, ctx1)))
    say("append two steps: step 2")
    case.idx = with_new_rows_selected(case)
    kn2, kr2, _, _ = split_rows(case, ctx, bt)
    _, o2, l2 = fused(case, d, d["bt"], d["ctx"], torch.from_numpy(case.idx).cuda(), None, kn2, kr2, 0, pool=pool)
    assert np.array_equal(pool.cpu().numpy(), case.oracle_pool()), "pool after two steps differs from the oracle's"
    ref_o, ref_l = case.oracle_decode()
    say(compare_outputs(bf16_to_np(o2).reshape(c.B * T, H, 512), ref_o, l2.cpu().numpy().astype(np.float64)
                        .reshape(c.B * T, H), ref_l, "step 2", vmax=case.vmax()))


def case_oracle_at(case, ctx, idx):
    """The oracle's decode with context lengths ctx and indices idx over the full pool (the rows beyond
    ctx are never selected: every index is at most the causal limit under ctx)."""
    import oracle
    c = case.cfg
    return oracle.sparse_decode(case.q, case.oracle_pool(), c.page_stride, case.lay.num_pages, case.lay.block_table,
                                ctx, idx, c.sm_scale, c.causal, fmt=c.fmt)[:2]


@pytest.mark.parametrize("name", ["sparse", "spec", "pages15", "short35"])
def test_full_size_fused_step_sampled(name):
    """The fused step at the full sizes bench.py times it (one mla_sparse_decode_append launch with the
    library's split choice): the cache holds every row but the step's new ones, whose slots are poisoned;
    after the call every new row is bit-exact against the oracle's writer, and sampled query tokens,
    which select their request's newest positions, match the oracle."""
    import oracle
    from cases import sampled_oracle
    cfg = W.CONFIGS[name]
    say(f"full-size fused {name}: generating inputs")
    inp = W.device_inputs(cfg, "cuda", n_sets=1)
    lay = inp["layout"]
    T = cfg.T
    rows = np.concatenate([inp["row_off"][b] + lay.ctx[b] - T + np.arange(T) for b in range(cfg.B)]).astype(np.int64)
    rows_d = torch.from_numpy(rows).cuda()
    old = inp["slots"].clone()
    old[rows_d] = -1
    pool = torch.zeros(lay.num_pages * cfg.page_stride, dtype=torch.uint8, device="cuda")
    inp["pool"] = pool
    M.mla_kv_quant_nvfp4(inp["lat"], inp["rope"], old, pool, cfg.page_stride, lay.num_pages)
    new_slots = inp["slots"][rows_d].cpu().numpy()
    offs = (new_slots // 64) * cfg.page_stride + (new_slots % 64) * cfg.row_bytes
    gidx = torch.from_numpy((offs[:, None] + np.arange(cfg.row_bytes)[None, :]).reshape(-1)).cuda()
    pool[gidx] = 255
    # every query token selects its request's newest positions first
    idx = inp["idx_sets"][0].cpu().numpy()
    for b in range(cfg.B):
        newest = np.arange(int(lay.ctx[b]) - T, int(lay.ctx[b]), dtype=np.int32)
        for t in range(T):
            r = idx[b, t]
            r = r[~np.isin(r, newest)]
            keep = np.concatenate([newest, r])[: cfg.topk]
            idx[b, t, :] = -1
            idx[b, t, : keep.size] = keep
    idx_d = torch.from_numpy(idx).cuda()
    q = inp["q_sets"][0]
    lse = torch.empty((cfg.B, T, cfg.H), dtype=torch.float32, device="cuda")
    say(f"full-size fused {name}: decode")
    out, _ = M.mla_sparse_decode_append(q, pool, cfg.page_stride, lay.num_pages, inp["bt"], inp["ctx"], idx_d,
                                        inp["lat"][rows_d].contiguous(), inp["rope"][rows_d].contiguous(),
                                        cfg.sm_scale, causal=cfg.causal, lse=lse)
    torch.cuda.synchronize()
    grows = pool[gidx].cpu().numpy().reshape(-1, cfg.row_bytes)
    lat = inp["lat"][rows_d].view(torch.int16).cpu().numpy().view(np.uint16)
    rope = inp["rope"][rows_d].view(torch.int16).cpu().numpy().view(np.uint16)
    for r in range(rows.size):
        assert np.array_equal(grows[r], oracle.quant_row_nvfp4(lat[r], rope[r])), f"new row {r} differs"
    nq = cfg.B * T
    qtoks = sorted(set([0, nq - 1] + list(np.random.default_rng(cfg.seed + 7).choice(nq, min(6, nq), replace=False))))
    say(f"full-size fused {name}: oracle on query tokens {qtoks}")
    ro, rl, vm, pools_ok = sampled_oracle(cfg, inp, qtoks, idx_d, q)
    assert pools_ok, "pool rows differ from the oracle's quantization"
    g = bf16_to_np(out).reshape(nq, cfg.H, 512)[qtoks]
    gl = lse.cpu().numpy().astype(np.float64).reshape(nq, cfg.H)[qtoks]
    say(compare_outputs(g, ro, gl, rl, f"full-size fused {name}", vmax=vm))
    del inp, pool
    torch.cuda.empty_cache()
