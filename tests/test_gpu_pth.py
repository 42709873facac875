"""GPU parity of TokenSpeed's per-token-head FP8 layout (writer bit-exact, sparse decode within the
attention tolerances of cases.py) through the C ABI, against the oracle."""
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from cases import Case, bf16_to_np, compare_outputs, selected_positions

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import nvfp4_compressed_sparse_amd as M  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def bf16_dev(bits):
    return dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def pth_buffers(case):
    """The case's rows written by the GPU and by the oracle: (gpu lat, scale, rope), (oracle ...)."""
    slots = case.lay.num_pages * 64
    lat_o = np.zeros((slots, 512), np.uint8)
    sc_o = np.zeros(slots, np.float32)
    rope_o = np.zeros((slots, 64), np.uint16)
    oracle.kv_quant_pth(case.lat, case.rope, case.slots, lat_o, sc_o, rope_o)
    lat_g = torch.zeros((slots, 512), dtype=torch.uint8, device="cuda")
    sc_g = torch.zeros(slots, dtype=torch.float32, device="cuda")
    rope_g = torch.zeros((slots, 64), dtype=torch.bfloat16, device="cuda")
    M.mla_kv_quant_pth(bf16_dev(case.lat), bf16_dev(case.rope), dev(case.slots), lat_g, sc_g, rope_g)
    torch.cuda.synchronize()
    return (lat_g, sc_g, rope_g), (lat_o, sc_o, rope_o)


def pth_vmax(case, lat_o, sc_o, idx=None):
    """Largest |V| = |code value * scale| per query token and column among its selected slots:
    [B, T, 1, 512]."""
    c = case.cfg
    e4 = np.array([oracle.e4m3_value(x) for x in range(256)])
    idx = case.idx if idx is None else idx
    out = np.zeros((c.B, c.T, 1, 512))
    num_pages = lat_o.shape[0] // 64
    for b in range(c.B):
        for t in range(c.T):
            pos = selected_positions(case.lay.ctx, c.T, c.causal, idx, b, t, case.lay.block_table, num_pages)
            if pos.size:
                slots = case.lay.block_table[b, pos // 64].astype(np.int64) * 64 + pos % 64
                out[b, t, 0] = np.abs(e4[lat_o[slots]] * sc_o[slots].astype(np.float64)[:, None]).max(0)
    return out


def small(B=2, T=1, H=16, topk=256, L=4096, causal=False, seed=7):
    return W.DecodeConfig("p", B=B, T=T, H=H, topk=topk, fmt="fp8", ctx=L, causal=causal, seed=seed)


def test_pth_write_bit_exact():
    rng = np.random.default_rng(95)
    n, slots = 700, 1024
    lat = W.bf16_bits((rng.standard_normal((n, 512)) * np.exp(rng.uniform(-20, 20, (n, 1)))).astype(np.float32))
    rope = W.bf16_bits((rng.standard_normal((n, 64)) * np.exp(rng.uniform(-20, 20, (n, 1)))).astype(np.float32))
    lat[0] = 0
    lat[1] = 0x8000  # -0
    rope[0, :4] = W.bf16_bits(np.array([1.0, 2.0 ** 33, -2.0 ** 33, -0.0], np.float32))  # inf from a tiny scale
    sm = rng.permutation(slots)[:n].astype(np.int64)
    sm[5] = -1
    sm[6] = slots + 3
    lat_o = np.zeros((slots, 512), np.uint8)
    sc_o = np.zeros(slots, np.float32)
    rope_o = np.zeros((slots, 64), np.uint16)
    oracle.kv_quant_pth(lat, rope, sm, lat_o, sc_o, rope_o)
    lat_g = torch.zeros((slots, 512), dtype=torch.uint8, device="cuda")
    sc_g = torch.zeros(slots, dtype=torch.float32, device="cuda")
    rope_g = torch.zeros((slots, 64), dtype=torch.bfloat16, device="cuda")
    M.mla_kv_quant_pth(bf16_dev(lat), bf16_dev(rope), dev(sm), lat_g, sc_g, rope_g)
    torch.cuda.synchronize()
    assert np.array_equal(lat_g.cpu().numpy(), lat_o)
    assert np.array_equal(sc_g.cpu().numpy().view(np.uint32), sc_o.view(np.uint32))
    assert np.array_equal(rope_g.view(torch.int16).cpu().numpy().view(np.uint16), rope_o)


def run_case(case, num_splits=0, idx=None, q=None, sm_scale=None, buffers=None, raw=False):
    (lat_g, sc_g, rope_g), (lat_o, sc_o, rope_o) = pth_buffers(case) if buffers is None else buffers
    c = case.cfg
    idx = case.idx if idx is None else idx
    q = case.q if q is None else q
    sm = c.sm_scale if sm_scale is None else sm_scale
    out, lse = M.mla_sparse_decode_pth(bf16_dev(q), lat_g, sc_g, rope_g, dev(case.lay.block_table),
                                       dev(case.lay.ctx), dev(idx), sm, causal=c.causal, num_splits=num_splits)
    torch.cuda.synchronize()
    g = bf16_to_np(out)
    if raw:
        return g, lse.cpu().numpy()
    ro, rl, _ = oracle.sparse_decode_pth(q, lat_o, sc_o, rope_o, case.lay.block_table, case.lay.ctx, idx, sm,
                                         c.causal)
    return compare_outputs(g, ro, lse.cpu().numpy(), rl, "pth", vmax=pth_vmax(case, lat_o, sc_o, idx))


@pytest.mark.parametrize("H", [16, 128])
def test_pth_query_times_power_of_two_gives_identical_results(H):
    """As for the NVFP4 decode: q * 2^k with sm_scale * 2^-k, k far outside FP16's range, gives bit-identical
    outputs (each head's query is normalised by a power of two), which match the oracle."""
    case = Case(small(B=2, H=H, topk=300, L=1500, seed=97 + H))
    bufs = pth_buffers(case)
    say(run_case(case, num_splits=1, buffers=bufs))
    for S in (1, 2):
        base = run_case(case, num_splits=S, buffers=bufs, raw=True)
        for k in (-100, -30, 30, 100):
            x = W.bf16_to_f32(case.q).astype(np.float64) * 2.0 ** k
            qk = W.bf16_bits(x.astype(np.float32))
            assert np.array_equal(W.bf16_to_f32(qk).astype(np.float64), x)
            got = run_case(case, num_splits=S, q=qk, sm_scale=case.cfg.sm_scale * 2.0 ** -k, buffers=bufs, raw=True)
            assert np.array_equal(got[0], base[0]) and np.array_equal(got[1], base[1]), f"k={k} S={S}"


def test_pth_query_outside_fp16_range_matches_oracle():
    """A 1e5 spike among N(0,1) values and whole heads at 1e30 or 1e-30, with sm_scale setting the scores to
    order one (one scale per run, checked on the heads it fits)."""
    case = Case(small(B=2, H=16, topk=256, L=1200, seed=99))
    bufs = pth_buffers(case)
    rng = np.random.default_rng(98)
    q = W.bf16_to_f32(case.q).astype(np.float64)
    g = np.arange(16) % 3
    for b in range(2):
        for h in np.nonzero(g == 0)[0]:
            q[b, 0, h, rng.integers(0, 512)] = 1.0e5
    q[:, :, g == 1, :] *= 1.0e30
    q[:, :, g == 2, :] *= 1.0e-30
    qbits = W.bf16_bits(q.astype(np.float32))
    for grp, sm in ((0, 1.0e-5), (1, 1.0 / 2.4e31), (2, 1.0 / 2.4e-29)):
        out, lse = run_case(case, num_splits=0, q=qbits, sm_scale=sm, buffers=bufs, raw=True)
        ro, rl, _ = oracle.sparse_decode_pth(qbits, bufs[1][0], bufs[1][1], bufs[1][2], case.lay.block_table,
                                             case.lay.ctx, case.idx, sm)
        sel = g == grp
        assert np.isfinite(out[:, :, sel]).all()  # other groups' scores may leave fp32's range at this scale
        say(compare_outputs(out[:, :, sel], ro[:, :, sel], lse[:, :, sel], rl[:, :, sel], f"pth group {grp}",
                            vmax=pth_vmax(case, bufs[1][0], bufs[1][1])))


@pytest.mark.parametrize("H", [16, 32, 128])
@pytest.mark.parametrize("topk", [1, 77, 300, 2048])
def test_pth_decode_heads_topk(H, topk):
    say(f"pth decode H={H} topk={topk}")
    case = Case(small(H=H, topk=topk, L=5000, seed=100 + topk))
    say(run_case(case))


@pytest.mark.parametrize("S", [1, 2, 5])
def test_pth_decode_splits(S):
    say(f"pth decode splits={S}")
    case = Case(small(H=32, topk=640, L=3000, seed=120))
    say(run_case(case, num_splits=S))


def test_pth_decode_causal_padding_and_bad_pages():
    say("pth decode causal T=2 with -1 runs and pages outside the pool")
    case = Case(small(B=3, T=2, H=16, topk=512, L=1500, causal=True, seed=130))
    idx = case.idx.copy()
    idx[0, 0, 100:300] = -1
    idx[1, 1, :] = -1       # an empty selection: out 0, lse -inf
    idx[2, 0, 5] = 99999    # past the context
    bt = case.lay.block_table
    bt[2, 3] = case.lay.num_pages + 4  # positions 192..255 of request 2 on a page outside the pool
    say(run_case(case, idx=idx))


def test_pth_decode_full_size_sampled():
    """The primary shape (64 query tokens, 32 heads, top-2048 over 140,000 positions) in the library's split
    choice; query tokens 0 and 41 checked against the oracle."""
    cfg = W.DecodeConfig("pthfull", B=64, T=1, H=32, topk=2048, fmt="fp8", ctx=140000, seed=140)
    say("pth decode full size")
    rng = np.random.default_rng(cfg.seed)
    lay = W.gen_layout(cfg, rng)
    slots_n = lay.num_pages * 64
    lat_g = torch.zeros((slots_n, 512), dtype=torch.uint8, device="cuda")
    sc_g = torch.zeros(slots_n, dtype=torch.float32, device="cuda")
    rope_g = torch.zeros((slots_n, 64), dtype=torch.bfloat16, device="cuda")
    idx = W.gen_indices(rng, lay.ctx, 1, 2048, False)
    q = W.gen_q(rng, 64, 1, 32)
    keep = {}
    for b in range(64):
        pos = np.arange(int(lay.ctx[b]))
        if b in (0, 41):  # only the selected rows of the sampled tokens need host copies
            sel = np.unique(idx[b, 0][idx[b, 0] >= 0])
            la, ro = W.gen_latent_rope(rng, sel.size)
            keep[b] = (sel, la, ro)
        la_all = torch.randn((pos.size, 512), device="cuda").to(torch.bfloat16)
        ro_all = torch.randn((pos.size, 64), device="cuda").to(torch.bfloat16)
        sm = dev(W.slots_for_request(lay, b, pos).astype(np.int64))
        M.mla_kv_quant_pth(la_all, ro_all, sm, lat_g, sc_g, rope_g)
    for b, (sel, la, ro) in keep.items():  # the sampled tokens' selected rows: known values
        M.mla_kv_quant_pth(bf16_dev(la), bf16_dev(ro), dev(W.slots_for_request(lay, b, sel).astype(np.int64)), lat_g,
                           sc_g, rope_g)
    out, lse = M.mla_sparse_decode_pth(bf16_dev(q), lat_g, sc_g, rope_g, dev(lay.block_table), dev(lay.ctx), dev(idx),
                                       cfg.sm_scale)
    got = bf16_to_np(out)
    lse_g = lse.cpu().numpy()
    for b, (sel, la, ro) in keep.items():
        n = sel.size
        lat_o = np.zeros((64 * ((n + 63) // 64), 512), np.uint8)
        sc_o = np.zeros(lat_o.shape[0], np.float32)
        rope_o = np.zeros((lat_o.shape[0], 64), np.uint16)
        oracle.kv_quant_pth(la, ro, np.arange(n), lat_o, sc_o, rope_o)
        # the token's selection renumbered onto a compact identity-paged copy of its rows
        pos_of = {int(p): i for i, p in enumerate(sel)}
        idx1 = np.array([[[pos_of[int(p)] if p >= 0 else -1 for p in idx[b, 0]]]], np.int32)
        bt1 = np.arange(lat_o.shape[0] // 64, dtype=np.int32)[None, :]
        ro_, rl_, _ = oracle.sparse_decode_pth(q[b:b + 1], lat_o, sc_o, rope_o, bt1, [n], idx1, cfg.sm_scale)
        e4 = np.array([oracle.e4m3_value(x) for x in range(256)])
        vm = np.abs(e4[lat_o[:n]] * sc_o[:n].astype(np.float64)[:, None]).max(0)[None, None, None, :]
        say(compare_outputs(got[b:b + 1], ro_, lse_g[b:b + 1], rl_, f"pth full token {b}", vmax=vm))
