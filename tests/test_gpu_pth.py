"""GPU parity of TokenSpeed's per-token-head FP8 layout (writer bit-exact, sparse decode within the
attention tolerances of cases.py) through the C ABI, against the oracle."""
import sys

import numpy as np
import pytest

import oracle
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


def run_case(case, num_splits=0, idx=None):
    (lat_g, sc_g, rope_g), (lat_o, sc_o, rope_o) = pth_buffers(case)
    c = case.cfg
    idx = case.idx if idx is None else idx
    out, lse = M.mla_sparse_decode_pth(bf16_dev(case.q), lat_g, sc_g, rope_g, dev(case.lay.block_table),
                                       dev(case.lay.ctx), dev(idx), c.sm_scale, causal=c.causal,
                                       num_splits=num_splits)
    torch.cuda.synchronize()
    ro, rl, _ = oracle.sparse_decode_pth(case.q, lat_o, sc_o, rope_o, case.lay.block_table, case.lay.ctx, idx,
                                         c.sm_scale, c.causal)
    g = bf16_to_np(out)
    return compare_outputs(g, ro, lse.cpu().numpy(), rl, "pth")


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
        say(compare_outputs(got[b:b + 1], ro_, lse_g[b:b + 1], rl_, f"pth full token {b}"))
