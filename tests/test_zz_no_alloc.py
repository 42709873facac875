"""The decode entry point that allocates nothing (mla_sparse_decode_noalloc), through the C ABI: the same
results as mla_sparse_decode with a workspace, on two calls in a row (the second smaller, so the scratch
array holds the first call's leftovers), and within the oracle tolerances."""
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


def _run(case, d, S, noalloc):
    c = case.cfg
    out = torch.full((c.B, c.T, c.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((c.B, c.T, c.H), float("nan"), dtype=torch.float32, device="cuda")
    fn = M.mla_sparse_decode_noalloc if noalloc else M.mla_sparse_decode
    fn(d["q"], d["pool"], c.page_stride, case.lay.num_pages, d["bt"], d["ctx"], d["idx"], c.sm_scale, causal=c.causal,
       num_splits=S, out=out, lse=lse)
    torch.cuda.synchronize()
    return bf16_to_np(out).reshape(c.B * c.T, c.H, 512), lse.cpu().numpy().astype(np.float64).reshape(c.B * c.T, c.H)


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_noalloc_decode_matches_workspace_decode(order):
    big = W.DecodeConfig("na1", B=5, T=1, H=32, topk=1024, fmt="nvfp4", ctx=6000, seed=301)
    small = W.DecodeConfig("na2", B=2, T=2, H=16, topk=300, fmt="nvfp4", ctx=2500, causal=True, seed=302)
    h128 = W.DecodeConfig("na3", B=2, T=1, H=128, topk=700, fmt="nvfp4", ctx=3000, seed=303)
    runs = [(big, 4), (small, 3), (h128, 2)] if order == "large_then_small" else [(small, 5), (big, 2), (h128, 3)]
    for cfg, S in runs:
        case = Case(cfg)
        say(f"{order}: {cfg.name} B={cfg.B} T={cfg.T} H={cfg.H} topk={cfg.topk} S={S}")
        d = case.to_device()
        M.mla_kv_quant_nvfp4(d["lat"], d["rope"], d["slots"], d["pool"], cfg.page_stride, case.lay.num_pages)
        ref_out, ref_lse = _run(case, d, S, noalloc=False)
        for rep in range(2):  # the scratch keeps the previous call's partials and (zeroed) counters
            out, lse = _run(case, d, S, noalloc=True)
            assert np.array_equal(out, ref_out), f"{cfg.name} call {rep}: output differs from mla_sparse_decode"
            assert np.array_equal(lse, ref_lse), f"{cfg.name} call {rep}: lse differs from mla_sparse_decode"
        ro, rl = case.oracle_decode()
        say(compare_outputs(out, ro, lse, rl, f"noalloc {cfg.name}", vmax=case.vmax()))


def test_noalloc_rejects_splits_beyond_the_scratch():
    cap = M.lib().mla_noalloc_scratch_bytes()
    B, H, topk, S = 256, 32, 2048, 64
    assert M.lib().mla_sparse_decode_workspace_bytes(B, 1, H, topk, S) > cap
    q = torch.zeros((B, 1, H, 576), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros(64 * 352, dtype=torch.uint8, device="cuda")
    bt = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    ctx = torch.ones(B, dtype=torch.int32, device="cuda")
    idx = torch.zeros((B, 1, topk), dtype=torch.int32, device="cuda")
    out = torch.zeros((B, 1, H, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MlaError) as e:
        M.mla_sparse_decode_noalloc(q, pool, 64 * 352, 1, bt, ctx, idx, 0.07, num_splits=S, out=out)
    assert e.value.status == 4
