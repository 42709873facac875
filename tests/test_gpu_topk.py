"""GPU parity of the index top-k (mla_index_topk through the C ABI) against the oracle's selection:
positions must match exactly (the selection is an integer result of exact comparisons)."""
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# lengths around k, the 8192-position chunk boundaries and the row stride
LENS = [0, 1, 5, 2047, 2048, 2049, 8191, 8192, 8193, 20000, 39999, 40000]


def run(x, lengths, k, workspace=None):
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    ld = torch.tensor(np.asarray(lengths, np.int32)).cuda()
    out = M.mla_index_topk(xd, ld, k, workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("kind", W.LOGIT_KINDS)
def test_index_topk_kinds(kind):
    say(f"index top-k kind={kind}")
    x = W.gen_logits(np.random.default_rng(70), len(LENS), 40000, kind)
    got = run(x, LENS, 2048)
    assert np.array_equal(got, oracle.topk_positions(x, LENS, 2048))


@pytest.mark.parametrize("k", [1, 3, 100, 1000, 2047])
def test_index_topk_k(k):
    say(f"index top-k k={k}")
    x = W.gen_logits(np.random.default_rng(71), len(LENS), 40000, "coarse")
    got = run(x, LENS, k)
    assert np.array_equal(got, oracle.topk_positions(x, LENS, k))


def test_index_topk_lengths_clamped():
    say("index top-k lengths outside [0, ld]")
    x = W.gen_logits(np.random.default_rng(72), 4, 12000, "normal")
    got = run(x, [-5, 12001, 1 << 30, 3], 2048)
    assert np.array_equal(got, oracle.topk_positions(x, [0, 12000, 12000, 3], 2048))


def test_index_topk_workspace_reuse():
    """Every call returns its histograms and counters to zero: calls on one workspace, alternating rows
    that use the candidate buffer with rows that overflow it, each match the oracle."""
    n, ldim = len(LENS), 40000
    ws = torch.zeros(M.mla_index_topk_workspace_bytes(n, ldim), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(73)
    for i, kind in enumerate(["normal", "ties", "coarse", "equal", "normal"]):
        say(f"workspace reuse call {i} kind={kind}")
        x = W.gen_logits(rng, n, ldim, kind)
        got = run(x, LENS, 2048, workspace=ws)
        assert np.array_equal(got, oracle.topk_positions(x, LENS, 2048)), (i, kind)
    assert int(ws[: n * 4096 * 4 + n * 32].count_nonzero()) == 0


def test_index_topk_full_size():
    """The decode workload's shape: 64 query tokens over 140,000-position contexts, top-2048."""
    cfg = W.CONFIGS["sparse"]
    say("index top-k full size 64 x 140000")
    x = W.gen_logits(np.random.default_rng(cfg.seed), cfg.B * cfg.T, cfg.ctx, "normal")
    lens = [cfg.ctx] * (cfg.B * cfg.T)
    got = run(x, lens, cfg.topk)
    assert np.array_equal(got, oracle.topk_positions(x, lens, cfg.topk))


def test_index_topk_long_row():
    """A row of more than 1024 chunks of 8192 positions takes the whole-row path even when its
    candidates would fit; a short row beside it takes the candidate path."""
    m = 1024 * 8192 + 5
    ld = m + 3
    say(f"index top-k long row m={m}")
    x = W.gen_logits(np.random.default_rng(74), 2, ld, "normal")
    lens = [m, 50000]
    got = run(x, lens, 2048)
    assert np.array_equal(got, oracle.topk_positions(x, lens, 2048))
