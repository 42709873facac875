"""Seeded synthetic inputs for NVFP4 sparse-MLA decode: shapes, value distributions and structure only.

This module holds none of the method's arithmetic (no quantization, no attention).  The oracle and
the HIP path both take what it produces; neither imports the other.

Recipe (the pages' workload is agent-session replay on a trained model, which is not available here;
these inputs stand in for it with the pages' shapes):
  * latent  x = N(0,1) * r_row, r_row ~ lognormal(0, 0.5) per token row, each element x8 with
    probability 0.01, rounded to bf16 (round to nearest even);
  * rope    N(0,1) -> bf16;
  * q       N(0,1) -> bf16, shape [B, T, H, 576];
  * indices per query token: topk distinct positions drawn uniformly without replacement from
    [0, limit], in random order, int32 (limit = L-1, or L-T+t under the causal rule); when the limit
    leaves fewer than topk positions the rest is -1;
  * page table: the ceil(L/64) logical pages of every request map to a random permutation of the
    physical pages; physical page 0 is a pad page no request uses; unused table entries are -1.
  * index logits (the input of the index top-k; the pages do not define the indexer's logits): one
    fp32 row per query token over its context, ld = context rounded up to a multiple of 4, values by
    kind: "normal" N(0,1); "coarse" N(0,1) rounded to multiples of 1/16 (ties at the threshold);
    "ties" integers 0..3 (bins far larger than the candidate buffer); "equal" all 0.5; "special" a mix
    of -0.0, +0.0, +-inf, subnormals, +-FLT_MAX and N(0,1); "ramp" N(0,1) + 6 * position / ld (the
    largest values crowd into the last positions, as a recency trend would put them).
  * sparse-indexer inputs (the pages give the key size only): keys N(0,1) -> bf16 [tokens, 128]; index
    queries N(0,1) -> bf16 [B, T, HI, 128]; head weights N(0,1) * HI^-1/2, fp32 [B, T, HI]; the
    indexer pool uses the MLA cache's page table.
CPU generators use numpy PCG64; device generators use a seeded torch generator on the GPU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

LATENT, ROPE, QK, PAGE = 512, 64, 576, 64
NVFP4_ROW_BYTES, FP8_ROW_BYTES = 352, 576


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    T: int
    H: int
    topk: int            # 0 = dense (every position up to the limit)
    fmt: str             # "nvfp4" (352-byte rows) or "fp8" (576-byte rows)
    ctx: int = 0         # fixed context length, or 0 when ctx_range is used
    ctx_range: tuple = ()  # (lo, hi): log-uniform context lengths
    causal: bool = False
    quant_chunk: int = 0  # tokens quantized into free slots as part of the step
    alloc_tokens: int = 0  # per-request allocation when larger than the used context
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def row_bytes(self) -> int:
        return NVFP4_ROW_BYTES if self.fmt == "nvfp4" else FP8_ROW_BYTES

    @property
    def page_stride(self) -> int:
        return PAGE * self.row_bytes

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(192.0)


CONFIGS = {
    "tiny": DecodeConfig("tiny", B=2, T=1, H=16, topk=256, fmt="nvfp4", ctx=4096, seed=20260001),
    "dense_b4": DecodeConfig("dense_b4", B=4, T=1, H=128, topk=0, fmt="fp8", ctx=8192, seed=20260002),
    "dense_b8": DecodeConfig("dense_b8", B=8, T=1, H=128, topk=0, fmt="fp8", ctx=8192, seed=20260002),
    "dense_b16": DecodeConfig("dense_b16", B=16, T=1, H=128, topk=0, fmt="fp8", ctx=8192, seed=20260002),
    "sparse": DecodeConfig("sparse", B=64, T=1, H=32, topk=2048, fmt="nvfp4", ctx=140000, seed=20260003),
    "spec": DecodeConfig("spec", B=128, T=4, H=32, topk=2048, fmt="nvfp4", ctx_range=(8192, 146000), causal=True,
                         seed=20260004),
    "mixed": DecodeConfig("mixed", B=256, T=1, H=128, topk=2048, fmt="nvfp4", ctx_range=(8192, 146000),
                          quant_chunk=4096, alloc_tokens=146000, seed=20260005),
    # the pages' native-vs-staged comparison shape: 15 query tokens per launch, one TP4 rank of a 64-head
    # model (16 heads), ~140K-token agent contexts, top-2048
    "pages15": DecodeConfig("pages15", B=15, T=1, H=16, topk=2048, fmt="nvfp4", ctx=140000, seed=20260006),
    # the pages' launch-size tunings: 20 query tokens per launch (cluster sizing) and a 35-token launch
    # whose short contexts leave -1 entries in the 2,048-position lists
    "pages20": DecodeConfig("pages20", B=20, T=1, H=16, topk=2048, fmt="nvfp4", ctx=140000, seed=20260007),
    "short35": DecodeConfig("short35", B=35, T=1, H=16, topk=2048, fmt="nvfp4", ctx_range=(256, 2048),
                            seed=20260008),
    # the third arm of the pages' comparison at the same shape and inputs as pages15 (same seed): the
    # selected rows read from a 576-byte FP8 cache
    "pages15_fp8": DecodeConfig("pages15_fp8", B=15, T=1, H=16, topk=2048, fmt="fp8", ctx=140000, seed=20260006),
}


# --------------------------------------------------------------------------- helpers (input synthesis)

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def context_lengths(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    if cfg.ctx:
        return np.full(cfg.B, cfg.ctx, np.int32)
    lo, hi = cfg.ctx_range
    return np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=cfg.B))).astype(np.int32)


def gen_latent_rope(rng: np.random.Generator, n: int):
    """n token rows -> (latent bf16 bits [n,512], rope bf16 bits [n,64])."""
    r = rng.lognormal(0.0, 0.5, size=(n, 1)).astype(np.float32)
    x = rng.standard_normal((n, LATENT), dtype=np.float32) * r
    x = np.where(rng.random((n, LATENT)) < 0.01, x * 8.0, x).astype(np.float32)
    y = rng.standard_normal((n, ROPE), dtype=np.float32)
    return bf16_bits(x), bf16_bits(y)


def gen_q(rng: np.random.Generator, B: int, T: int, H: int) -> np.ndarray:
    return bf16_bits(rng.standard_normal((B, T, H, QK), dtype=np.float32))


def position_limit(L: int, T: int, t: int, causal: bool) -> int:
    return L - T + t if causal else L - 1


def gen_indices(rng: np.random.Generator, ctx: np.ndarray, T: int, topk: int, causal: bool) -> np.ndarray:
    B = ctx.shape[0]
    out = np.full((B, T, topk), -1, np.int32)
    for b in range(B):
        for t in range(T):
            lim = position_limit(int(ctx[b]), T, t, causal)
            n = min(topk, lim + 1)
            if n <= 0:
                continue
            sel = rng.choice(lim + 1, size=n, replace=False).astype(np.int32)
            out[b, t, :n] = sel
            rng.shuffle(out[b, t])
    return out


@dataclass
class PoolLayout:
    ctx: np.ndarray            # int32 [B]
    block_table: np.ndarray    # int32 [B, max_pages]
    num_pages: int             # physical pages (page 0 = pad)
    free_pages: np.ndarray     # physical pages no request uses


def gen_layout(cfg: DecodeConfig, rng: np.random.Generator, ctx: np.ndarray | None = None) -> PoolLayout:
    if ctx is None:
        ctx = context_lengths(cfg, rng)
    pages_per = (ctx.astype(np.int64) + PAGE - 1) // PAGE
    alloc_per = max(int(pages_per.max()), (cfg.alloc_tokens + PAGE - 1) // PAGE if cfg.alloc_tokens else 0)
    used = int(pages_per.sum())
    total = 1 + (cfg.B * alloc_per if cfg.alloc_tokens else used)
    if cfg.quant_chunk and not cfg.alloc_tokens:
        total += (cfg.quant_chunk + PAGE - 1) // PAGE
    perm = rng.permutation(np.arange(1, total, dtype=np.int64))
    bt = np.full((cfg.B, int(pages_per.max())), -1, np.int32)
    off = 0
    for b in range(cfg.B):
        n = int(pages_per[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    return PoolLayout(ctx=ctx.astype(np.int32), block_table=bt, num_pages=int(total), free_pages=perm[off:])


def slots_for_request(layout: PoolLayout, b: int, positions: np.ndarray) -> np.ndarray:
    pages = layout.block_table[b, positions // PAGE].astype(np.int64)
    return pages * PAGE + (positions % PAGE)


def gen_chunk_slots(layout: PoolLayout, rng: np.random.Generator, n: int) -> np.ndarray:
    """n slots on free pages, spread over the pool (the mixed step's write chunk)."""
    npg = (n + PAGE - 1) // PAGE
    pages = rng.choice(layout.free_pages, size=npg, replace=False).astype(np.int64)
    slots = (pages[:, None] * PAGE + np.arange(PAGE)[None, :]).reshape(-1)[:n]
    return rng.permutation(slots)


# --------------------------------------------------------------------------- device generators (torch)

def torch_bf16_normal(gen, shape, device, scale_rows=False, outliers=False):
    """Seeded N(0,1) bf16 tensor on the device; with scale_rows, each row (last axis) is multiplied by
    lognormal(0, 0.5); with outliers, each element is x8 with probability 0.01."""
    import torch
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if scale_rows:
        r = torch.empty(shape[:-1] + (1,), device=device, dtype=torch.float32).log_normal_(0.0, 0.5, generator=gen)
        x = x * r
    if outliers:
        m = torch.rand(shape, generator=gen, device=device) < 0.01
        x = torch.where(m, x * 8.0, x)
    return x.to(torch.bfloat16)


def torch_logits(gen, n: int, ld: int, device, kind: str = "normal"):
    """Seeded fp32 [n, ld] index logits on the device: the "normal" or the "ramp" kind."""
    import torch
    x = torch.randn((n, ld), generator=gen, device=device, dtype=torch.float32)
    if kind == "ramp":
        x += 6.0 * torch.arange(ld, device=device, dtype=torch.float32) / ld
    elif kind != "normal":
        raise ValueError(kind)
    return x


def torch_indices(gen, ctx: np.ndarray, T: int, topk: int, causal: bool, device):
    """[B,T,topk] int32 on the device: distinct uniform positions in [0, limit], random order, -1 pad."""
    import torch
    B = ctx.shape[0]
    lims = np.array([[position_limit(int(ctx[b]), T, t, causal) for t in range(T)] for b in range(B)], np.int64)
    Lmax = int(lims.max()) + 1
    out = torch.empty((B, T, topk), dtype=torch.int32, device=device)
    lim_t = torch.as_tensor(lims, device=device)
    pos = torch.arange(Lmax, device=device)
    rows_per = max(1, (1 << 26) // max(Lmax, 1))
    flat_lim = lim_t.reshape(-1)
    flat_out = out.view(-1, topk)
    for s in range(0, B * T, rows_per):
        e = min(B * T, s + rows_per)
        keys = torch.rand((e - s, Lmax), generator=gen, device=device)
        keys = torch.where(pos[None, :] <= flat_lim[s:e, None], keys, torch.full_like(keys, -1.0))
        k = min(topk, Lmax)
        v, i = torch.topk(keys, k, dim=1, sorted=True)
        i = torch.where(v >= 0, i, torch.full_like(i, -1)).to(torch.int32)
        if k < topk:
            i = torch.cat([i, torch.full((e - s, topk - k), -1, dtype=torch.int32, device=device)], dim=1)
        flat_out[s:e] = i
    return out


# --------------------------------------------------------------------------- full-size device inputs

def device_inputs(cfg: DecodeConfig, device="cuda", n_sets: int = 1, row_chunk: int = 1 << 20):
    """Every input of one step of `cfg`, generated on the device from the config's seed.

    Returns a dict: layout (PoolLayout, host), row_off (host int64 [B+1]: request b's source rows are
    lat[row_off[b]:row_off[b+1]], position order), lat / rope (bf16 source rows of every cached
    position), slots (int64 slot of every source row), bt / ctx (device int32), q_sets / idx_sets
    (n_sets independent query and index sets), and for a config with a write chunk, chunk_lat /
    chunk_rope / chunk_slots.
    """
    import torch
    rng = np.random.default_rng(cfg.seed)
    lay = gen_layout(cfg, rng)
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed)
    ctx = lay.ctx.astype(np.int64)
    row_off = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int64)
    total = int(row_off[-1])
    lat = torch.empty((total, LATENT), dtype=torch.bfloat16, device=device)
    rope = torch.empty((total, ROPE), dtype=torch.bfloat16, device=device)
    for s in range(0, total, row_chunk):
        e = min(total, s + row_chunk)
        lat[s:e] = torch_bf16_normal(gen, (e - s, LATENT), device, scale_rows=True, outliers=True)
        rope[s:e] = torch_bf16_normal(gen, (e - s, ROPE), device)
    bt = torch.from_numpy(lay.block_table).to(device)
    slots = torch.empty(total, dtype=torch.int64, device=device)
    for b in range(cfg.B):
        pos = torch.arange(int(ctx[b]), device=device)
        slots[row_off[b]:row_off[b + 1]] = bt[b][pos >> 6].long() * PAGE + (pos & (PAGE - 1))
    out = dict(layout=lay, row_off=row_off, lat=lat, rope=rope, slots=slots, bt=bt,
               ctx=torch.from_numpy(lay.ctx).to(device))
    out["q_sets"] = [torch_bf16_normal(gen, (cfg.B, cfg.T, cfg.H, QK), device) for _ in range(n_sets)]
    out["idx_sets"] = ([torch_indices(gen, lay.ctx, cfg.T, cfg.topk, cfg.causal, device) for _ in range(n_sets)]
                       if cfg.topk else [])
    if cfg.quant_chunk:
        out["chunk_lat"] = torch_bf16_normal(gen, (cfg.quant_chunk, LATENT), device, scale_rows=True, outliers=True)
        out["chunk_rope"] = torch_bf16_normal(gen, (cfg.quant_chunk, ROPE), device)
        out["chunk_slots"] = torch.from_numpy(gen_chunk_slots(lay, rng, cfg.quant_chunk)).to(device)
    return out


# --------------------------------------------------------------------------- index logits
LOGIT_KINDS = ("normal", "coarse", "ties", "equal", "special", "ramp")


def gen_logits(rng: np.random.Generator, n: int, ld: int, kind: str = "normal") -> np.ndarray:
    """fp32 [n, ld] logits of one kind (see the module recipe)."""
    if kind == "normal":
        return rng.standard_normal((n, ld), dtype=np.float32)
    if kind == "coarse":
        return np.round(rng.standard_normal((n, ld), dtype=np.float32) * 16.0) / np.float32(16.0)
    if kind == "ties":
        return rng.integers(0, 4, (n, ld)).astype(np.float32)
    if kind == "equal":
        return np.full((n, ld), 0.5, np.float32)
    if kind == "special":
        specials = np.array([-0.0, 0.0, np.inf, -np.inf, 1e-45, -1e-45, 1e-40, -1e-40, 3.4028235e38, -3.4028235e38],
                            np.float32)
        x = rng.standard_normal((n, ld), dtype=np.float32)
        pick = rng.random((n, ld)) < 0.3
        x[pick] = specials[rng.integers(0, specials.size, int(pick.sum()))]
        return x
    if kind == "ramp":
        x = rng.standard_normal((n, ld), dtype=np.float32)
        return x + (np.float32(6.0) * np.arange(ld, dtype=np.float32) / np.float32(ld))[None, :]
    raise ValueError(kind)


# --------------------------------------------------------------------------- sparse-indexer inputs
INDEX_DIM = 128


def gen_index_keys(rng: np.random.Generator, n: int) -> np.ndarray:
    """bf16 bits [n, 128] of N(0,1) indexer keys."""
    return bf16_bits(rng.standard_normal((n, INDEX_DIM)).astype(np.float32))


def gen_index_query(rng: np.random.Generator, B: int, T: int, HI: int):
    """(q bf16 bits [B, T, HI, 128], w float32 [B, T, HI])."""
    q = bf16_bits(rng.standard_normal((B, T, HI, INDEX_DIM)).astype(np.float32))
    w = (rng.standard_normal((B, T, HI)) / math.sqrt(HI)).astype(np.float32)
    return q, w
