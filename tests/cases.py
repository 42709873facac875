"""Shared builders for the tests: seeded inputs (workloads), the oracle's results, and the device copies
the HIP path gets.  Both sides receive the same bf16 inputs; the oracle quantizes its own pool."""
from __future__ import annotations

import numpy as np

import oracle
import workloads as W

# Tolerances for bf16 attention outputs against the FP64 oracle.  Every element o of the output must
# satisfy |g - o| <= 2e-2 + half a bf16 ulp of o + 2^-9 * vmax, where vmax is the largest |V| in that
# column among the query token's selected rows, and the relative L2 error of the whole tensor must stay
# within 1e-2.  The terms:
#   - 2e-2: the stated max-abs bound;
#   - half a bf16 ulp: the output is stored as bf16, so an output of magnitude 8 or more cannot be held
#     to 2e-2 (below 8 this adds at most 2^-6);
#   - 2^-9 * vmax: the matrix operands are FP16, as on the pages.  Rounding a softmax weight to FP16
#     changes it by at most 2^-11 of itself, which moves the output by at most
#     2^-11 * sum_j w_j |V_j - o| <= 2^-10 * vmax; a split's normalized result stored as FP16 adds at most
#     2^-11 of its magnitude, weighted by that split's share, <= 2^-11 * vmax.  Their sum, 1.5 * 2^-10 *
#     vmax, is rounded up to 2^-9 * vmax (fp32 accumulation adds far less).
# lse (natural log, fp32) within 1e-3 absolute, its -inf pattern exact.
MAX_ERR = 2e-2
REL_L2 = 1e-2
LSE_ABS = 1e-3
FP16_OPERAND_FACTOR = 2.0 ** -9


def half_ulp_bf16(x):
    """Half the spacing of bf16 values at |x| (2^(e-8) for |x| in [2^(e-1), 2^e)); subnormal spacing below."""
    ax = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(ax)
    e = np.where(ax > 0, np.maximum(e, -125), -125)  # bf16 subnormals (and zero's neighbours) are 2^-133 apart
    return np.ldexp(1.0, e - 9)


def output_bound(ref, vmax=None):
    b = MAX_ERR + half_ulp_bf16(ref)
    return b if vmax is None else b + FP16_OPERAND_FACTOR * vmax


def compare_outputs(gpu_out: np.ndarray, ref_out: np.ndarray, gpu_lse=None, ref_lse=None, what="", lse_tol=LSE_ABS,
                    vmax=None):
    """vmax: largest |V| per query token and column among its selected rows, shaped to broadcast against
    the outputs ([n, 1, 512] for outputs [n, H, 512]); None leaves out the FP16-operand term."""
    g = gpu_out.astype(np.float64)
    d = np.abs(g - ref_out)
    excess = d - output_bound(ref_out, vmax)
    nrm = np.linalg.norm(ref_out)
    rel = np.linalg.norm(g - ref_out) / (nrm if nrm > 0 else 1.0)
    info = f"{what}: max|d|={d.max():.3e} rel-L2={rel:.3e}"
    if excess.max() > 0:
        i = np.unravel_index(np.argmax(excess), d.shape)
        raise AssertionError(f"{info}: |d|={d[i]:.3e} at {i} exceeds 2e-2 + half ulp of ref {ref_out[i]:.4g}")
    assert rel <= REL_L2, info
    if ref_lse is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(gpu_lse)), what + ": -inf pattern of lse"
        if fin.any():
            dl = np.abs(gpu_lse[fin] - ref_lse[fin]).max()
            info += f" lse max|d|={dl:.3e}"
            assert dl <= lse_tol, info
    return info


class Case:
    """A complete decode problem on the host: pool source rows, layout, queries, indices."""

    def __init__(self, cfg: W.DecodeConfig, seed_offset: int = 0, ctx=None, indices=None, q=None):
        rng = np.random.default_rng(cfg.seed + seed_offset)
        self.cfg = cfg
        self.lay = W.gen_layout(cfg, rng, ctx=None if ctx is None else np.asarray(ctx, np.int32))
        lat, rope, slots = [], [], []
        for b in range(cfg.B):
            pos = np.arange(int(self.lay.ctx[b]))
            la, ro = W.gen_latent_rope(rng, pos.size)
            lat.append(la)
            rope.append(ro)
            slots.append(W.slots_for_request(self.lay, b, pos))
        self.lat = np.concatenate(lat)
        self.rope = np.concatenate(rope)
        self.slots = np.concatenate(slots).astype(np.int64)
        self.q = W.gen_q(rng, cfg.B, cfg.T, cfg.H) if q is None else q
        if indices is not None:
            self.idx = indices
        elif cfg.topk:
            self.idx = W.gen_indices(rng, self.lay.ctx, cfg.T, cfg.topk, cfg.causal)
        else:
            self.idx = None
        self.rng = rng
        self._pool = None

    @property
    def pool_bytes(self):
        return self.lay.num_pages * self.cfg.page_stride

    def oracle_pool(self):
        if self._pool is None:
            pool = np.zeros(self.pool_bytes, np.uint8)
            oracle.kv_quant(self.cfg.fmt, self.lat, self.rope, self.slots, pool, self.cfg.page_stride,
                            self.lay.num_pages)
            self._pool = pool
        return self._pool

    def oracle_decode(self, idx=None, units=None):
        pool = self.oracle_pool()
        c = self.cfg
        if c.topk:
            return oracle.sparse_decode(self.q, pool, c.page_stride, self.lay.num_pages, self.lay.block_table,
                                        self.lay.ctx, self.idx if idx is None else idx, c.sm_scale, c.causal,
                                        units=units, fmt=c.fmt)[:2]
        return oracle.dense_decode_fp8(self.q, pool, c.page_stride, self.lay.num_pages, self.lay.block_table,
                                       self.lay.ctx, c.sm_scale, c.causal, units=units)[:2]

    def vmax(self, idx=None, ctx=None):
        """Largest |V| per query token and latent column among its selected rows (under context lengths
        ctx, the case's own by default): [B*T, 1, 512]."""
        c = self.cfg
        pool = self.oracle_pool()
        idx = (self.idx if idx is None else idx) if c.topk else None
        out = np.zeros((c.B * c.T, 1, 512))
        for b in range(c.B):
            for t in range(c.T):
                pos = selected_positions(self.lay.ctx if ctx is None else ctx, c.T, c.causal, idx, b, t,
                                         self.lay.block_table,
                                         self.lay.num_pages)
                if pos.size == 0:
                    continue
                pg = self.lay.block_table[b, pos // 64].astype(np.int64)
                off = pg * c.page_stride + (pos % 64) * c.row_bytes
                rows = pool[(off[:, None] + np.arange(c.row_bytes)[None, :])]
                out[b * c.T + t, 0] = v_abs_of_rows(rows, c.fmt).max(0)
        return out

    # ---- device side
    def to_device(self):
        import torch
        dev = "cuda"
        c = self.cfg
        d = {}
        d["lat"] = torch.from_numpy(self.lat.view(np.int16)).to(dev).view(torch.bfloat16)
        d["rope"] = torch.from_numpy(self.rope.view(np.int16)).to(dev).view(torch.bfloat16)
        d["slots"] = torch.from_numpy(self.slots).to(dev)
        d["q"] = torch.from_numpy(self.q.view(np.int16)).to(dev).view(torch.bfloat16)
        d["bt"] = torch.from_numpy(self.lay.block_table).to(dev)
        d["ctx"] = torch.from_numpy(self.lay.ctx).to(dev)
        if self.idx is not None:
            d["idx"] = torch.from_numpy(self.idx).to(dev)
        d["pool"] = torch.zeros(self.pool_bytes, dtype=torch.uint8, device=dev)
        return d


_E2M1 = None
_E4M3 = None


def _tables():
    """Value tables from the oracle's decoders (pinned against torch's float8 and a minifloat decoder)."""
    global _E2M1, _E4M3
    if _E2M1 is None:
        _E2M1 = np.array([oracle.e2m1_value(c) for c in range(16)])
        _E4M3 = np.array([oracle.e4m3_value(c) for c in range(256)])
    return _E2M1, _E4M3


def v_abs_of_rows(rows: np.ndarray, fmt: str) -> np.ndarray:
    """|V| (the 512 latent values) of cache rows [n, row_bytes] -> [n, 512]."""
    e2, e4 = _tables()
    rows = np.asarray(rows, np.uint8)
    if fmt == "fp8":
        return np.abs(e4[rows[:, :512]])
    nib = np.empty((rows.shape[0], 512), np.int64)
    nib[:, 0::2] = rows[:, :256] & 15
    nib[:, 1::2] = rows[:, :256] >> 4
    return np.abs(e2[nib] * np.repeat(e4[rows[:, 256:288]], 16, axis=1))


def selected_positions(ctx, T, causal, idx, b, t, block_table, num_pages):
    """The decoders' selection rule restated: entries 0 <= i <= limit whose page entry is in the pool (all
    positions up to the limit when idx is None, the dense decode)."""
    L = int(ctx[b])
    lim = L - T + t if causal else L - 1
    pos = np.arange(lim + 1) if idx is None else np.asarray(idx[b, t], np.int64)
    pos = pos[(pos >= 0) & (pos <= lim) & (pos // 64 < block_table.shape[1])]
    pg = block_table[b, pos // 64]
    return pos[(pg >= 0) & (pg < num_pages)]


def bf16_to_np(t) -> np.ndarray:
    """bf16 device tensor -> float64 numpy array (exact)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def sampled_oracle(cfg, inp, qtoks, idx_d, q_d):
    """Oracle results for sampled query tokens of a full-size device case: the selected source rows are
    copied to the host and quantized by the oracle into a small pool of their own."""
    import torch
    lay = inp["layout"]
    outs, lses, vmaxes, pools_ok = [], [], [], True
    idx_all = idx_d.cpu().numpy() if idx_d is not None else None
    q_all = q_d.view(torch.int16).cpu().numpy().view(np.uint16)
    for qt in qtoks:
        b, t = divmod(int(qt), cfg.T)
        L = int(lay.ctx[b])
        lim = W.position_limit(L, cfg.T, t, cfg.causal)
        if idx_all is not None:
            ids = idx_all[b, t]
            pos = np.unique(ids[(ids >= 0) & (ids <= lim)])
        else:
            pos = np.arange(lim + 1)
        pages = np.unique(pos // 64)
        mini_bt = np.full((1, lay.block_table.shape[1]), -1, np.int32)
        mini_bt[0, pages] = np.arange(1, pages.size + 1)
        rows = torch.from_numpy(inp["row_off"][b] + pos).cuda()
        lat = inp["lat"][rows].view(torch.int16).cpu().numpy().view(np.uint16)
        rope = inp["rope"][rows].view(torch.int16).cpu().numpy().view(np.uint16)
        npg = pages.size + 1
        pool = np.zeros(npg * cfg.page_stride, np.uint8)
        slots = (mini_bt[0, pos // 64].astype(np.int64) * 64 + pos % 64)
        oracle.kv_quant(cfg.fmt, lat, rope, slots, pool, cfg.page_stride, npg)
        ctx = np.array([L], np.int32)
        q1 = q_all[b:b + 1]
        if idx_all is not None:
            o, l, _ = oracle.sparse_decode(q1, pool, cfg.page_stride, npg, mini_bt, ctx, idx_all[b:b + 1],
                                           cfg.sm_scale, cfg.causal, units=[t], fmt=cfg.fmt)
        else:
            o, l, _ = oracle.dense_decode_fp8(q1, pool, cfg.page_stride, npg, mini_bt, ctx, cfg.sm_scale, cfg.causal,
                                              units=[t])
        outs.append(o[0])
        lses.append(l[0])
        # the device pool holds the same bytes for these rows
        gslots = lay.block_table[b, pos // 64].astype(np.int64) * 64 + pos % 64
        offs = (gslots // 64) * cfg.page_stride + (gslots % 64) * cfg.row_bytes
        rb = cfg.row_bytes
        gidx = torch.from_numpy((offs[:, None] + np.arange(rb)[None, :]).reshape(-1)).cuda()
        grows = inp["pool"][gidx].cpu().numpy().reshape(-1, rb)
        oidx = (slots // 64) * cfg.page_stride + (slots % 64) * rb
        orows = pool[(oidx[:, None] + np.arange(rb)[None, :]).reshape(-1)].reshape(-1, rb)
        pools_ok &= np.array_equal(grows, orows)
        vmaxes.append(v_abs_of_rows(orows, cfg.fmt).max(0)[None, :] if orows.size else np.zeros((1, 512)))
    return np.stack(outs), np.stack(lses), np.stack(vmaxes), pools_ok
