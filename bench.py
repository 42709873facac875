#!/usr/bin/env python3
"""Benchmark of one NVFP4 sparse-MLA decode step on one MI355X.

A step is the whole hot path over one batch: quantize-on-write of the step's new cache rows (the B*T
query tokens' own rows; for the mixed workload the 4,096-token write chunk) followed by the decode
(split decode kernel + LSE merge) of the B*T query tokens.  Inputs are seeded synthetic data of the
workload's shapes, resident in HBM before timing starts.  Eight independent (query, index) sets
rotate across steps so the 256 MB last-level cache cannot hold the working set.

Prints one JSON line (rank 0).  `roofline` covers the decode call (the dominant work), timed with
HIP events on its stream inside the timed steps; `cpu_baseline` times the FP64 oracle on the host
cores over a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
N_SETS = 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(cfg, valid_rows: int):
    """Bytes the method must move per decode call and its MFMA flops (QK^T + PV)."""
    nq = cfg.B * cfg.T
    rows_bytes = valid_rows * cfg.row_bytes
    qo_bytes = nq * cfg.H * (576 * 2 + 512 * 2)
    list_bytes = (valid_rows * 8) if cfg.topk else 0  # index + page-table entry per selected row
    flops = 2.0 * (576 + 512) * cfg.H * valid_rows
    return rows_bytes + qo_bytes + list_bytes, flops


def source_hash(cfg):
    """Hash of the sources of the decode kernel this workload runs (shared headers and the ABI included)
    and of the compile flags of its source (include paths left out: they differ between machines)."""
    from nvfp4_compressed_sparse_amd.build import HIPCC_FLAGS, SOURCE_FLAGS
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nvfp4_compressed_sparse_amd", "csrc")
    for f in ("mla_abi.hip", "mla_device.h", "mla_internal.h", "mla_decode.hip"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    flags = [x for x in HIPCC_FLAGS if not os.path.isabs(x)] + SOURCE_FLAGS.get("mla_decode.hip", [])
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def profile_record(cfg, kind: str, key: str, variant: str = ""):
    """A figure from a rocprofv3 counter summary of this workload's decode kernel, if it was taken on the
    current kernel source: profiles/decode_<workload><variant>_<kind>.md holds lines `source_hash: ...` and
    `<key>: ...`."""
    p = os.path.join(ROOT, "profiles", f"decode_{cfg.name}{variant}_{kind}.md")
    if not os.path.exists(p):
        return None
    rec = {}
    with open(p) as f:
        for line in f:
            if ":" in line and line.split(":", 1)[0].strip() in ("source_hash", key):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip().strip("`")
    if rec.get("source_hash") != source_hash(cfg) or key not in rec:
        return None
    return float(rec[key])


def copy_calibration(nbytes: int, reps: int):
    """A plain device copy of known size (reads nbytes, writes nbytes), for scaling the FETCH_SIZE /
    WRITE_SIZE counters of a rocprofv3 --pmc run to bytes."""
    import torch
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sparse", choices=sorted(W.CONFIGS))
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's choice")
    ap.add_argument("--pad-as-row0", action="store_true",
                    help="sparse workloads: replace the lists' -1 entries by position 0 before timing (the pages' "
                         "first version read row zero for each of them; a comparison, not the method's result)")
    ap.add_argument("--path", default="native", choices=["native", "staged", "pth"],
                    help="sparse workloads: native NVFP4 decode, the staged path (unpack the selected rows "
                         "to an FP8 copy, then the FP8 decoder reads it), or the per-token-head FP8 layout "
                         "(FP8 latent, fp32 scale, bf16 rope in three buffers) and its decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="sparse NVFP4 decode: write the step's new rows with the writer's own launch before the "
                         "decode (two launches per step) instead of inside the decode launch")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-rate probes (streaming read, row gather, MFMA loop) run after the timing")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step's calls as captured HIP graphs instead of prepared launches")
    ap.add_argument("--cpu-sample", type=int, default=0, help="query tokens in the oracle sample (0 = auto)")
    ap.add_argument("--timeline", action="store_true",
                    help="decode kernel phase timeline: run the step on the instrumented build of the library "
                         "(libmla_nvfp4_timeline.so, the same kernels with phase timestamps compiled in) and print "
                         "the last launch's phase times (medians over workgroups) instead of the metric line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration) and exit")
    ap.add_argument("--op", default="decode", choices=["decode", "index-topk", "index-logits", "dsa-step"],
                    help="decode: the decode step (default); index-topk: the indexer's top-k selection over fp32 "
                         "logits of the workload's query tokens and contexts; index-logits: the indexer's logits "
                         "over FP8 keys (a DeepSeek-style reading); dsa-step: indexer logits, top-k and the sparse "
                         "decode in sequence, each timed")
    ap.add_argument("--index-heads", type=int, default=64, help="index-logits: index heads (16, 32 or 64)")
    ap.add_argument("--logits", default="normal", choices=["normal", "ramp"],
                    help="index-topk: N(0,1) logits, or N(0,1) plus a rising trend over positions")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the sharding across GPUs is a design note, "
                                   "but not implemented", "n_gpus": args.gpus}))
        sys.exit(2)
    if args.op == "index-topk":
        bench_index_topk(args)
        return
    if args.op == "index-logits":
        bench_index_logits(args)
        return
    if args.op == "dsa-step":
        bench_dsa_step(args)
        return

    import torch
    import nvfp4_compressed_sparse_amd as M

    if args.timeline:
        M.use_timeline_library()
        args.no_cpu_baseline = args.no_peaks = True
    cfg = W.CONFIGS[args.workload]
    staged_path = args.path == "staged"
    pth_path = args.path == "pth"
    if (staged_path or pth_path) and not (cfg.topk and cfg.fmt == "nvfp4"):
        raise SystemExit("--path staged / pth apply to the sparse NVFP4 workloads")
    dev = "cuda"
    torch.cuda.set_device(0)
    log(f"[bench] workload {cfg.name}: B={cfg.B} T={cfg.T} H={cfg.H} topk={cfg.topk} fmt={cfg.fmt}")
    t0 = time.time()
    inp = W.device_inputs(cfg, dev, n_sets=N_SETS)
    lay = inp["layout"]
    pool = torch.zeros(lay.num_pages * cfg.page_stride, dtype=torch.uint8, device=dev)
    quant = M.mla_kv_quant_nvfp4 if cfg.fmt == "nvfp4" else M.mla_kv_quant_fp8
    quant(inp["lat"], inp["rope"], inp["slots"], pool, cfg.page_stride, lay.num_pages)
    torch.cuda.synchronize()
    log(f"[bench] pool filled: {pool.numel() / 1e9:.2f} GB, {inp['slots'].numel()} rows ({time.time() - t0:.1f} s)")

    # the step's own new rows: position L-T+t of every request (or the mixed step's write chunk)
    if cfg.quant_chunk:
        w_lat, w_rope, w_slots = inp["chunk_lat"], inp["chunk_rope"], inp["chunk_slots"]
    else:
        rows = torch.from_numpy(np.concatenate([inp["row_off"][b] + lay.ctx[b] - cfg.T + np.arange(cfg.T)
                                                for b in range(cfg.B)]).astype(np.int64)).to(dev)
        w_lat, w_rope, w_slots = inp["lat"][rows].contiguous(), inp["rope"][rows].contiguous(), inp["slots"][rows]

    if pth_path:  # the same rows in the per-token-head layout
        pth_slots = lay.num_pages * 64
        pth_lat = torch.zeros((pth_slots, 512), dtype=torch.uint8, device=dev)
        pth_sc = torch.zeros(pth_slots, dtype=torch.float32, device=dev)
        pth_rope = torch.zeros((pth_slots, 64), dtype=torch.bfloat16, device=dev)
        M.mla_kv_quant_pth(inp["lat"], inp["rope"], inp["slots"], pth_lat, pth_sc, pth_rope)
        torch.cuda.synchronize()

    # oracle sample (built before the source rows are released)
    cpu = None
    if not args.no_cpu_baseline and not pth_path:  # the oracle sample covers the NVFP4 rows
        cpu = prepare_cpu_sample(cfg, inp, args.cpu_sample)
    del inp["lat"], inp["rope"], inp["slots"]
    torch.cuda.empty_cache()

    q_sets, idx_sets = inp["q_sets"], inp["idx_sets"]
    sparse_fp8 = bool(cfg.topk) and cfg.fmt == "fp8"  # the FP8-cache arm of the pages' comparison
    sparse_fn = M.mla_sparse_decode_fp8 if sparse_fp8 else M.mla_sparse_decode
    # the sparse NVFP4 step in one launch: the decode kernel writes the step's new rows in its prologue
    fusable = bool(cfg.topk) and not sparse_fp8 and not cfg.quant_chunk and not staged_path and not pth_path
    fused = fusable and not args.unfused
    if cfg.topk:
        S = args.splits or (M.mla_sparse_decode_fp8_splits if sparse_fp8 else M.mla_sparse_decode_splits)(
            cfg.B, cfg.T, cfg.H, cfg.topk)
    else:
        S = args.splits or M.mla_dense_decode_splits(cfg.B, cfg.T, cfg.H, int(lay.ctx.max()))
    if cfg.topk:
        ws_bytes = (M.mla_sparse_decode_fp8_workspace_bytes if sparse_fp8 else M.mla_sparse_decode_workspace_bytes)(
            cfg.B, cfg.T, cfg.H, cfg.topk, S)
    else:
        ws_bytes = M.mla_dense_decode_workspace_bytes(cfg.B, cfg.T, cfg.H, int(lay.ctx.max()), S)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)  # split counters start at zero
    out = torch.empty((cfg.B, cfg.T, cfg.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((cfg.B, cfg.T, cfg.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    max_ctx = int(lay.ctx.max())
    if staged_path:
        # the FP8 copy of every query token's selected rows, read by the FP8 decoder as a paged cache
        nq = cfg.B * cfg.T
        st_pages = (cfg.topk + 63) // 64
        staged = torch.empty(nq * st_pages * 64 * 576, dtype=torch.uint8, device=dev)
        st_bt = torch.empty((nq, st_pages), dtype=torch.int32, device=dev)
        st_len = torch.empty(nq, dtype=torch.int32, device=dev)
        S = args.splits or M.mla_dense_decode_splits(nq, 1, cfg.H, st_pages * 64)
        ws_bytes = M.mla_dense_decode_workspace_bytes(nq, 1, cfg.H, st_pages * 64, S)
        ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        out1 = out.view(nq, 1, cfg.H, 512)
        lse1 = lse.view(nq, 1, cfg.H)

    # valid selected rows per set (algorithmic work)
    if cfg.topk:
        lims = np.array([[W.position_limit(int(lay.ctx[b]), cfg.T, t, cfg.causal) for t in range(cfg.T)]
                         for b in range(cfg.B)])
        lim_d = torch.from_numpy(lims).to(dev)[..., None]
        valid = [int(((ix >= 0) & (ix <= lim_d)).sum().item()) for ix in idx_sets]
        if args.pad_as_row0:  # after counting: the padding reads are not work the method asks for
            idx_sets = [torch.where(ix < 0, torch.zeros_like(ix), ix).contiguous() for ix in idx_sets]
    else:
        valid = [int(sum(min(W.position_limit(int(lay.ctx[b]), cfg.T, t, cfg.causal) + 1, int(lay.ctx[b]))
                         for b in range(cfg.B) for t in range(cfg.T)))] * N_SETS

    if pth_path:
        S = args.splits or 0
        pth_ws = M.lib().mla_sparse_decode_pth_workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.topk, S)

    def write(i):
        """The step's quantize-on-write (the same new rows every step), on the current stream."""
        st = torch.cuda.current_stream()
        if pth_path:
            M.mla_kv_quant_pth(w_lat, w_rope, w_slots, pth_lat, pth_sc, pth_rope, stream=st)
        else:
            quant(w_lat, w_rope, w_slots, pool, cfg.page_stride, lay.num_pages, stream=st)

    def decode(i):
        """The step's decode call over index set i % N_SETS, on the current stream."""
        k = i % N_SETS
        st = torch.cuda.current_stream()
        if pth_path:
            M.mla_sparse_decode_pth(q_sets[k], pth_lat, pth_sc, pth_rope, inp["bt"], inp["ctx"], idx_sets[k],
                                    cfg.sm_scale, causal=cfg.causal, num_splits=S, out=out, lse=lse, stream=st)
        elif staged_path:
            M.mla_stage_nvfp4_fp8(pool, cfg.page_stride, lay.num_pages, inp["bt"], inp["ctx"], idx_sets[k],
                                  causal=cfg.causal, staged=staged, staged_block_table=st_bt, staged_lens=st_len,
                                  stream=st)
            M.mla_dense_decode_fp8(q_sets[k].view(nq, 1, cfg.H, 576), staged, 64 * 576, nq * st_pages, st_bt, st_len,
                                   st_pages * 64, cfg.sm_scale, num_splits=S, out=out1, lse=lse1, workspace=ws,
                                   stream=st)
        elif fused:
            M.mla_sparse_decode_append(q_sets[k], pool, cfg.page_stride, lay.num_pages, inp["bt"], inp["ctx"],
                                       idx_sets[k], w_lat, w_rope, cfg.sm_scale, causal=cfg.causal, num_splits=S,
                                       out=out, lse=lse, workspace=ws, stream=st)
        elif cfg.topk:
            sparse_fn(q_sets[k], pool, cfg.page_stride, lay.num_pages, inp["bt"], inp["ctx"], idx_sets[k], cfg.sm_scale,
                      causal=cfg.causal, num_splits=S, out=out, lse=lse, workspace=ws, stream=st)
        else:
            M.mla_dense_decode_fp8(q_sets[k], pool, cfg.page_stride, lay.num_pages, inp["bt"], inp["ctx"], max_ctx,
                                   cfg.sm_scale, causal=cfg.causal, num_splits=S, out=out, lse=lse, workspace=ws,
                                   stream=st)

    for i in range(args.warmup):
        if not fused:
            write(i)
        decode(i)
    torch.cuda.synchronize()
    if args.graph:
        # The step's calls captured once as HIP graphs (the write, and the decode of each index set) and replayed.
        # Nothing in a captured call allocates or clears memory (the split counters return to zero inside the
        # decode kernel).  Measured slower than the prepared launches below on this software stack.
        g_write = None
        if not fused:
            g_write = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_write):
                write(0)
        g_dec = []
        for k in range(N_SETS):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                decode(k)
            g_dec.append(g)
        torch.cuda.synchronize()
        for i in range(max(args.warmup, N_SETS)):
            if g_write is not None:
                g_write.replay()
            g_dec[i % N_SETS].replay()
        torch.cuda.synchronize()

        def step(i):
            if g_write is not None:
                g_write.replay()
            g_dec[i % N_SETS].replay()

        def dec_call(i):
            g_dec[i % N_SETS].replay()
    else:
        # The step's calls with their arguments checked and converted once (the binding's prepared calls): each
        # step then costs the host two plain C-ABI calls, so the host stays ahead of the GPU and the timed loop
        # measures the GPU rather than the host's launch path.
        w_call = None if fused else M.prepare(write, 0)
        d_calls = [M.prepare(decode, k) for k in range(N_SETS)]

        def step(i):
            if w_call is not None:
                w_call()
            d_calls[i % N_SETS]()

        def dec_call(i):
            d_calls[i % N_SETS]()

        for i in range(N_SETS):
            step(i)
        torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps), splits={S}, {'graph replay' if args.graph else 'prepared launches'}")

    # The timed steps: HIP events on the launch stream at the two ends only.  An event recorded between the
    # calls of a step puts a marker between the kernels, which costs several microseconds per step here.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / args.steps
    # The decode call's average duration: the same decode calls back to back, events at the two ends.
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    d0.record(stream)
    for i in range(args.steps):
        dec_call(i)
    d1.record(stream)
    torch.cuda.synchronize()
    dec_avg_us = d0.elapsed_time(d1) * 1e3 / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.2f} us/step (events), wall {wall / args.steps * 1e6:.2f} "
        f"us/step; decode call avg {dec_avg_us:.2f} us over {args.steps} back-to-back calls")
    if fused:  # the timed steps are themselves back-to-back launches of the one call
        dec_avg_us = ms_per_step * 1e3
    if args.timeline:
        if staged_path or pth_path:
            raise SystemExit("--timeline covers decode_kernel (the native paths)")
        print_timeline(M, cfg, S, ms_per_step, dec_avg_us, fused)
        return

    nq = cfg.B * cfg.T
    value = nq / (ms_per_step * 1e-3)
    vrows = float(np.mean([valid[i % N_SETS] for i in range(args.steps)]))
    bytes_per, flops_per = algorithmic_work(cfg, vrows)
    if fused:  # the new rows: bf16 read, quantized row written
        bytes_per += nq * (1152 + cfg.row_bytes)
    if staged_path:
        # the staged path moves a selected row three times: 352 B read, 576 B FP8 copy written and read
        bytes_per += int(vrows * 2 * 576)
    if pth_path:  # a per-token-head row is 512 + 4 + 128 bytes
        bytes_per += int(vrows * (644 - cfg.row_bytes))
    if cfg.H <= 32:
        ach = bytes_per / (dec_avg_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = flops_per / (dec_avg_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4)}
    variant = "_unfused" if (fusable and not fused) else ""
    t = None if (staged_path or pth_path) else profile_record(cfg, "traffic", "traffic_bytes_per_launch", variant)
    roof["traffic"] = None if t is None else int(t)
    if cfg.H > 32:
        roof["mfma_util_counter"] = profile_record(cfg, "mfma", "mfma_util_percent", variant)
    if staged_path:
        roof["kernel"] = ("mla_stage_nvfp4_fp8 + mla_dense_decode_fp8 calls: stage_rows_kernel then decode_kernel "
                          "over the FP8 copy, back-to-back calls timed together with HIP events on their stream")
    elif pth_path:
        roof["kernel"] = ("mla_sparse_decode_pth call: pth_decode_kernel (+ pth_merge_kernel when split), "
                          "back-to-back calls timed with HIP events on their stream")
    elif fused:
        roof["kernel"] = ("mla_sparse_decode_append call: decode_kernel (the step's new rows quantized and "
                          "written in its prologue, split merge inside), back-to-back calls timed with HIP "
                          "events on its stream")
    else:
        roof["kernel"] = (("mla_sparse_decode_fp8" if sparse_fp8 else "mla_sparse_decode") if cfg.topk
                          else "mla_dense_decode_fp8") + \
            " call: decode_kernel (split merge inside), back-to-back calls timed with HIP events on its stream"
    roof["algorithmic_bytes_per_launch"] = int(bytes_per)
    roof["flops_per_launch"] = flops_per
    roof["launch_us"] = round(dec_avg_us, 3)

    if not args.no_peaks:
        peaks = measure_achievable(cfg, pool if not pth_path else None, inp, idx_sets if cfg.topk else None, lay, lim_d
                                   if cfg.topk else None)
        roof["achievable"] = peaks
        if roof["bound"] == "hbm":
            roof["frac_of_stream_read"] = round(roof["achieved"] / peaks["stream_read_GBs"], 4)
            if peaks.get("row_gather_GBs"):
                roof["frac_of_row_gather"] = round(roof["achieved"] / peaks["row_gather_GBs"], 4)
        else:
            roof["frac_of_mfma_loop"] = round(roof["achieved"] / peaks["mfma_f16_TFLOPs"], 4)

    res = {
        "metric": "NVFP4 sparse-MLA decode query-tokens/s at B=64, top-2048; % of roofline",
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "q_len": cfg.T, "H": cfg.H, "topk": cfg.topk,
                   "context": cfg.ctx or list(cfg.ctx_range), "row_bytes": cfg.row_bytes, "page_tokens": 64,
                   "causal": cfg.causal, "splits": S, "path": args.path,
                   "row_bytes_read": 644 if pth_path else cfg.row_bytes,
                   "index_padding": "position 0" if args.pad_as_row0 else "-1 (skipped)",
                   "step": ("quantize %d rows + %s" % (cfg.quant_chunk or nq,
                                                       "stage + FP8 decode" if staged_path else "decode")),
                   "launch": ("one launch per step (the decode writes the new rows), " if fused else
                              "write + decode launches per step, ") +
                             ("hip graph replay" if args.graph else
                              "prepared C-ABI calls (arguments checked once)")},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if cpu is not None:
        res["cpu_baseline"] = run_cpu_baseline(cfg, cpu)
    print(json.dumps(res), flush=True)


TIMELINE_PHASES = [(1, "prologue loads issued (query DMA, list entries, page table; new rows loaded)"),
                   (2, "loads landed, page table staged (new rows quantized)"),
                   (3, "row list compacted (new rows stored and complete)"),
                   (4, "first gathers: step 0 visible"),
                   (5, "last step done"),
                   (6, "split result tile normalized"),
                   (7, "split result stored, arrival counter taken")]


def print_timeline(M, cfg, S, ms_per_step, dec_avg_us, fused):
    """Phase times of the last decode launch from the instrumented library: per workgroup, the stamps of
    its wave 0 (10 ns ticks) relative to the first workgroup's start; medians and 90th percentiles over the
    workgroups that reach each phase."""
    n = int(M.timeline(1)[0, 11])  # the launch's workgroups (16- or 32-head groups, or 64 at 64/128 heads)
    if n > 4096:
        raise SystemExit(f"--timeline records at most 4096 workgroups (this launch has {n})")
    st = M.timeline(n)
    hg = n // (cfg.B * cfg.T * S)
    t0 = st[:, 0].min()
    rel = (st[:, :9] - t0) * 0.01  # us
    merged = st[:, 13] == 1
    rows = [("workgroup start", rel[:, 0])]
    rows += [(name, rel[st[:, i] != 0, i]) for i, name in TIMELINE_PHASES]
    rows += [("end, merging workgroups" if S > 1 else "end", rel[merged, 8])]
    if S > 1:
        rows += [("end, other workgroups", rel[~merged, 8])]
    steps = st[:, 15]
    per_step = (st[:, 5] - st[:, 4]) * 0.01 / np.maximum(steps, 1)
    out = {"workload": cfg.name, "workgroups": int(n), "splits": S, "steps_per_workgroup": int(np.median(steps)),
           "launch_us": round(dec_avg_us, 2), "ms_per_step": round(ms_per_step, 6), "fused": fused,
           "span_us": round(float(rel[:, 8].max()), 2), "step_us_median": round(float(np.median(per_step)), 3),
           "xcds_per_query_token": None, "phases_us": []}
    for name, v in rows:
        if v.size:
            out["phases_us"].append({"phase": name, "median": round(float(np.median(v)), 2),
                                     "p90": round(float(np.percentile(v, 90)), 2), "workgroups": int(v.size)})
    # the XCC each workgroup ran on, grouped by query token (logical index / (head groups * splits))
    tok = st[:, 14] // (hg * S)
    out["xcds_per_query_token"] = int(max(len(set(st[tok == q, 12].tolist())) for q in np.unique(tok)))
    log(f"[bench] timeline of the last launch ({n} workgroups, {S} splits, median "
        f"{out['steps_per_workgroup']} steps; step {out['step_us_median']} us):")
    for ph in out["phases_us"]:
        log(f"[bench]   {ph['phase']:<64s} median {ph['median']:7.2f} us   p90 {ph['p90']:7.2f} us")
    print(json.dumps({"timeline": out}), flush=True)


def measure_achievable(cfg, pool, inp, idx_sets, lay, lim_d):
    """Rates this GPU reaches, measured here with the probe kernels (libmla_probe.so), each timed with HIP
    events over back-to-back calls: a streaming read of a 4 GiB buffer, a gather of the step's selected rows from the pool (the decode's
    access pattern: the valid rows of each index set, rotating over the sets), and a loop of independent FP16 and
    bf16 MFMAs."""
    import torch
    from nvfp4_compressed_sparse_amd import probe
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def timed(fn, reps):
        # back-to-back calls, events at the two ends only (as the decode call is timed): seconds per call
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    out = {}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    wg = 256 * 8
    sink = torch.empty(wg * 256, dtype=torch.int32, device="cuda")
    probe.stream_read(buf, sink, wg, sh)
    t = timed(lambda i: probe.stream_read(buf, sink, wg, sh), 10)
    out["stream_read_GBs"] = round(nbytes / t / 1e9, 1)
    out["stream_read_bytes"] = nbytes
    del buf
    torch.cuda.empty_cache()
    if pool is not None and idx_sets:
        addrs = []
        for ix in idx_sets:
            b = torch.arange(cfg.B, device="cuda").view(cfg.B, 1, 1).expand_as(ix)
            ok = (ix >= 0) & (ix <= lim_d)
            pos = ix[ok].long()
            bb = b[ok]
            page = inp["bt"][bb, torch.clamp(pos >> 6, max=inp["bt"].shape[1] - 1)].long()
            keep = (page >= 0) & (page < lay.num_pages) & ((pos >> 6) < inp["bt"].shape[1])
            a16 = (page[keep] * cfg.page_stride + (pos[keep] & 63) * cfg.row_bytes) // 16
            addrs.append(a16.to(torch.int32).contiguous())
        chunks = cfg.row_bytes // 16
        n = max(a.numel() for a in addrs)
        gwg = (n * chunks + 256 * 6 - 1) // (256 * 6)
        gsink = torch.empty(gwg * 256, dtype=torch.int32, device="cuda")
        for a in addrs:
            probe.row_gather(pool, a, cfg.row_bytes, gsink, gwg, sh)
        t = timed(lambda i: probe.row_gather(pool, addrs[i % len(addrs)], cfg.row_bytes, gsink, gwg, sh), 24)
        rows = float(np.mean([a.numel() for a in addrs]))
        out["row_gather_GBs"] = round(rows * cfg.row_bytes / t / 1e9, 1)
        out["row_gather_us"] = round(t * 1e6, 2)
        out["row_gather_rows"] = int(rows)
    iters, mwg = 4000, 256 * 16
    mout = torch.empty(mwg * 256 * 4, dtype=torch.float32, device="cuda")
    for bf16, key in ((0, "mfma_f16_TFLOPs"), (1, "mfma_bf16_TFLOPs")):
        probe.mfma(bf16, iters, mout, mwg, sh)
        t = timed(lambda i: probe.mfma(bf16, iters, mout, mwg, sh), 5)
        out[key] = round(probe.mfma_flops(iters, mwg) / t / 1e12, 1)
    log(f"[bench] achievable: {out}")
    return out


def bench_index_topk(args):
    """The index top-k over one step's logits: B*T query tokens, each over its context, top-`topk`."""
    import torch
    import nvfp4_compressed_sparse_amd as M

    cfg = W.CONFIGS[args.workload]
    if not cfg.topk:
        raise SystemExit("--op index-topk applies to the sparse workloads")
    dev = "cuda"
    torch.cuda.set_device(0)
    rng = np.random.default_rng(cfg.seed)
    ctx = W.context_lengths(cfg, rng)
    n = cfg.B * cfg.T
    # each query token ranks the positions it may attend to (its causal limit, or the whole context)
    lengths = np.array([W.position_limit(int(ctx[b]), cfg.T, t, cfg.causal) + 1 for b in range(cfg.B)
                        for t in range(cfg.T)], np.int32)
    ld = int(-(-int(lengths.max()) // 4) * 4)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    sets = [W.torch_logits(gen, n, ld, dev, args.logits) for _ in range(N_SETS)]
    lens_d = torch.from_numpy(lengths).to(dev)
    out = torch.empty((n, cfg.topk), dtype=torch.int32, device=dev)
    ws = torch.zeros(M.mla_index_topk_workspace_bytes(n, ld), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    log(f"[bench] index top-k: {n} rows, ld={ld}, k={cfg.topk}, {N_SETS} logit sets of "
        f"{n * ld * 4 / 1e6:.1f} MB")

    def step(i):
        M.mla_index_topk(sets[i % N_SETS], lens_d, cfg.topk, out=out, workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    chosen = int((out >= 0).sum().item())
    if chosen != int(np.minimum(lengths, cfg.topk).sum()):
        raise SystemExit(f"index top-k chose {chosen} positions, expected {int(np.minimum(lengths, cfg.topk).sum())}")
    # a step is one call: back-to-back calls, HIP events on their stream at the two ends only
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    call_avg = ms_per_step * 1e3
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.2f} us/step (one call each)")
    # algorithmic bytes: every logit of every row read once, the lists written
    bytes_per = int(lengths.astype(np.int64).sum() * 4 + n * cfg.topk * 4)
    ach = bytes_per / (call_avg * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "mla_index_topk call: topk_hist_kernel, topk_collect_kernel, topk_finish_kernel, timed with "
                      "HIP events on their stream",
            "algorithmic_bytes_per_launch": bytes_per, "launch_us": round(call_avg, 3)}
    res = {
        "metric": "index top-k query-tokens/s (fp32 logits over each context, top-%d); %% of roofline" % cfg.topk,
        "value": round(n / (ms_per_step * 1e-3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "rows": n, "context": cfg.ctx or list(cfg.ctx_range), "ld": ld,
                   "topk": cfg.topk, "logits": "N(0,1) fp32" if args.logits == "normal" else
                   "N(0,1) + 6 * position / ld, fp32", "step": "index top-k"},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        x = sets[0].cpu().numpy()
        rows = min(n, args.cpu_sample or n)
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.topk_positions(x[:rows], lengths[:rows], cfg.topk)
            times.append(time.perf_counter() - t0)
        tmed = float(np.median(times))
        res["cpu_baseline"] = {"value": round(rows / tmed, 3), "unit": "query-tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{rows} of {n} rows of one step, median of 3 runs of {tmed:.2f} s "
                                         "(numpy, one thread)"}
    print(json.dumps(res), flush=True)


def bench_index_logits(args):
    """The indexer's logits for one step: B*T query tokens, each over the FP8 keys of its request's
    context (128 codes + an fp32 scale per position), HI index heads."""
    import torch
    import nvfp4_compressed_sparse_amd as M

    cfg = W.CONFIGS[args.workload]
    if not cfg.topk:
        raise SystemExit("--op index-logits applies to the sparse workloads")
    HI = args.index_heads
    dev = "cuda"
    torch.cuda.set_device(0)
    rng = np.random.default_rng(cfg.seed)
    lay = W.gen_layout(cfg, rng)
    n = cfg.B * cfg.T
    maxc = int(lay.ctx.max())
    ps = M.INDEX_PAGE_BYTES
    t0 = time.time()
    pool = torch.zeros(lay.num_pages * ps, dtype=torch.uint8, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    for b in range(cfg.B):  # every position of every request, keys N(0,1)
        L = int(lay.ctx[b])
        slots = torch.from_numpy(W.slots_for_request(lay, b, np.arange(L))).to(dev)
        keys = torch.randn((L, 128), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        M.mla_index_key_quant(keys, slots, pool, ps, lay.num_pages)
    torch.cuda.synchronize()
    log(f"[bench] index logits: {n} query tokens, HI={HI}, contexts up to {maxc}, pool {pool.numel() / 1e9:.2f} GB "
        f"({time.time() - t0:.1f} s)")
    bt = torch.from_numpy(lay.block_table).to(dev)
    ctx = torch.from_numpy(lay.ctx).to(dev)
    q_sets = [torch.randn((cfg.B, cfg.T, HI, 128), generator=gen, device=dev).to(torch.bfloat16) for _ in range(N_SETS)]
    w_sets = [torch.randn((cfg.B, cfg.T, HI), generator=gen, device=dev) / HI ** 0.5 for _ in range(N_SETS)]
    out = torch.empty((n, (maxc + 3) // 4 * 4), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        M.mla_index_logits(q_sets[i % N_SETS], w_sets[i % N_SETS], pool, ps, lay.num_pages, bt, ctx, maxc,
                           causal=cfg.causal, out=out, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # a step is one call: back-to-back calls, HIP events on their stream at the two ends only
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    call_avg = ms_per_step * 1e3
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.2f} us/step (one call each)")
    # algorithmic work: each request's keys (128 code bytes + a 4-byte scale per position) read once, the
    # query tokens' q and w read, one fp32 logit written per (query token, visible position)
    visible = sum(W.position_limit(int(lay.ctx[b]), cfg.T, t, cfg.causal) + 1
                  for b in range(cfg.B) for t in range(cfg.T))
    bytes_per = int(int(lay.ctx.astype(np.int64).sum()) * 132 + n * HI * (128 * 2 + 4) + visible * 4)
    flops = 2.0 * HI * 128 * visible
    ach = bytes_per / (call_avg * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
            # q and w of a request's tokens go to LDS when they fit 72 KB (272 + 4 bytes per token and
            # head), else q stays in registers
            "kernel": "mla_index_logits call: %s<%d>, timed with HIP events on its stream"
                      % ("index_logits_multi_kernel" if cfg.T * HI * 276 <= 72 * 1024 else "index_logits_kernel", HI),
            "algorithmic_bytes_per_launch": bytes_per, "flops_per_launch": flops,
            "mfma_tflops": round(flops / (call_avg * 1e-6) / 1e12, 1), "launch_us": round(call_avg, 3)}
    res = {
        "metric": "indexer logits query-tokens/s (FP8 keys of each context, %d index heads); %% of roofline" % HI,
        "value": round(n / (ms_per_step * 1e-3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "q_len": cfg.T, "index_heads": HI,
                   "context": cfg.ctx or list(cfg.ctx_range), "causal": cfg.causal, "key_bytes": 132,
                   "step": "index logits"},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        # the oracle over the first few requests (a bounded sample, one query-token group per host thread):
        # their pool pages copied out and renumbered
        nthreads = len(os.sched_getaffinity(0))
        S = max(1, min(cfg.B, nthreads, 16))
        pages = [lay.block_table[b][lay.block_table[b] >= 0] for b in range(S)]
        allp = np.concatenate(pages).astype(np.int64)
        host = pool.view(-1, ps)[torch.from_numpy(allp).to(dev)].cpu().numpy().reshape(-1)
        bt1 = np.full((S, max(p.size for p in pages)), -1, np.int32)
        off = 0
        for b in range(S):
            bt1[b, :pages[b].size] = np.arange(off, off + pages[b].size)
            off += pages[b].size
        q1 = q_sets[0][:S].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        w1 = w_sets[0][:S].contiguous().cpu().numpy()
        times, used = [], 1
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.index_logits(q1, w1, host, ps, off, bt1, lay.ctx[:S], causal=cfg.causal, nthreads=nthreads)
            times.append(time.perf_counter() - t0)
        used = min(nthreads, S * cfg.T)
        tmed = float(np.median(times))
        res["cpu_baseline"] = {"value": round(S * cfg.T / tmed, 3), "unit": "query-tokens/s", "cores": used,
                               "kind": "oracle", "sample": f"{S * cfg.T} of {n} query tokens (requests 0..{S - 1}), "
                                                           f"median of 3 runs of {tmed:.2f} s on {used} threads"}
    print(json.dumps(res), flush=True)


def bench_dsa_step(args):
    """A whole sparse decode step on one layer: indexer logits over each query token's context, the
    top-k of them, then the NVFP4 sparse decode over the chosen rows (the new rows' quantize-on-write
    included), each stage timed with HIP events on the one stream."""
    import torch
    import nvfp4_compressed_sparse_amd as M

    cfg = W.CONFIGS[args.workload]
    if not (cfg.topk and cfg.fmt == "nvfp4"):
        raise SystemExit("--op dsa-step applies to the sparse NVFP4 workloads")
    HI = args.index_heads
    dev = "cuda"
    torch.cuda.set_device(0)
    inp = W.device_inputs(cfg, dev, n_sets=2)
    lay = inp["layout"]
    pool = torch.zeros(lay.num_pages * cfg.page_stride, dtype=torch.uint8, device=dev)
    M.mla_kv_quant_nvfp4(inp["lat"], inp["rope"], inp["slots"], pool, cfg.page_stride, lay.num_pages)
    rows = torch.from_numpy(np.concatenate([inp["row_off"][b] + lay.ctx[b] - cfg.T + np.arange(cfg.T)
                                            for b in range(cfg.B)]).astype(np.int64)).to(dev)
    w_lat, w_rope, w_slots = inp["lat"][rows].contiguous(), inp["rope"][rows].contiguous(), inp["slots"][rows]
    del inp["lat"], inp["rope"]
    ips = M.INDEX_PAGE_BYTES
    ipool = torch.zeros(lay.num_pages * ips, dtype=torch.uint8, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed + 1)
    keys = torch.randn((inp["slots"].numel(), 128), generator=gen, device=dev).to(torch.bfloat16)
    M.mla_index_key_quant(keys, inp["slots"], ipool, ips, lay.num_pages)
    del keys
    torch.cuda.synchronize()
    n, maxc = cfg.B * cfg.T, int(lay.ctx.max())
    lens = torch.from_numpy(np.array([W.position_limit(int(lay.ctx[b]), cfg.T, t, cfg.causal) + 1
                                      for b in range(cfg.B) for t in range(cfg.T)], np.int32)).to(dev)
    qi = [torch.randn((cfg.B, cfg.T, HI, 128), generator=gen, device=dev).to(torch.bfloat16) for _ in range(2)]
    wi = [torch.randn((cfg.B, cfg.T, HI), generator=gen, device=dev) / HI ** 0.5 for _ in range(2)]
    logits = torch.empty((n, (maxc + 3) // 4 * 4), dtype=torch.float32, device=dev)
    tk_ws = torch.zeros(M.mla_index_topk_workspace_bytes(n, logits.shape[1]), dtype=torch.uint8, device=dev)
    idx = torch.empty((cfg.B, cfg.T, cfg.topk), dtype=torch.int32, device=dev)
    S = M.mla_sparse_decode_splits(cfg.B, cfg.T, cfg.H, cfg.topk)
    ws = torch.zeros(max(M.mla_sparse_decode_workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.topk, S), 256),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.B, cfg.T, cfg.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((cfg.B, cfg.T, cfg.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        k = i % 2
        if ev is not None:
            ev[0].record(stream)
        M.mla_index_logits(qi[k], wi[k], ipool, ips, lay.num_pages, inp["bt"], inp["ctx"], maxc, causal=cfg.causal,
                           out=logits, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        M.mla_index_topk(logits, lens, cfg.topk, out=idx.view(n, cfg.topk), workspace=tk_ws, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        if args.unfused:
            M.mla_kv_quant_nvfp4(w_lat, w_rope, w_slots, pool, cfg.page_stride, lay.num_pages, stream=stream)
            M.mla_sparse_decode(inp["q_sets"][k], pool, cfg.page_stride, lay.num_pages, inp["bt"], inp["ctx"], idx,
                                cfg.sm_scale, causal=cfg.causal, num_splits=S, out=out, lse=lse, workspace=ws,
                                stream=stream)
        else:  # the new rows written by the decode launch itself
            M.mla_sparse_decode_append(inp["q_sets"][k], pool, cfg.page_stride, lay.num_pages, inp["bt"], inp["ctx"],
                                       idx, w_lat, w_rope, cfg.sm_scale, causal=cfg.causal, num_splits=S, out=out,
                                       lse=lse, workspace=ws, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed steps with events at the two ends only; then the same steps with an event between stages (the
    # markers add a few microseconds each) for the per-stage split
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    stage = [float(np.mean([e[j].elapsed_time(e[j + 1]) * 1e3 for e in evs])) for j in range(3)]
    log(f"[bench] dsa step: {ms_per_step * 1e3:.1f} us/step; with stage markers: logits {stage[0]:.1f}, "
        f"top-k {stage[1]:.1f}, write + decode {stage[2]:.1f} us")
    res = {
        "metric": "sparse decode step (indexer logits + top-k + NVFP4 sparse-MLA decode) query-tokens/s",
        "value": round(n / (ms_per_step * 1e-3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/f16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "q_len": cfg.T, "H": cfg.H, "index_heads": HI,
                   "topk": cfg.topk, "context": cfg.ctx or list(cfg.ctx_range), "splits": S,
                   "step": "index logits + top-k + quantize %d rows + decode" % n},
        "stages_us": {"index_logits": round(stage[0], 2), "index_topk": round(stage[1], 2),
                      "write_and_decode": round(stage[2], 2)},
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def prepare_cpu_sample(cfg, inp, n_sample):
    """Host copies for the oracle over a bounded sample of the step's query tokens: the selected source
    rows of the sampled tokens, and the tokens' own new rows."""
    import torch
    lay = inp["layout"]
    nq = cfg.B * cfg.T
    if n_sample <= 0:
        n_sample = min(nq, 64)
    units = np.arange(nq)[:n_sample]
    idx_all = inp["idx_sets"][0].cpu().numpy() if cfg.topk else None
    q_all = inp["q_sets"][0].view(torch.int16).cpu().numpy().view(np.uint16)
    positions = {}
    for u in units:
        b, t = divmod(int(u), cfg.T)
        lim = W.position_limit(int(lay.ctx[b]), cfg.T, t, cfg.causal)
        if cfg.topk:
            ids = idx_all[b, t]
            pos = ids[(ids >= 0) & (ids <= lim)]
        else:
            pos = np.arange(lim + 1)
        positions[b] = np.union1d(positions.get(b, np.zeros(0, np.int64)), pos)
    src = {}
    for b, pos in positions.items():
        rows = torch.from_numpy(inp["row_off"][b] + pos).to("cuda")
        src[b] = (pos, inp["lat"][rows].view(torch.int16).cpu().numpy().view(np.uint16),
                  inp["rope"][rows].view(torch.int16).cpu().numpy().view(np.uint16))
    new_rows = torch.from_numpy(np.array([inp["row_off"][u // cfg.T] + lay.ctx[u // cfg.T] - cfg.T + u % cfg.T
                                          for u in units], np.int64)).to("cuda")
    new_lat = inp["lat"][new_rows].view(torch.int16).cpu().numpy().view(np.uint16)
    new_rope = inp["rope"][new_rows].view(torch.int16).cpu().numpy().view(np.uint16)
    return dict(units=units, src=src, idx=idx_all, q=q_all, ctx=lay.ctx.copy(), new_lat=new_lat, new_rope=new_rope,
                max_pages=lay.block_table.shape[1])


def run_cpu_baseline(cfg, cpu):
    """Time the FP64 oracle (as it stands) on this host: quantize-on-write of the sampled tokens' own
    rows plus the decode of the sampled tokens (one call, threaded over query tokens)."""
    import oracle
    nthreads = len(os.sched_getaffinity(0))
    # setup (untimed): a pool holding the pages of the selected rows, quantized by the oracle
    bt = np.full((cfg.B, cpu["max_pages"]), -1, np.int32)
    npg = 1
    for b, (pos, _, _) in cpu["src"].items():
        pages = np.unique(pos // 64)
        bt[b, pages] = np.arange(npg, npg + pages.size)
        npg += pages.size
    pool = np.zeros(npg * cfg.page_stride, np.uint8)
    for b, (pos, lat, rope) in cpu["src"].items():
        slots = bt[b, pos // 64].astype(np.int64) * 64 + pos % 64
        oracle.kv_quant(cfg.fmt, lat, rope, slots, pool, cfg.page_stride, npg)
    n = cpu["units"].size
    scratch = np.zeros(((n + 63) // 64) * cfg.page_stride, np.uint8)
    wslots = np.arange(n, dtype=np.int64)
    times, used = [], 1
    for rep in range(3):
        t0 = time.perf_counter()
        oracle.kv_quant(cfg.fmt, cpu["new_lat"], cpu["new_rope"], wslots, scratch, cfg.page_stride, (n + 63) // 64)
        if cfg.topk:
            _, _, used = oracle.sparse_decode(cpu["q"], pool, cfg.page_stride, npg, bt, cpu["ctx"], cpu["idx"],
                                              cfg.sm_scale, cfg.causal, units=cpu["units"], nthreads=nthreads,
                                              fmt=cfg.fmt)
        else:
            _, _, used = oracle.dense_decode_fp8(cpu["q"], pool, cfg.page_stride, npg, bt, cpu["ctx"], cfg.sm_scale,
                                                 cfg.causal, units=cpu["units"], nthreads=nthreads)
        times.append(time.perf_counter() - t0)
    tmed = float(np.median(times))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(n / tmed, 3), "unit": "query-tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"{n} of {cfg.B * cfg.T} query tokens of one step (their row writes + decode), "
                      f"median of {len(times)} runs of {tmed:.2f} s on {used} threads; {cpu_model}"}


if __name__ == "__main__":
    main()
