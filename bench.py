#!/usr/bin/env python3
"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = one pass of the whole path for the workload over one batch of
synthetic input already resident in HBM: the arrow block layout
(bsa_build_arrow_layout) followed by the block-sparse forward (bsa_forward)
for the 2K MMDiT shape (B=1, H=24, N=16896 = 512 text + 128x128 image
tokens, D=128, block 128, arrow window 8 on every head).  Content-driven
workloads (--workload C1/C3/C5) run the block selection (mean-pool scoring
fused with top-k in one call where it applies, else pool_scores +
select_topk) + forward.

Prints ONE JSON line.  `value` is the actual (kept-block) TFLOP/s of the
step; the dense-equivalent rate, the fraction of the bf16 MFMA peak, the
forward kernel's roofline entry (timed with HIP events on the launch stream)
and the CPU oracle's rate on a bounded sample are reported beside it.
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

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "block-sparse attn fwd TFLOP/s (actual + dense-equiv) and % bf16 MFMA peak"


def _src_hash(fp8: bool) -> str:
    h = hashlib.sha256()
    p = os.path.join(ROOT, "block_sparse_attention_18_amd", "csrc", "fp8.hip" if fp8 else "forward.hip")
    h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _traffic(workload: str, fp8: bool = False):
    """HBM bytes per forward launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    name = "forward_fp8" if fp8 else "forward"
    p = os.path.join(ROOT, "profiles", f"{name}_{workload.lower()}_traffic.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("forward_src_sha") != _src_hash(fp8):
        return None
    return d.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="C4")
    ap.add_argument("--window", type=int, default=None, help="override the arrow window")
    ap.add_argument("--no-split", action="store_true", help="run every row in one workgroup")
    ap.add_argument("--stride", default=None, help="neighbourhood workloads: stride 'rows,cols'")
    ap.add_argument("--nb-window", default=None, help="neighbourhood workloads: window 'rows,cols'")
    ap.add_argument("--nb-permuted", action="store_true",
                    help="neighbourhood workloads: permute Q, K, V to tile-major order and O, LSE back in "
                         "separate passes instead of the kernels' "
                         "natural-order gather")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="time a large dense bf16 GEMM (torch.mm, hipBLASLt) as the practical MFMA ceiling")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample (0 disables it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for HBM byte counters)")
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward (dQ, dK, dV) of the forward on the workload's "
                         "layout, for a synthetic output gradient")
    ap.add_argument("--score-grad", action="store_true",
                    help="also time the gradient of the mean-pool / projection block score "
                         "(dW and the pooled dQ, dK) for a seeded upstream gradient")
    ap.add_argument("--fp8", action="store_true",
                    help="run the forward in the FP8 (E4M3) mode on inputs quantised once "
                         "before the timed region (quantisation timed separately)")
    ap.add_argument("--reuse", type=int, default=0, metavar="T",
                    help="only run a T-step select-once / reuse loop (full attention for the first "
                         "T*skip steps, one selection, then the reused mask) with RSE and Jaccard "
                         "diagnostics, on --reuse-workload")
    ap.add_argument("--reuse-workload", default="C5")
    ap.add_argument("--reuse-skip", type=float, default=0.2)
    ap.add_argument("--reuse-diag-every", type=int, default=16,
                    help="diagnose every this many sparse steps (and the selection step)")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step (layout + forward [+ permutation back]) in a HIP graph, "
                         "check three replays against the eager step bit for bit, and time replays")
    ap.add_argument("--sweep-select", default=None, metavar="WORKLOAD",
                    help="only run the forward-time sweep over the top-k budget on a content-driven "
                         "workload (C3: k of the 64 image key blocks; C5: the fraction rho of each "
                         "column group) with a least-squares fit")
    ap.add_argument("--pool-probe", action="store_true",
                    help="only time the mean-pool scoring (bsa_pool_scores, MEANPOOL_PROJ) on Q and K of "
                         "the long-context shape (B=1, H=32, N=65536, D=128, block 128: 1.07 GB read), "
                         "with the last-level cache flushed before every call; a bandwidth probe, "
                         "not a workload")
    ap.add_argument("--unfused", action="store_true",
                    help="content-driven mean-pool workloads: score (bsa_pool_scores) and select "
                         "(bsa_select_topk) in two calls instead of the fused bsa_select_meanpool")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the kept-pairs sweep of the forward at the C4 shape "
                         "(arrow windows 0..127 and all-FULL) with a least-squares fit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only: the block-sparse path shards by (batch, head) "
              f"with no exchange, so a multi-GPU figure is not measured here (asked for "
              f"{args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_18_amd as bsa
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # a plain copy kernel of known size: reads and writes exactly MIB MiB
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": max(args.steps, 1)}))
        return
    if args.pool_probe:
        pool_probe(torch, bsa, dev, reps=max(args.steps // 5, 5))
        return
    if args.gemm_ceiling:
        # the practical bf16 MFMA rate on this machine: a large dense GEMM of
        # contiguous operands through the vendor library
        n = 8192
        a = torch.randn(n, n, device=dev).to(torch.bfloat16)
        b = torch.randn(n, n, device=dev).to(torch.bfloat16)
        for _ in range(3):
            torch.mm(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(args.steps, 1)
        e0.record()
        for _ in range(reps):
            torch.mm(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
        print(json.dumps({"gemm_ceiling": {"m": n, "n": n, "k": n, "dtype": "bf16", "ms": round(ms, 4),
                                           "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}}))
        return
    bsa.load()
    if args.sweep:
        print(json.dumps(sweep(torch, bsa, synth, dev)), flush=True)
        return
    if args.sweep_select:
        print(json.dumps(select_sweep(torch, bsa, synth, dev, args.sweep_select)), flush=True)
        return
    if args.reuse:
        print(json.dumps(reuse_loop(torch, bsa, synth, dev, args)), flush=True)
        return

    wl = synth.WORKLOADS[args.workload]
    if args.window is not None:
        wl = wl.replace(arrow_window=args.window)
    x = synth.make_inputs(wl)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    B, H, N, D, block = wl.B, wl.H, wl.N, wl.D, wl.block
    nB = wl.n_blocks
    q, k, v = d(x["q"]), d(x["k"]), d(x["v"])
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    post = None
    token_pairs = None
    nb_natural = False
    if wl.layout == "neighborhood":
        # inputs arrive in natural order: the step builds the layout and runs the
        # forward, which gathers the tile-major tiles from natural order and
        # scatters O, LSE back (FP8: the quantisation writes tile-major codes
        # from natural-order inputs; the backward gathers and scatters too);
        # with --nb-permuted it permutes Q, K, V to tile-major order and O, LSE
        # back in separate passes
        stride = tuple(int(v2) for v2 in args.stride.split(",")) if args.stride else wl.nb_stride
        window = tuple(int(v2) for v2 in args.nb_window.split(",")) if args.nb_window else wl.nb_window
        wl = wl.replace(nb_stride=stride, nb_window=window)
        nb = bsa.neighborhood(wl.text_len, wl.nb_grid, wl.nb_tile, wl.nb_window, wl.nb_stride)
        cap = bsa.neighborhood_capacity(B, H, nb)
        row_ptr = torch.empty(B * H * nB + 1, dtype=torch.int32, device=dev)
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        flags = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        kept_pairs = cap
        computed_heads = B * H
        R_, C_ = wl.nb_grid
        token_pairs = B * H * (wl.text_len * N + R_ * C_ * (wl.text_len + wl.nb_window[0] * wl.nb_window[1]))
        nb_natural = not args.nb_permuted
        if nb_natural:
            out_t, lse_t = out, lse

            def layout(mark=None):
                bsa.build_neighborhood_layout(B, H, nb, row_ptr=row_ptr, col_idx=col_idx, flags=flags)
            layout_parts = ("layout",)
        else:
            qn, kn, vn = q, k, v
            q, k, v = torch.empty_like(qn), torch.empty_like(kn), torch.empty_like(vn)
            out_t = torch.empty_like(q)
            lse_t = torch.empty_like(lse)

            def layout(mark=None):
                for src, dst in ((qn, q), (kn, k), (vn, v)):
                    bsa.permute_tokens(src, nb, out=dst)
                if mark is not None:
                    mark()
                bsa.build_neighborhood_layout(B, H, nb, row_ptr=row_ptr, col_idx=col_idx, flags=flags)
            layout_parts = ("permute_in", "layout")
        # the split policy from the geometry's closed-form row lengths
        split = bsa.neighborhood_split_policy(B, H, nb, block)
        fwd_kw = {}

        if not nb_natural:
            def post():
                bsa.permute_tokens(out_t, nb, inverse=True, lse=lse_t, out=out, lse_out=lse)
    elif wl.layout == "arrow":
        modes, wins = x["head_modes"], x["head_windows"]
        cap = bsa.arrow_capacity(B, H, N, block, wl.text_len, modes, wins)
        row_ptr = torch.empty(B * H * nB + 1, dtype=torch.int32, device=dev)
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        o_cache = d(x["o_cache"]) if "o_cache" in x else None
        lse_cache = torch.from_numpy(x["lse_cache"]).to(dev) if "lse_cache" in x else None
        kept_pairs = cap
        computed_heads = B * int((modes != bsa.HEAD_SKIP).sum())

        def layout(mark=None):
            bsa.build_arrow_layout(B, H, N, block, wl.text_len, modes, wins, device=dev,
                                   row_ptr=row_ptr, col_idx=col_idx)
        layout_parts = ("arrow",)
        fwd_kw = dict(head_modes=modes, o_cache=o_cache, lse_cache=lse_cache)
        split = bsa.arrow_split_policy(B, H, N, block, wl.text_len, modes, wins)
    else:
        w = torch.from_numpy(x["w"]).to(dev) if "w" in x else None
        scores = torch.empty((B, H, nB, nB), dtype=torch.float32, device=dev)
        ws_s = torch.empty(max(bsa.pool_scores_workspace_size(B, H, N, D, block, wl.score_mode,
                                                              wl.r if w is not None else 0), 16),
                           dtype=torch.uint8, device=dev)
        cap = bsa.select_capacity(B, H, nB, wl.text_blocks, wl.groups)
        row_ptr = torch.empty(B * H * nB + 1, dtype=torch.int32, device=dev)
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        ws_sel = torch.empty(max(int(bsa.load().bsa_select_workspace_size(B, H, nB)), 16),
                             dtype=torch.uint8, device=dev)

        fused = (wl.score_mode == synth.SCORE_MEANPOOL_PROJ and not args.unfused and
                 bsa.select_meanpool_applies(nB, wl.r, wl.text_blocks, wl.groups))
        if fused:
            ws_f = bsa.select_meanpool_workspace(B, H, N, block, wl.r, dev)

            def layout(mark=None):
                bsa.select_meanpool(q, k, block, w, wl.text_blocks, wl.groups, row_ptr=row_ptr,
                                    col_idx=col_idx, workspace=ws_f)
            layout_parts = ("select_meanpool",)
        else:
            def layout(mark=None):
                bsa.pool_scores(q, k, block, wl.score_mode, w=w, out=scores, workspace=ws_s)
                if mark is not None:
                    mark()
                bsa.select_topk(scores, wl.text_blocks, wl.groups, row_ptr=row_ptr, col_idx=col_idx,
                                workspace=ws_sel)
            layout_parts = ("pool_scores", "select")
        fwd_kw = {}
        computed_heads = B * H
        split = bsa.select_split_policy(B, H, nB, wl.text_blocks, wl.groups, block=block)
    if args.no_split or (args.fp8 and wl.layout == "neighborhood"):
        split = None
    if split is not None:   # workspace allocated once, outside the timed region
        split["workspace"] = torch.empty(
            bsa.split_workspace_size(B, H, N, D, block, split["max_chunks"], split["max_split_rows"]),
            dtype=torch.uint8, device=dev)
        fwd_kw["split"] = split

    quant = None
    if args.fp8:
        if wl.layout == "neighborhood":
            layout()                      # (permuted runs: the tile-major Q, K, V that are quantised)
        qnb = nb if nb_natural else None  # natural-order inputs, tile-major codes
        qkv8 = bsa.quantize_fp8(q, k, v, nb=qnb)
        ws_q = torch.empty(max(bsa.quantize_fp8_workspace_size(B, H, N, D), 16), dtype=torch.uint8,
                           device=dev)

        if wl.layout == "neighborhood":
            def forward():
                bsa.forward_fp8_neighborhood(qkv8, row_ptr, col_idx, flags, nb, out=out_t, lse=lse_t,
                                             natural=nb_natural)
        else:
            def forward():
                bsa.forward_fp8(qkv8, block, row_ptr, col_idx, out=out, lse=lse, **fwd_kw)

        def quantize():
            bsa.quantize_fp8(q, k, v, out=qkv8, workspace=ws_q, nb=qnb)
    elif wl.layout == "neighborhood":
        def forward():
            bsa.forward_neighborhood(q, k, v, row_ptr, col_idx, flags, nb, out=out_t, lse=lse_t, natural=nb_natural,
                                     **({"split": fwd_kw["split"]} if "split" in fwd_kw else {}))
    else:
        def forward():
            bsa.forward(q, k, v, block, row_ptr, col_idx, out=out, lse=lse, **fwd_kw)

    # warmup (also fixes kept_pairs for content-driven selection)
    for _ in range(max(args.warmup, 1)):
        layout()
        forward()
        if post is not None:
            post()
    torch.cuda.synchronize()
    if wl.layout != "arrow":
        kept_pairs = int(row_ptr[-1].item())

    flop_pair = 4.0 * block * block * D
    actual_flop = flop_pair * kept_pairs
    dense_flop = 4.0 * N * N * D * B * H

    # timed region: K steps; events on the launch stream mark the boundary
    # between the layout parts, the start and the end of the forward, and the
    # end of the step (a step starts where the previous one ended: no event
    # is recorded twice at one point of the stream)
    def new_ev():
        return torch.cuda.Event(enable_timing=True)
    ev = [[new_ev() for _ in range(len(layout_parts) + 3)] for _ in range(args.steps)]
    t0 = new_ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    prev = t0
    for s in range(args.steps):
        e = ev[s]
        e[0] = prev
        layout(mark=lambda: e[1].record(stream))
        e[-3].record(stream)
        forward()
        e[-2].record(stream)
        if post is not None:
            post()
            e[-1].record(stream)
        else:
            e[-1] = e[-2]
        prev = e[-1]
    t1 = prev
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    fwd_ms = [e[-3].elapsed_time(e[-2]) for e in ev]
    post_ms = float(np.median([e[-2].elapsed_time(e[-1]) for e in ev])) if post is not None else None
    fwd_avg = float(np.mean(fwd_ms))
    part_ms = {name: float(np.median([e[j].elapsed_time(e[j + 1]) for e in ev]))
               for j, name in enumerate(layout_parts)}
    graph = graph_step(torch, stream, layout, forward, post, [out, lse, row_ptr, col_idx], args.steps) \
        if args.graph else None
    if args.fp8:
        # quantisation of Q, K, V: reads them (V twice: channel maxima, then
        # codes) and writes the codes; the scales are negligible
        for _ in range(3):
            quantize()
        qe = [new_ev() for _ in range(11)]
        for j in range(10):
            qe[j].record(stream)
            quantize()
        qe[10].record(stream)
        torch.cuda.synchronize()
        q_ms = float(np.median([qe[j].elapsed_time(qe[j + 1]) for j in range(10)]))
        elems = B * H * N * D
        quant = {"ms": round(q_ms, 4), "hbm_bytes": 4 * 2 * elems + 3 * elems,
                 "GBps": round((4 * 2 * elems + 3 * elems) / (q_ms * 1e-3) / 1e9, 1)}
    cold = None
    if wl.layout == "select":
        cold = cold_layout_parts(torch, dev, stream, layout, B, H, N, D, nB, row_ptr,
                                 wl.score_mode == synth.SCORE_EXACT_AVGPOOL, fused=len(layout_parts) == 1)

    value = actual_flop / (ms_step * 1e-3) / 1e12
    achieved = actual_flop / (fwd_avg * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if args.fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.description}",
            "B": B, "H": H, "N": N, "D": D, "block": block,
            "layout": (f"arrow w={wl.arrow_window}" if wl.layout == "arrow" else
                       (f"neighbourhood grid={list(wl.nb_grid)} tile={list(wl.nb_tile)} "
                        f"window={list(wl.nb_window)} stride={list(wl.nb_stride)}"
                        if wl.layout == "neighborhood" else
                        f"select groups={list(wl.groups)} text_blocks={wl.text_blocks}")),
            "kept_pairs": kept_pairs,
            "kept_fraction": round(kept_pairs / (B * H * nB * nB), 4),
            "long_row_split": (None if split is None else
                               {k2: split[k2] for k2 in ("chunk_blocks", "max_chunks", "max_split_rows")}),
            "parallelism": "single GPU",
            "precision": ("E4M3 Q (per-token scale), K (per-64-key-tile scale), V (per-channel "
                          "scale) and P; fp32 accumulation; bf16 O" if args.fp8 else
                          "bf16 Q, K, V, P; fp32 accumulation; bf16 O"),
        },
        "dense_equiv_tflops": round(dense_flop / (ms_step * 1e-3) / 1e12, 2),
        "frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "forward_ms": round(fwd_avg, 4),
        "forward_ms_p10_p50_p90": [round(float(np.percentile(fwd_ms, q_)), 4) for q_ in (10, 50, 90)],
        "layout_ms": {k2: round(v2, 4) for k2, v2 in part_ms.items()},
        "scoring_ratio": (round(sum(part_ms.values()) / fwd_avg, 4) if wl.layout == "select" else None),
        "permute_out_ms": None if post_ms is None else round(post_ms, 4),
        "token_pairs": token_pairs,
        "token_level_tflops": (None if token_pairs is None else
                               round(4.0 * D * token_pairs / (fwd_avg * 1e-3) / 1e12, 2)),
        "layout_cold_cache": cold,
        "forward_dense_equiv_tflops": round(dense_flop / (fwd_avg * 1e-3) / 1e12, 2),
        "step_wall_ms": round(wall * 1e3 / args.steps, 4),
        "fp8_quantize": quant,
        "graph": graph,
        "roofline": {
            "bound": "mfma",
            "kernel": ("bsa::fwd8_kernel" if args.fp8 else
                       "bsa::fwd_kernel (+ split plan / combine when long rows are split)"),
            "achieved": round(achieved, 2),
            "peak": PEAK_FP8_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / (PEAK_FP8_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS), 4),
            "traffic": _traffic(wl.name, args.fp8),
            "algorithmic_flop_per_launch": actual_flop,
        },
        "cpu_baseline": None,
    }

    if args.backward:
        if args.fp8 or ("head_modes" in fwd_kw and fwd_kw["head_modes"] is not None
                        and np.any(fwd_kw["head_modes"] == bsa.HEAD_SKIP)):
            raise SystemExit("--backward: layouts without SKIP heads, bf16 only")
        nbk = (nb, flags, token_pairs, nb_natural) if wl.layout == "neighborhood" else None
        res["backward"] = backward_bench(torch, bsa, synth, dev, stream, wl, q, k, v, row_ptr, col_idx, kept_pairs,
                                         nbk=nbk)
    if args.score_grad:
        if wl.score_mode != bsa.SCORE_MEANPOOL_PROJ or wl.layout in ("arrow", "neighborhood"):
            raise SystemExit("--score-grad: a workload scored by mean-pool / projection (C1, C3)")
        res["score_grad"] = score_grad_bench(torch, bsa, dev, stream, wl, q, k, w)
    if args.cpu_seconds > 0 and not args.fp8:
        res["cpu_baseline"] = cpu_baseline(wl, x, row_ptr, col_idx, args.cpu_seconds,
                                           fwd_kw.get("head_modes"))
    print(json.dumps(res), flush=True)


def _evict_buffer(torch, dev):
    """512 MB, twice the last-level cache, written once here."""
    return torch.ones(128 << 20, dtype=torch.int32, device=dev)


def _evict(buf):
    """Read the eviction buffer (a reduction): the cache then holds its clean
    lines instead of the next call's inputs, and no dirty lines are left to
    be written back while the timed call runs."""
    buf.max()


def pool_probe(torch, bsa, dev, reps: int = 10):
    """Mean-pool scoring bandwidth at the long-context shape: Q and K (bf16
    [1, 32, 65536, 128], 1.07 GB) read once by the pooling kernel; the call
    also projects (r = 32) and scores the 512 x 512 block pairs of every head.
    Inputs are random (the rate does not depend on the values); a 512 MB
    read before every call evicts them from the 256 MB last-level cache."""
    B, H, N, D, block, r = 1, 32, 65536, 128, 128, 32
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    q = torch.randn((B, H, N, D), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((B, H, N, D), generator=g, device=dev).to(torch.bfloat16)
    w = torch.randn((D, r), generator=g, device=dev) / math.sqrt(D)
    nB = N // block
    S = torch.empty((B, H, nB, nB), dtype=torch.float32, device=dev)
    ws = torch.empty(bsa.pool_scores_workspace_size(B, H, N, D, block, bsa.SCORE_MEANPOOL_PROJ, r),
                     dtype=torch.uint8, device=dev)
    scratch = _evict_buffer(torch, dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(2):
        bsa.pool_scores(q, k, block, bsa.SCORE_MEANPOOL_PROJ, w=w, out=S, workspace=ws)
    ts = []
    for _ in range(reps):
        _evict(scratch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        bsa.pool_scores(q, k, block, bsa.SCORE_MEANPOOL_PROJ, w=w, out=S, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    nbytes = 2 * B * H * N * D * 2
    print(json.dumps({"pool_probe": {"shape": [B, H, N, D], "block": block, "r": r, "bytes_read": nbytes,
                                     "ms": round(ms, 4), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                     "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                     "note": "pool + projection + the 512 x 512 scores of 32 heads, cold cache"}}),
          flush=True)


def cold_layout_parts(torch, dev, stream, layout, B, H, N, D, nB, row_ptr, exact: bool, iters: int = 10,
                      fused: bool = False):
    """pool_scores and select timed with a 512 MB read before every
    call, so the 256 MB last-level cache does not serve their inputs.  Rates
    against the algorithmic work: mean-pool scores are HBM-bound (Q and K
    read once); exact scores are MFMA-bound (one Q K^T over all pairs, plus
    one exp per pair); select reads the score matrix once and writes the
    CSR once.  The fused mean-pool selection is one call: its rate counts Q
    and K read once."""
    scratch = _evict_buffer(torch, dev)
    if fused:
        t = []
        for _ in range(iters):
            _evict(scratch)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            layout()
            e[1].record(stream)
            torch.cuda.synchronize()
            t.append(e[0].elapsed_time(e[1]))
        ms = float(np.median(t))
        return {"select_meanpool_ms": round(ms, 4),
                "qk_read_GBps": round(2.0 * B * H * N * D * 2 / (ms * 1e-3) / 1e9, 1),
                "hbm_peak_GBps": PEAK_HBM_GBS}
    pool, sel = [], []
    for _ in range(iters):
        _evict(scratch)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        layout(mark=lambda: e[1].record(stream))
        e[2].record(stream)
        torch.cuda.synchronize()
        pool.append(e[0].elapsed_time(e[1]))
        sel.append(e[1].elapsed_time(e[2]))
    pool_ms, sel_ms = float(np.median(pool)), float(np.median(sel))
    nnz = int(row_ptr[-1].item())
    sel_bytes = 4.0 * B * H * nB * nB + 4.0 * (nnz + B * H * nB + 1)
    res = {"pool_scores_ms": round(pool_ms, 4)}
    if exact:
        flop = 2.0 * B * H * N * N * D
        res["pool_scores_tflops"] = round(flop / (pool_ms * 1e-3) / 1e12, 1)
        res["pool_scores_frac_mfma_peak"] = round(flop / (pool_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    else:
        res["pool_GBps"] = round(2.0 * B * H * N * D * 2 / (pool_ms * 1e-3) / 1e9, 1)
        res["hbm_peak_GBps"] = PEAK_HBM_GBS
    res["select_ms"] = round(sel_ms, 4)
    res["select_GBps"] = round(sel_bytes / (sel_ms * 1e-3) / 1e9, 1)
    return res


def sweep(torch, bsa, synth, dev, windows=(0, 1, 2, 4, 8, 18, 32, 64, 127), reps: int = 30):
    """Forward time against kept pairs at the C4 shape: arrow windows plus
    all-FULL heads; least-squares fit t = a + b * pairs."""
    base = synth.WORKLOADS["C4"]
    x = synth.make_inputs(base)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = d(x["q"]), d(x["k"]), d(x["v"])
    B, H, N, D, block = base.B, base.H, base.N, base.D, base.block
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    pts = []
    for w in list(windows) + ["full"]:
        modes = np.full(H, bsa.HEAD_FULL if w == "full" else bsa.HEAD_ARROW, dtype=np.int8)
        wins = np.full(H, 0 if w == "full" else w, dtype=np.int32)
        rp, ci = bsa.build_arrow_layout(B, H, N, block, base.text_len, modes, wins, device=dev)
        pairs = bsa.arrow_capacity(B, H, N, block, base.text_len, modes, wins)
        for _ in range(10):
            bsa.forward(q, k, v, block, rp, ci, out=out, lse=lse)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            bsa.forward(q, k, v, block, rp, ci, out=out, lse=lse)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        t = float(np.median(ts))
        pts.append({"window": w, "kept_pairs": pairs, "forward_ms": round(t, 4),
                    "tflops": round(4.0 * block * block * D * pairs / (t * 1e-3) / 1e12, 1)})
    xs = np.array([p_["kept_pairs"] for p_ in pts], dtype=np.float64)
    ys = np.array([p_["forward_ms"] for p_ in pts], dtype=np.float64)
    A = np.stack([np.ones_like(xs), xs], axis=1)
    (a, b), *_ = np.linalg.lstsq(A, ys, rcond=None)
    r2 = 1.0 - float(((ys - (a + b * xs)) ** 2).sum() / ((ys - ys.mean()) ** 2).sum())
    full = pts[-1]
    for p_ in pts:
        realised = full["forward_ms"] / p_["forward_ms"]
        theoretical = full["kept_pairs"] / p_["kept_pairs"]
        p_["speedup_realised_over_theoretical"] = round(realised / theoretical, 3)
    return {"sweep": "forward time vs kept pairs, C4 shape (B1 H24 N16896 D128 block 128)",
            "fit_ms": {"intercept": round(float(a), 4), "us_per_kept_pair": round(float(b) * 1e3, 6),
                       "r2": round(r2, 5)},
            "points": pts}


def graph_step(torch, stream, layout, forward, post, outs, steps):
    """One step captured in a HIP graph (torch.cuda.graph: the library's
    launches go to the capturing stream).  Three replays, each after an eager
    step, must reproduce the eager outputs bit for bit; then `steps` replays
    are timed with events."""
    def step():
        layout()
        forward()
        if post is not None:
            post()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        step()
        torch.cuda.synchronize()
        eager = [t.clone() for t in outs]
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(outs, eager)):
            raise SystemExit("a graph replay differs from the eager step")
    for _ in range(3):
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return {"ms_per_step": round(e0.elapsed_time(e1) / steps, 4), "replays_checked_bitwise": 3}


def select_sweep(torch, bsa, synth, dev, name, reps=None):
    """Forward time against kept pairs over the top-k budget of a
    content-driven workload: the scores are computed once, then each budget
    (every group's k scaled to the fraction rho of its width, up to all
    columns) is selected and its forward timed; least-squares fit
    t = a + b * pairs and realised over theoretical speedup against the
    all-columns point."""
    wl = synth.WORKLOADS[name]
    if wl.layout != "select":
        raise SystemExit("--sweep-select needs a content-driven (select) workload")
    x = synth.make_inputs(wl)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = d(x["q"]), d(x["k"]), d(x["v"])
    w = torch.from_numpy(x["w"]).to(dev) if "w" in x else None
    B, H, N, D, block, nB = wl.B, wl.H, wl.N, wl.D, wl.block, wl.n_blocks
    S = bsa.pool_scores(q, k, block, wl.score_mode, w=w)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    reps = reps or (30 if N <= 8192 else 5)
    pts = []
    for rho in (0.0625, 0.125, 0.25, 0.5, 0.75, 1.0):
        groups = tuple((c0, c1, max(1, int(round(rho * (c1 - c0))))) for c0, c1, _ in wl.groups)
        rp, ci = bsa.select_topk(S, wl.text_blocks, groups)
        split = bsa.select_split_policy(B, H, nB, wl.text_blocks, groups, block=block)
        kw = {"split": split} if split is not None else {}
        for _ in range(3):
            bsa.forward(q, k, v, block, rp, ci, out=out, lse=lse, **kw)
        torch.cuda.synchronize()
        pairs = int(rp[-1].item())
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            bsa.forward(q, k, v, block, rp, ci, out=out, lse=lse, **kw)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        t = float(np.median(ts))
        pts.append({"rho": rho, "groups": [list(g) for g in groups], "kept_pairs": pairs, "forward_ms": round(t, 4),
                    "tflops": round(4.0 * block * block * D * pairs / (t * 1e-3) / 1e12, 1)})
    xs = np.array([p_["kept_pairs"] for p_ in pts], dtype=np.float64)
    ys = np.array([p_["forward_ms"] for p_ in pts], dtype=np.float64)
    A = np.stack([np.ones_like(xs), xs], axis=1)
    (a, b), *_ = np.linalg.lstsq(A, ys, rcond=None)
    r2 = 1.0 - float(((ys - (a + b * xs)) ** 2).sum() / ((ys - ys.mean()) ** 2).sum())
    full = pts[-1]
    for p_ in pts:
        p_["speedup_realised_over_theoretical"] = round(
            (full["forward_ms"] / p_["forward_ms"]) / (full["kept_pairs"] / p_["kept_pairs"]), 3)
    return {"sweep": f"forward time vs top-k budget, {wl.name} shape (B{B} H{H} N{N} D{D} block {block})",
            "fit_ms": {"intercept": round(float(a), 4), "us_per_kept_pair": round(float(b) * 1e3, 6),
                       "r2": round(r2, 5)},
            "points": pts}


def reuse_loop(torch, bsa, synth, dev, args):
    """Select-once / reuse over T denoising steps (SparseD's schedule) on a
    content-driven workload.  Step s runs on X_s = X + a_s Z for X = the
    workload's Q, K, V, Z a seeded N(0, 1) drift and a_s = 0.5 (1 - s / T)
    (inputs that change less and less from step to step); the inputs of a
    step are formed before its timed region.  Full steps run the forward on
    the dense block list; the selection step runs scoring + top-k + the
    sparse forward; later steps reuse the mask.  At sampled steps the sparse
    output is compared with full attention (per-head RSE) and the reused
    mask with that step's own selection (per-head Jaccard); those extra
    computations are not timed."""
    wl = synth.WORKLOADS[args.reuse_workload]
    if wl.layout != "select":
        raise SystemExit("--reuse needs a content-driven (select) workload")
    T = args.reuse
    sched = bsa.ReuseSchedule(T, args.reuse_skip)
    B, H, N, D, block, nB = wl.B, wl.H, wl.N, wl.D, wl.block, wl.n_blocks
    x = synth.make_inputs(wl)
    z = synth.random_qkv(B, H, N, D, seed=wl.seed + 1000)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    base = [d(x["q"]), d(x["k"]), d(x["v"])]
    drift = [d(a) for a in z]
    w = torch.from_numpy(x["w"]).to(dev) if "w" in x else None
    del x, z
    cur = [torch.empty_like(t) for t in base]

    def set_inputs(s):
        a = 0.5 * (1.0 - s / T)
        for c, b0, z0 in zip(cur, base, drift):
            torch.add(b0, z0, alpha=a, out=c)

    full_modes = np.zeros(H, np.int8)
    rp_full, ci_full = bsa.build_arrow_layout(B, H, N, block, 0, full_modes, np.zeros(H, np.int32), device=dev)
    cap = bsa.select_capacity(B, H, nB, wl.text_blocks, wl.groups)
    rp_s = torch.empty(B * H * nB + 1, dtype=torch.int32, device=dev)
    ci_s = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    rp_f = torch.empty_like(rp_s)
    ci_f = torch.empty_like(ci_s)
    scores = torch.empty((B, H, nB, nB), dtype=torch.float32, device=dev)
    ws = torch.empty(max(bsa.pool_scores_workspace_size(B, H, N, D, block, wl.score_mode,
                                                        wl.r if w is not None else 0), 16),
                     dtype=torch.uint8, device=dev)
    ws_sel = torch.empty(max(int(bsa.load().bsa_select_workspace_size(B, H, nB)), 16), dtype=torch.uint8,
                         device=dev)
    out = torch.empty_like(cur[0])
    out_full = torch.empty_like(cur[0])
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def select(rp, ci):
        bsa.pool_scores(cur[0], cur[1], block, wl.score_mode, w=w, out=scores, workspace=ws)
        bsa.select_topk(scores, wl.text_blocks, wl.groups, row_ptr=rp, col_idx=ci, workspace=ws_sel)

    def fwd(rp, ci, o):
        bsa.forward(cur[0], cur[1], cur[2], block, rp, ci, out=o, lse=lse)

    # warm-up of every kernel the loop uses
    set_inputs(0)
    select(rp_s, ci_s)
    fwd(rp_s, ci_s, out)
    fwd(rp_full, ci_full, out_full)
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)
    times = {"full": [], "select": [], "sparse": []}
    diag = []
    for s in range(T):
        set_inputs(s)
        act = sched.action(s)
        e0, e1, e2 = ev(), ev(), ev()
        e0.record(stream)
        if act == "select":
            select(rp_s, ci_s)
        e1.record(stream)
        if act == "full":
            fwd(rp_full, ci_full, out)
        else:
            fwd(rp_s, ci_s, out)
        e2.record(stream)
        torch.cuda.synchronize()
        if act == "full":
            times["full"].append(e0.elapsed_time(e2))
        else:
            times["sparse"].append(e1.elapsed_time(e2))
            if act == "select":
                times["select"].append(e0.elapsed_time(e1))
        if act != "full" and (s - sched.n_full) % args.reuse_diag_every == 0 or (act == "sparse" and s == T - 1):
            fwd(rp_full, ci_full, out_full)
            rse = bsa.output_rse(out, out_full).cpu().numpy().reshape(-1)
            select(rp_f, ci_f)
            jac = bsa.mask_jaccard(B, H, nB, rp_s, ci_s, rp_f, ci_f).cpu().numpy().reshape(-1)
            diag.append({"step": s, "rse_mean": round(float(rse.mean()), 5),
                         "rse_max": round(float(rse.max()), 5),
                         "jaccard_mean": round(float(jac.mean()), 4),
                         "jaccard_min": round(float(jac.min()), 4)})
    med = {k2: (float(np.median(v2)) if v2 else None) for k2, v2 in times.items()}
    total = sum(sum(v2) for v2 in times.values())
    t_full = med["full"] if med["full"] is not None else None
    kept = int(rp_s[-1].item())
    res = {
        "mode": "reuse",
        "workload": f"{wl.name}: {wl.description}",
        "steps": T, "skip": args.reuse_skip, "schedule": sched.counts(),
        "step_ms_median": {k2: (round(v2, 3) if v2 is not None else None) for k2, v2 in med.items()},
        "attention_ms_total": round(total, 2),
        "kept_fraction": round(kept / (B * H * nB * nB), 4),
        "data": "synthetic: workload inputs plus a seeded drift that shrinks over the steps",
    }
    if t_full is not None and med["sparse"] is not None:
        res["full_every_step_ms"] = round(T * t_full, 2)
        res["amortised_speedup"] = round(sched.amortised_speedup(t_full, med["select"] or 0.0, med["sparse"]), 3)
        res["amortised_speedup_measured"] = round(T * t_full / total, 3)
    res["diagnostics"] = diag
    return res


def backward_bench(torch, bsa, synth, dev, stream, wl, q, k, v, row_ptr, col_idx, kept_pairs, reps=20, nbk=None):
    """Times bsa_backward (Delta/LSE prep, dQ kernel, dK/dV kernel) after one
    forward, for a seeded N(0, 1) output gradient.  Algorithmic work: the five
    products of the backward (S recomputed, dP, dV, dK, dQ), 10 * block^2 * D
    FLOP per kept block pair; the dQ and dK/dV kernels each recompute S and
    dP, so 14 * block^2 * D are executed.  nbk = (geometry, entry flags,
    token pairs, natural) runs the neighbourhood backward (on natural-order
    tensors if natural, else tile-major ones) and also reports the
    token-level rate (10 * D FLOP per kept token pair)."""
    B, H, N, D, block = wl.B, wl.H, wl.N, wl.D, wl.block
    g = synth.random_qkv(B, H, N, D, seed=wl.seed + 2000)[0]
    gd = torch.from_numpy(np.ascontiguousarray(g).view(np.int16)).view(torch.bfloat16).to(dev)
    if nbk is None:
        O, L = bsa.forward(q, k, v, block, row_ptr, col_idx)
    else:
        O, L = bsa.forward_neighborhood(q, k, v, row_ptr, col_idx, nbk[1], nbk[0], natural=nbk[3])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(int(bsa.load().bsa_backward_workspace_size(B, H, N)), dtype=torch.uint8, device=dev)

    def run():
        if nbk is None:
            bsa.backward(q, k, v, O, gd, block, row_ptr, col_idx, L, dq=dq, dk=dk, dv=dv, workspace=ws)
        else:
            bsa.backward_neighborhood(q, k, v, O, gd, row_ptr, col_idx, nbk[1], nbk[0], L, dq=dq, dk=dk, dv=dv,
                                      workspace=ws, natural=nbk[3])
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    for r in range(reps):
        ev[r].record(stream)
        run()
    ev[reps].record(stream)
    torch.cuda.synchronize()
    ms = [ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]
    med = float(np.median(ms))
    alg = 10.0 * block * block * D * kept_pairs
    return {"ms": round(med, 4), "ms_p10_p50_p90": [round(float(np.percentile(ms, x)), 4) for x in (10, 50, 90)],
            "algorithmic_tflops": round(alg / (med * 1e-3) / 1e12, 2),
            "executed_tflops": round(1.4 * alg / (med * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(alg / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "token_level_tflops": (None if nbk is None else
                                   round(10.0 * D * nbk[2] / (med * 1e-3) / 1e12, 2)),
            "flop_per_pair": "10 * block^2 * D (dQ, dK, dV, dP, S); 14 executed"}


def score_grad_bench(torch, bsa, dev, stream, wl, q, k, w, reps=50):
    """Times bsa_score_grad (pooling, g = dS p' and dS^T p, W g, the per-head
    partial dW and its reduction) for a seeded N(0, 1) upstream gradient.
    Algorithmic bytes: Q and K read once (bf16), dS read once, dW and the
    pooled gradients written once (fp32)."""
    B, H, N, D, block = wl.B, wl.H, wl.N, wl.D, wl.block
    nB, r = bsa.n_blocks(N, block), int(w.shape[1])
    g = np.random.default_rng(wl.seed + 3000).standard_normal((B, H, nB, nB)).astype(np.float32)
    dS = torch.from_numpy(g).to(dev)
    dw = torch.empty((D, r), dtype=torch.float32, device=dev)
    dqp = torch.empty((B, H, nB, D), dtype=torch.float32, device=dev)
    dkp = torch.empty_like(dqp)
    ws = torch.empty(bsa.score_grad_workspace_size(B, H, N, D, block, r), dtype=torch.uint8, device=dev)

    def run():
        bsa.score_grad(q, k, block, w, dS, dw=dw, dq_pool=dqp, dk_pool=dkp, workspace=ws)
    for _ in range(5):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    for i in range(reps):
        ev[i].record(stream)
        run()
    ev[reps].record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
    alg = 2 * B * H * N * D * 2 + B * H * nB * nB * 4 + D * r * 4 + 2 * B * H * nB * D * 4
    return {"ms": round(ms, 4), "algorithmic_bytes": alg, "GB_per_s": round(alg / (ms * 1e-3) / 1e9, 1),
            "kernels": "pool_proj, score_grad_p, score_grad_w, score_grad_reduce"}


def cpu_baseline(wl, x, row_ptr, col_idx, seconds, modes):
    """The fp64 CPU oracle's forward on a bounded sample of the workload's rows."""
    import oracle
    rp = row_ptr.cpu().numpy()
    ci = col_idx.cpu().numpy()[:rp[-1]]
    B, H, N, D, block = wl.B, wl.H, wl.N, wl.D, wl.block
    nB = wl.n_blocks
    rng = np.random.default_rng(0)
    comp = [h for h in range(H) if modes is None or modes[h] != 2]

    def rows_of(n):
        b = rng.integers(0, B, n)
        h = np.array(comp)[rng.integers(0, len(comp), n)]
        t = rng.integers(0, N, n)
        return ((b * H + h) * N + t).astype(np.int64)

    if wl.layout == "neighborhood":
        # the block list is in tile-major order; the oracle works in natural order
        perm = oracle.tile_permutation(wl.text_len, wl.nb_grid, wl.nb_tile)
        pos = np.empty_like(perm)
        pos[perm] = np.arange(N)

        def run(rows):
            oracle.forward_neighborhood(x["q"], x["k"], x["v"], wl.text_len, wl.nb_grid, wl.nb_window,
                                        wl.nb_stride, rows=rows)
    else:
        pos = np.arange(N)

        def run(rows):
            oracle.forward(x["q"], x["k"], x["v"], block, rp, ci, rows=rows)

    def flop(rows):
        # the metric's unit: 4 * block * D per kept block of the row's block row
        bh = rows // N
        r = bh * nB + pos[rows % N] // block
        kept = (rp[r + 1] - rp[r]).astype(np.float64)
        return float((4.0 * block * D * kept).sum())

    # grow the sample until it takes at least half the target time (a small
    # probe overestimates the per-row cost: thread start-up dominates it)
    n = 64
    while True:
        rows = rows_of(n)
        t = time.perf_counter()
        run(rows)
        dt = time.perf_counter() - t
        if dt >= 0.5 * seconds or n >= 1000000:
            break
        n = int(min(max(n * seconds / max(dt, 1e-3), 2 * n), 1000000))
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(flop(rows) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "cpu_model": cpu_model,
            "sample": f"{n} random query rows of the {wl.name} forward (fp64, kept blocks only), "
                      f"{dt:.1f} s"}


if __name__ == "__main__":
    main()
