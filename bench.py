#!/usr/bin/env python3
"""CoWA benchmark on one MI355X: 128K single-rank prefill and 128K decode.

One step = one prefill forward of the 128K single-rank workload at global KV
head g = 0 (B=1, N=131072, H_q=5, H_kv=1 of 8, d=128, S=128, W=8192, L=15360;
g = 0 carries the most band work, so it bounds a tensor-parallel step) and one
decode step of the 128K decode workload (B=16, H_q=40, H_kv=8, d=128, cached
lengths uniform in [98304, 131072]).  Inputs are seeded synthetic data already
resident in HBM.  Prints one JSON line.

value = prefill tokens/s (B*N / prefill time).  The decode figures, the other
seven global heads, the full-causal (FullAttn) mode and the backward of the
same prefill (training) sit in extra keys.  Kernel times come from HIP events
on the stream the library launches on.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CoWA prefill tokens/s + decode tokens/s at 128K, % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def visible_counts(t, g, sink, window, band):
    """Keys visible from query positions t (numpy array) for global head g:
    sink + band + local, made disjoint (metric accounting only)."""
    t = np.asarray(t, dtype=np.int64)
    s_end = np.minimum(sink, t + 1)
    l_lo = np.maximum(np.maximum(t - window + 1, 0), s_end)
    n = s_end + (t + 1 - l_lo)
    if band > 0:
        b_lo = np.maximum(t - (window + (g + 1) * band) + 1, s_end)
        b_hi = np.minimum(t - (window + g * band) + 1, l_lo)
        n = n + np.maximum(b_hi - b_lo, 0)
    return n


# headers every kernel source includes: a change to any of them, or to the
# kernel source itself, invalidates the counters recorded for that kernel
KERNEL_HEADERS = tuple(f"structured_sparse_attention_cowa_amd/csrc/{h}"
                       for h in ("cowa_internal.h", "cowa_pattern.h", "kernel_util.h",
                                  "cowa_layout.h"))


def source_digest(source: str) -> str:
    """sha256 of the kernel source followed by KERNEL_HEADERS."""
    import hashlib
    h = hashlib.sha256()
    for path in (source,) + KERNEL_HEADERS:
        h.update(open(os.path.join(ROOT, path), "rb").read())
    return h.hexdigest()


def traffic_record(kernel: str, source: str):
    """Calibrated HBM bytes per launch from the committed rocprofv3 summaries
    (profiles/*.md), or None when the kernel source or its headers changed
    since then."""
    import glob
    digest = source_digest(source)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if not line.startswith("traffic-record:"):
                continue
            f = dict(kv.split("=", 1) for kv in line.split()[1:])
            if f.get("kernel") == kernel and f.get("source_sha256") == digest:
                fb, wb = float(f["fetch_bytes"]), float(f["write_bytes"])
                return {"bytes": fb + wb, "fetch_bytes": fb, "write_bytes": wb,
                        "source": os.path.relpath(path, ROOT)}
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-head sweep and the full-causal comparison")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--only", choices=["prefill", "decode", "backward", "copy"], default=None,
                    help="profile a single kernel (rocprofv3 runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operator's tensor-parallel ranks are modelled by the global KV-head "
              "offset on one device)", file=sys.stderr)
        sys.exit(2)

    import torch

    from structured_sparse_attention_cowa_amd import binding as C
    from structured_sparse_attention_cowa_amd import workloads as W

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    need_prefill = args.only in (None, "prefill", "backward")
    need_decode = args.only in (None, "decode")
    need_backward = args.only == "backward" or (args.only is None and not args.no_backward)

    # ---------------- prefill setup ----------------
    wp = W.P128K
    B, N, Hq, Hkv, d = wp.B, wp.N, wp.H_q, wp.H_kv, wp.d
    if need_prefill:
        x = W.prefill_inputs(wp)
        q, k, v = to_dev(x.q_bits), to_dev(x.k_bits), to_dev(x.v_bits)
    o = torch.empty((B, N, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    bm, bn = C.cowa_fwd_block_sizes(d)
    scale = 1.0 / np.sqrt(d)

    def make_plan(g, mode=0):
        p = C.make_pattern(N, wp.sink, wp.window, 0, wp.h_kv_global, g, mode)
        rp, col, fl = C.cowa_plan(p, N, Hkv, bm, bn)
        return (p, torch.from_numpy(rp).to(dev), torch.from_numpy(col).to(dev),
                torch.from_numpy(fl).to(dev), len(col))

    t_plan0 = time.perf_counter()
    plan0 = make_plan(0) if need_prefill else None
    plan_ms = (time.perf_counter() - t_plan0) * 1e3

    fws = torch.empty(C.cowa_fwd_workspace_size(B, N, Hkv, d), dtype=torch.uint8, device=dev)

    def prefill(plan):
        p, rp, col, fl, nnz = plan
        C.cowa_fwd(p, rp, col, fl, nnz, bm, bn, q, k, v, o, lse, scale, workspace=fws)

    # ---------------- backward setup (same prefill, training) ----------------
    if need_backward:
        bmk, bnk = C.cowa_bwd_block_sizes(d)
        dout = to_dev(W.grad_output(7, B, N, Hq, d))
        dq = torch.empty((B, N, Hq, d), dtype=torch.bfloat16, device=dev)
        dk = torch.empty((B, N, Hkv, d), dtype=torch.bfloat16, device=dev)
        dv = torch.empty((B, N, Hkv, d), dtype=torch.bfloat16, device=dev)
        ws_bytes = max(C.cowa_bwd_workspace_size(C.make_pattern(N, wp.sink, wp.window, 0,
                                                                wp.h_kv_global, 0, mode),
                                                 B, Hq, Hkv, N) for mode in (0, 1))
        ws_b = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def make_plan_kv(plan):
        p = plan[0]
        rp, col, fl = C.cowa_plan_kv(p, N, Hkv, bmk, bnk)
        return (torch.from_numpy(rp).to(dev), torch.from_numpy(col).to(dev),
                torch.from_numpy(fl).to(dev), len(col))

    def backward(plan, plan_kv):
        p, rp, col, fl, nnz = plan
        rpk, colk, flk, nnzk = plan_kv
        C.cowa_bwd(p, rp, col, fl, nnz, bm, bn, rpk, colk, flk, nnzk, bmk, bnk, q, k, v, o,
                   dout, lse, dq, dk, dv, scale, ws_b)

    t_all = np.arange(N)
    G = Hq // Hkv
    pairs = [int(visible_counts(t_all, g, wp.sink, wp.window, wp.stated_band).sum())
             for g in range(wp.h_kv_global)]
    flops = [4.0 * d * G * B * pg for pg in pairs]

    # ---------------- decode setup ----------------
    wd = W.D128K
    lens = W.decode_lens(wd)
    qd = to_dev(W.decode_query(wd))
    if need_decode:
        kc, vc = W.decode_cache_device(wd, lens, device=dev)
    pd = C.make_pattern(wd.n_ctx, wd.sink, wd.window, 0, wd.h_kv_global, 0, 0)
    # the decode workspace needs no initialisation (partials are written before read)
    ws = torch.empty(C.cowa_decode_workspace_size(pd, wd.B, wd.H_q, wd.H_kv, wd.d, wd.n_max),
                     dtype=torch.uint8, device=dev)
    od = torch.empty((wd.B, wd.H_q, wd.d), dtype=torch.float32, device=dev)
    lsed = torch.empty((wd.B, wd.H_q), dtype=torch.float32, device=dev)
    sl = torch.from_numpy(lens).to(dev)
    vis_dec = sum(int(visible_counts(np.array([int(L) - 1]), g, wd.sink, wd.window,
                                     wd.stated_band)[0])
                  for L in lens for g in range(wd.H_kv))
    dec_bytes = vis_dec * wd.d * 2 * 2

    def decode():
        C.cowa_decode(pd, qd, kc, vc, sl, od, lsed, 1.0 / np.sqrt(wd.d), ws)

    torch.cuda.synchronize()

    if args.only is not None:
        # a few launches of one kernel for counter / trace runs
        if args.only == "copy":
            src = torch.empty(1 << 28, dtype=torch.uint8, device=dev)  # 256 MiB
            dst = torch.empty_like(src)
            for _ in range(args.steps):
                dst.copy_(src)
        if args.only == "backward":
            plan_kv0 = make_plan_kv(plan0)
            prefill(plan0)
        for _ in range(args.steps):
            if args.only == "prefill":
                prefill(plan0)
            elif args.only == "decode":
                decode()
            elif args.only == "backward":
                backward(plan0, plan_kv0)
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "steps": args.steps}))
        return

    # ---------------- timed steps ----------------
    for _ in range(args.warmup):
        prefill(plan0)
        decode()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        prefill(plan0)
        evs[i][1].record()
        decode()
        evs[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_per_step = wall * 1e3 / args.steps

    pre_tps = B * N / (pre_ms * 1e-3)
    dec_tps = wd.B / (dec_ms * 1e-3)
    pre_tflops = flops[0] / (pre_ms * 1e-3) / 1e12
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9

    def time_it(fn, reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fn()
        torch.cuda.synchronize()
        e[0].record()
        for _ in range(reps):
            fn()
        e[1].record()
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / reps

    extras = {}
    if not args.no_extras:
        per_g = []
        for g in range(wp.h_kv_global):
            pl = plan0 if g == 0 else make_plan(g)
            per_g.append(time_it(lambda: prefill(pl), 3))
        causal_plan = make_plan(0, mode=1)
        causal_ms = time_it(lambda: prefill(causal_plan), 2)
        causal_flops = 4.0 * d * G * B * (N * (N + 1) // 2)
        pd_c = C.make_pattern(wd.n_ctx, wd.sink, wd.window, 0, wd.h_kv_global, 0, 1)
        ws_c = torch.empty(C.cowa_decode_workspace_size(pd_c, wd.B, wd.H_q, wd.H_kv, wd.d,
                                                        wd.n_max), dtype=torch.uint8, device=dev)
        dec_causal_ms = time_it(lambda: C.cowa_decode(pd_c, qd, kc, vc, sl, od, lsed,
                                                      1.0 / np.sqrt(wd.d), ws_c), 3)
        # pattern variants on the same kernels: sliding-window attention with
        # sinks (no band) at the 128K rank, and the 8K ablation setting (8 KV
        # heads) with 1, 2, 4, 8 distinct long-range windows
        sl_plan = make_plan(0, mode=2)
        sl_ms = time_it(lambda: prefill(sl_plan), 3)
        sl_pairs = int(visible_counts(t_all, 0, wp.sink, wp.window, 0).sum())
        sl_flops = 4.0 * d * G * B * sl_pairs
        variants = {"sink_local_128k": {"ms": round(sl_ms, 4),
                                        "tflops": round(sl_flops / (sl_ms * 1e-3) / 1e12, 1),
                                        "mfma_frac": round(sl_flops / (sl_ms * 1e-3) / 1e12
                                                           / PEAK_BF16_TFLOPS, 4)},
                    "ablation_8k": ablation_8k(C, W, torch, dev, to_dev, time_it)}
        # decode on windowed caches (each KV head keeps its sink and a ring of
        # the positions later queries can still see)
        rows, total_rows = C.cowa_kv_window_rows(pd, wd.H_kv, wd.n_max)
        kw = torch.empty((wd.B, total_rows, wd.d), dtype=torch.bfloat16, device=dev)
        vw = torch.empty_like(kw)
        C.cowa_kv_window_fill(pd, kc, vc, sl, kw, vw)
        dec_win_ms = time_it(lambda: C.cowa_decode_window(pd, qd, kw, vw, sl, od, lsed, wd.H_kv,
                                                          wd.n_max, 1.0 / np.sqrt(wd.d), ws), 5)
        del kw, vw
        decode_window = {
            "us": round(dec_win_ms * 1e3, 2),
            "tokens_per_s": round(wd.B / (dec_win_ms * 1e-3), 1),
            "hbm_frac": round(dec_bytes / (dec_win_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "kv_rows_per_sequence": int(total_rows),
            "full_cache_rows_per_sequence": wd.H_kv * wd.n_max,
            "memory_ratio_all_heads": round(wd.H_kv * wd.n_max / total_rows, 3),
            "rows_per_head": [int(r) for r in rows],
            "memory_ratio_per_rank": [round(wd.n_max / int(r), 3) for r in rows],
        }
        extras = {
            "prefill_32k": prefill_32k(C, W, torch, dev, to_dev, time_it),
            "prefill_8k": prefill_8k(C, W, torch, dev, to_dev, time_it),
            "varlen_prefill": varlen_prefill(C, W, torch, dev, time_it),
            "decode_window": decode_window,
            "variants": variants,
            "prefill_per_g": [{"g": g, "ms": round(per_g[g], 4),
                               "tflops": round(flops[g] / (per_g[g] * 1e-3) / 1e12, 1),
                               "mfma_frac": round(flops[g] / (per_g[g] * 1e-3) / 1e12
                                                  / PEAK_BF16_TFLOPS, 4)}
                              for g in range(wp.h_kv_global)],
            # the eight g together are one tensor-parallel step's ranks run
            # one after another on this GPU
            "prefill_all_g": {"ms_sum": round(float(np.sum(per_g)), 4),
                              "tflops": round(float(np.sum(flops)) / (np.sum(per_g) * 1e-3)
                                              / 1e12, 1),
                              "mfma_frac": round(float(np.sum(flops)) / (np.sum(per_g) * 1e-3)
                                                 / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "prefill_causal_mode": {"ms": round(causal_ms, 4),
                                    "tflops": round(causal_flops / (causal_ms * 1e-3) / 1e12, 1),
                                    "cowa_speedup_g0": round(causal_ms / per_g[0], 3),
                                    "cowa_speedup_mean_g": round(causal_ms / np.mean(per_g), 3)},
            "decode_causal_mode": {"us": round(dec_causal_ms * 1e3, 2),
                                   "cowa_speedup": round(dec_causal_ms / dec_ms, 3)},
        }

    if need_backward:
        # O and LSE of the forward at g = 0 feed the backward, as in training
        plan_kv0 = make_plan_kv(plan0)
        prefill(plan0)
        bwd_ms = time_it(lambda: backward(plan0, plan_kv0), max(3, args.steps // 2))
        causal_plan_b = make_plan(0, mode=1)
        causal_kv = make_plan_kv(causal_plan_b)
        prefill(causal_plan_b)
        bwd_causal_ms = time_it(lambda: backward(causal_plan_b, causal_kv), 2)
        prefill(plan0)
        # dQ, dK, dV from S, P, dP, dS: five products of the visible pairs
        # (the kernels recompute S and dP once more for dQ)
        bwd_flops = 2.5 * flops[0]
        bwd_tflops = bwd_flops / (bwd_ms * 1e-3) / 1e12
        extras["backward"] = {
            "workload": "backward of the 128K single-rank prefill at g=0 (O fp32 from the "
                        "forward, dO N(0,1) bf16, dQ/dK/dV bf16)",
            "ms": round(bwd_ms, 4),
            "tokens_per_s": round(B * N / (bwd_ms * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(bwd_tflops, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
                         "algorithmic_flops_per_call": bwd_flops},
            "fwd_plus_bwd_ms": round(pre_ms + bwd_ms, 4),
            "causal_mode_ms": round(bwd_causal_ms, 4),
            "cowa_speedup_vs_causal": round(bwd_causal_ms / bwd_ms, 3),
        }

    tr_pre = traffic_record("cowa_fwd_kernel", "structured_sparse_attention_cowa_amd/csrc/fwd.hip")
    tr_dec = traffic_record("cowa_decode_split",
                            "structured_sparse_attention_cowa_amd/csrc/decode.hip")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, wp, scale)

    out = {
        "metric": METRIC,
        "value": round(pre_tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "CoWA 128K single-rank prefill (B=1, N=131072, H_q=5, H_kv=1 of 8, "
                        "g=0, d=128, S=128, W=8192, L=15360) + 128K decode step (B=16, "
                        "H_q=40, H_kv=8, d=128, lens U[98304,131072])",
            "global_batch": B, "seq_len": N, "parallelism": "single-gpu (one TP rank)",
        },
        "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": tr_pre["bytes"] if tr_pre else None,
                     "traffic_detail": tr_pre,
                     "kernel": "cowa_fwd_kernel<128,true>",
                     "algorithmic_flops_per_launch": flops[0]},
        "cpu_baseline": cpu,
        "prefill": {"ms": round(pre_ms, 4), "tokens_per_s": round(pre_tps, 1),
                    "visible_flops": flops[0], "plan_host_ms": round(plan_ms, 2)},
        "decode": {"us": round(dec_ms * 1e3, 2), "tokens_per_s": round(dec_tps, 1),
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                                "traffic": tr_dec["bytes"] if tr_dec else None,
                                "traffic_detail": tr_dec,
                                "algorithmic_bytes_per_step": dec_bytes}},
    }
    out.update(extras)
    print(json.dumps(out), flush=True)


def _prefill_modes(C, W, torch, dev, to_dev, time_it, w):
    """CoWA and full-causal prefill of one workload (all KV heads, offset 0)."""
    x = W.prefill_inputs(w)
    q, k, v = to_dev(x.q_bits), to_dev(x.k_bits), to_dev(x.v_bits)
    o = torch.empty((w.B, w.N, w.H_q, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H_q, w.N), dtype=torch.float32, device=dev)
    bm, bn = C.cowa_fwd_block_sizes(w.d)
    fws = torch.empty(C.cowa_fwd_workspace_size(w.B, w.N, w.H_kv, w.d), dtype=torch.uint8,
                      device=dev)
    G = w.H_q // w.H_kv
    t = np.arange(w.N)
    res = {}
    for mode, name in ((0, "cowa"), (1, "causal")):
        p = C.make_pattern(w.N, w.sink, w.window, 0, w.h_kv_global, 0, mode)
        rp, col, fl = [torch.from_numpy(a).to(dev) for a in C.cowa_plan(p, w.N, w.H_kv, bm, bn)]
        ms = time_it(lambda: C.cowa_fwd(p, rp, col, fl, col.numel(), bm, bn, q, k, v, o, lse,
                                        1.0 / np.sqrt(w.d), workspace=fws), 5)
        if mode == 0:
            pairs = sum(int(visible_counts(t, g, w.sink, w.window, w.stated_band).sum())
                        for g in range(w.H_kv))
        else:
            pairs = w.H_kv * w.N * (w.N + 1) // 2
        flops = 4.0 * w.d * G * w.B * pairs
        res[name] = {"ms": round(ms, 4), "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1),
                     "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                     "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    res["cowa_speedup"] = round(res["causal"]["ms"] / res["cowa"]["ms"], 3)
    return res


def prefill_32k(C, W, torch, dev, to_dev, time_it):
    """The 32K workload (B=1, N=32768, H_q=40, H_kv=8, d=128, S=128, W=4096,
    L=3584, Q rows RMS 1.5), CoWA and full-causal mode."""
    r = _prefill_modes(C, W, torch, dev, to_dev, time_it, W.P32K)
    r["workload"] = "B=1, N=32768, H_q=40, H_kv=8, d=128, S=128, W=4096, L=3584"
    return r


def prefill_8k(C, W, torch, dev, to_dev, time_it):
    """The 8K workload (B=2, N=8192, H_q=32, H_kv=8, d=128, S=64, W=1024,
    L=896, 5% of keys x4), CoWA and full-causal mode."""
    r = _prefill_modes(C, W, torch, dev, to_dev, time_it, W.P8K)
    r["workload"] = "B=2, N=8192, H_q=32, H_kv=8, d=128, S=64, W=1024, L=896"
    return r


def ablation_8k(C, W, torch, dev, to_dev, time_it):
    """Prefill of the 8K workload (B=2, N=8192, H_q=32, H_kv=8, S=64, W=1024,
    L=896) with m distinct long-range windows shared out over the 8 KV heads."""
    w = W.P8K
    x = W.prefill_inputs(w)
    q, k, v = to_dev(x.q_bits), to_dev(x.k_bits), to_dev(x.v_bits)
    o = torch.empty((w.B, w.N, w.H_q, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H_q, w.N), dtype=torch.float32, device=dev)
    bm, bn = C.cowa_fwd_block_sizes(w.d)
    fws = torch.empty(C.cowa_fwd_workspace_size(w.B, w.N, w.H_kv, w.d), dtype=torch.uint8,
                      device=dev)
    G = w.H_q // w.H_kv
    t = np.arange(w.N)
    out = []
    for m in (1, 2, 4, 8):
        p = C.make_pattern(w.N, w.sink, w.window, 0, w.h_kv_global, 0, 0, m)
        rp, col, fl = [torch.from_numpy(a).to(dev) for a in C.cowa_plan(p, w.N, w.H_kv, bm, bn)]
        ms = time_it(lambda: C.cowa_fwd(p, rp, col, fl, col.numel(), bm, bn, q, k, v, o, lse,
                                        1.0 / np.sqrt(w.d), workspace=fws), 5)
        pairs = sum(int(visible_counts(t, g % m, w.sink, w.window, w.stated_band).sum())
                    for g in range(w.H_kv))
        flops = 4.0 * w.d * G * w.B * pairs
        out.append({"distinct_windows": m, "ms": round(ms, 4),
                    "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                    "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
    return out


def varlen_prefill(C, W, torch, dev, time_it):
    """Packed prefill of 8 sequences of seeded lengths in [4096, 32768] (the
    32K workload's heads: H_q=40, H_kv=8, d=128, S=128, W=4096, L=3584)."""
    w = W.VARLEN32K
    lens = w.lengths()
    T, max_len = int(lens.sum()), int(lens.max())
    q, k, v, cu = W.varlen_device(w, dev)
    o = torch.empty((T, w.H_q, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.H_q, T), dtype=torch.float32, device=dev)
    p = C.make_pattern(w.n_ctx, w.sink, w.window, 0, w.h_kv_global, 0, 0)
    bm, bn = C.cowa_fwd_block_sizes(w.d)
    rp, col, fl = [torch.from_numpy(a).to(dev) for a in C.cowa_plan(p, max_len, w.H_kv, bm, bn)]
    fws = torch.empty(C.cowa_fwd_workspace_size(len(lens), max_len, w.H_kv, w.d),
                      dtype=torch.uint8, device=dev)
    ms = time_it(lambda: C.cowa_fwd_varlen(p, rp, col, fl, col.numel(), bm, bn, q, k, v, o, lse,
                                           cu, max_len, 1.0 / np.sqrt(w.d), workspace=fws), 5)
    band = C.cowa_band_length(p)
    G = w.H_q // w.H_kv
    pairs = 0
    for n in lens:
        t = np.arange(int(n))
        pairs += sum(int(visible_counts(t, g, w.sink, w.window, band).sum())
                     for g in range(w.H_kv))
    flops = 4.0 * w.d * G * pairs
    # the packed backward of the same batch (O and LSE from the forward above,
    # dO N(0,1) drawn on the device; bf16 gradients): five products of the pairs
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 1)
    do = torch.randn((T, w.H_q, w.d), generator=gen, device=dev).to(torch.bfloat16)
    dq = torch.empty((T, w.H_q, w.d), dtype=torch.bfloat16, device=dev)
    dk = torch.empty((T, w.H_kv, w.d), dtype=torch.bfloat16, device=dev)
    dv = torch.empty((T, w.H_kv, w.d), dtype=torch.bfloat16, device=dev)
    bmk, bnk = C.cowa_bwd_block_sizes(w.d)
    rpk, colk, flk = [torch.from_numpy(a).to(dev)
                      for a in C.cowa_plan_kv(p, max_len, w.H_kv, bmk, bnk)]
    ws = torch.empty(C.cowa_bwd_workspace_size(p, len(lens), w.H_q, w.H_kv, max_len),
                     dtype=torch.uint8, device=dev)
    ms_b = time_it(lambda: C.cowa_bwd_varlen(p, rp, col, fl, col.numel(), bm, bn, rpk, colk, flk,
                                             colk.numel(), bmk, bnk, q, k, v, o, do, lse, dq,
                                             dk, dv, cu, max_len, 1.0 / np.sqrt(w.d), ws), 3)
    flops_b = 2.5 * flops
    return {"workload": f"{w.n_seqs} packed sequences, lengths {[int(x) for x in lens]} "
                        f"({T} tokens), H_q=40, H_kv=8, d=128, S=128, W=4096, L={band}",
            "ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "backward": {"ms": round(ms_b, 4), "tokens_per_s": round(T / (ms_b * 1e-3), 1),
                         "tflops": round(flops_b / (ms_b * 1e-3) / 1e12, 1),
                         "mfma_frac": round(flops_b / (ms_b * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                            4)}}


def cpu_baseline(x, wp, scale, target_s=12.0):
    """The fp64 oracle on a seeded sample of query rows of the same prefill
    workload (all 5 query heads per row), timed on the host cores."""
    import oracle.cowa_oracle as O

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    p = O.Pattern(wp.N, wp.sink, wp.window, 0, wp.h_kv_global, 0, 0)
    q, k, v = x.q(), x.k(), x.v()
    rng = np.random.Generator(np.random.PCG64(1234))
    rows_all = np.sort(rng.choice(wp.N, 4096, replace=False))
    n = 16
    t0 = time.perf_counter()
    O.attention(q, k, v, p, scale, rows=rows_all[:n])
    dt = time.perf_counter() - t0
    n2 = int(min(len(rows_all), max(n, n * target_s / max(dt, 1e-3))))
    rows = np.sort(rng.choice(rows_all, n2, replace=False))
    t0 = time.perf_counter()
    O.attention(q, k, v, p, scale, rows=rows)
    dt = time.perf_counter() - t0
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(len(rows) / dt, 3), "unit": "tokens/s", "cores": cores,
            "cpu_model": cpu_model, "kind": "oracle",
            "sample": f"{len(rows)} seeded random query rows (all 5 heads) of the 128K "
                      f"single-rank prefill at g=0, dense masked fp64 softmax, {dt:.1f} s"}


if __name__ == "__main__":
    main()
