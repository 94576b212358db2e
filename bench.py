"""Benchmark of the DCOCO corrector hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--workload q8b_32]

A step is one dcoco_correct_block call: top-K, representations, pair states,
transition scores and the greedy walk for N draft blocks.  The default
workload is 32 streams of B = 16 slots, K = 16 candidates, d = 4096,
V = 151936 (bf16 storage, fp32 accumulation).  Inputs are seeded synthetic
tensors resident in HBM before timing starts; R >= 4 independently seeded
input sets (logits and hidden states; the embedding table and the weights are
shared) rotate from step to step so that one step's logits are not still in
the 256 MB Infinity Cache from the step before.

Prints one JSON line: blocks/s over the timed steps, plus per-stage times
from HIP events on the stream the stages run on, the roofline of the dominant
kernel and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
# fp32 vector issue: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-ops/s
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
# a grid element costs 7 lane-op slots: fma, rcp (quarter rate: 4 slots), add, fma
GRID_ELEM_PEAK = VALU_LANE_OPS / 7


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="q8b_32")
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--stage-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-blocks", type=int, default=64)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (1/4/8/16 streams, K = 64, d = 8192)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for scaling HBM counters)")
    ap.add_argument("--no-btable", action="store_true", help="skip the table-path timing")
    ap.add_argument("--no-lm-head", action="store_true", help="skip the fused LM-head top-K timing")
    ap.add_argument("--no-stress", action="store_true", help="skip the top-K stress-row timing")
    ap.add_argument("--no-attainable", action="store_true", help="skip the copy / library-GEMM reference rates")
    ap.add_argument("--null-stream", action="store_true",
                    help="launch on the null stream instead of a stream of our own")
    return ap.parse_args()


def algorithmic_work(D):
    """Bytes and flops the method itself must move / compute per call, by
    stage (weights read once per call)."""
    e = 2 if D.dtype == "bf16" else 4
    R = D.n_blocks * D.B
    RK = R * D.K
    P = D.n_blocks * (D.B - 1)
    w_params = (D.r * D.e + D.r * D.d + D.r_z * 2 * D.r + D.r_s * 2 * D.d
                + D.H * (2 * D.r_z + D.r_s) + 2 * D.H)
    w = {
        "logit_bytes": R * D.V * e,
        "gather_bytes": RK * D.e * e,
        "h_bytes": R * D.d * e,
        "slot_weight_bytes": (D.r + 2 * D.r_s) * D.d * e,
        "weight_bytes": w_params * e,
        # representation stage: P_e E[c], [P_h; W_L; W_R] h, and the fusion
        # W_f [b; g] (its g half once per slot, its b half once per candidate)
        "cand_flops": 2.0 * RK * D.e * D.r,
        "slot_flops": 2.0 * R * D.d * (D.r + 2 * D.r_s),
        "fuse_flops": 2.0 * (R * D.r * D.r_z + RK * D.r * D.r_z),
        # scoring stage: W1a z and W1b z per candidate, W1s s_p per pair
        "ab_flops": 2.0 * RK * D.r_z * 2 * D.H,
        "pair_flops": 2.0 * P * D.r_s * D.H,
        # representation backward: P_e E[c] and P_h h again, dz W_f, dW_f,
        # dP_e, [dP_h; dW_pair] and dh (each product counted once)
        "rep_bwd_flops": 2.0 * (2 * RK * D.e * D.r + R * D.d * D.r + 2 * RK * D.r_z * 2 * D.r
                                + 2 * R * D.d * (D.r + 2 * D.r_s)),
        "grid_elems": P * D.K * D.K * D.H,
        "transitions": P * D.K * D.K,
    }
    w["represent_flops"] = w["cand_flops"] + w["slot_flops"] + w["fuse_flops"]
    w["score_mfma_flops"] = w["ab_flops"] + w["pair_flops"]
    w["total_bytes"] = w["logit_bytes"] + w["gather_bytes"] + w["h_bytes"] + w["weight_bytes"]
    return w


def copy_calibration():
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give the
    factor between what those counters read and the bytes actually moved."""
    import torch
    n = 256 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 5}), flush=True)


def source_digest(paths):
    """Digest of kernel sources with comments and blank lines removed; a stored
    counter figure is used only while it matches (comment edits keep it)."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p)) as f:
            txt = f.read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        txt = re.sub(r"//[^\n]*", "", txt)
        lines = [ln.rstrip() for ln in txt.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


def stored_traffic(kernel, digest):
    """HBM bytes per launch read from a committed counter summary, or None when
    the summary is missing or was taken from other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        m = re.match(r"^- (\w+): (\S+)$", line.strip())
        if m:
            vals[m.group(1)] = m.group(2)
    if vals.get("source_digest") != digest or "hbm_bytes_per_launch" not in vals:
        return None
    return float(vals["hbm_bytes_per_launch"])


KERNEL_SOURCES = ["topk.hip", "gemm.hip", "rep.hip", "score.hip", "score_slab.hip", "api.cpp", "common.h", "dma.h", "gemm_tile.h", "kernels.h",
                  "ln_tile.h", "select.h", "wave.h"]


def stored_kernel_figures(name, digest):
    """Per-kernel figures from a committed rocprofv3 summary
    (profiles/<name>.md: lines '- <kernel>.<field>: <value>'), or None when the
    file is missing or was taken from other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{name}.md")
    if not os.path.exists(path):
        return None
    vals, figs = {}, {}
    for line in open(path):
        m = re.match(r"^- ([\w.]+): (\S+)$", line.strip())
        if not m:
            continue
        key, v = m.group(1), m.group(2)
        if "." in key:
            k, f = key.split(".", 1)
            figs.setdefault(k, {})[f] = float(v)
        else:
            vals[key] = v
    if vals.get("source_digest") != digest:
        return None
    return figs


def kernel_rooflines(figs, work):
    """Each profiled kernel against the bound of its own work: algorithmic
    bytes or flops per launch over its profiled duration, and the counters'
    HBM bytes against the algorithmic ones where they were taken."""
    bounds = {
        # kernel key: (bound, algorithmic work per launch, unit)
        "topk": ("hbm", work["logit_bytes"]),
        "cand_gemm": ("mfma", work["cand_flops"]),
        "slot_gemm": ("mfma", work["slot_flops"]),
        "ab_gemm": ("mfma", work["ab_flops"]),
        "pair_term": ("mfma", work["pair_flops"]),
        "grid": ("alu", work["grid_elems"]),
        "slab": ("alu", work["grid_elems"]),
        # top-K rows and the slot GEMM in one launch: the logits, h and the
        # slot weights read once
        "topk_gemm": ("hbm", work["logit_bytes"] + work["h_bytes"] + work["slot_weight_bytes"]),
    }
    out = {}
    for k, f in figs.items():
        us = f.get("us")
        if us is None:
            continue
        e = {"us": us}
        if k in bounds:
            bound, amount = bounds[k]
            rate = amount / (us * 1e-6)
            if bound == "hbm":
                e.update(bound="hbm", achieved_GBps=round(rate / 1e9, 1), frac=round(rate / 1e9 / HBM_PEAK_GBS, 4))
            elif bound == "mfma":
                e.update(bound="mfma", achieved_TFLOPs=round(rate / 1e12, 1),
                         frac=round(rate / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4))
            else:
                e.update(bound="alu", elems_per_s=round(rate, 1), frac=round(rate / GRID_ELEM_PEAK, 4))
        if "hbm_bytes" in f:
            e["hbm_bytes_per_launch"] = f["hbm_bytes"]
            e["hbm_GBps"] = round(f["hbm_bytes"] / (us * 1e-6) / 1e9, 1)
            if "algo_bytes" in f:
                e["traffic_over_algorithmic"] = round(f["hbm_bytes"] / f["algo_bytes"], 3)
        if "mfma_busy" in f:
            e["mfma_busy_frac"] = f["mfma_busy"]
        out[k] = e
    return out


def time_workload(dc, torch, dims, w, E, dsets, stream, desc, steps=20, reps=10):
    """Whole-path and per-stage times of one workload on rotating input sets;
    each figure is one event pair around calls queued back to back."""
    N, B, K = dims.n_blocks, dims.B, dims.K
    dev = E.device
    dt = dims.dtype
    ws = torch.empty(dc.correct_block_workspace_bytes(dims, w), dtype=torch.uint8, device=dev)
    sel = torch.empty((N, B), dtype=torch.int32, device=dev)

    def timed(fn, n):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    us = timed(lambda i: dc.correct_block(dims, w, dsets[i % len(dsets)][0], dsets[i % len(dsets)][1], E,
                                          sel_tok=sel, workspace=ws, stream=stream), steps)
    R = N * B
    ids = torch.empty((R, K), dtype=torch.int32, device=dev)
    cl = torch.empty((R, K), dtype=torch.float32, device=dev)
    z = torch.empty((N, B, K, dims.d_z), dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device=dev)
    s = torch.empty((N, max(B - 1, 1), dims.d_pair), dtype=torch.float32, device=dev)
    S = torch.empty((N, max(B - 1, 1), K, K), dtype=torch.float32, device=dev)
    si = torch.empty((N, B), dtype=torch.int32, device=dev)
    st = {
        "topk": timed(lambda i: dc.topk(dims, dsets[i % len(dsets)][0], ids, cl, workspace=ws, stream=stream), reps),
        "represent": timed(lambda i: dc.represent(dims, w, dsets[i % len(dsets)][1], E, ids, z, s, workspace=ws,
                                                  stream=stream), reps),
        "score": timed(lambda i: dc.score(dims, w, z, s, cl, S, workspace=ws, stream=stream), reps),
        "select": timed(lambda i: dc.select(dims, S, cl, ids, si, sel, stream=stream), reps),
    }

    class _D:
        pass
    Dw = _D()
    Dw.n_blocks, Dw.B, Dw.K, Dw.V = N, B, K, dims.V
    Dw.d, Dw.e, Dw.r, Dw.r_z, Dw.r_s, Dw.H, Dw.dtype = (dims.d_hidden, dims.d_embed, dims.d_proj, dims.d_z,
                                                        dims.d_pair, dims.d_mlp, dt)
    wk = algorithmic_work(Dw)
    del ws, ids, cl, z, s, S, si, sel
    return {"workload": desc, "us_per_call": round(us, 2), "blocks_per_s": round(N / (us * 1e-6), 1),
            "transitions_per_s": round(wk["transitions"] / (us * 1e-6), 1),
            "stage_us": {k: round(v, 2) for k, v in st.items()},
            "hbm_frac_topk": round(wk["logit_bytes"] / (st["topk"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac_represent": round(wk["represent_flops"] / (st["represent"] * 1e-6) / 1e12
                                         / MFMA_BF16_PEAK_TFLOPS, 4),
            "alu_frac_score": round(wk["grid_elems"] / (st["score"] * 1e-6) / GRID_ELEM_PEAK, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(blocks are independent; sharding would split the streams).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration()
        return
    import draft_block_contextual_amd as dc
    import synth

    def to_dev(a, dtype, device):
        if dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return t.to(device)

    if not os.path.exists(dc.LIB_PATH):
        from draft_block_contextual_amd import build as _b
        _b.build()
    dc.load()
    cfg = synth.get_config(args.workload)
    D = cfg.dims
    dev = "cuda:0"
    torch.cuda.set_device(0)
    print(f"# generating inputs for {cfg.name}: {cfg.desc}", file=sys.stderr, flush=True)
    base = synth.make_inputs(cfg)
    sets = [{"logits": base["logits"], "h": base["h"]}]
    for j in range(1, args.sets):
        sets.append(synth.make_stream_inputs(cfg, cfg.seed + 100 * j))
    dims = dc.Dims.from_synth(D)
    dt = D.dtype
    w = dc.Weights(P_e=to_dev(base["P_e"], dt, dev), P_h=to_dev(base["P_h"], dt, dev),
                   W_f=to_dev(base["W_f"], dt, dev), W_pair=to_dev(base["W_pair"], dt, dev),
                   W1=to_dev(base["W1"], dt, dev), b1=to_dev(base["b1"], dt, dev),
                   w2=to_dev(base["w2"], dt, dev), b2=base["b2"])
    E = to_dev(base["E"], dt, dev)
    dsets = [(to_dev(s["logits"].reshape(D.n_blocks * D.B, D.V), dt, dev), to_dev(s["h"], dt, dev))
             for s in sets]
    N, B, K = D.n_blocks, D.B, D.K
    sel_tok = torch.empty((N, B), dtype=torch.int32, device=dev)
    ws = torch.empty(dc.correct_block_workspace_bytes(dims, w), dtype=torch.uint8, device=dev)
    # a stream of our own (default priority), as a serving loop would use
    stream = torch.cuda.current_stream() if args.null_stream else torch.cuda.Stream()
    print("# inputs resident; warming up", file=sys.stderr, flush=True)

    def step(i):
        lg, h = dsets[i % len(dsets)]
        dc.correct_block(dims, w, lg, h, E, sel_tok=sel_tok, workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / args.steps
    blocks_per_s = N * args.steps / (gpu_ms / 1e3)
    print(f"# timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (wall {wall * 1e3 / args.steps:.1f})",
          file=sys.stderr, flush=True)

    # ---- per-call latency: the same steps one at a time, an event pair each
    # (outside the timed region above; the host waits between calls)
    call_us = []
    for i in range(min(args.steps, 100)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step(i)
        b.record(stream)
        b.synchronize()
        call_us.append(a.elapsed_time(b) * 1e3)
    call_us = np.asarray(call_us)
    latency = {"p10": round(float(np.percentile(call_us, 10)), 2), "p50": round(float(np.median(call_us)), 2),
               "p90": round(float(np.percentile(call_us, 90)), 2), "calls": int(call_us.size)}

    # ---- the table path (a next step beyond the per-call path): b_v = LN(P_e E_v)
    # built once for the weight set, outside the timed region, then the same
    # steps with b gathered from the table.  Reported beside `value`, not as it.
    btable = None
    if dt == "bf16" and not args.no_btable:
        tb0 = torch.cuda.Event(enable_timing=True)
        tb1 = torch.cuda.Event(enable_timing=True)
        tb0.record(stream)
        tab = dc.build_btable(dims, w, E, stream=stream)
        tb1.record(stream)
        torch.cuda.synchronize()
        build_ms = tb0.elapsed_time(tb1)
        wsb = torch.empty(dc.correct_block_workspace_bytes(dims, w, btable=True), dtype=torch.uint8, device=dev)

        def step_t(i):
            lg, h = dsets[i % len(dsets)]
            dc.correct_block(dims, w, lg, h, None, sel_tok=sel_tok, workspace=wsb, stream=stream, btable=tab)

        for i in range(args.warmup):
            step_t(i)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(args.steps):
            step_t(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        t_ms = ev0.elapsed_time(ev1) / args.steps
        btable = {"value": round(N / (t_ms / 1e3), 1), "unit": "blocks/s", "ms_per_step": round(t_ms, 5),
                  "table_build_ms": round(build_ms, 3),
                  "table": f"[V={D.V}, d_proj={D.r}] bf16, built once per weight set"}
        print(f"# table path: {t_ms * 1e3:.1f} us/step (table built in {build_ms:.2f} ms)", file=sys.stderr,
              flush=True)
        del tab, wsb

    # ---- per-stage times: each entry point alone, between events on the same stream
    R = N * B
    ids = torch.empty((R, K), dtype=torch.int32, device=dev)
    cl = torch.empty((R, K), dtype=torch.float32, device=dev)
    z = torch.empty((N, B, K, D.r_z), dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device=dev)
    s = torch.empty((N, max(B - 1, 1), D.r_s), dtype=torch.float32, device=dev)
    S = torch.empty((N, max(B - 1, 1), K, K), dtype=torch.float32, device=dev)
    si = torch.empty((N, B), dtype=torch.int32, device=dev)
    stages = {
        "topk": lambda i: dc.topk(dims, dsets[i % len(dsets)][0], ids, cl, workspace=ws, stream=stream),
        "represent": lambda i: dc.represent(dims, w, dsets[i % len(dsets)][1], E, ids, z, s, workspace=ws,
                                            stream=stream),
        "score": lambda i: dc.score(dims, w, z, s, cl, S, workspace=ws, stream=stream),
        "select": lambda i: dc.select(dims, S, cl, ids, si, sel_tok, stream=stream),
        # the whole-path rules on the same grid (reported beside the stages)
        "select_global_sum": lambda i: dc.select_path(dims, S, cl, ids, "global_sum", 1.0, si, sel_tok,
                                                      stream=stream),
        "select_discount": lambda i: dc.select_path(dims, S, cl, ids, "discount", 0.75, si, sel_tok,
                                                    stream=stream),
        # the training side on the same grid: loss and dL/dS, then the MLP backward
        "train_loss": lambda i: dc.loss(dims, S, ids, targets(), 4.0, stream=stream),
        "train_backward": lambda i: dc.score_backward(dims, w, z, s, S, stream=stream),
    }
    if dt == "bf16":
        # and on through the representations (P_e, P_h, W_f, W_pair and dh)
        gen = torch.Generator(device=dev).manual_seed(7)
        dzr = torch.randn((N, B, K, D.r_z), generator=gen, device=dev) / N
        dsr = torch.randn((N, max(B - 1, 1), D.r_s), generator=gen, device=dev) / N
        torch.cuda.synchronize()     # made on torch's stream, read on the bench stream
        stages["train_rep_backward"] = lambda i: dc.represent_backward(dims, w, dsets[i % len(dsets)][1], E, ids,
                                                                       dzr, dsr, stream=stream)
    tgt_cache = []

    def targets():
        # one of each slot's candidates, drawn once (seeded) after top-K has run
        if not tgt_cache:
            pick = torch.from_numpy(np.random.default_rng(5).integers(0, K, (N, B, 1))).to(dev)
            with torch.cuda.stream(stream):     # ids were written on this stream
                tgt_cache.append(torch.gather(ids.view(N, B, K), 2, pick).view(N, B).to(torch.int32).contiguous())
        return tgt_cache[0]
    stage_us = {}
    for name, fn in stages.items():
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        # one event pair around stage_reps calls queued back to back, so the
        # host's enqueue time between calls does not show as idle GPU time
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(args.stage_reps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        stage_us[name] = float(a.elapsed_time(b) * 1e3 / args.stage_reps)
    print(f"# stage us: {stage_us}", file=sys.stderr, flush=True)

    # ---- next row: the drafter's LM head fused with top-K (head tied to E),
    # beside the same product through the BLAS library followed by dcoco_topk
    lm_head = None
    if dt == "bf16" and D.d == D.e and not args.no_lm_head:
        L = synth.make_lm_head_inputs(cfg, base["E"])
        hd = to_dev(L["hd"], dt, dev)
        for _ in range(3):
            dc.lm_head_topk(dims, hd, E, ids, cl, stream=stream)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        reps = 10
        a.record(stream)
        for _ in range(reps):
            dc.lm_head_topk(dims, hd, E, ids, cl, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        fused_us = a.elapsed_time(b) * 1e3 / reps
        with torch.cuda.stream(stream):
            for _ in range(3):
                lg = torch.matmul(hd, E.t())
                dc.topk(dims, lg, ids, cl, stream=stream)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(reps):
                lg = torch.matmul(hd, E.t())
                dc.topk(dims, lg, ids, cl, stream=stream)
            b.record(stream)
        torch.cuda.synchronize()
        unfused_us = a.elapsed_time(b) * 1e3 / reps
        flops = 2.0 * N * B * D.V * D.d
        lm_head = {"us": round(fused_us, 1), "tflops": round(flops / (fused_us * 1e-6) / 1e12, 1),
                   "mfma_frac": round(flops / (fused_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                   "unfused_us": round(unfused_us, 1),
                   "shape": f"[{N * B}, {D.d}] x [{D.V}, {D.d}]^T, top-{K}, bf16"}
        print(f"# lm head + top-K: {fused_us:.1f} us fused, {unfused_us:.1f} us as library GEMM + dcoco_topk",
              file=sys.stderr, flush=True)
        del lg, hd

    # ---- top-K on stress rows (not in the metric): no planted peaks, rising
    # and falling ramps, constant rows; same shape as the timed logits
    topk_stress = None
    if dt == "bf16" and not args.no_stress:
        R_, V_ = N * B, D.V
        gen = torch.Generator(device=dev).manual_seed(11)
        cases = {
            "flat_normal_sd2": lambda: (torch.randn(R_, V_, generator=gen, device=dev) * 2).to(torch.bfloat16),
            "ramp_up": lambda: torch.linspace(-12, 12, V_, device=dev).to(torch.bfloat16).repeat(R_, 1),
            "ramp_down": lambda: torch.linspace(12, -12, V_, device=dev).to(torch.bfloat16).repeat(R_, 1),
            "constant": lambda: torch.full((R_, V_), 1.5, device=dev, dtype=torch.bfloat16),
        }
        topk_stress = {}
        for cname, make in cases.items():
            with torch.cuda.stream(stream):     # made on the stream that reads them
                lgs = make()
            for _ in range(2):
                dc.topk(dims, lgs, ids, cl, workspace=ws, stream=stream)
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(5):
                dc.topk(dims, lgs, ids, cl, workspace=ws, stream=stream)
            b.record(stream)
            torch.cuda.synchronize()
            topk_stress[cname] = round(a.elapsed_time(b) * 1e3 / 5, 1)
            del lgs
        topk_stress["unit"] = "us per dcoco_topk call"
        print(f"# top-K stress rows: {topk_stress}", file=sys.stderr, flush=True)

    # ---- attainable rates on this GPU, beside the spec-sheet peaks: a device
    # copy (read + write bytes) and a large bf16 GEMM through the BLAS library
    attain = None
    if not args.no_attainable:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        ga = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        gb = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        torch.cuda.synchronize()     # made on torch's stream, read on the bench stream
        with torch.cuda.stream(stream):
            for _ in range(3):
                dst.copy_(src)
                torch.matmul(ga, gb)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            a.record(stream)
            for _ in range(10):
                dst.copy_(src)
            b.record(stream)
        torch.cuda.synchronize()
        copy_gbs = 2 * src.numel() * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
        with torch.cuda.stream(stream):
            a.record(stream)
            for _ in range(10):
                torch.matmul(ga, gb)
            b.record(stream)
        torch.cuda.synchronize()
        gemm_tf = 2.0 * 8192 ** 3 * 10 / (a.elapsed_time(b) * 1e-3) / 1e12
        attain = {"copy_GBps": round(copy_gbs, 1), "bf16_gemm_TFLOPs": round(gemm_tf, 1),
                  "how": "256 MiB device copy (bytes read + written); 8192^3 bf16 matmul through torch"}
        del src, dst, ga, gb
        print(f"# attainable: {attain}", file=sys.stderr, flush=True)

    work = algorithmic_work(D)
    # Dominant kernel: top-K, one launch per dcoco_topk call, so the events
    # around that call time exactly that kernel.  It is bound by reading the
    # logits once from HBM.
    kname = "topk_bf16_row_reg_kernel" if dt == "bf16" else "topk_partial_kernel+topk_merge_kernel"
    topk_us = stage_us["topk"]
    ach = work["logit_bytes"] / (topk_us * 1e-6) / 1e9
    digest = source_digest([f"draft_block_contextual_amd/csrc/{f}"
                            for f in ("topk.hip", "common.h", "dma.h", "gemm_tile.h", "kernels.h", "select.h",
                                      "wave.h")])
    traffic = stored_traffic(f"topk_{cfg.name}", digest)
    roof = {"bound": "hbm", "kernel": kname, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic / (topk_us * 1e-6) / 1e9, 1),
            "traffic_bytes_per_launch": traffic,
            "algorithmic_bytes_per_launch": work["logit_bytes"], "launch_us": round(topk_us, 2),
            "source_digest": digest}
    if attain is not None:
        # the same achieved rate against the device-copy rate measured above
        roof["frac_of_copy"] = round(ach / attain["copy_GBps"], 4)
    # ---- CPU oracle on a bounded sample of the same workload, its BLAS on
    # every core of this process's affinity mask; then single-threaded on the
    # tiny workload and on one block of this workload (the one-stream shape)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import dcoco_oracle as O
        from threadpoolctl import threadpool_limits
        cores = len(os.sched_getaffinity(0))
        nb = max(1, min(args.cpu_blocks, N * len(sets)))
        with threadpool_limits(cores):
            t = time.perf_counter()
            done = 0
            for j, sj in enumerate(sets):
                take = min(N, nb - done)
                if take <= 0:
                    break
                O.correct_block({**base, "logits": sj["logits"], "h": sj["h"]}, blocks=list(range(take)))
                done += take
            el = time.perf_counter() - t
        single = {}
        with threadpool_limits(1):
            tiny = synth.make_inputs("tiny")
            t = time.perf_counter()
            reps = 0
            while time.perf_counter() - t < 1.0:
                O.correct_block(tiny)
                reps += 1
            single["tiny"] = round(reps / (time.perf_counter() - t), 2)
            t = time.perf_counter()
            O.correct_block(base, blocks=[0])
            single[f"one_block_of_{cfg.name}"] = round(1.0 / (time.perf_counter() - t), 3)
        cpu = {"value": round(nb / el, 4), "unit": "blocks/s", "cores": cores, "kind": "oracle",
               "sample": f"{nb} blocks ({nb // N} whole input sets of {N} blocks"
                         f"{f' + {nb % N} blocks' if nb % N else ''}, same shapes as the timed steps), "
                         f"NumPy float64 with BLAS on {cores} threads, {el:.1f} s",
               "single_thread_blocks_per_s": single}

    # ---- every kernel of the step against its own bound, from the committed
    # rocprofv3 summaries of this command (durations, HBM counters, MFMA busy
    # cycles), used only while the kernel sources match the ones profiled
    kdig = source_digest([f"draft_block_contextual_amd/csrc/{f}" for f in KERNEL_SOURCES])
    figs = stored_kernel_figures(f"kernels_{cfg.name}", kdig)
    kernels = {"source_digest": kdig, "from": f"profiles/kernels_{cfg.name}.md" if figs else None}
    if figs:
        kernels.update(kernel_rooflines(figs, work))

    out = {
        "metric": "corrected draft blocks/sec @B=16,K=16,d=4096,32 streams; % HBM/MFMA peak",
        "value": round(blocks_per_s, 1),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == "bf16" else "f32",
        "data": f"synthetic, seeded; {len(dsets)} rotating input sets",
        "config": {"workload": f"{cfg.name}: {cfg.desc}", "streams": N, "B": B, "K": K, "d": D.d,
                   "V": D.V, "embed": D.e, "proj": D.r, "mlp_hidden": D.H},
        "transitions_per_s": round(work["transitions"] * args.steps / (gpu_ms / 1e3), 1),
        "stage_us": {k: round(v, 2) for k, v in stage_us.items()},
        # each stage against its own work, timed live (the stage's entry point
        # alone, between events on the stream it runs on)
        "mfma_frac_represent": round(work["represent_flops"] / (stage_us["represent"] * 1e-6) / 1e12
                                     / MFMA_BF16_PEAK_TFLOPS, 4),
        "mfma_frac_score": round(work["score_mfma_flops"] / (stage_us["score"] * 1e-6) / 1e12
                                 / MFMA_BF16_PEAK_TFLOPS, 4),
        "alu_frac_score": round(work["grid_elems"] / (stage_us["score"] * 1e-6) / GRID_ELEM_PEAK, 4),
        "mfma_frac_rep_backward": (round(work["rep_bwd_flops"] / (stage_us["train_rep_backward"] * 1e-6) / 1e12
                                         / MFMA_BF16_PEAK_TFLOPS, 4) if "train_rep_backward" in stage_us else None),
        "latency_us": latency,
        "roofline": roof,
        "kernels": kernels,
        "attainable": attain,
        "topk_stress": topk_stress,
        "cpu_baseline": cpu,
        "btable_path": btable,
        "lm_head_topk": lm_head,
    }
    # ---- the other workloads: one stream, the 4/8/16-stream sweep (the
    # first n blocks of the same rotating input sets), the K = 64 stress shape
    # and the d = 8192 shape (drawn on the GPU: see synth.make_inputs_device)
    if not args.no_configs:
        other = {}
        for n in (1, 4, 8, 16):
            dn = dc.Dims.from_synth(D)
            dn.n_blocks = n
            sub = [(lg[: n * B], h[:n]) for lg, h in dsets]
            other[f"q8b_{n}" if cfg.name == "q8b_32" else f"{cfg.name}@{n}"] = time_workload(
                dc, torch, dn, w, E, sub, stream, f"{n} streams of the {cfg.name} shapes")
        if dt == "bf16" and cfg.name == "q8b_32":
            for name in ("kstress", "large"):
                xc = synth.get_config(name)
                print(f"# drawing {name} on the GPU: {xc.desc}", file=sys.stderr, flush=True)
                g = synth.make_inputs_device(xc, sets=args.sets, device=dev)
                torch.cuda.synchronize()     # drawn on torch's stream, read on the bench stream
                wx = dc.Weights(P_e=g["P_e"], P_h=g["P_h"], W_f=g["W_f"], W_pair=g["W_pair"], W1=g["W1"],
                                b1=g["b1"], w2=g["w2"], b2=g["b2"])
                other[name] = time_workload(dc, torch, dc.Dims.from_synth(xc.dims), wx, g["E"], g["sets"], stream,
                                            xc.desc)
                del g, wx
                torch.cuda.empty_cache()
        out["workloads"] = other
        print(f"# other workloads: { {k: v['us_per_call'] for k, v in other.items()} }", file=sys.stderr,
              flush=True)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
