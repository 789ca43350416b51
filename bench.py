#!/usr/bin/env python3
"""MoE-layer throughput of the intra-expert-sparse expert FFN on one MI355X.

Workload: a synthetic Qwen-MoE-style decode layer (hidden 2048, 128 experts of
intermediate 768, top-8 softmax routing, bf16 weights, fp32 accumulation), the
gate bias channel and correlated tokens of the synthetic generator, threshold
calibrated on the GPU to 85% intra-expert sparsity.  One step is one call of
moe_sparse_expert_ffn on a batch of T tokens (default 64): routing, grouping,
dense gate + SiLU + threshold + ballot, gathered up, gathered down, combine.
Batches rotate over 16 draws so that expert weights are not reused from the
256 MB Infinity Cache between steps.  The timed calls are replayed from a HIP
graph that holds the calls on all 16 batches in order, as a caller that
captures a whole forward pass replays them; the time per call with one call
per graph, and with eager launches, is reported beside it.

Prints ONE JSON line (rank 0) with the headline tokens/s, the roofline of the
dominant kernel (expert projection: gate, score, mask, up), the speedup over
the library's own dense mode, a batch sweep, the time of the top-k neuron
selection variant at the same sparsity, and the CPU oracle's throughput on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at 1 MI355X + HBM GB/s fraction; speedup vs dense"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16
ROTATE = 16
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_expert_projection_qwen_decode_T64.json")
# sources compiled into the expert projection kernel: a stored HBM-traffic
# measurement is used only while they are unchanged
KERNEL_SRCS = [os.path.join(ROOT, "intra_expert_activation_amd", "csrc", f)
               for f in ("proj.hip", "gemv_rows.h", "mfma_body.h", "moe_internal.h", "wave_reduce.h")]


def kernel_src_sha256():
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


# name: (config id, default batch, default q, default sweep, description)
WORKLOADS = {
    "decode": (2, 64, 0.85, "1,8,16,32", "qwen-moe-style decode layer: H 2048, 128 experts x I 768, top-8"),
    "prefill": (5, 4096, 0.70, "", "qwen-moe-style prefill layer: H 2048, 128 experts x I 768, top-8"),
    "mixtral": (3, 16, 0.90, "1,128", "mixtral-style layer: H 4096, 8 experts x I 14336, top-2"),
    "deepseek": (4, 64, 0.85, "1,8,32", "deepseek-v2-lite-style layer: H 2048, 64 experts x I 1408 top-6 "
                                          "+ 2 shared experts, zipf routing"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="decode")
    ap.add_argument("--tokens", type=int, default=None, help="batch size (default: the workload's)")
    ap.add_argument("--q", type=float, default=None, help="target sparsity of the calibration")
    ap.add_argument("--sweep", default=None, help="extra batch sizes reported beside the headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run 5 plain device copies of this many bytes (HBM counter scale)")
    return ap.parse_args()


def copy_probe(nbytes):
    """A plain device-to-device copy of known size, used to scale HBM counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 5}))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only: run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.copy_bytes:
        copy_probe(args.copy_bytes)
        return

    import torch

    from intra_expert_activation_amd import moe, synth

    if not os.path.exists(moe.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg_id, T_def, q_def, sweep_def, desc = WORKLOADS[args.workload]
    T = args.tokens or T_def
    args.q = q_def if args.q is None else args.q
    args.sweep = sweep_def if args.sweep is None else args.sweep
    c = synth.config(cfg_id)
    rotate = ROTATE if T <= 256 else 2
    t_gen = time.time()
    L = synth.make_layer(c)
    x_all, l_all = synth.make_tokens(c, 2, rotate * max(T, max(c["T"])))
    xc, lc = synth.make_tokens(c, 1)
    gen_s = time.time() - t_gen

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    Wg, Wu, Wd = bf16(L["w_gate"]), bf16(L["w_up"]), bf16(L["w_down"])
    H, E, I, K, S, Is = L["H"], L["E"], L["I"], L["K"], L["S"], L["I_shared"]
    renorm = bool(L["renormalize"])
    shared = (bf16(L["ws_gate"]), bf16(L["ws_up"]), bf16(L["ws_down"])) if S else None
    Imax = max(I, Is) if S else I
    rows = np.array([I] * E + [Is] * S)
    tau = moe.calibrate_threshold(bf16(xc), torch.from_numpy(lc).to(dev), Wg, args.q, K=K,
                                  shared_gate=shared[0] if S else None)
    torch.cuda.synchronize()

    def batches(Tb):
        out = []
        for r in range(rotate):
            sl = slice(r * Tb, (r + 1) * Tb)
            out.append((bf16(x_all[sl]), torch.from_numpy(np.ascontiguousarray(l_all[sl])).to(dev)))
        return out

    def make_outputs(Tb):
        return dict(y=torch.empty((Tb, H), dtype=torch.float32, device=dev),
                    mask_bits=torch.empty((Tb, K + S, Imax // 32), dtype=torch.int32, device=dev),
                    union_idx=torch.empty((E + S, Imax), dtype=torch.int32, device=dev),
                    union_cnt=torch.empty((E + S,), dtype=torch.int32, device=dev),
                    topk_ids=torch.empty((Tb, K), dtype=torch.int32, device=dev),
                    topk_w=torch.empty((Tb, K), dtype=torch.float32, device=dev))

    def run(Tb, mode, steps, warmup, kernel_timing, graph, chain=True, budget=0):
        bs = batches(Tb)
        outs = [make_outputs(Tb) for _ in range(rotate)]
        shape = moe.layer_shape(bs[0][0], Wg, K, renorm, shared[0] if S else None)
        ws = moe.alloc_workspace(moe.workspace_size(shape, mode), dev)

        def call(r, ev=None):
            x, lg = bs[r]
            moe.sparse_expert_ffn(x, lg, Wg, Wu, Wd, tau, K=K, renormalize=renorm, shared=shared, mode=mode,
                                  out=outs[r], workspace=ws, prof_events=ev, neuron_budget=budget)

        # per-batch algorithmic bytes and flops from the returned unions
        for r in range(rotate):
            call(r)
        torch.cuda.synchronize()
        proj_bytes, call_bytes, proj_flops, call_flops, active = [], [], [], [], []
        for r in range(rotate):
            ucnt = outs[r]["union_cnt"].cpu().numpy().astype(np.int64)
            ne = np.bincount(outs[r]["topk_ids"].cpu().numpy().ravel(), minlength=E + S).astype(np.int64)
            ne[E:] = Tb
            t = ne > 0
            u = rows if mode == moe.MOE_DENSE else ucnt
            gate_rows, union_rows = int(rows[t].sum()), int(u[t].sum())
            proj_bytes.append((gate_rows + union_rows) * H * 2 + Tb * H * 2)
            call_bytes.append((gate_rows + 2 * union_rows) * H * 2 + Tb * H * 2 + Tb * E * 4 + Tb * H * 4)
            proj_flops.append(float((2 * H * ne * (rows + u))[t].sum()))
            call_flops.append(float((2 * H * ne * (rows + 2 * u))[t].sum()))
            active.append(union_rows / gate_rows)
        active = float(np.mean(active))

        for s in range(warmup):
            call(s % rotate)
        torch.cuda.synchronize()

        # graphs: one per batch, and (chain) one holding the calls on all the
        # batches in order, as a caller that captures a whole forward pass
        # replays them; a step is still one call on one batch
        graphs, whole = None, None
        if graph:
            try:
                graphs = []
                st = torch.cuda.Stream()
                st.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(st):
                    for r in range(rotate):
                        g = torch.cuda.CUDAGraph()
                        with torch.cuda.graph(g, stream=st):
                            call(r)
                        graphs.append(g)
                    if chain:
                        whole = torch.cuda.CUDAGraph()
                        with torch.cuda.graph(whole, stream=st):
                            for r in range(rotate):
                                call(r)
                torch.cuda.current_stream().wait_stream(st)
                for r in range(rotate):
                    graphs[r].replay()
                if whole is not None:
                    whole.replay()
                torch.cuda.synchronize()
            except Exception as exc:  # capture unsupported: time eager calls
                print(f"# graph capture failed ({exc}); timing eager calls", file=sys.stderr)
                graphs, whole = None, None

        timers = [moe.Timer() for _ in range(steps)] if kernel_timing else None
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        s = 0
        if timers is None and whole is not None:
            while s + rotate <= steps:  # calls s .. s + rotate - 1, batches 0 .. rotate - 1
                whole.replay()
                s += rotate
        while s < steps:
            r = s % rotate
            if timers is not None:
                call(r, timers[s].events)
            elif graphs is not None:
                graphs[r].replay()
            else:
                call(r)
            s += 1
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        res = dict(ms_per_step=elapsed * 1e3 / steps, tokens_per_s=Tb * steps / elapsed,
                   call_bytes=float(np.mean(call_bytes)), proj_bytes=float(np.mean(proj_bytes)),
                   proj_flops=float(np.mean(proj_flops)), call_flops=float(np.mean(call_flops)),
                   union_fraction=active, graph=graphs is not None and timers is None,
                   calls_per_graph=(rotate if whole is not None and steps >= rotate else 1) if graphs else 0)
        if timers is not None:
            kms = np.array([t.elapsed_ms() for t in timers])
            for t in timers:
                t.close()
            kb = np.array([proj_bytes[s % rotate] for s in range(steps)])
            kf = np.array([proj_flops[s % rotate] for s in range(steps)])
            res["proj_ms"] = float(kms.mean())
            res["proj_gbs"] = float(kb.sum() / (kms.sum() * 1e-3) / 1e9)
            res["proj_tflops"] = float(kf.sum() / (kms.sum() * 1e-3) / 1e12)
        res["call_gbs"] = res["call_bytes"] / (res["ms_per_step"] * 1e-3) / 1e9
        res["call_tflops"] = res["call_flops"] / (res["ms_per_step"] * 1e-3) / 1e12
        return res

    use_graph = not args.no_graph
    # headline: eager calls with events around the expert projection kernel,
    # then the whole call timed from graph replays
    head = run(T, moe.MOE_SPARSE, args.steps, args.warmup, kernel_timing=True, graph=False)
    head_g = run(T, moe.MOE_SPARSE, args.steps, args.warmup, kernel_timing=False, graph=use_graph)
    head_1 = run(T, moe.MOE_SPARSE, args.steps, args.warmup, kernel_timing=False, graph=use_graph, chain=False)
    dense_g = run(T, moe.MOE_DENSE, args.steps, args.warmup, kernel_timing=False, graph=use_graph)
    dense_k = run(T, moe.MOE_DENSE, max(20, args.steps // 4), 5, kernel_timing=True, graph=False)

    sweep = []
    for Ts in [int(v) for v in args.sweep.split(",") if v.strip()]:
        sp = run(Ts, moe.MOE_SPARSE, args.steps, args.warmup, kernel_timing=False, graph=use_graph)
        de = run(Ts, moe.MOE_DENSE, args.steps, args.warmup, kernel_timing=False, graph=use_graph)
        sweep.append(dict(T=Ts, sparse_us=round(sp["ms_per_step"] * 1e3, 2),
                          dense_us=round(de["ms_per_step"] * 1e3, 2),
                          speedup_vs_dense=round(de["ms_per_step"] / sp["ms_per_step"], 3),
                          tokens_per_s=round(sp["tokens_per_s"], 1),
                          hbm_frac_call=round(sp["call_gbs"] / HBM_PEAK_GBS, 4),
                          union_fraction=round(sp["union_fraction"], 4)))

    # the top-k alternative at the same sparsity: the budget largest |a| of
    # every pair instead of the threshold (a score pass, a per-pair selection
    # and a masked projection in place of the one fused threshold pass)
    topk = None
    if T < 1024:
        budget = int(round((1.0 - args.q) * I))
        tk = run(T, moe.MOE_TOPK, args.steps, args.warmup, kernel_timing=False, graph=use_graph, budget=budget)
        topk = dict(neuron_budget=budget, ms_per_step=round(tk["ms_per_step"], 5),
                    time_vs_threshold=round(tk["ms_per_step"] / head_g["ms_per_step"], 3),
                    speedup_vs_dense=round(dense_g["ms_per_step"] / tk["ms_per_step"], 3),
                    union_fraction=round(tk["union_fraction"], 4))

    best = head_g if head_g["ms_per_step"] < head["ms_per_step"] else head
    traffic = None
    if args.workload == "decode" and T == 64 and os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("kernel_src_sha256") == kernel_src_sha256():
            traffic = tr.get("hbm_bytes_per_launch")

    if T >= 1024:  # prefill: the projection is a dense contraction on MFMA
        roof = {"bound": "mfma", "achieved": round(head["proj_tflops"], 1), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(head["proj_tflops"] / MFMA_PEAK_TFLOPS, 4),
                "traffic": traffic, "kernel": "k_proj_mfma (gate, SiLU, threshold, ballot, up; bf16 MFMA)",
                "kernel_avg_us": round(head["proj_ms"] * 1e3, 2),
                "algorithmic_flops_per_launch": round(head["proj_flops"])}
    else:
        roof = {"bound": "hbm", "achieved": round(head["proj_gbs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(head["proj_gbs"] / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": "k_proj (gate, SiLU, threshold, ballot, up)",
                "kernel_avg_us": round(head["proj_ms"] * 1e3, 2),
                "algorithmic_bytes_per_launch": round(head["proj_bytes"])}
    line = {
        "metric": METRIC,
        "value": round(best["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(best["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{desc}, T {T}, bf16 weights, tau at q={args.q}",
                   "global_batch": T, "q": args.q,
                   "timing": (f"graph replay, {best['calls_per_graph']} calls per graph" if best["graph"]
                              else "eager")},
        "roofline": roof,
        "speedup_vs_dense": round(dense_g["ms_per_step"] / head_g["ms_per_step"], 3),
        "dense_ms_per_step": round(dense_g["ms_per_step"], 5),
        "ms_per_step_one_call_per_graph": round(head_1["ms_per_step"], 5),
        "ms_per_step_eager": round(head["ms_per_step"], 5),
        "dense_proj_frac": round((dense_k["proj_tflops"] / MFMA_PEAK_TFLOPS) if T >= 1024
                                 else (dense_k["proj_gbs"] / HBM_PEAK_GBS), 4),
        "call_hbm_frac": round(head_g["call_gbs"] / HBM_PEAK_GBS, 4),
        "call_tflops": round(head_g["call_tflops"], 1),
        "union_fraction": round(head["union_fraction"], 4),
        "sweep": sweep,
        "topk_variant": topk,
        "setup_s": round(gen_s, 1),
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(L, x_all, l_all, xc, lc, T, args)

    print(json.dumps(line))


def cpu_baseline(L, x_all, l_all, xc, lc, T, args):
    """The CPU oracle as it stands (float64 loops, OpenMP over tokens) on a
    bounded sample of the same workload: batches of min(T, 64) tokens of the
    same draw, repeated until about --cpu-seconds of work."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or oracle.default_threads()
    threads = max(1, min(threads, oracle.default_threads()))
    tau = oracle.calibrate(L, xc, lc, args.q, threads=threads)
    Tb = min(T, 64)
    nb = x_all.shape[0] // Tb
    done, t0 = 0, time.perf_counter()
    r = 0
    while True:
        sl = slice(r * Tb, (r + 1) * Tb)
        oracle.moe(L, x_all[sl], l_all[sl], tau, threads=threads)
        done += Tb
        r = (r + 1) % nb
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(done / el, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done // Tb} batches of {Tb} tokens of the same layer (float64 oracle, sparse mode)"}


if __name__ == "__main__":
    main()
