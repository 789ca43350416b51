#!/usr/bin/env python3
"""MoE-layer throughput of the intra-expert-sparse expert FFN on one MI355X.

Headline workload: a synthetic Qwen-MoE-style decode layer (hidden 2048, 128
experts of intermediate 768, top-8 softmax routing, bf16 weights, fp32
accumulation), with the gate bias channel and correlated tokens of the
synthetic generator, threshold calibrated on the GPU to 85% intra-expert
sparsity.  One step is one call of moe_sparse_expert_ffn on a batch of T
tokens (default 64): routing, grouping, dense gate + SiLU + threshold +
ballot, gathered up, gathered down, combine.  Batches rotate over 16 token
draws, and for batches of at most 8 tokens over 4 device copies of the
weights too, so that expert weights are not served from the 256 MB Infinity
Cache between steps.  The timed calls are replayed from a HIP graph that holds
the calls on all 16 batches in order, as a caller that captures a whole
forward pass replays them; single-call latency percentiles (graphs of one
call, each replay bracketed by events) and eager timing are reported beside
it.

Prints ONE JSON line with the headline tokens/s, the roofline of the dominant
kernel (expert projection: gate, score, mask, up), the speedup over the
library's own dense mode, a batch sweep, the top-k neuron selection variant at
the same sparsity, lines for the Mixtral-, DeepSeek-style and prefill layers,
and the CPU oracle (dense and sparse) on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at 1 MI355X + HBM GB/s fraction; speedup vs dense"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16
TOKEN_DRAWS = 16
SMALL_BATCH_REPLICAS = 4   # weight copies rotated for batches of at most 8 tokens
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
    "mixtral": (3, 16, 0.90, "1,128,256", "mixtral-style layer: H 4096, 8 experts x I 14336, top-2"),
    "deepseek": (4, 64, 0.85, "1,8,32", "deepseek-v2-lite-style layer: H 2048, 64 experts x I 1408 top-6 "
                                          "+ 2 shared experts, zipf routing"),
}
# reported beside the default headline: (workload, batch, q)
EXTRA = [("mixtral", 16, 0.90), ("mixtral", 256, 0.90), ("deepseek", 64, 0.85), ("prefill", 4096, 0.70)]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="decode")
    ap.add_argument("--tokens", type=int, default=None, help="batch size (default: the workload's)")
    ap.add_argument("--q", type=float, default=None, help="target sparsity of the calibration")
    ap.add_argument("--sweep", default=None, help="extra batch sizes reported beside the headline")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads' lines")
    ap.add_argument("--no-topk", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=6.0, help="per leg of the CPU baseline (4 legs)")
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


class DeviceLayer:
    """One synthetic layer on the device: its weights (and replicas of them),
    the threshold calibrated on the GPU, and the host token draws."""

    def __init__(self, name, q, dev, replicas=1):
        import torch

        from intra_expert_activation_amd import moe, synth
        self.moe, self.torch = moe, torch
        cfg_id, _, _, _, self.desc = WORKLOADS[name]
        self.name, self.q, self.dev = name, q, dev
        t0 = time.time()
        self.c = c = synth.config(cfg_id)
        self.L = L = synth.make_layer(c)
        self.xc, self.lc = synth.make_tokens(c, 1)
        self.gen_s = time.time() - t0
        self.H, self.E, self.I, self.K = L["H"], L["E"], L["I"], L["K"]
        self.S, self.Is = L["S"], L["I_shared"]
        self.renorm = bool(L["renormalize"])
        self.Imax = max(self.I, self.Is) if self.S else self.I
        self.rows = np.array([self.I] * self.E + [self.Is] * self.S)
        keys = ("w_gate", "w_up", "w_down") + (("ws_gate", "ws_up", "ws_down") if self.S else ())
        base = tuple(self.bf16(L[k]) for k in keys)
        self.weights = [base]
        self.set_replicas(replicas)
        sg = base[3] if self.S else None
        self.tau = moe.calibrate_threshold(self.bf16(self.xc), torch.from_numpy(self.lc).to(dev), base[0], q,
                                           K=self.K, shared_gate=sg)
        torch.cuda.synchronize()
        self._tokens = {}

    def bf16(self, a):
        t = self.torch
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t.bfloat16).to(self.dev)

    def set_replicas(self, n):
        self.weights = self.weights[:1] + [tuple(w.clone() for w in self.weights[0]) for _ in range(n - 1)]

    def tokens(self, T, draws):
        from intra_expert_activation_amd import synth
        key = (T, draws)
        if key not in self._tokens:
            x_all, l_all = synth.make_tokens(self.c, 2, draws * T)
            self._tokens[key] = [(x_all[r * T:(r + 1) * T], np.ascontiguousarray(l_all[r * T:(r + 1) * T]))
                                 for r in range(draws)]
        return self._tokens[key]

    def free(self):
        self.weights = []
        self.torch.cuda.empty_cache()


def measure(layer, T, mode, steps, warmup, *, kernel_timing=False, graph=True, chain=True, budget=0,
            percentiles=False):
    """Time `steps` calls of one mode on batches of T tokens (rotating over the
    token draws and the weight replicas).  Returns a dict of figures."""
    torch, moe = layer.torch, layer.moe
    dev = layer.dev
    draws = TOKEN_DRAWS if T <= 256 else 2
    host = layer.tokens(T, draws)
    bs = [(layer.bf16(x), torch.from_numpy(lg).to(dev)) for x, lg in host]
    H, E, K, S, Imax = layer.H, layer.E, layer.K, layer.S, layer.Imax
    nrep = len(layer.weights)
    ncall = draws * nrep // np.gcd(draws, nrep)  # every (batch, replica) pairing once

    def outputs():
        return dict(y=torch.empty((T, H), dtype=torch.float32, device=dev),
                    mask_bits=torch.empty((T, K + S, Imax // 32), dtype=torch.int32, device=dev),
                    union_idx=torch.empty((E + S, Imax), dtype=torch.int32, device=dev),
                    union_cnt=torch.empty((E + S,), dtype=torch.int32, device=dev),
                    topk_ids=torch.empty((T, K), dtype=torch.int32, device=dev),
                    topk_w=torch.empty((T, K), dtype=torch.float32, device=dev))

    outs = [outputs() for _ in range(draws)]
    w0 = layer.weights[0]
    shape = moe.layer_shape(bs[0][0], w0[0], K, layer.renorm, w0[3] if S else None)
    ws = moe.alloc_workspace(moe.workspace_size(shape, mode), dev)

    def call(i, ev=None):
        x, lg = bs[i % draws]
        w = layer.weights[i % nrep]
        moe.sparse_expert_ffn(x, lg, w[0], w[1], w[2], layer.tau, K=K, renormalize=layer.renorm,
                              shared=w[3:6] if S else None, mode=mode, out=outs[i % draws], workspace=ws,
                              prof_events=ev, neuron_budget=budget)

    # per-batch algorithmic bytes and flops from the returned unions
    for r in range(draws):
        call(r)
    torch.cuda.synchronize()
    rows = layer.rows
    proj_bytes, call_bytes, proj_flops, call_flops, active = [], [], [], [], []
    for r in range(draws):
        ucnt = outs[r]["union_cnt"].cpu().numpy().astype(np.int64)
        ne = np.bincount(outs[r]["topk_ids"].cpu().numpy().ravel(), minlength=E + S).astype(np.int64)
        ne[E:] = T
        t = ne > 0
        u = rows if mode == moe.MOE_DENSE else ucnt
        gate_rows, union_rows = int(rows[t].sum()), int(u[t].sum())
        proj_bytes.append((gate_rows + union_rows) * H * 2 + T * H * 2)
        call_bytes.append((gate_rows + 2 * union_rows) * H * 2 + T * H * 2 + T * E * 4 + T * H * 4)
        proj_flops.append(float((2 * H * ne * (rows + u))[t].sum()))
        call_flops.append(float((2 * H * ne * (rows + 2 * u))[t].sum()))
        active.append(union_rows / gate_rows)

    for s in range(warmup):
        call(s)
    torch.cuda.synchronize()

    # graphs: one per (batch, replica) pairing, and (chain) one holding the
    # calls on all of them in order; a step is still one call on one batch
    graphs, whole = None, None
    if graph:
        try:
            graphs = []
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                for i in range(ncall):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=st):
                        call(i)
                    graphs.append(g)
                if chain:
                    whole = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(whole, stream=st):
                        for i in range(ncall):
                            call(i)
            torch.cuda.current_stream().wait_stream(st)
            for g in graphs:
                g.replay()
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
        while s + ncall <= steps:
            whole.replay()
            s += ncall
    while s < steps:
        if timers is not None:
            call(s, timers[s].events)
        elif graphs is not None:
            graphs[s % ncall].replay()
        else:
            call(s)
        s += 1
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    res = dict(ms_per_step=elapsed * 1e3 / steps, tokens_per_s=T * steps / elapsed,
               call_bytes=float(np.mean(call_bytes)), proj_bytes=float(np.mean(proj_bytes)),
               proj_flops=float(np.mean(proj_flops)), call_flops=float(np.mean(call_flops)),
               union_fraction=float(np.mean(active)), graph=graphs is not None and timers is None,
               calls_per_graph=(ncall if whole is not None and steps >= ncall else 1) if graphs else 0,
               weight_replicas=nrep, token_draws=draws)
    if timers is not None:
        kms = np.array([t.elapsed_ms() for t in timers])
        for t in timers:
            t.close()
        kb = np.array([proj_bytes[s % draws] for s in range(steps)])
        kf = np.array([proj_flops[s % draws] for s in range(steps)])
        res["proj_ms"] = float(kms.mean())
        res["proj_gbs"] = float(kb.sum() / (kms.sum() * 1e-3) / 1e9)
        res["proj_tflops"] = float(kf.sum() / (kms.sum() * 1e-3) / 1e12)
    if percentiles and graphs is not None:
        n = max(200, steps)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            evs[i][0].record()
            graphs[i % ncall].replay()
            evs[i][1].record()
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        res["latency_us"] = dict(p10=round(float(np.percentile(us, 10)), 2), p50=round(float(np.median(us)), 2),
                                 p90=round(float(np.percentile(us, 90)), 2), replays=n,
                                 how="single-call graph replays, each bracketed by events")
    res["call_gbs"] = res["call_bytes"] / (res["ms_per_step"] * 1e-3) / 1e9
    res["call_tflops"] = res["call_flops"] / (res["ms_per_step"] * 1e-3) / 1e12
    return res


def roofline(res, T, traffic=None):
    if T >= 1024:  # prefill: the projection is a dense contraction on MFMA
        return {"bound": "mfma", "achieved": round(res["proj_tflops"], 1), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(res["proj_tflops"] / MFMA_PEAK_TFLOPS, 4),
                "traffic": traffic, "kernel": "expert projection (gate, SiLU, threshold, ballot, up; bf16 MFMA)",
                "kernel_avg_us": round(res["proj_ms"] * 1e3, 2),
                "algorithmic_flops_per_launch": round(res["proj_flops"])}
    return {"bound": "hbm", "achieved": round(res["proj_gbs"], 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(res["proj_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic, "kernel": "expert projection (gate, SiLU, threshold, ballot, up)",
            "kernel_avg_us": round(res["proj_ms"] * 1e3, 2),
            "algorithmic_bytes_per_launch": round(res["proj_bytes"])}


def workload_line(layer, T, args, use_graph):
    """ms/call, tokens/s, the projection's roofline fraction and the speedup
    over dense for one (layer, batch)."""
    moe = layer.moe
    sp = measure(layer, T, moe.MOE_SPARSE, args.steps, args.warmup, graph=use_graph, percentiles=True)
    de = measure(layer, T, moe.MOE_DENSE, args.steps, args.warmup, graph=use_graph)
    kt = measure(layer, T, moe.MOE_SPARSE, max(20, args.steps // 4), 5, kernel_timing=True, graph=False)
    rf = roofline(kt, T)
    return dict(workload=f"{layer.desc}, T {T}, bf16 weights, tau at q={layer.q}", T=T, q=layer.q,
                ms_per_step=round(sp["ms_per_step"], 5), tokens_per_s=round(sp["tokens_per_s"], 1),
                latency_us=sp.get("latency_us"), dense_ms_per_step=round(de["ms_per_step"], 5),
                speedup_vs_dense=round(de["ms_per_step"] / sp["ms_per_step"], 3),
                call_hbm_frac=round(sp["call_gbs"] / HBM_PEAK_GBS, 4), call_tflops=round(sp["call_tflops"], 1),
                union_fraction=round(sp["union_fraction"], 4), weight_replicas=sp["weight_replicas"],
                roofline={k: rf[k] for k in ("bound", "achieved", "unit", "frac", "kernel_avg_us")})


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

    from intra_expert_activation_amd import moe

    if not os.path.exists(moe.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    _, T_def, q_def, sweep_def, desc = WORKLOADS[args.workload]
    T = args.tokens or T_def
    args.q = q_def if args.q is None else args.q
    args.sweep = sweep_def if args.sweep is None else args.sweep
    use_graph = not args.no_graph
    t_setup = time.time()
    layer = DeviceLayer(args.workload, args.q, dev, replicas=SMALL_BATCH_REPLICAS if T <= 8 else 1)

    # headline: eager calls with events around the expert projection kernel,
    # then the whole call timed from graph replays
    head = measure(layer, T, moe.MOE_SPARSE, args.steps, args.warmup, kernel_timing=True, graph=False)
    head_g = measure(layer, T, moe.MOE_SPARSE, args.steps, args.warmup, graph=use_graph, percentiles=True)
    head_1 = measure(layer, T, moe.MOE_SPARSE, args.steps, args.warmup, graph=use_graph, chain=False)
    dense_g = measure(layer, T, moe.MOE_DENSE, args.steps, args.warmup, graph=use_graph)
    dense_k = measure(layer, T, moe.MOE_DENSE, max(20, args.steps // 4), 5, kernel_timing=True, graph=False)

    # the top-k alternative at the same sparsity: the budget largest |a| of
    # every pair instead of the threshold (a score pass, a per-pair selection
    # and a masked projection in place of the one fused threshold pass)
    topk = None
    if T < 1024 and not args.no_topk:
        budget = int(round((1.0 - args.q) * layer.I))
        tk = measure(layer, T, moe.MOE_TOPK, args.steps, args.warmup, graph=use_graph, budget=budget)
        topk = dict(neuron_budget=budget, ms_per_step=round(tk["ms_per_step"], 5),
                    time_vs_threshold=round(tk["ms_per_step"] / head_g["ms_per_step"], 3),
                    speedup_vs_dense=round(dense_g["ms_per_step"] / tk["ms_per_step"], 3),
                    union_fraction=round(tk["union_fraction"], 4))

    sweep = []
    for Ts in [int(v) for v in args.sweep.split(",") if v.strip()]:
        layer.set_replicas(SMALL_BATCH_REPLICAS if Ts <= 8 else 1)
        sp = measure(layer, Ts, moe.MOE_SPARSE, args.steps, args.warmup, graph=use_graph, percentiles=True)
        de = measure(layer, Ts, moe.MOE_DENSE, args.steps, args.warmup, graph=use_graph)
        sweep.append(dict(T=Ts, sparse_us=round(sp["ms_per_step"] * 1e3, 2),
                          dense_us=round(de["ms_per_step"] * 1e3, 2),
                          speedup_vs_dense=round(de["ms_per_step"] / sp["ms_per_step"], 3),
                          tokens_per_s=round(sp["tokens_per_s"], 1),
                          hbm_frac_call=round(sp["call_gbs"] / HBM_PEAK_GBS, 4),
                          union_fraction=round(sp["union_fraction"], 4),
                          p50_us=sp["latency_us"]["p50"] if "latency_us" in sp else None,
                          weight_replicas=sp["weight_replicas"]))

    best = head_g if head_g["ms_per_step"] < head["ms_per_step"] else head
    traffic = None
    if args.workload == "decode" and T == 64 and os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("kernel_src_sha256") == kernel_src_sha256():
            traffic = tr.get("hbm_bytes_per_launch")

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
        "roofline": roofline(head, T, traffic),
        "latency_us": head_g.get("latency_us"),
        "speedup_vs_dense": round(dense_g["ms_per_step"] / head_g["ms_per_step"], 3),
        "dense_ms_per_step": round(dense_g["ms_per_step"], 5),
        "ms_per_step_one_call_per_graph": round(head_1["ms_per_step"], 5),
        "ms_per_step_eager": round(head["ms_per_step"], 5),
        "dense_proj_frac": round((dense_k["proj_tflops"] / MFMA_PEAK_TFLOPS) if T >= 1024
                                 else (dense_k["proj_gbs"] / HBM_PEAK_GBS), 4),
        "call_hbm_frac": round(head_g["call_gbs"] / HBM_PEAK_GBS, 4),
        "call_tflops": round(head_g["call_tflops"], 1),
        "union_fraction": round(head["union_fraction"], 4),
        "weight_replicas": head_g["weight_replicas"],
        "sweep": sweep,
        "topk_variant": topk,
    }

    host_layer = (layer.L, layer.xc, layer.lc, layer.tokens(T, TOKEN_DRAWS if T <= 256 else 2))
    layer.free()
    del layer

    # the other workloads (the default line only)
    if args.workload == "decode" and args.tokens is None and not args.no_extra:
        extra = []
        by_name = {}
        for name, Te, qe in EXTRA:
            by_name.setdefault(name, []).append((Te, qe))
        for name, runs in by_name.items():
            for qe in sorted({q for _, q in runs}):
                wl = DeviceLayer(name, qe, dev)
                for Te, q2 in runs:
                    if q2 == qe:
                        extra.append(workload_line(wl, Te, args, use_graph))
                wl.free()
                del wl
        line["workloads"] = extra
    line["setup_and_extra_s"] = round(time.time() - t_setup, 1)

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(*host_layer, T, args)

    print(json.dumps(line))


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(L, xc, lc, draws, T, args):
    """The CPU oracle as it stands (float64 loops, OpenMP over tokens) on a
    bounded sample of the same workload: batches of min(T, 64) tokens of the
    same draws in sparse and in dense mode on every host core, then single
    tokens on one core, each leg for about --cpu-seconds."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or oracle.default_threads()
    threads = max(1, min(threads, oracle.default_threads()))
    tau = oracle.calibrate(L, xc, lc, args.q, threads=threads)
    Tb = min(T, 64)
    batches = [(x[:Tb], lg[:Tb]) for x, lg in draws]

    def leg(dense, nthreads, tokens):
        done, r, t0 = 0, 0, time.perf_counter()
        while True:
            x, lg = batches[r % len(batches)]
            oracle.moe(L, x[:tokens], lg[:tokens], tau, dense=dense, threads=nthreads)
            done += tokens
            r += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        return done / (time.perf_counter() - t0), r

    sp, nsp = leg(False, threads, Tb)
    de, nde = leg(True, threads, Tb)
    sp1, n1 = leg(False, 1, 1)
    de1, n1d = leg(True, 1, 1)
    return {"value": round(sp, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"{nsp} sparse and {nde} dense batches of {Tb} tokens of the same layer and draws "
                       f"(float64 oracle, {threads} threads), then {n1} sparse and {n1d} dense single tokens "
                       f"on 1 thread"),
            "cpu_model": cpu_model(),
            "dense_tokens_per_s": round(de, 2),
            "sparse_over_dense": round(sp / de, 3),
            "single_core_T1": {"sparse_tokens_per_s": round(sp1, 2), "dense_tokens_per_s": round(de1, 2),
                               "sparse_over_dense": round(sp1 / de1, 3)}}


if __name__ == "__main__":
    main()
