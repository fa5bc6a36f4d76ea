"""Benchmark of the fused-MoE layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W]                       # headline + every config's sweep
    python bench.py --config mixtral [--tokens 4096] [--sweep 1,32,256]   # one config only

A step is one moe_forward (route, align, [fp8 quantisation], GEMM1, GEMM2, reduce) over one
batch of T tokens of seeded synthetic inputs already resident in HBM; steps are replayed
from a captured hipGraph.  Prints one JSON line.  The headline (value, ms_per_step, config)
is the largest single-GPU layer, Llama-4-Scout at T=8192 (bf16, 4.2 GB of weights, 2.06
TFLOP per step); its line also carries a short T sweep of every layer (Mixtral TP2,
Qwen2-57B TP4 fp8, DeepSeek-V3 int4, Scout).  Each point reports whole-layer tokens/s (K
replays back to back, after W warm-up replays, themselves after the cold replays below), the
same step with cold caches (a 512 MiB buffer read before each replay, outside the timed
region; median, p10, p90), TFLOP/s and HBM GB/s with their
fractions of the MI355X peaks, and the step's kernels' durations.  The headline adds the
dominant kernel's roofline (its duration from HIP events recorded on the launch stream
around each step of the forward) and the CPU oracle's throughput on a bounded sample of the
same workload, on the host's cores.
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
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from moe_layer_02_amd import abi, synth  # noqa: E402

METRIC = "fused-MoE layer tokens/s + TFLOP/s & HBM GB/s (% of roofline) vs T, 1 GPU"
PEAK_HBM = 8.0e12                                  # B/s, MI355X HBM3E
FLUSH_BYTES = 512 << 20                            # > 256 MB last-level cache + 8 x 4 MB L2
PEAK_MFMA = {synth.WDT_BF16: 2.5e15, synth.WDT_FP8: 5.0e15, synth.WDT_INT4: 2.5e15}   # dense, fp16 for int4
DTYPE_NAME = {synth.WDT_BF16: "bf16", synth.WDT_FP8: "fp8-e4m3 w8a8", synth.WDT_INT4: "int4-g128 w / fp16 mfma"}
WORKLOAD = {
    "mixtral": "Mixtral-8x7B MoE layer, one TP2 shard (E=8, top-2 softmax renormalised, H=4096, I=7168, bf16)",
    "qwen2": "Qwen2-57B-A14B routed experts, one TP4 shard (E=64, top-8 softmax, H=3584, I=640, fp8 w8a8)",
    "deepseek": "DeepSeek-V3 routed experts (E=256, grouped sigmoid top-8, H=7168, I=2048, int4 g128)",
    "scout": "Llama-4-Scout MoE layer (E=16, top-1 sigmoid, Zipf(1.2) load, H=5120, I=8192, bf16)",
    "tiny": "tiny MoE layer (E=8, top-2 softmax, H=128, I=256, bf16)",
}


# the headline: the largest layer that fits one GPU (4.2 GB of bf16 weights, 2.06 TFLOP per step)
HEADLINE = ("scout", 8192)
# each layer's short T sweep in the same line: small batches stream weights, large ones are
# MFMA work
SWEEPS = {"scout": (1, 32, 2048, 8192), "mixtral": (1, 32, 1024, 4096), "qwen2": (1, 32, 1024, 4096),
          "deepseek": (1, 32, 512)}


def sweep_point(name, m):
    d = {"config": name}
    d.update({k: (round(v, 4) if isinstance(v, float) else v) for k, v in m.items()})
    return d


def bytes_per_weight(cfg):
    return {synth.WDT_BF16: 2.0, synth.WDT_FP8: 1.0, synth.WDT_INT4: 0.5 + 4.0 / 128.0}[cfg.wdtype]


def layer_flops(cfg, T):
    """2*T*k*(2I*H) (gate/up) + 2*T*k*(H*I) (down); routing and elementwise work excluded."""
    return 6.0 * T * cfg.k * cfg.H * cfg.I


def layer_min_bytes(cfg, T, active):
    """Weights of the experts in use, hidden in, output out (bf16), logits in (bf16)."""
    return active * 3.0 * cfg.H * cfg.I * bytes_per_weight(cfg) + 4.0 * T * cfg.H + 2.0 * T * cfg.E


def gemm_algorithmic(cfg, T, active, stage):
    """(flops, bytes) one launch of a GEMM stage must do / move at the minimum:
    gemm1 reads the active experts' w13 and the T hidden rows, writes T*k rows of h (bf16);
    gemm2 reads the active experts' w2 and the T*k rows of h, writes T*k output rows (bf16)."""
    bpw = bytes_per_weight(cfg)
    a_bytes = 1.0 if cfg.wdtype == synth.WDT_FP8 else 2.0
    if stage == "gemm1":
        return (4.0 * T * cfg.k * cfg.H * cfg.I,
                active * 2.0 * cfg.I * cfg.H * bpw + T * cfg.H * a_bytes + T * cfg.k * cfg.I * 2.0)
    return (2.0 * T * cfg.k * cfg.H * cfg.I,
            active * 1.0 * cfg.H * cfg.I * bpw + T * cfg.k * cfg.I * a_bytes + T * cfg.k * cfg.H * 2.0)


class Bench:
    def __init__(self, cfg, plan_override=None, plan_T=None):
        self.cfg = cfg
        self.plan_override, self.plan_T = plan_override, plan_T
        t0 = time.time()
        self.w = synth.expert_weights(cfg, device="cuda")
        self.bias = synth.correction_bias(cfg)
        d = self.w.tensors()
        self.layer = abi.MoELayer.create(
            cfg.E, cfg.H, cfg.I, cfg.k, cfg.route_kind, cfg.wdtype, d["w13"], d["w2"],
            renormalize=cfg.renormalize, n_group=cfg.n_group, topk_group=cfg.topk_group,
            routed_scaling=cfg.routed_scaling, w13_scale=d.get("w13_scale"), w2_scale=d.get("w2_scale"),
            w13_s=d.get("w13_s"), w13_z=d.get("w13_z"), w2_s=d.get("w2_s"), w2_z=d.get("w2_z"),
            correction_bias=None if self.bias is None else self.bias.cuda())
        self.flush = torch.ones((FLUSH_BYTES // 4096, 1024), dtype=torch.float32, device="cuda")
        self.flush_out = torch.empty(1024, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        print("[bench] %s weights generated on the GPU in %.1f s" % (cfg.name, time.time() - t0),
              file=sys.stderr, flush=True)

    def prepare(self, T):
        x = synth.hidden_states(self.cfg, T).cuda()
        lg = synth.router_logits(self.cfg, T).cuda()
        plan = self.plan_override if self.plan_override and T == self.plan_T else self.layer.plan(T)
        ws = self.layer.workspace(T, plan)
        out = torch.empty((T, self.cfg.H), dtype=torch.bfloat16, device="cuda")
        return x, lg, plan, ws, out

    def active_experts(self, T, plan, ws):
        off = abi.moe_workspace_offsets(self.layer.struct, T, plan)["expert_counts"]
        counts = ws[off:off + 4 * self.cfg.E].view(torch.int32).cpu().numpy()
        return int((counts > 0).sum())

    def time_graph(self, T, steps, warmup, stage_steps):
        """The step captured in a graph.  The cold-cache replays first (untimed for the
        headline), then W warm-up replays and the K timed replays back to back, so the timed
        replays do not start on a clock that is still ramping up from idle; then the
        per-kernel event timing (eager forwards) on the same warm clock."""
        x, lg, plan, ws, out = self.prepare(T)
        self.layer.forward(x, lg, out=out, workspace=ws, plan=plan)        # eager once (first-use setup)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                self.layer.forward(x, lg, out=out, workspace=ws, plan=plan)
        torch.cuda.current_stream().wait_stream(s)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # cold caches: before each timed replay, read a buffer larger than the 256 MB
        # last-level cache and the L2s together, outside the timed region (a read leaves
        # clean lines; a write would leave dirty ones whose write-back lands in the replay)
        cold = []
        for _ in range(max(steps, 10)):
            torch.amax(self.flush, dim=0, out=self.flush_out)
            t0.record()
            g.replay()
            t1.record()
            torch.cuda.synchronize()
            cold.append(t0.elapsed_time(t1))
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(steps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        stages = self.time_stages(T, plan, (x, lg, ws, out), stage_steps)
        active = self.active_experts(T, plan, ws)
        return ms, np.array(cold), active, plan, stages

    def time_stages(self, T, plan, bufs, steps):
        """Average duration of each step of the forward, from HIP events recorded on the
        launch stream before and after each kernel: `steps` eager forwards launched back to
        back (one warm-up call first), read after one synchronisation."""
        x, lg, ws, out = bufs
        abi.moe_forward_profiled(self.layer.struct, T, x, lg, out, ws,
                                 [torch.cuda.Event(enable_timing=True) for _ in range(abi.STAGE_COUNT + 1)], plan)
        torch.cuda.synchronize()
        evs, names = [], None
        for _ in range(steps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(abi.STAGE_COUNT + 1)]
            names = abi.moe_forward_profiled(self.layer.struct, T, x, lg, out, ws, ev, plan)
            evs.append(ev)
        torch.cuda.synchronize()
        acc = {}
        for ev in evs:
            for j, n in enumerate(names):
                acc[n] = acc.get(n, 0.0) + ev[j].elapsed_time(ev[j + 1]) * 1e3
        return {n: acc[n] / steps for n in names}


def measure(b: Bench, T, steps, warmup, stage_steps):
    cfg = b.cfg
    ms, cold, active, plan, stages = b.time_graph(T, steps, warmup, stage_steps)
    sec = ms / 1e3
    flops, mbytes = layer_flops(cfg, T), layer_min_bytes(cfg, T, active)
    t_hbm, t_mfma = mbytes / PEAK_HBM, flops / PEAK_MFMA[cfg.wdtype]
    c50, c10, c90 = (float(np.percentile(cold, q)) for q in (50, 10, 90))
    return dict(T=T, ms_per_step=ms, tokens_per_s=T / sec, tflops=flops / sec / 1e12, hbm_gbps=mbytes / sec / 1e9,
                frac_hbm=mbytes / sec / PEAK_HBM, frac_mfma=flops / sec / PEAK_MFMA[cfg.wdtype],
                roofline_frac=max(t_hbm, t_mfma) / sec, bound="hbm" if t_hbm >= t_mfma else "mfma",
                cold_ms={"median": round(c50, 4), "p10": round(c10, 4), "p90": round(c90, 4), "n": len(cold)},
                cold_tokens_per_s=T / (c50 / 1e3), cold_roofline_frac=max(t_hbm, t_mfma) / (c50 / 1e3),
                active_experts=active, plan=abi.moe_plan_describe(b.layer.struct, T, plan),
                stages_us={k: round(v, 2) for k, v in stages.items()})


def kernel_roofline(cfg, m):
    """Roofline of the longest-running kernel of the step."""
    gemms = {k: v for k, v in m["stages_us"].items() if k in ("gemm1", "gemm2")}
    name = max(gemms, key=gemms.get)
    dur = gemms[name] * 1e-6
    flops, nbytes = gemm_algorithmic(cfg, m["T"], m["active_experts"], name)
    if flops / PEAK_MFMA[cfg.wdtype] >= nbytes / PEAK_HBM:
        ach, peak, unit, bound = flops / dur / 1e12, PEAK_MFMA[cfg.wdtype] / 1e12, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = nbytes / dur / 1e9, PEAK_HBM / 1e9, "GB/s", "hbm"
    return dict(kernel=name, bound=bound, achieved=round(ach, 2), peak=peak, unit=unit, frac=round(ach / peak, 4),
                traffic=measured_traffic(cfg, m["T"], name), avg_us=round(gemms[name], 2),
                algorithmic_flops=flops, algorithmic_bytes=nbytes)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_sources(wdtype):
    """The sources of the GEMM kernels a layer of this weight type runs at large T: the
    pipelined kernels (bf16, fp8) or the int4 kernels, and the headers they share."""
    own = "gemm_i4.hip" if wdtype == synth.WDT_INT4 else "gemm_pipe.hip"
    return tuple("moe_layer_02_amd/csrc/" + f for f in (own, "pipe.h", "common.h", "kernels.h"))


def kernel_source_sha(wdtype):
    h = hashlib.sha256()
    for f in kernel_sources(wdtype):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(cfg, T, kernel):
    """HBM-side bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by a device copy of known size), or None when no
    summary exists for this workload or the GEMM sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    rec = data.get("%s:T%d:%s" % (cfg.name, T, kernel))
    if not rec or rec.get("kernel_sha") != kernel_source_sha(cfg.wdtype):
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def host_cpu():
    """(threads this process may use, the host CPU's model name)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def cpu_baseline(b: Bench, T, budget_s=15.0):
    """The oracle (plain C, fp64, tokens spread over the host's cores, at most 16 threads) on
    a sample of the same workload: routing of all T tokens, then the layer output of random
    tokens in batches until the time budget is spent (w8a8 fp8 needs every token's
    intermediate for its second scale, so there the whole layer runs at a smaller T)."""
    import oracle
    cfg = b.cfg
    x, lg = synth.hidden_states(cfg, T), synth.router_logits(cfg, T)
    bits = lambda t: t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    h = {k: v.cpu() for k, v in b.w.tensors().items()}
    wd = {synth.WDT_BF16: oracle.BF16, synth.WDT_FP8: oracle.FP8_E4M3, synth.WDT_INT4: oracle.INT4_G128}[cfg.wdtype]
    if cfg.wdtype == synth.WDT_BF16:
        W = oracle.Weights(wd, cfg.E, cfg.H, cfg.I, bits(h["w13"]), bits(h["w2"]))
    elif cfg.wdtype == synth.WDT_FP8:
        W = oracle.Weights(wd, cfg.E, cfg.H, cfg.I, h["w13"].numpy(), h["w2"].numpy(),
                           w13_scale=h["w13_scale"].numpy(), w2_scale=h["w2_scale"].numpy())
    else:
        W = oracle.Weights(wd, cfg.E, cfg.H, cfg.I, h["w13"].numpy(), h["w2"].numpy(), w13_s=bits(h["w13_s"]),
                           w13_z=bits(h["w13_z"]), w2_s=bits(h["w2_s"]), w2_z=bits(h["w2_z"]))
    ncpu, model = host_cpu()
    threads = oracle.default_threads()
    t0 = time.time()
    ids, w = oracle.route(cfg.route_kind, cfg.E, cfg.k, bits(lg), renormalize=cfg.renormalize, n_group=cfg.n_group,
                          topk_group=cfg.topk_group, routed_scaling=cfg.routed_scaling,
                          bias=None if b.bias is None else b.bias.numpy())
    t_route = time.time() - t0
    common = dict(unit="tokens/s", cores=threads, kind="oracle", host_cpus=ncpu, cpu_model=model)
    if cfg.wdtype == synth.WDT_FP8:
        Ts = max(1, min(T, 8 * threads))
        t0 = time.time()
        oracle.forward(W, bits(x[:Ts]), ids[:Ts], w[:Ts], threads=threads)
        el = time.time() - t0
        return dict(value=round(Ts / el, 4), sample="whole w8a8 layer at T=%d (first %d tokens of the batch), "
                    "%d threads, %.1f s" % (Ts, Ts, threads, el), **common)
    order = np.random.default_rng(0).permutation(T)
    n, el, batch = 0, 0.0, threads
    xb = bits(x)
    while n < T and (el < budget_s or n == 0):
        toks = [int(t) for t in order[n:n + batch]]
        t0 = time.time()
        oracle.forward(W, xb, ids, w, tokens=toks, threads=threads)
        el += time.time() - t0
        n += len(toks)
    per_token = el / n + t_route / T
    return dict(value=round(1.0 / per_token, 4), sample="%d of %d tokens (random, in batches of %d), routing of "
                "all %d; %d threads, %.1f s" % (n, T, batch, T, threads, el + t_route), **common)


# ---- the EP-MoE grouped GEMM (pre-permuted contiguous segments) ------------------------

GG_METRIC = "EP-MoE grouped GEMM tokens/s + TFLOP/s & HBM GB/s (% of roofline) vs batch, 1 GPU"


def grouped_gemm_bench(args):
    """moe_grouped_gemm on Qwen2-57B-A14B TP4's w13 (E = 64 experts, N = 1280, K = 3584) with
    the batch's T*8 routed rows grouped by expert (synthetic sizes): the pages' FBGEMM vs
    SGLang grouped-GEMM sweep.  The op (the segment-layout kernel and the GEMM) is timed by
    HIP events around graph replays on its stream."""
    base = synth.CONFIGS["qwen2"]
    cfg = base if args.dtype == "fp8" else base.with_shape(name="qwen2_bf16", wdtype=synth.WDT_BF16)
    fp8 = cfg.wdtype == synth.WDT_FP8
    w = synth.expert_weights(cfg, device="cuda")
    W, Ws = w.w13, w.w13_scale
    desc = abi.grouped_gemm_desc(W, abi.DT_FP8_E4M3 if fp8 else abi.DT_BF16, Ws)
    N, K = 2 * cfg.I, cfg.H
    flush = torch.ones((FLUSH_BYTES // 4096, 1024), dtype=torch.float32, device="cuda")
    flush_out = torch.empty(1024, dtype=torch.float32, device="cuda")

    def run_T(T, steps, warmup):
        x, xs, sizes = synth.grouped_gemm_inputs(cfg, T)
        M = x.shape[0]
        x, sizes = x.cuda(), sizes.cuda()
        xs = None if xs is None else xs.cuda()
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        tile = abi.moe_grouped_gemm_default_tile(desc, M)
        ws = torch.empty(abi.moe_grouped_gemm_workspace_bytes(desc, M, tile), dtype=torch.uint8, device="cuda")
        abi.moe_grouped_gemm(desc, x, sizes, y, ws, x_scale=xs, tile=tile)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                abi.moe_grouped_gemm(desc, x, sizes, y, ws, x_scale=xs, tile=tile)
        torch.cuda.current_stream().wait_stream(s)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        cold = []
        for _ in range(max(steps, 10)):
            torch.amax(flush, dim=0, out=flush_out)
            t0.record()
            g.replay()
            t1.record()
            torch.cuda.synchronize()
            cold.append(t0.elapsed_time(t1))
        active = int((sizes > 0).sum())
        flops = 2.0 * M * N * K
        mbytes = active * N * K * (1.0 if fp8 else 2.0) + M * K * (1.0 if fp8 else 2.0) + M * N * 2.0
        peak = PEAK_MFMA[cfg.wdtype]
        sec = ms / 1e3
        c50 = float(np.median(cold))
        return dict(T=T, rows=M, tile=tile, ms_per_step=round(ms, 4), tokens_per_s=round(T / sec, 2),
                    tflops=round(flops / sec / 1e12, 3), hbm_gbps=round(mbytes / sec / 1e9, 2),
                    roofline_frac=round(max(mbytes / PEAK_HBM, flops / peak) / sec, 4),
                    bound="hbm" if mbytes / PEAK_HBM >= flops / peak else "mfma",
                    cold_ms=round(c50, 4), flops=flops, min_bytes=mbytes, active_experts=active)

    T = args.tokens or 4096
    head = run_T(T, args.steps, args.warmup)
    sweep = [run_T(t, args.steps, args.warmup) for t in [int(v) for v in args.sweep.split(",") if v.strip()]
             if t != T]
    bound_mfma = head["bound"] == "mfma"
    dur = head["ms_per_step"] * 1e-3
    roof = dict(kernel="grouped_gemm (segment layout + GEMM)", bound=head["bound"],
                achieved=round(head["flops"] / dur / 1e12, 2) if bound_mfma else round(head["min_bytes"] / dur / 1e9, 2),
                peak=PEAK_MFMA[cfg.wdtype] / 1e12 if bound_mfma else PEAK_HBM / 1e9,
                unit="TFLOP/s" if bound_mfma else "GB/s", frac=head["roofline_frac"], traffic=None,
                avg_us=round(head["ms_per_step"] * 1e3, 2))
    cpu = None
    if not args.no_cpu_baseline:   # the oracle on a bounded sample of rows
        import oracle
        x, xs, sizes = synth.grouped_gemm_inputs(cfg, T)
        sizes = sizes.numpy()
        xb = x.numpy() if fp8 else x.contiguous().view(torch.int16).numpy().view(np.uint16)
        wh = W.cpu()
        wb = wh.numpy() if fp8 else wh.view(torch.int16).numpy().view(np.uint16)
        rows, el = 0, 0.0
        starts = np.concatenate([[0], np.cumsum(sizes)])
        for e in range(cfg.E):
            if el > 15.0:
                break
            if sizes[e] == 0:
                continue
            sub = np.zeros(cfg.E, np.int32)
            sub[e] = 1
            t0 = time.time()
            oracle.grouped_gemm(oracle.FP8_E4M3 if fp8 else oracle.BF16, cfg.E, N, K, xb[starts[e]:starts[e] + 1], wb,
                                sub, x_scale=1.0 if xs is None else float(xs[0]),
                                w_scale=None if Ws is None else Ws.cpu().numpy())
            el += time.time() - t0
            rows += 1
        cpu = dict(value=round(rows / el / cfg.k, 4), unit="tokens/s", cores=1, kind="oracle",
                   sample="%d rows (one per expert), %.1f s; tokens/s = rows/s / k" % (rows, el))
    line = {
        "metric": GG_METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE_NAME[cfg.wdtype], "data": "synthetic (seeded sizes and inputs)",
        "config": {"workload": "EP-MoE grouped GEMM, Qwen2-57B-A14B TP4 w13 (E=64, N=1280, K=3584, top-8 rows, %s)"
                   % ("fp8 per-tensor" if fp8 else "bf16"), "T": T, "rows": head["rows"], "tile": head["tile"]},
        "tflops": head["tflops"], "hbm_gbps": head["hbm_gbps"], "roofline_frac": head["roofline_frac"],
        "cold_ms": head["cold_ms"], "roofline": roof, "cpu_baseline": cpu,
        "sweep": [{k: v for k, v in m.items() if k not in ("flops", "min_bytes")} for m in sweep],
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None, choices=sorted(synth.CONFIGS),
                    help="one layer only (default: the Scout T=8192 headline and every layer's sweep)")
    ap.add_argument("--tokens", type=int, default=None, help="T of the headline step (default: the layer's largest)")
    ap.add_argument("--sweep", default=None, help="comma-separated T values of the headline layer's sweep "
                    "('' for none; default: its standard sweep)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--plan", default=None, help="block_m,gemm1_tile,gemm2_tile,split_k[,split_k1[,split_tail"
                    "[,max_workgroups[,split_tail1]]]] for the headline T")
    ap.add_argument("--workload", default="layer", choices=("layer", "grouped_gemm"),
                    help="the fused layer (default) or the EP-MoE grouped GEMM over pre-grouped rows")
    ap.add_argument("--dtype", default="fp8", choices=("bf16", "fp8"), help="grouped_gemm: operand type")
    ap.add_argument("--copy-probe-mib", type=int, default=256,
                    help="after timing, one device copy of this size (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the layer is one GPU's expert/TP shard and this build has no "
              "multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    torch.cuda.init()
    if args.workload == "grouped_gemm":
        if args.sweep is None:
            args.sweep = "1,2,4,8,16,32,64,128,256,512,1024,2048"
        grouped_gemm_bench(args)
        return
    if args.config is None:
        cfg, T = synth.CONFIGS[HEADLINE[0]], args.tokens or HEADLINE[1]
        others = [c for c in SWEEPS if c != cfg.name]
    else:
        cfg, T = synth.CONFIGS[args.config], args.tokens or synth.CONFIGS[args.config].t_max
        others = []
    plan = abi.Plan(*[int(v) for v in args.plan.split(",")]) if args.plan else None
    b = Bench(cfg, plan, T)
    head = measure(b, T, args.steps, args.warmup, stage_steps=max(3, min(args.steps, 10)))
    print("[bench] %s T=%d %.3f ms/step %s" % (cfg.name, T, head["ms_per_step"], head["plan"]),
          file=sys.stderr, flush=True)
    head_ts = SWEEPS.get(cfg.name, ()) if args.sweep is None else \
        tuple(int(s) for s in args.sweep.split(",") if s.strip())
    sweep = [sweep_point(cfg.name, head)]
    for t in head_ts:
        if t != T and t <= cfg.t_max:
            sweep.append(sweep_point(cfg.name, measure(b, t, args.steps, args.warmup, stage_steps=3)))
            print("[bench] %s T=%d %.3f ms/step" % (cfg.name, t, sweep[-1]["ms_per_step"]), file=sys.stderr, flush=True)
    if args.copy_probe_mib > 0:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cpu = None if args.no_cpu_baseline else cpu_baseline(b, T)
    roof = kernel_roofline(cfg, head)
    del b
    torch.cuda.empty_cache()
    for name in others:   # the other layers' sweeps, one layer's weights on the GPU at a time
        ob = Bench(synth.CONFIGS[name])
        for t in SWEEPS[name]:
            sweep.append(sweep_point(name, measure(ob, t, args.steps, args.warmup, stage_steps=3)))
            print("[bench] %s T=%d %.3f ms/step" % (name, t, sweep[-1]["ms_per_step"]), file=sys.stderr, flush=True)
        del ob
        torch.cuda.empty_cache()
    line = {
        "metric": METRIC, "value": round(head["tokens_per_s"], 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_NAME[cfg.wdtype],
        "data": "synthetic (seeded; random-init weights of the layer's shape)",
        "config": {"workload": WORKLOAD[cfg.name], "T": T, "E": cfg.E, "top_k": cfg.k, "H": cfg.H, "I": cfg.I,
                   "plan": head["plan"]},
        "tflops": round(head["tflops"], 3), "hbm_gbps": round(head["hbm_gbps"], 2),
        "frac_mfma": round(head["frac_mfma"], 4), "frac_hbm": round(head["frac_hbm"], 4),
        "layer_roofline_frac": round(head["roofline_frac"], 4), "layer_bound": head["bound"],
        "cold_ms": head["cold_ms"], "cold_tokens_per_s": round(head["cold_tokens_per_s"], 2),
        "cold_layer_roofline_frac": round(head["cold_roofline_frac"], 4),
        "stages_us": head["stages_us"], "roofline": roof, "cpu_baseline": cpu, "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
