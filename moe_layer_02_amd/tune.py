"""Plan sweep: time every plan the library accepts for a layer at each T and report the
fastest (per-batch-size tuning, as vLLM PR #2979 "Optimized fused MoE Kernel, take 2" does
for its Triton kernel's knobs; here the knobs are the compiled tile shapes, the align
block height and GEMM2's split-K factor).

    python -m moe_layer_02_amd.tune --config mixtral --tokens 1,32,256,4096

Each plan is captured in a hipGraph and replayed; the median of several timed replays is
kept.  Output: one JSON line per (config, T) with every plan's time and the best plan.
"""
from __future__ import annotations

import argparse
import json
import sys

import torch

from moe_layer_02_amd import abi, synth


def valid_plans(layer: abi.MoELayer, T: int, max_tile: int = 40, bms=(16, 32, 64, 128, 256), tiles=None,
                split1=(1,), tails=(0,), tails1=(0,)):
    out = []
    for bm in bms:
        for g1 in (tiles if tiles is not None else range(max_tile)):
            for g2 in (tiles if tiles is not None else range(max_tile)):
                for sk in (1, 2, 3, 4, 5, 6, 7, 8):
                    for s1 in split1:
                        for st in tails:
                            for st1 in tails1:
                                p = abi.Plan(bm, g1, g2, sk, s1, st, 0, st1)
                                try:
                                    abi.moe_workspace_bytes(layer.struct, T, p)
                                except abi.MoEError:
                                    continue
                                out.append(p)
    return out


def time_plan(layer, x, lg, T, plan, reps=20):
    ws = layer.workspace(T, plan)
    out = torch.empty((T, layer.H), dtype=torch.bfloat16, device="cuda")
    layer.forward(x, lg, out=out, workspace=ws, plan=plan)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            layer.forward(x, lg, out=out, workspace=ws, plan=plan)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    times.sort()
    return times[len(times) // 2]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="mixtral", choices=sorted(synth.CONFIGS))
    ap.add_argument("--tokens", default="1,32,256,4096")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--bm", default="16,32,64,128,256", help="block heights to try")
    ap.add_argument("--tiles", default=None, help="tile ids to try for both GEMMs (default: all)")
    ap.add_argument("--split1", default="1", help="GEMM1 K splits to try (small-T tiles only)")
    ap.add_argument("--split-tail", default="0", help="GEMM2 split-tail factors to try (0: off)")
    ap.add_argument("--split-tail1", default="0", help="GEMM1 split-tail factors to try (0: off)")
    args = ap.parse_args()
    cfg = synth.CONFIGS[args.config]
    w = synth.expert_weights(cfg, device="cuda")
    bias = synth.correction_bias(cfg)
    d = w.tensors()
    layer = abi.MoELayer.create(cfg.E, cfg.H, cfg.I, cfg.k, cfg.route_kind, cfg.wdtype, d["w13"], d["w2"],
                                renormalize=cfg.renormalize, n_group=cfg.n_group, topk_group=cfg.topk_group,
                                routed_scaling=cfg.routed_scaling, w13_scale=d.get("w13_scale"),
                                w2_scale=d.get("w2_scale"), w13_s=d.get("w13_s"), w13_z=d.get("w13_z"),
                                w2_s=d.get("w2_s"), w2_z=d.get("w2_z"),
                                correction_bias=None if bias is None else bias.cuda())
    for T in [int(t) for t in args.tokens.split(",")]:
        x = synth.hidden_states(cfg, T).cuda()
        lg = synth.router_logits(cfg, T).cuda()
        res = []
        bms = tuple(int(b) for b in args.bm.split(","))
        tiles = None if args.tiles is None else [int(t) for t in args.tiles.split(",")]
        split1 = tuple(int(v) for v in args.split1.split(","))
        tails = tuple(int(v) for v in args.split_tail.split(","))
        tails1 = tuple(int(v) for v in args.split_tail1.split(","))
        plans = valid_plans(layer, T, bms=bms, tiles=tiles, split1=split1, tails=tails, tails1=tails1)
        if plans:   # bring the clocks up before the first timed plan
            time_plan(layer, x, lg, T, plans[0], 5 * args.reps)
        for p in plans:
            us = time_plan(layer, x, lg, T, p, args.reps)
            res.append((us, p.as_tuple()))
            print("[tune] %s T=%d plan=%s %.1f us" % (cfg.name, T, p.as_tuple(), us), file=sys.stderr, flush=True)
        res.sort()
        default = layer.plan(T).as_tuple()
        dus = next((u for u, p in res if p == default), None)
        if dus is None:
            dus = time_plan(layer, x, lg, T, layer.plan(T), args.reps)
        print(json.dumps({"config": cfg.name, "T": T, "best": res[0][1], "best_us": round(res[0][0], 2),
                          "default": default, "default_us": round(dus, 2),
                          "all": [[round(u, 2), p] for u, p in res]}), flush=True)


if __name__ == "__main__":
    main()
