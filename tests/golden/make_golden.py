"""Write the golden regression fixture of the tiny layer (E=8, top-2 softmax renormalised,
H=128, I=256, bf16 weights, T=16, seed 1001).

The pages print no worked example of a layer, so this fixture holds the oracle's own
answer on the seeded tiny layer; it detects drift of the input generator's random stream
or of the oracle.  It calls only the oracle and the input generator.

    python tests/golden/make_golden.py    # rewrites tests/golden/tiny_T16.txt
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from moe_layer_02_amd import synth  # noqa: E402


def bits(t):
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def compute():
    cfg = synth.CONFIGS["tiny"]
    T = 16
    x = bits(synth.hidden_states(cfg, T))
    lg = bits(synth.router_logits(cfg, T))
    wts = synth.expert_weights(cfg)
    ids, w = oracle.route(oracle.ROUTE_SOFTMAX, cfg.E, cfg.k, lg, renormalize=True)
    a = oracle.align(ids, T, cfg.k, cfg.E, 16)
    W = oracle.Weights(oracle.BF16, cfg.E, cfg.H, cfg.I, bits(wts.w13), bits(wts.w2))
    out = oracle.to_bf16(oracle.forward(W, x, ids, w))
    return dict(hidden_sum=float(x.astype(np.uint64).sum()), logits_sum=float(lg.astype(np.uint64).sum()),
                w13_sum=float(bits(wts.w13).astype(np.uint64).sum()), topk_ids=ids, topk_weights=w,
                sorted_token_ids=a["sorted_token_ids"], expert_counts=a["expert_counts"], out_bf16=out)


def serialise(d):
    lines = ["# tiny layer, T=16, seed 1001; oracle answer (see make_golden.py)"]
    for key, v in d.items():
        if isinstance(v, float):
            lines.append("%s %d" % (key, int(v)))
        elif v.dtype == np.float32:
            lines.append(key + " " + " ".join("%08x" % u for u in v.ravel().view(np.uint32)))
        else:
            lines.append(key + " " + " ".join(str(int(u)) for u in v.ravel()))
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_T16.txt"), "w") as f:
        f.write(serialise(compute()))
