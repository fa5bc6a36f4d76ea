"""Helpers of the GPU parity tests: device layers from the seeded generator, the oracle's
view of the same inputs, comparison metrics.  (Not a test module.)"""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_layer_02_amd import abi, synth

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

# spec tolerances on the layer output (relative L2 over the whole [T, H] output)
TOL = {synth.WDT_BF16: 1e-2, synth.WDT_FP8: 3e-2, synth.WDT_INT4: 3e-2}


def say(*a):
    """Name the case about to run on the GPU (flushed, so a crash still shows it)."""
    print(*a, file=sys.stderr, flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 / fp16 tensor -> its uint16 bit patterns (host numpy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


@functools.lru_cache(maxsize=2)
def weights(name: str, device: str):
    """Expert weights of a config: 'cpu' draws them on the host, 'cuda' on the GPU."""
    return synth.expert_weights(synth.CONFIGS[name], device=device)


def oracle_weights(cfg, w: synth.ExpertWeights) -> oracle.Weights:
    wd = {synth.WDT_BF16: oracle.BF16, synth.WDT_FP8: oracle.FP8_E4M3, synth.WDT_INT4: oracle.INT4_G128}[cfg.wdtype]
    if cfg.wdtype == synth.WDT_BF16:
        return oracle.Weights(wd, cfg.E, cfg.H, cfg.I, bits(w.w13), bits(w.w2))
    if cfg.wdtype == synth.WDT_FP8:
        return oracle.Weights(wd, cfg.E, cfg.H, cfg.I, u8(w.w13), u8(w.w2),
                              w13_scale=w.w13_scale.cpu().numpy(), w2_scale=w.w2_scale.cpu().numpy())
    return oracle.Weights(wd, cfg.E, cfg.H, cfg.I, u8(w.w13), u8(w.w2), w13_s=bits(w.w13_s), w13_z=bits(w.w13_z),
                          w2_s=bits(w.w2_s), w2_z=bits(w.w2_z))


def device_layer(cfg, w: synth.ExpertWeights, bias=None) -> abi.MoELayer:
    d = {k: v.cuda().contiguous() for k, v in w.tensors().items()}
    return abi.MoELayer.create(cfg.E, cfg.H, cfg.I, cfg.k, cfg.route_kind, cfg.wdtype, d["w13"], d["w2"],
                               renormalize=cfg.renormalize, n_group=cfg.n_group, topk_group=cfg.topk_group,
                               routed_scaling=cfg.routed_scaling, w13_scale=d.get("w13_scale"),
                               w2_scale=d.get("w2_scale"), w13_s=d.get("w13_s"), w13_z=d.get("w13_z"),
                               w2_s=d.get("w2_s"), w2_z=d.get("w2_z"),
                               correction_bias=None if bias is None else bias.cuda().contiguous())


def oracle_route(cfg, logits_bits, bias):
    return oracle.route(cfg.route_kind, cfg.E, cfg.k, logits_bits, renormalize=cfg.renormalize,
                        n_group=cfg.n_group, topk_group=cfg.topk_group, routed_scaling=cfg.routed_scaling,
                        bias=None if bias is None else bias.numpy())


def workspace_view(layer, T, plan, ws, region, dtype, count):
    off = abi.moe_workspace_offsets(layer.struct, T, plan)[region]
    return ws[off:off + count * torch.tensor([], dtype=dtype).element_size()].view(dtype)


def valid_plans(layer, T, split1=(1, 2, 4), splits=(1, 2, 4, 8), tails=(0,), max_workgroups=0, tails1=(0,),
                ragged=(0,)):
    """Every (block_m, tile1, tile2, split, split1, split_tail, split_tail1, ragged) the
    library accepts for this layer (grids capped at max_workgroups)."""
    n = 64   # every tile id the library compiles (ids run below 64)
    out = []
    for rg in ragged:
        for g1 in range(n):
            for g2 in range(n):
                for sk in splits:
                    for s1 in split1:
                        for st in tails:
                            for st1 in tails1:
                                for bm in (16, 32, 64, 128, 256):
                                    p = abi.Plan(bm, g1, g2, sk, s1, st, max_workgroups, st1, rg)
                                    try:
                                        abi.moe_workspace_bytes(layer.struct, T, p)
                                    except abi.MoEError:
                                        continue
                                    out.append(p)
    return out


def gemm1_tile(layer, T, plan):
    """(BM, BN, BK) of the plan's GEMM1 tile, from moe_plan_describe."""
    return gemm2_tile(layer, T, plan, "gemm1=")


def gemm2_tile(layer, T, plan, which="gemm2="):
    """(BM, BN, BK) of the plan's GEMM2 tile, from moe_plan_describe."""
    d = abi.moe_plan_describe(layer.struct, T, plan)
    g2 = d.split(which)[1]
    f = {k: int(v) for k, v in (("BM", g2.split("BM")[1].split()[0]), ("BN", g2.split("BN")[1].split()[0]),
                                   ("BK", g2.split("BK")[1].split()[0]))}
    return f["BM"], f["BN"], f["BK"]


def expected_tail(npp, cap, H, I, tile, max_workgroups, split_tail, units=256, gemm1=False):
    """The split tail GEMM2 (GEMM1: gemm1=True) takes with its grid capped at max_workgroups
    (fewer than the compute units): (first tail row, S), S = 0 when it splits nothing -- the
    rule of the split_tail / split_tail1 plan fields restated.  The grid is also at most the
    tiles the capacity allows, and a multiple of 8 from 8 on.  GEMM1's tiles cover BN / 2
    of the I outputs and its K is H."""
    BM, BN, BK = tile
    if gemm1:
        H, I, BN = I, H, BN // 2
    mblocks, ntiles = npp // BM, H // BN
    grid = min(max_workgroups, cap // BM * ntiles)
    if grid >= 8:
        grid -= grid % 8
    mn = mblocks * ntiles
    rem = mn % grid
    if rem:
        tmb = -(-rem // ntiles)
        tt = tmb * ntiles
        s = min(split_tail, grid // tt, units // tt, I // BK)
        if s >= 2:
            return (mblocks - tmb) * BM, s
    return mblocks * BM, 0


def block_cover_tokens(sorted_ids, npp, BM, k, pairs, extra=(), blk_start=None):
    """Tokens whose pairs lie in every row block of an align layout: block by block, a
    block with a real row that no chosen token covers adds the token of its last real row
    (the ragged edge of an expert's rows) -- so each block, the split-tail blocks included,
    holds at least one row the oracle computes.  Plus the tokens in `extra`.  blk_start:
    the block table of the layout without padding (block b = sorted_ids[blk_start[b] :
    blk_start[b + 1]])."""
    chosen = set(int(t) for t in extra)
    sorted_ids = np.asarray(sorted_ids)
    for b in range(int(npp) // BM):
        if blk_start is None:
            rows = sorted_ids[b * BM:(b + 1) * BM]
        else:
            rows = sorted_ids[int(blk_start[b]):int(blk_start[b + 1])]
        real = rows[rows < pairs]                      # pairs = T*k is the filler value
        if real.size == 0:
            continue
        if not any(int(p) // k in chosen for p in real):
            chosen.add(int(real[-1]) // k)
    return sorted(chosen)
