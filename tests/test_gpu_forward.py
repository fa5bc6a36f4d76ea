"""moe_forward on the GPU vs the oracle.

Layer outputs within the relative-L2 budget (bf16 weights 1e-2, fp8 and int4 3e-2) on all
five configs; the routing and align intermediates the forward leaves in its workspace
bit-exact; every plan the library accepts on the tiny layer; the full-size Mixtral and
Llama-4-Scout shapes at the largest T on tokens the oracle computes one by one; bitwise
determinism, hipGraph replay equal to eager, split-K on and off in agreement; routing that
sends every token to the same one or two experts.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_layer_02_amd import abi, synth
from tests.gpu_util import (TOL, bits, bf16_to_f64, block_cover_tokens, device_layer, expected_tail, gemm1_tile,
                            gemm2_tile, needs_gpu, oracle_route, oracle_weights, rel_l2, say, valid_plans, weights,
                            workspace_view)

pytestmark = [pytest.mark.gpu, needs_gpu]


class Case:
    """A config with its device layer and the oracle's view of the same weights."""

    def __init__(self, name, device_for_weights, cfg=None):
        self.cfg = cfg or synth.CONFIGS[name]
        say("generating weights", name, "on", device_for_weights)
        w = synth.expert_weights(cfg, device=device_for_weights) if cfg else weights(name, device_for_weights)
        self.bias = synth.correction_bias(self.cfg)
        self.layer = device_layer(self.cfg, w, self.bias)
        self.W = oracle_weights(self.cfg, w)

    def inputs(self, T):
        return synth.hidden_states(self.cfg, T), synth.router_logits(self.cfg, T)

    def gpu(self, T, plan=None, ws=None):
        x, lg = self.inputs(T)
        say("forward", self.cfg.name, "T=%d" % T, "plan", None if plan is None else plan.as_tuple())
        if ws is None:
            ws = self.layer.workspace(T, plan)
        out = self.layer.forward(x.cuda(), lg.cuda(), workspace=ws, plan=plan)
        torch.cuda.synchronize()
        return out, ws

    def oracle(self, T, tokens=None):
        x, lg = self.inputs(T)
        ids, w = oracle_route(self.cfg, bits(lg), self.bias)
        return oracle.forward(self.W, bits(x), ids, w, tokens=tokens), ids, w


_cases = {}


def case(name):
    if name not in _cases:
        dev = "cpu" if name == "tiny" else "cuda"
        _cases[name] = Case(name, dev)
    return _cases[name]


def check_intermediates(c, T, plan, ws):
    """Route and align results inside the forward's workspace equal the oracle's."""
    cfg = c.cfg
    plan = plan or c.layer.plan(T)
    _, lg = c.inputs(T)
    rids, rw = oracle_route(cfg, bits(lg), c.bias)
    ids = workspace_view(c.layer, T, plan, ws, "topk_ids", torch.int32, T * cfg.k).cpu().numpy().reshape(T, cfg.k)
    assert (ids == rids).all()
    w = workspace_view(c.layer, T, plan, ws, "topk_weights", torch.float32, T * cfg.k).cpu().numpy()
    np.testing.assert_allclose(w.reshape(T, cfg.k), rw, rtol=1e-5, atol=1e-7)
    ref = oracle.align(rids, T, cfg.k, cfg.E, plan.block_m)
    cap = abi.moe_align_capacity(T, cfg.k, cfg.E, plan.block_m)
    pairs = T * cfg.k
    if plan.ragged:
        # no padding: the oracle's stable order with its filler entries removed, each pair's
        # row in that order, and the blocks cut at expert ends
        want = ref["sorted_token_ids"][ref["sorted_token_ids"] < pairs]
        srt = workspace_view(c.layer, T, plan, ws, "sorted_ids", torch.int32, pairs).cpu().numpy()
        assert (srt == want).all()
        inv = workspace_view(c.layer, T, plan, ws, "inv_pos", torch.int32, pairs).cpu().numpy()
        assert (inv == np.argsort(want, kind="stable")).all()
        nb = cap // plan.block_m
        blk = workspace_view(c.layer, T, plan, ws, "block_start", torch.int32, nb + 1).cpu().numpy()
        coff = np.concatenate([[0], np.cumsum(ref["expert_counts"])])
        poff = np.concatenate([[0], np.cumsum((ref["expert_counts"] + plan.block_m - 1) // plan.block_m
                                              * plan.block_m)])
        for b in range(nb + 1):
            e = ref["expert_ids"][b] if b < nb else -1
            assert blk[b] == (coff[e] + b * plan.block_m - poff[e] if e >= 0 else pairs), b
    else:
        srt = workspace_view(c.layer, T, plan, ws, "sorted_ids", torch.int32, cap).cpu().numpy()
        assert (srt == ref["sorted_token_ids"]).all()
        inv = workspace_view(c.layer, T, plan, ws, "inv_pos", torch.int32, pairs).cpu().numpy()
        assert (inv == ref["inv_pos"]).all()
    npp = workspace_view(c.layer, T, plan, ws, "num_post_pad", torch.int32, 1).cpu().numpy()
    assert npp[0] == ref["num_tokens_post_padded"][0]
    eids = workspace_view(c.layer, T, plan, ws, "expert_ids", torch.int32, cap // plan.block_m).cpu().numpy()
    assert (eids == ref["expert_ids"]).all()
    counts = workspace_view(c.layer, T, plan, ws, "expert_counts", torch.int32, cfg.E).cpu().numpy()
    assert (counts == ref["expert_counts"]).all()


def check_full(name, T, plan=None):
    c = case(name)
    out, ws = c.gpu(T, plan)
    ref, _, _ = c.oracle(T)
    err = rel_l2(bf16_to_f64(out), ref)
    say("  rel-L2 %.3e" % err)
    assert err <= TOL[c.cfg.wdtype], "rel-L2 %.3e" % err
    check_intermediates(c, T, plan, ws)
    return out


def check_sampled(name, T, tokens=None, plan=None):
    """The forward at T against the oracle on sampled tokens: by default one token in every
    row block of the layout the forward used (so every GEMM tile row range, the split-tail
    blocks included, holds a compared row).  Each sampled row is within the tolerance on its
    own, and so is the set."""
    c = case(name)
    out, ws = c.gpu(T, plan)
    plan = plan or c.layer.plan(T)
    cap = abi.moe_align_capacity(T, c.cfg.k, c.cfg.E, plan.block_m)
    srt = workspace_view(c.layer, T, plan, ws, "sorted_ids", torch.int32,
                         T * c.cfg.k if plan.ragged else cap).cpu().numpy()
    npp = int(workspace_view(c.layer, T, plan, ws, "num_post_pad", torch.int32, 1).cpu()[0])
    blk = None
    if plan.ragged:
        blk = workspace_view(c.layer, T, plan, ws, "block_start", torch.int32, cap // plan.block_m + 1).cpu().numpy()
    if tokens is None:
        tokens = block_cover_tokens(srt, npp, plan.block_m, c.cfg.k, T * c.cfg.k, extra=(0, T - 1), blk_start=blk)
        # the split tails GEMM1 / GEMM2 took (rows from row0 on) are among the covered blocks
        inv = workspace_view(c.layer, T, plan, ws, "inv_pos", torch.int32, T * c.cfg.k).cpu().numpy()
        inv = inv.reshape(T, c.cfg.k)
        for region, on in (("gemm2_tail", plan.split_tail > 1), ("gemm1_tail", plan.split_tail1 > 1)):
            if on:
                row0, S = (int(v) for v in workspace_view(c.layer, T, plan, ws, region, torch.int32, 4).cpu()[:2])
                if S:
                    assert any((inv[t] >= row0).any() for t in tokens), region
                    say("  %s from row %d, S=%d: sampled" % (region, row0, S))
    say("  %d sampled tokens over %d row blocks" % (len(tokens), npp // plan.block_m))
    ref, _, _ = c.oracle(T, tokens=tokens)
    got = bf16_to_f64(out[tokens])
    err = rel_l2(got, ref)
    worst = max(rel_l2(got[i], ref[i]) for i in range(len(tokens)))
    say("  sampled rel-L2 %.3e, worst row %.3e" % (err, worst))
    assert err <= TOL[c.cfg.wdtype], "rel-L2 %.3e" % err
    assert worst <= TOL[c.cfg.wdtype], "worst row rel-L2 %.3e" % worst
    assert torch.isfinite(out.float()).all()
    check_intermediates(c, T, plan, ws)


# ---- tiny layer: every plan, ragged sizes -----------------------------------------------

@pytest.mark.parametrize("T", [1, 2, 3, 16, 37, 64, 100])
def test_tiny_every_plan(T):
    c = case("tiny")
    plans = valid_plans(c.layer, T)
    assert len(plans) >= 8
    ref, _, _ = c.oracle(T)
    for p in plans:
        out, ws = c.gpu(T, p)
        err = rel_l2(bf16_to_f64(out), ref)
        assert err <= TOL[c.cfg.wdtype], "plan %s rel-L2 %.3e" % (p.as_tuple(), err)
    check_intermediates(c, T, plans[-1], ws)


TINY_TOP1 = synth.CONFIGS["tiny"].with_shape(name="tiny_top1", k=1, route_kind=abi.ROUTE_SIGMOID, renormalize=False)


@pytest.mark.parametrize("T", [1, 37])
def test_tiny_top1_every_plan(T):
    """Top-1 routing: plans without a K split write GEMM2's rows straight into the output
    (no reduce pass), split plans go through the reduce; both match the oracle."""
    if "tiny_top1" not in _cases:
        _cases["tiny_top1"] = Case("tiny_top1", "cpu", TINY_TOP1)
    c = _cases["tiny_top1"]
    plans = valid_plans(c.layer, T)
    assert any(p.split_k == 1 for p in plans) and any(p.split_k > 1 for p in plans)
    ref, _, _ = c.oracle(T)
    x, lg = c.inputs(T)
    for p in plans:
        out, ws = c.gpu(T, p)
        err = rel_l2(bf16_to_f64(out), ref)
        assert err <= TOL[c.cfg.wdtype], "plan %s rel-L2 %.3e" % (p.as_tuple(), err)
        if p.gemm1_tile == plans[0].gemm1_tile and p.block_m == plans[0].block_m:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(abi.STAGE_COUNT + 1)]
            o2 = torch.empty_like(out)
            stages = abi.moe_forward_profiled(c.layer.struct, T, x.cuda(), lg.cuda(), o2, ws, ev, p)
            torch.cuda.synchronize()
            assert ("reduce" in stages) == (p.split_k > 1 or p.split_tail > 1), (p.as_tuple(), stages)
            assert torch.equal(o2.view(torch.int16), out.view(torch.int16))


def test_tiny_zero_tokens():
    c = case("tiny")
    out = torch.empty((0, c.cfg.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    abi.moe_forward(c.layer.struct, 0, out, out, out, ws)


# ---- bf16 full shapes ------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 4])
def test_mixtral_small_T(T):
    check_full("mixtral", T)


def test_mixtral_largest_T_sampled():
    check_sampled("mixtral", 4096)


def test_mixtral_mid_T_sampled():
    check_sampled("mixtral", 256)


@pytest.mark.parametrize("T", [32, 1024])
def test_mixtral_sweep_T_sampled(T):
    check_sampled("mixtral", T)


def test_mixtral_every_large_tile_plan_sampled():
    """Every plan with block_m >= 64 on the full-size Mixtral shard (the tile shapes the
    large-T bench uses), against one oracle computation of sampled tokens."""
    c = case("mixtral")
    T, tokens = 512, [0, 211, 511]
    ref, _, _ = c.oracle(T, tokens=tokens)
    plans = [p for p in valid_plans(c.layer, T) if p.block_m >= 64]
    assert len(plans) >= 10
    for p in plans:
        out, ws = c.gpu(T, p)
        err = rel_l2(bf16_to_f64(out[tokens]), ref)
        assert err <= TOL[c.cfg.wdtype], "plan %s rel-L2 %.3e" % (p.as_tuple(), err)


@pytest.mark.parametrize("T", [1, 5])
def test_scout_small_T(T):
    check_full("scout", T)


def test_scout_largest_T_sampled():
    check_sampled("scout", 8192)


@pytest.mark.parametrize("T", [32, 2048])
def test_scout_sweep_T_sampled(T):
    check_sampled("scout", T)


# ---- fp8 w8a8 --------------------------------------------------------------------------

def test_qwen2_largest_T_route_and_align():
    """T*k = 32768 pairs: the forward's multi-workgroup align must lay rows out exactly as
    the oracle's stable sort does."""
    c = case("qwen2")
    out, ws = c.gpu(4096)
    assert torch.isfinite(out.float()).all()
    check_intermediates(c, 4096, None, ws)


QWEN2_NARROW = synth.CONFIGS["qwen2"].with_shape(name="qwen2_narrow", H=512, I=256, wdtype=synth.WDT_BF16)


@pytest.mark.parametrize("T", [2000, 8192, 8193, 9000])
def test_align_paths_in_forward(T):
    """Qwen2's routing (64 experts, top-8) on narrow bf16 weights (per-token work, so the
    oracle computes the sampled tokens alone): 16000 and 65536 pairs take the
    one-launch align whose workgroups each count the whole batch, 65544 and 72000 pairs the
    count / scan / scatter launches; either way the rows are laid out exactly as the
    oracle's stable sort does, and sampled tokens match the oracle."""
    if "qwen2_narrow" not in _cases:
        _cases["qwen2_narrow"] = Case("qwen2_narrow", "cuda", QWEN2_NARROW)
    c = _cases["qwen2_narrow"]
    out, ws = c.gpu(T)
    tokens = [0, T // 2, T - 1]
    ref, _, _ = c.oracle(T, tokens=tokens)
    err = rel_l2(bf16_to_f64(out[tokens]), ref)
    say("  sampled rel-L2 %.3e" % err)
    assert err <= TOL[c.cfg.wdtype]
    check_intermediates(c, T, None, ws)


@pytest.mark.parametrize("T", [1, 8, 24, 128, 512, 2048])
def test_qwen2_fp8(T):
    """The whole [T, H] output: T = 128, 512 and 2048 run the 32-, 128- and 256-row fp8
    plans of the Qwen2 shard (with GEMM1's and GEMM2's split tails) at its real shape."""
    check_full("qwen2", T)


def test_qwen2_fp8_largest_T_sampled():
    """T = 4096 (the 256x256 fp8 tiles with GEMM2's split tail): one token per row block."""
    check_sampled("qwen2", 4096)


@pytest.mark.parametrize("T", [16, 40])
def test_qwen2_fp8_activation_codes_exact(T):
    """The hidden states' E4M3 codes are decided in fp32 on both sides: bit-exact (T=16:
    the one-launch prologue; T=40: the separate absmax and quantisation kernels)."""
    c = case("qwen2")
    out, ws = c.gpu(T)
    plan = c.layer.plan(T)
    x, _ = c.inputs(T)
    xf = x.float().numpy()
    amax = np.float32(np.abs(xf).max())
    inv = np.float32(np.float32(448.0) / amax)
    ref_codes = oracle.f32_to_e4m3((xf * inv).astype(np.float32))
    got = workspace_view(c.layer, T, plan, ws, "x_q", torch.uint8, T * c.cfg.H).cpu().numpy().reshape(T, -1)
    same = (got == ref_codes) | ((got & 0x7F) == 0) & ((ref_codes & 0x7F) == 0)   # +-0 either way
    assert same.all(), "%d codes differ" % (~same).sum()
    sc = workspace_view(c.layer, T, plan, ws, "scalars", torch.float32, 4).cpu().numpy()
    assert sc[2] == np.float32(amax / np.float32(448.0))


@pytest.mark.parametrize("T", [16, 512])
@pytest.mark.parametrize("ragged", [0, 1])
def test_qwen2_fp8_intermediate_codes(T, ragged):
    """The intermediate h is quantised from fp32 on both sides (T=16: the one-workgroup
    finishing pass quantises it; T=512: GEMM1's epilogue and the quantisation kernel).
    - The GPU's codes are exactly the oracle's codec applied to the GPU's own fp32 h and
      scale (RNE to E4M3 of h * (448 / amax) in fp32), bit for bit, and its amax is the
      exact maximum of its |h| over the valid rows.
    - The GPU's h (fp32 accumulation) and the oracle's (fp64, rounded to fp32) differ by
      the accumulation order only: a length-3584 dot product in fp32 is off by at most
      ~n * 2^-24 = 2e-4 of the sum of its terms' magnitudes, which for these rows stays
      within 1e-3 of the largest |h|; the two scales agree to 2e-4.
    - So a code differs from the oracle's only where the two h values straddle an E4M3
      rounding midpoint: each differing code is one step from the oracle's, and the
      midpoint between them lies between the two scaled values."""
    c = case("qwen2")
    plan = abi.Plan(*(c.layer.plan(T).as_tuple() + (0,) * 9)[:8], ragged)   # the default, in either layout
    out, ws = c.gpu(T, plan)
    x, lg = c.inputs(T)
    ids, _ = oracle_route(c.cfg, bits(lg), c.bias)
    ref_h, ref_codes, ref_sc = oracle.fp8_intermediate(c.W, bits(x), ids)
    sc = workspace_view(c.layer, T, plan, ws, "scalars", torch.float32, 4).cpu().numpy()
    amax_gpu = np.float32(sc[1])                       # word 1: |h| max as fp32 bits
    assert abs(sc[3] / ref_sc[1] - 1) < 2e-4
    # h's rows: the padded capacity, or exactly the T*k pairs without padding
    rows = T * c.cfg.k if plan.ragged else abi.moe_align_capacity(T, c.cfg.k, c.cfg.E, plan.block_m)
    inv = workspace_view(c.layer, T, plan, ws, "inv_pos", torch.int32, T * c.cfg.k).cpu().numpy()
    hq = workspace_view(c.layer, T, plan, ws, "h_q", torch.uint8, rows * c.cfg.I).cpu().numpy().reshape(rows, -1)[inv]
    h = workspace_view(c.layer, T, plan, ws, "h", torch.float32, rows * c.cfg.I).cpu().numpy().reshape(rows, -1)[inv]
    # the GPU's own quantisation, exactly
    assert np.float32(np.abs(h).max()) == amax_gpu
    assert sc[3] == np.float32(amax_gpu / np.float32(448.0))
    inv_gpu = np.float32(np.float32(448.0) / amax_gpu)
    own = oracle.f32_to_e4m3((h * inv_gpu).astype(np.float32))
    same = (own == hq) | (((own & 0x7F) == 0) & ((hq & 0x7F) == 0))
    assert same.all(), "%d codes differ from the codec applied to the GPU's h" % (~same).sum()
    # the GPU's h against the oracle's
    dh = np.abs(h.astype(np.float64) - ref_h) / np.abs(ref_h).max()
    say("  h max diff %.2e of max|h|" % dh.max())
    assert dh.max() <= 1e-3
    # differing codes straddle a midpoint
    val = lambda q: oracle.e4m3_to_f32(q).astype(np.float64)  # noqa: E731
    diff = (hq != ref_codes) & ~(((hq & 0x7F) == 0) & ((ref_codes & 0x7F) == 0))
    say("  h codes differing from the oracle's: %d of %d (%.2e)" % (diff.sum(), diff.size, diff.mean()))
    a, b = val(hq[diff]), val(ref_codes[diff])
    assert (np.abs(a - b) <= np.maximum(np.abs(a), np.abs(b)) * 0.125 + 2.0 ** -9).all()   # one step
    mid = (a + b) / 2
    vg = (h[diff] * inv_gpu).astype(np.float64)
    inv_ref = np.float32(np.float32(448.0) / np.float32(np.abs(ref_h).max()))   # the oracle's own factor
    vr = (ref_h[diff] * inv_ref).astype(np.float64)
    lo, hi = np.minimum(vg, vr), np.maximum(vg, vr)
    slack = 1e-6 * np.abs(mid)
    assert ((lo - slack <= mid) & (mid <= hi + slack)).all(), "a differing code does not straddle a midpoint"


# ---- int4 group 128 --------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 3])
def test_deepseek_int4(T):
    check_full("deepseek", T)


def test_deepseek_int4_largest_T_sampled():
    check_sampled("deepseek", 512)


def test_deepseek_int4_mid_T_sampled():
    check_sampled("deepseek", 64)


# Qwen2's w8a8 fp8 format at a size where every fp8 tile runs (four K steps of 128 in GEMM1,
# two in GEMM2): every plan against the oracle
FP8_SMALL = synth.CONFIGS["qwen2"].with_shape(name="fp8small", E=16, k=4, H=512, I=256)


@pytest.mark.parametrize("T", [1, 6, 40, 300])
def test_fp8_every_plan(T):
    if "fp8small" not in _cases:
        _cases["fp8small"] = Case("fp8small", "cpu", FP8_SMALL)
    c = _cases["fp8small"]
    plans = valid_plans(c.layer, T)
    tiles = {p.gemm1_tile for p in plans}
    assert {0, 1, 2, 7, 9, 12, 14} <= tiles, tiles       # staged and pipelined, 8 and 16 waves
    ref, _, _ = c.oracle(T)
    for p in plans:
        out, ws = c.gpu(T, p)
        err = rel_l2(bf16_to_f64(out), ref)
        assert err <= TOL[c.cfg.wdtype], "plan %s rel-L2 %.3e" % (p.as_tuple(), err)
    check_intermediates(c, T, plans[-1], ws)


# DeepSeek-V3's gate and int4 format at a size the oracle runs in well under a second: three
# K steps of 256 in GEMM1 (a ragged start for the K rotation), two in GEMM2 (split-K 2)
I4_SMALL = synth.CONFIGS["deepseek"].with_shape(name="i4small", E=16, k=4, n_group=4, topk_group=2, H=768, I=512)


@pytest.mark.parametrize("T", [1, 5, 37, 200])
def test_int4_every_plan(T):
    if "i4small" not in _cases:
        _cases["i4small"] = Case("i4small", "cpu", I4_SMALL)
    c = _cases["i4small"]
    plans = valid_plans(c.layer, T)
    tiles = {p.gemm1_tile for p in plans}
    assert {0, 4, 5, 6, 7, 8, 9, 10} <= tiles, tiles       # staged and pipelined tiles both run
    ref, _, _ = c.oracle(T)
    for p in plans:
        out, ws = c.gpu(T, p)
        err = rel_l2(bf16_to_f64(out), ref)
        assert err <= TOL[c.cfg.wdtype], "plan %s rel-L2 %.3e" % (p.as_tuple(), err)
    check_intermediates(c, T, plans[-1], ws)


@pytest.mark.parametrize("scale", [3e4, 1e5, 1e6])
def test_int4_outlier_channels(scale):
    """Hidden states with outlier channels far past fp16's range (65504), as real DeepSeek
    activations carry: the int4 kernels keep activations and the intermediate in bf16 (bf16
    MFMA), so every plan of both tile kinds stays finite and within tolerance of the oracle
    on the same bf16 inputs."""
    if "i4small" not in _cases:
        _cases["i4small"] = Case("i4small", "cpu", I4_SMALL)
    c = _cases["i4small"]
    T = 37
    x, lg = c.inputs(T)
    xf = x.float()
    xf[:, [5, 300, 701]] = torch.tensor([scale, -scale, 0.5 * scale])
    xf[3, 100] = -2.0 * scale
    x = xf.to(torch.bfloat16)
    ids, w = oracle_route(c.cfg, bits(lg), c.bias)
    ref = oracle.forward(c.W, bits(x), ids, w)
    assert np.isfinite(ref).all()
    plans = valid_plans(c.layer, T)
    kinds = {p.gemm1_tile >= 4 for p in plans}
    assert kinds == {False, True}                       # register-staged and pipelined tiles
    for p in plans[::3] + [plans[-1]]:
        say("int4 outliers %.0e plan %s" % (scale, p.as_tuple()))
        out = c.layer.forward(x.cuda(), lg.cuda(), plan=p)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all(), p.as_tuple()
        err = rel_l2(bf16_to_f64(out), ref)
        assert err <= TOL[c.cfg.wdtype], "plan %s rel-L2 %.3e" % (p.as_tuple(), err)


# ---- the layout without padding (ragged plans) -------------------------------------------

def ragged_of(plan):
    return abi.Plan(*(plan.as_tuple() + (0,) * (8 - len(plan.as_tuple()))), 1) if not plan.ragged else plan


@pytest.mark.parametrize("name,T", [("tiny", 37), ("tiny", 100), ("tiny_top1", 37), ("fp8small", 40),
                                    ("fp8small", 300), ("i4small", 37), ("i4small", 200)])
def test_ragged_every_plan(name, T):
    """Every plan of the layout without padding (the pairs expert by expert, no filler rows;
    GEMM tiles cut at expert ends) on the small shapes of all three weight types: output
    within tolerance, routing and the unpadded layout bit-exact."""
    cfg = {"tiny_top1": TINY_TOP1, "fp8small": FP8_SMALL, "i4small": I4_SMALL}.get(name)
    c = case(name) if cfg is None else small_case(cfg)
    plans = valid_plans(c.layer, T, ragged=(1,))
    assert len(plans) >= 8 and all(p.ragged for p in plans)
    ref, _, _ = c.oracle(T)
    for p in plans:
        out, ws = c.gpu(T, p)
        err = rel_l2(bf16_to_f64(out), ref)
        assert err <= TOL[c.cfg.wdtype], "plan %s rel-L2 %.3e" % (p.as_tuple(), err)
    for p in (plans[0], plans[len(plans) // 2], plans[-1]):
        check_intermediates(c, T, p, c.gpu(T, p)[1])


@pytest.mark.parametrize("name", ["tiny", "tiny_top1", "fp8small", "i4small"])
def test_one_token_layouts(name):
    """One token (a decode step): its k distinct experts are laid out directly by the
    prologue. Every block height, with and without padding: routing and the layout
    bit-exact against the oracle's align, the output within tolerance."""
    cfg = {"tiny_top1": TINY_TOP1, "fp8small": FP8_SMALL, "i4small": I4_SMALL}.get(name)
    c = case(name) if cfg is None else small_case(cfg)
    plans = valid_plans(c.layer, 1, split1=(1,), splits=(1,), ragged=(0, 1))
    picked = {}
    for p in plans:   # the first plan of every (block height, layout)
        picked.setdefault((p.block_m, p.ragged), p)
    assert len(picked) >= 4
    ref, _, _ = c.oracle(1)
    for (bm, rg), p in sorted(picked.items()):
        out, ws = c.gpu(1, p)
        assert rel_l2(bf16_to_f64(out), ref) <= TOL[c.cfg.wdtype], p.as_tuple()
        check_intermediates(c, 1, p, ws)


@pytest.mark.parametrize("name", ["mixtral", "qwen2", "deepseek", "scout"])
def test_one_token_full_layers(name):
    """The layers' own plans at T = 1, and the same tiles with the other layout."""
    c = case(name)
    dp = c.layer.plan(1)
    head = (dp.as_tuple() + (0,) * 9)[:8]
    for p in (dp, abi.Plan(*head, 1 - dp.ragged)):
        out, ws = c.gpu(1, p)
        ref, _, _ = c.oracle(1)
        assert rel_l2(bf16_to_f64(out), ref) <= TOL[c.cfg.wdtype], p.as_tuple()
        check_intermediates(c, 1, p, ws)


@pytest.mark.parametrize("T", [100, 300])
def test_ragged_split_tails(T):
    """Both split tails and the K splits on grids capped so that whole tiles are followed by
    a split tail, without padding: the tails' first rows are rows of the unpadded layout."""
    c = small_case(TAIL_SMALL)
    ref, _, _ = c.oracle(T)
    n = 0
    for g in (24, 48):
        for p in valid_plans(c.layer, T, split1=(1,), splits=(1, 2), tails=(0, 4), max_workgroups=g, tails1=(0, 4),
                             ragged=(1,))[::2]:
            out, ws = c.gpu(T, p)
            err = rel_l2(bf16_to_f64(out), ref)
            assert err <= TOL[c.cfg.wdtype], "plan %s rel-L2 %.3e" % (p.as_tuple(), err)
            n += 1
    assert n >= 10


@pytest.mark.parametrize("name,T,whole", [("mixtral", 4096, False), ("mixtral", 512, False), ("scout", 8192, False),
                                          ("qwen2", 512, True), ("qwen2", 4096, False), ("deepseek", 512, False),
                                          ("mixtral", 8, True)])
def test_ragged_full_size(name, T, whole):
    """The full-size layers under their default plans made unpadded: the whole output (or one
    token per row block), routing and the unpadded layout bit-exact."""
    c = case(name)
    p = ragged_of(c.layer.plan(T))
    if whole:
        check_full(name, T, p)
    else:
        check_sampled(name, T, plan=p)


def test_ragged_equals_padded_bitwise():
    """A row's products do not depend on where it sits: with the same tiles and splits, the
    unpadded layout gives the padded layout's output bit for bit."""
    c = case("mixtral")
    for T in (64, 1024):
        p = c.layer.plan(T)
        a, _ = c.gpu(T, p)
        b, _ = c.gpu(T, ragged_of(p))
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), T


# ---- properties ------------------------------------------------------------------------

@pytest.mark.parametrize("name,T", [("mixtral", 1), ("qwen2", 3), ("deepseek", 2), ("scout", 5)])
def test_gemm1_split_k(name, T):
    """GEMM1 split into 2 and 4 K ranges (fp32 partial planes of gate and up, added in order
    by the finishing pass) on the full-size layers: output within tolerance, routing and
    align bit-exact, and the same output for a repeated call."""
    c = case(name)
    base = c.layer.plan(T)
    ran = 0
    for s1 in (2, 4, 7):
        p = abi.Plan(base.block_m, base.gemm1_tile, base.gemm2_tile, base.split_k, s1)
        try:
            abi.moe_workspace_bytes(c.layer.struct, T, p)
        except abi.MoEError:
            continue                  # H is not a multiple of s1 K steps for this tile
        out = check_full(name, T, p)
        again, _ = c.gpu(T, p)
        assert torch.equal(out.view(torch.int16), again.view(torch.int16))
        ran += 1
    assert ran >= 2


def test_deterministic_bitwise():
    c = case("mixtral")
    a, ws = c.gpu(64)
    b, _ = c.gpu(64, ws=ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_split_k_on_and_off_agree():
    c = case("mixtral")
    T = 4
    p = c.layer.plan(T)
    p1 = abi.Plan(p.block_m, p.gemm1_tile, p.gemm2_tile, 1)
    p4 = abi.Plan(p.block_m, p.gemm1_tile, p.gemm2_tile, 4)
    a, _ = c.gpu(T, p1)
    b, _ = c.gpu(T, p4)
    assert rel_l2(bf16_to_f64(a), bf16_to_f64(b)) < 5e-3


@pytest.mark.parametrize("name,T,ragged", [("tiny", 37, 0), ("mixtral", 8, 0), ("qwen2", 8, 0), ("qwen2", 300, 1)])
def test_graph_replay_matches_eager(name, T, ragged):
    c = case(name)
    x, lg = c.inputs(T)
    x, lg = x.cuda(), lg.cuda()
    plan = c.layer.plan(T)
    if ragged:
        plan = ragged_of(plan)
    ws = c.layer.workspace(T, plan)
    out = torch.empty((T, c.cfg.H), dtype=torch.bfloat16, device="cuda")
    eager = c.layer.forward(x, lg, out=torch.empty_like(out), workspace=ws, plan=plan).clone()
    say("graph capture", name, "T=%d" % T)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            c.layer.forward(x, lg, out=out, workspace=ws, plan=plan)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        out.zero_()
        ws.fill_(0xAB)                    # eager work between replays; the workspace is scratch
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), "replay %d" % i


@pytest.mark.parametrize("name,T,expect", [
    ("qwen2", 1, ["prologue", "gemm1", "h_quant", "gemm2", "reduce"]),
    ("qwen2", 16, ["prologue", "gemm1", "h_quant", "gemm2", "reduce"]),
    ("qwen2", 17, ["route", "align", "act_quant", "gemm1", "h_quant", "gemm2", "reduce"]),
    ("deepseek", 3, ["prologue", "gemm1", "gemm2", "reduce"]),
    ("deepseek", 16, ["prologue", "gemm1", "gemm2", "reduce"]),
    ("deepseek", 17, ["route", "align", "act_quant", "gemm1", "gemm2", "reduce"]),
    ("mixtral", 64, ["prologue", "gemm1", "gemm2", "reduce"]),
    ("mixtral", 65, ["route", "align", "gemm1", "gemm2", "reduce"])])
def test_small_batch_prologue(name, T, expect):
    """Up to 64 tokens (16 where a token's routing is long: more than 64 experts or top-k
    above 2; for fp8 also at most 131072 elements of hidden states), route, align and the
    activation pass run as one launch;
    the forward's routing and align results stay bit-exact and the output within tolerance."""
    c = case(name)
    x, lg = c.inputs(T)
    plan = c.layer.plan(T)
    ws = c.layer.workspace(T, plan)
    out = torch.empty((T, c.cfg.H), dtype=torch.bfloat16, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(abi.STAGE_COUNT + 1)]
    say("profiled forward", name, "T=%d" % T)
    stages = abi.moe_forward_profiled(c.layer.struct, T, x.cuda(), lg.cuda(), out, ws, ev, plan)
    torch.cuda.synchronize()
    if plan.split_k1 > 1 or plan.split_tail1 > 1:   # a K-split GEMM1 is followed by its finishing pass
        expect = expect[:expect.index("gemm1") + 1] + ["gemm1_finish"] + expect[expect.index("gemm1") + 1:]
        if c.cfg.wdtype == synth.WDT_FP8 and plan.split_k1 > 1 and T * c.cfg.k * c.cfg.I * plan.split_k1 <= 32768:
            expect.remove("h_quant")   # which also quantises h in a tiny batch
    assert stages == expect
    tokens = list(range(T)) if T <= 16 else [0, 1, T // 2, T - 1]   # the oracle token by token
    ref, _, _ = c.oracle(T, tokens=tokens)
    assert rel_l2(bf16_to_f64(out[tokens]), ref) <= TOL[c.cfg.wdtype]
    check_intermediates(c, T, plan, ws)


FP8_WIDE = synth.CONFIGS["qwen2"].with_shape(name="fp8wide", E=8, k=2, H=8192, I=256)


@pytest.mark.parametrize("T", [15, 16, 17])
def test_fp8_prologue_register_limit(T):
    """fp8 with short routing and H=8192: the prologue's activation pass holds the batch in
    registers, 131072 elements at most, so it takes T <= 16 (T=16 fills every register
    group, T=15 leaves the last ones reading the final group again) and T=17 goes to the
    separate kernels.  Codes bit-exact, output within tolerance."""
    c = small_case(FP8_WIDE)
    x, lg = c.inputs(T)
    plan = c.layer.plan(T)
    ws = c.layer.workspace(T, plan)
    out = torch.empty((T, c.cfg.H), dtype=torch.bfloat16, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(abi.STAGE_COUNT + 1)]
    say("profiled forward fp8wide T=%d" % T)
    stages = abi.moe_forward_profiled(c.layer.struct, T, x.cuda(), lg.cuda(), out, ws, ev, plan)
    torch.cuda.synchronize()
    assert ("prologue" in stages) == (T <= 16), stages
    xf = x.float().numpy()
    amax = np.float32(np.abs(xf).max())
    ref_codes = oracle.f32_to_e4m3((xf * np.float32(np.float32(448.0) / amax)).astype(np.float32))
    got = workspace_view(c.layer, T, plan, ws, "x_q", torch.uint8, T * c.cfg.H).cpu().numpy().reshape(T, -1)
    same = (got == ref_codes) | ((got & 0x7F) == 0) & ((ref_codes & 0x7F) == 0)
    assert same.all(), "%d codes differ" % (~same).sum()
    ref, _, _ = c.oracle(T)
    assert rel_l2(bf16_to_f64(out), ref) <= TOL[c.cfg.wdtype]


def test_profiled_forward_records_every_stage():
    c = case("qwen2")
    T = 32
    x, lg = c.inputs(T)
    ws = c.layer.workspace(T)
    out = torch.empty((T, c.cfg.H), dtype=torch.bfloat16, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(abi.STAGE_COUNT + 1)]
    stages = abi.moe_forward_profiled(c.layer.struct, T, x.cuda(), lg.cuda(), out, ws, ev)
    torch.cuda.synchronize()
    expect = ["route", "align", "act_quant", "gemm1", "h_quant", "gemm2", "reduce"]
    if c.layer.plan(T).split_k1 > 1 or c.layer.plan(T).split_tail1 > 1:
        expect.insert(4, "gemm1_finish")
    assert stages == expect
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(stages))]
    assert all(t >= 0 for t in times)
    ref, _, _ = c.oracle(T)
    assert rel_l2(bf16_to_f64(out), ref) <= TOL[c.cfg.wdtype]


# ---- GEMM2 split tail ------------------------------------------------------------------

def tail_taken(c, T, plan, ws):
    """(first tail row, S) that GEMM2 recorded in the workspace."""
    info = workspace_view(c.layer, T, plan, ws, "gemm2_tail", torch.int32, 4).cpu().numpy()
    return int(info[0]), int(info[1])


def check_tail_plans(c, T, grids, tails=(2, 8)):
    """Every split-tail plan on grids of `grids` workgroups against the oracle; GEMM2's
    recorded tail is the rule's.  Returns how many runs split a tail after whole tiles and
    how many split everything."""
    ref, _, _ = c.oracle(T)
    mixed = whole = 0
    for g in grids:
        plans = valid_plans(c.layer, T, split1=(1,), splits=(1,), tails=tails, max_workgroups=g)
        assert plans, "no split-tail plan"
        for p in plans:
            out, ws = c.gpu(T, p)
            err = rel_l2(bf16_to_f64(out), ref)
            assert err <= TOL[c.cfg.wdtype], "plan %s rel-L2 %.3e" % (p.as_tuple(), err)
            npp = int(workspace_view(c.layer, T, p, ws, "num_post_pad", torch.int32, 1).cpu()[0])
            got = tail_taken(c, T, p, ws)
            cap = abi.moe_align_capacity(T, c.cfg.k, c.cfg.E, p.block_m)
            want = expected_tail(npp, cap, c.cfg.H, c.cfg.I, gemm2_tile(c.layer, T, p), g, p.split_tail)
            assert got == want, (p.as_tuple(), got, want)
            if got[1]:
                mixed += got[0] > 0
                whole += got[0] == 0
    return mixed, whole


# a layer wide enough for several GEMM2 column tiles and K steps in every tile shape
TAIL_SMALL = synth.CONFIGS["tiny"].with_shape(name="tailsmall", H=512, I=512)
TAIL_SMALL_TOP1 = TAIL_SMALL.with_shape(name="tailsmall_top1", k=1, route_kind=abi.ROUTE_SIGMOID, renormalize=False)


def small_case(cfg):
    if cfg.name not in _cases:
        _cases[cfg.name] = Case(cfg.name, "cpu", cfg)
    return _cases[cfg.name]


@pytest.mark.parametrize("T", [100, 300])
def test_split_tail_every_plan(T):
    """GEMM2's last partial round as K splits (fp32 planes the reduce adds in order) on grids
    of 24 and 48 workgroups, every tile shape: whole tiles, then the split tail."""
    mixed, _ = check_tail_plans(small_case(TAIL_SMALL), T, (24, 48))
    assert mixed > 0


def test_split_tail_every_plan_fp8():
    mixed, _ = check_tail_plans(small_case(FP8_SMALL), 300, (8, 24))
    assert mixed > 0


@pytest.mark.parametrize("T", [100, 300])
def test_split_tail_top1(T):
    """Top-1: GEMM2 writes the whole-tile rows' tokens itself and the reduce writes only the
    tail's tokens."""
    mixed, _ = check_tail_plans(small_case(TAIL_SMALL_TOP1), T, (24,))
    assert mixed > 0


# ---- GEMM1 split tail ------------------------------------------------------------------

def tail1_taken(c, T, plan, ws):
    """(first tail row, S) that GEMM1 recorded in the workspace."""
    info = workspace_view(c.layer, T, plan, ws, "gemm1_tail", torch.int32, 4).cpu().numpy()
    return int(info[0]), int(info[1])


def check_tail1_plans(c, T, grids, tails2=(0,)):
    """Every GEMM1 split-tail plan on grids of `grids` workgroups against the oracle (with
    GEMM2's split tail off, or on as well); GEMM1's recorded tail is the rule's.  Returns
    how many runs split a tail after whole tiles."""
    ref, _, _ = c.oracle(T)
    mixed = 0
    for g in grids:
        plans = valid_plans(c.layer, T, split1=(1,), splits=(1,), tails=tails2, max_workgroups=g, tails1=(2, 8))
        assert plans, "no GEMM1 split-tail plan"
        for p in plans:
            out, ws = c.gpu(T, p)
            err = rel_l2(bf16_to_f64(out), ref)
            assert err <= TOL[c.cfg.wdtype], "plan %s rel-L2 %.3e" % (p.as_tuple(), err)
            npp = int(workspace_view(c.layer, T, p, ws, "num_post_pad", torch.int32, 1).cpu()[0])
            got = tail1_taken(c, T, p, ws)
            cap = abi.moe_align_capacity(T, c.cfg.k, c.cfg.E, p.block_m)
            want = expected_tail(npp, cap, c.cfg.H, c.cfg.I, gemm1_tile(c.layer, T, p), g, p.split_tail1, gemm1=True)
            assert got == want, (p.as_tuple(), got, want)
            mixed += got[1] > 0 and got[0] > 0
    return mixed


@pytest.mark.parametrize("T", [100, 300])
def test_split_tail1_every_plan(T):
    """GEMM1's last partial round as K splits (fp32 gate and up planes, finished in order
    before GEMM2) on grids of 24 and 48 workgroups, every pipelined GEMM1 tile."""
    assert check_tail1_plans(small_case(TAIL_SMALL), T, (24, 48)) > 0


def test_split_tail1_fp8_and_both_tails():
    """fp8 (the finishing pass also folds |h| of the tail rows), and both GEMMs' tails at once."""
    assert check_tail1_plans(small_case(FP8_SMALL), 300, (8, 24)) > 0
    assert check_tail1_plans(small_case(TAIL_SMALL), 300, (24,), tails2=(4,)) > 0


def test_split_tail1_mixtral_sampled():
    """The full-size Mixtral shard at T=1024 (a last GEMM1 round of a sixth) with GEMM1's
    split tail on the whole device: tokens whose rows lie in the tail against the oracle,
    and the same output on a second call."""
    c = case("mixtral")
    T = 1024
    p = abi.Plan(128, 22, 22, 1, 1, 8, 0, 8)
    out, ws = c.gpu(T, p)
    row0, S = tail1_taken(c, T, p, ws)
    say("  GEMM1 tail rows from %d, S=%d" % (row0, S))
    assert S >= 2 and row0 > 0
    inv = workspace_view(c.layer, T, p, ws, "inv_pos", torch.int32, T * c.cfg.k).cpu().numpy().reshape(T, c.cfg.k)
    in_tail = [t for t in range(T) if (inv[t] >= row0).any()]
    tokens = sorted(set(in_tail[:3] + [0, T - 1]))
    ref, _, _ = c.oracle(T, tokens=tokens)
    err = rel_l2(bf16_to_f64(out[tokens]), ref)
    say("  sampled rel-L2 %.3e" % err)
    assert err <= TOL[c.cfg.wdtype]
    again, _ = c.gpu(T, p, ws=ws)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))


@pytest.mark.parametrize("cfg,hot", [(TAIL_SMALL, (0, 1)), (TAIL_SMALL_TOP1, (3,))], ids=["top2_two_experts", "top1_one_expert"])
def test_degenerate_routing(cfg, hot):
    """Every token routed to the same expert(s), all others empty: one or two experts hold
    every pair in several row blocks.  A spread of plans (split-K, both split tails, grids
    capped so that tails are taken) against the oracle."""
    c = small_case(cfg)
    T = 300
    x, lg = c.inputs(T)
    lg = lg.float()
    top = lg.max(dim=1).values
    for i, e in enumerate(hot):
        lg[:, e] = top + 4.0 - 2.0 * i
    lg = lg.to(torch.bfloat16)
    ids, w = oracle_route(c.cfg, bits(lg), c.bias)
    assert set(np.unique(ids).tolist()) == set(hot)
    ref = oracle.forward(c.W, bits(x), ids, w)
    n = 0
    for g in (24, 0):
        plans = valid_plans(c.layer, T, split1=(1,), splits=(1, 2), tails=(0, 4), max_workgroups=g, tails1=(0, 4))
        for p in plans[::5]:
            say("degenerate routing", cfg.name, "plan", p.as_tuple())
            out = c.layer.forward(x.cuda(), lg.cuda(), plan=p)
            torch.cuda.synchronize()
            err = rel_l2(bf16_to_f64(out), ref)
            assert err <= TOL[c.cfg.wdtype], "plan %s rel-L2 %.3e" % (p.as_tuple(), err)
            n += 1
    assert n >= 10


def test_degenerate_routing_mixtral_sampled():
    """The full-size Mixtral shard at T=4096 with every token sent to experts 5 and 6: two
    experts of 4096 rows each, six empty, under the default plan.  Sampled tokens against the
    oracle, and the same output on a second call."""
    c = case("mixtral")
    T = 4096
    x, lg = c.inputs(T)
    lg = lg.float()
    top = lg.max(dim=1).values
    lg[:, 5] = top + 4.0
    lg[:, 6] = top + 2.0
    lg = lg.to(torch.bfloat16)
    ids, w = oracle_route(c.cfg, bits(lg), c.bias)
    assert set(np.unique(ids).tolist()) == {5, 6}
    say("degenerate routing mixtral T=%d plan %s" % (T, c.layer.plan(T).as_tuple()))
    ws = c.layer.workspace(T)
    out = c.layer.forward(x.cuda(), lg.cuda(), workspace=ws)
    torch.cuda.synchronize()
    tokens = [0, 1, 2047, 4094, 4095]
    ref = oracle.forward(c.W, bits(x), ids, w, tokens=tokens)
    err = rel_l2(bf16_to_f64(out[tokens]), ref)
    say("  sampled rel-L2 %.3e" % err)
    assert err <= TOL[c.cfg.wdtype]
    again = c.layer.forward(x.cuda(), lg.cuda(), workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))


@pytest.mark.parametrize("grid", [112, 0])
def test_split_tail_mixtral_sampled(grid):
    """The full-size Mixtral shard with its large-T tile: tokens whose expert rows lie in
    the split tail (and two others) against the oracle."""
    c = case("mixtral")
    T = 512
    p = abi.Plan(256, 25, 25, 1, 1, 4, grid)
    out, ws = c.gpu(T, p)
    row0, S = tail_taken(c, T, p, ws)
    if grid:   # with the whole device the grid is the capacity's tile bound: no tail here
        npp = int(workspace_view(c.layer, T, p, ws, "num_post_pad", torch.int32, 1).cpu()[0])
        cap = abi.moe_align_capacity(T, c.cfg.k, c.cfg.E, 256)
        assert (row0, S) == expected_tail(npp, cap, c.cfg.H, c.cfg.I, (256, 256, 64), grid, 4)
        assert S >= 2 and row0 > 0
    inv = workspace_view(c.layer, T, p, ws, "inv_pos", torch.int32, T * c.cfg.k).cpu().numpy().reshape(T, c.cfg.k)
    in_tail = [t for t in range(T) if S and (inv[t] >= row0).any()]
    tokens = sorted(set(in_tail[:2] + [0, T - 1]))
    ref, _, _ = c.oracle(T, tokens=tokens)
    err = rel_l2(bf16_to_f64(out[tokens]), ref)
    say("  tail rows from %d, S=%d, sampled rel-L2 %.3e" % (row0, S, err))
    assert err <= TOL[c.cfg.wdtype]
    again, _ = c.gpu(T, p, ws=ws)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
