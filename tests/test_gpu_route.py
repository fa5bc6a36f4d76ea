"""moe_route on the GPU vs the oracle: expert ids bit-exact in slot order, weights within
1e-5 relative, on every config's logits, forced ties, fp32 logits, and the sigmoid over
every finite bf16 input."""
import numpy as np
import pytest
import torch

import oracle
from moe_layer_02_amd import abi, synth
from tests.gpu_util import bits, needs_gpu, oracle_route, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def gpu_route(cfg, logits, bias, logits_dtype=abi.DT_BF16):
    T = logits.shape[0]
    c = abi.route_cfg(cfg.E, cfg.k, cfg.route_kind, cfg.renormalize, cfg.n_group, cfg.topk_group,
                      cfg.routed_scaling, logits_dtype)
    ids = torch.full((T, cfg.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, cfg.k), -7.0, dtype=torch.float32, device="cuda")
    b = None if bias is None else bias.cuda()
    abi.moe_route(c, T, logits.cuda(), b, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def check(cfg, logits, bias, logits_dtype=abi.DT_BF16):
    say("route", cfg.name, "E=%d k=%d kind=%d T=%d" % (cfg.E, cfg.k, cfg.route_kind, logits.shape[0]))
    ids, w = gpu_route(cfg, logits, bias, logits_dtype)
    lg = bits(logits) if logits_dtype == abi.DT_BF16 else logits.numpy()
    rids, rw = oracle_route(cfg, lg, bias)
    mism = np.nonzero((ids != rids).any(1))[0]
    assert mism.size == 0, "token %d: gpu %s oracle %s" % (mism[0], ids[mism[0]], rids[mism[0]])
    np.testing.assert_allclose(w, rw, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("name", sorted(synth.CONFIGS))
def test_route_on_config_logits(name):
    cfg = synth.CONFIGS[name]
    bias = synth.correction_bias(cfg)
    for T in sorted({1, 3, 64, 333, cfg.t_max}):
        check(cfg, synth.router_logits(cfg, T), bias)


@pytest.mark.parametrize("E,k,kind,ng,tg", [(8, 2, 0, 1, 1), (64, 8, 0, 1, 1), (256, 8, 0, 1, 1),
                                            (16, 1, 1, 1, 1), (64, 6, 1, 1, 1), (256, 8, 2, 8, 4),
                                            (128, 6, 2, 16, 3), (32, 4, 2, 32, 32), (256, 64, 2, 4, 4),
                                            (48, 4, 2, 4, 3), (96, 5, 2, 4, 2), (200, 8, 2, 8, 4)])
def test_route_forced_ties(E, k, kind, ng, tg):
    cfg = synth.CONFIGS["tiny"].with_shape(name="ties", E=E, k=k, route_kind=kind, n_group=ng, topk_group=tg,
                                            renormalize=True, routed_scaling=1.5)
    g = torch.Generator().manual_seed(E * 1000 + k)
    logits = torch.randint(-1, 2, (500, E), generator=g).to(torch.bfloat16)
    bias = None
    if kind != 0:
        bias = (torch.randint(0, 3, (E,), generator=g).float() * 0.125).contiguous()   # equal biases: ties
    check(cfg, logits, bias)


@pytest.mark.parametrize("kind,E,k", [(0, 8, 2), (0, 64, 8), (1, 64, 6)])
def test_route_signed_zero_ties(kind, E, k):
    """-0.0 and +0.0 logits are equal keys (the index decides between them), on both sides."""
    cfg = synth.CONFIGS["tiny"].with_shape(name="zeros", E=E, k=k, route_kind=kind, renormalize=True)
    g = torch.Generator().manual_seed(E + k + 7 * kind)
    logits = torch.randint(0, 3, (300, E), generator=g).float()
    logits = torch.where(logits == 0, torch.tensor(-0.0), torch.where(logits == 1, torch.tensor(0.0), -logits))
    check(cfg, logits.to(torch.bfloat16), None)


def test_route_fp32_logits():
    cfg = synth.CONFIGS["deepseek"]
    logits = torch.randn(300, cfg.E, generator=torch.Generator().manual_seed(5))
    check(cfg, logits, synth.correction_bias(cfg), abi.DT_FP32)
    cfg = synth.CONFIGS["qwen2"]
    check(cfg, torch.randn(300, cfg.E, generator=torch.Generator().manual_seed(6)), None, abi.DT_FP32)


def test_sigmoid_exhaustive_over_bf16():
    """E=1, top-1 sigmoid, no renormalisation: the weight is the sigmoid itself, so every
    finite bf16 input checks the kernel's sigmoid bit for bit against the oracle's."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16)
    x = x[torch.isfinite(x.float())].reshape(-1, 1).contiguous()
    cfg = synth.CONFIGS["scout"].with_shape(name="sigmoid", E=1, k=1, renormalize=False)
    say("route sigmoid exhaustive T=%d" % x.shape[0])
    ids, w = gpu_route(cfg, x, None)
    ref = oracle.sigmoid(x.float().numpy().ravel())
    assert (ids == 0).all()
    assert (w.ravel().view(np.uint32) == ref.view(np.uint32)).all()


def test_route_zero_tokens():
    cfg = synth.CONFIGS["tiny"]
    c = abi.route_cfg(cfg.E, cfg.k, cfg.route_kind)
    abi.moe_route(c, 0, None, None, None, None)
