"""moe_grouped_gemm (the EP-MoE grouped GEMM over contiguous per-expert segments) on the GPU
vs the oracle: every pipelined tile on a reduced shape with ragged segments (empty ones,
one segment holding every row, rows past the segments left untouched), the Qwen2-57B TP4
w13 shape at the default tiles on sampled rows, bf16 and fp8 per-tensor, and bitwise
determinism.  Relative L2 over the compared rows <= 1e-2: the op takes its operands as they
are (no quantisation inside), so only the fp32 accumulation order and the bf16 output
rounding differ from the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_layer_02_amd import abi, synth
from tests.gpu_util import bf16_to_f64, bits, needs_gpu, rel_l2, say

pytestmark = [pytest.mark.gpu, needs_gpu]

TOL = 1e-2
SENTINEL = 0x7FC1    # a bf16 NaN pattern: rows the op must not write keep it

# reduced Qwen2 shape (W = w13 [8, 256, 512]: N = 256, K = 512): every tile width divides it
SMALL_FP8 = synth.CONFIGS["qwen2"].with_shape(name="ggsmall_fp8", E=8, k=4, H=512, I=128)
SMALL_BF16 = SMALL_FP8.with_shape(name="ggsmall_bf16", wdtype=synth.WDT_BF16)
QWEN2_BF16 = synth.CONFIGS["qwen2"].with_shape(name="qwen2_bf16", wdtype=synth.WDT_BF16)

_weights = {}


def weights(cfg, device):
    key = (cfg.name, device)
    if key not in _weights:
        say("generating weights", cfg.name, "on", device)
        w = synth.expert_weights(cfg, device=device)
        _weights[key] = (w.w13.cuda(), None if w.w13_scale is None else w.w13_scale.cuda(), w.w13.cpu(),
                         None if w.w13_scale is None else w.w13_scale.cpu())
    return _weights[key]


def oracle_dtype(cfg):
    return oracle.FP8_E4M3 if cfg.wdtype == synth.WDT_FP8 else oracle.BF16


def host_bits(t):
    return t.numpy() if t.dtype == torch.uint8 else bits(t)


def run(cfg, w, ws_scale, x, x_scale, sizes, tile, M=None, y=None):
    """One call; y is pre-filled with SENTINEL so that rows the op skips are visible."""
    desc = abi.grouped_gemm_desc(w, abi.DT_FP8_E4M3 if cfg.wdtype == synth.WDT_FP8 else abi.DT_BF16, ws_scale)
    M = x.shape[0] if M is None else M
    if y is None:
        y = torch.full((M, desc.N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ws = torch.empty(abi.moe_grouped_gemm_workspace_bytes(desc, M, tile), dtype=torch.uint8, device="cuda")
    abi.moe_grouped_gemm(desc, x, sizes, y, ws, x_scale=x_scale, tile=tile)
    torch.cuda.synchronize()
    return y


def tiles_for(cfg, w, ws_scale, M):
    desc = abi.grouped_gemm_desc(w, abi.DT_FP8_E4M3 if cfg.wdtype == synth.WDT_FP8 else abi.DT_BF16, ws_scale)
    out = []
    for t in range(48):
        try:
            abi.moe_grouped_gemm_workspace_bytes(desc, M, t)
        except abi.MoEError:
            continue
        out.append(t)
    return out


@pytest.mark.parametrize("cfg", [SMALL_BF16, SMALL_FP8], ids=lambda c: c.name)
@pytest.mark.parametrize("sizes", [[5, 0, 17, 1, 0, 40, 3, 9],        # ragged, empty segments
                                   [0, 0, 0, 0, 0, 0, 300, 0],         # one segment holds every row
                                   [1, 1, 1, 1, 1, 1, 1, 1]])          # one row per expert
def test_every_tile_ragged_segments(cfg, sizes):
    w, ws_scale, w_host, s_host = weights(cfg, "cpu")
    x_all, x_scale, _ = synth.grouped_gemm_inputs(cfg, 300)
    total = sum(sizes)
    M = total + 7                                    # rows past the last segment: untouched
    x = x_all[:M]
    ref = oracle.grouped_gemm(oracle_dtype(cfg), cfg.E, 2 * cfg.I, cfg.H, host_bits(x), host_bits(w_host),
                              np.array(sizes, np.int32), x_scale=1.0 if x_scale is None else float(x_scale[0]),
                              w_scale=None if s_host is None else s_host.numpy())
    tiles = tiles_for(cfg, w, ws_scale, M)
    assert len(tiles) >= 6, tiles
    m_sizes = torch.tensor(sizes, dtype=torch.int32, device="cuda")
    xs = None if x_scale is None else x_scale.cuda()
    for t in tiles:
        say("grouped gemm", cfg.name, "sizes", sizes, "tile", t)
        y = run(cfg, w, ws_scale, x.cuda(), xs, m_sizes, t)
        err = rel_l2(bf16_to_f64(y[:total]), ref[:total])
        assert err <= TOL, "tile %d rel-L2 %.3e" % (t, err)
        assert (y[total:].view(torch.int16) == SENTINEL).all(), "tile %d wrote past the segments" % t


@pytest.mark.parametrize("cfg", [QWEN2_BF16, synth.CONFIGS["qwen2"]], ids=lambda c: c.name)
@pytest.mark.parametrize("T", [1, 64, 4096])
def test_qwen2_w13_default_tile_sampled(cfg, T):
    """The Qwen2-57B-A14B TP4 w13 shape (E = 64, N = 1280, K = 3584; M = 8T rows) at the
    default tile: rows at both ends of several segments against the oracle."""
    w, ws_scale, w_host, s_host = weights(cfg, "cuda")
    x, x_scale, sizes = synth.grouped_gemm_inputs(cfg, T)
    M = x.shape[0]
    y = run(cfg, w, ws_scale, x.cuda(), None if x_scale is None else x_scale.cuda(), sizes.cuda(), -1)
    starts = np.concatenate([[0], np.cumsum(sizes.numpy())])
    busy = [e for e in range(cfg.E) if sizes[e] > 0]
    busy = busy[::max(1, len(busy) // 12)]
    rows = sorted({int(r) for e in busy for r in (starts[e], starts[e + 1] - 1)})[:24]
    # the sampled rows as their own segments (they are in segment order)
    sub_sizes = np.array([sum(1 for r in rows if starts[e] <= r < starts[e + 1]) for e in range(cfg.E)], np.int32)
    ref = oracle.grouped_gemm(oracle_dtype(cfg), cfg.E, 2 * cfg.I, cfg.H, host_bits(x[rows]), host_bits(w_host),
                              sub_sizes, x_scale=1.0 if x_scale is None else float(x_scale[0]),
                              w_scale=None if s_host is None else s_host.numpy())
    err = rel_l2(bf16_to_f64(y[rows]), ref)
    say("  %d sampled rows, rel-L2 %.3e" % (len(rows), err))
    assert err <= TOL
    assert torch.isfinite(y.float()).all()


def test_deterministic_and_graph_capturable():
    cfg = SMALL_BF16
    w, ws_scale, _, _ = weights(cfg, "cpu")
    x, _, sizes = synth.grouped_gemm_inputs(cfg, 300)
    x, sizes = x.cuda(), sizes.cuda()
    a = run(cfg, w, ws_scale, x, None, sizes, -1)
    b = run(cfg, w, ws_scale, x, None, sizes, -1)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    desc = abi.grouped_gemm_desc(w, abi.DT_BF16)
    ws = torch.empty(abi.moe_grouped_gemm_workspace_bytes(desc, x.shape[0]), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(a)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            abi.moe_grouped_gemm(desc, x, sizes, y, ws)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), a.view(torch.int16))
