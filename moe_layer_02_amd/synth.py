"""Seeded synthetic inputs for the fused-MoE layer: shapes, distributions, storage formats.

This module draws random numbers and stores them in the formats the layer reads; it holds
none of the layer's arithmetic (no routing, permutation, GEMM or reduction).  It serves
the GPU path, the CPU oracle, the tests and the benchmark alike.

The five layer shapes follow the models the pages serve (one GPU's share at its real
shape):
  tiny      E=8,  top-2 softmax (renormalised), H=128,  I=256,  bf16
  mixtral   Mixtral-8x7B, one TP2 shard (vLLM PR #2979 tunes Mixtral for H100 TP2):
            E=8, top-2 softmax (renormalised), H=4096, I=7168, bf16
  qwen2     Qwen2-57B-A14B routed experts, one TP4 shard (SGLang PR #2333 serves the
            FP8 checkpoint at TP4): E=64, top-8 softmax (not renormalised), H=3584,
            I=640, fp8 E4M3 w8a8 with per-expert per-tensor weight scales
  deepseek  DeepSeek-V3 routed experts (vLLM PR #12185 serves the AWQ checkpoint;
            SGLang PR #3191 adds its grouped gate): E=256, top-8 grouped sigmoid gate
            with correction bias (8 groups, keep 4, renormalise, scale 2.5), H=7168,
            I=2048, int4 with group size 128, fp16 scales and zero points
  scout     Llama-4-Scout (in the FBGEMM article's benchmark list): E=16, top-1
            sigmoid, H=5120, I=8192, bf16, router logits skewed so that expert
            popularity follows Zipf(1.2)

Distribution conventions: N(0, v) names the variance v; weights ~ N(0, 1/fan_in) with
fan_in the reduction length (H for w13, I for w2).  Every tensor is drawn in fp32 and
rounded to nearest even into its storage type.  Hidden states, logits and biases come from
numpy's PCG64 seeded by SeedSequence([seed, tensor id, block]); hidden states and logits
are drawn in blocks of 64 rows, so the first T rows do not depend on how many rows are
drawn (the T-prefix property).  Expert weights are drawn per expert, either on the host
(numpy PCG64, SeedSequence([seed, tensor id, expert])) or, for the multi-GB full-size
layers, on the GPU (torch's Philox generator seeded from the same SeedSequence); the two
streams differ, so a test or benchmark uses one of them for both the GPU and the oracle.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

ROUTE_SOFTMAX, ROUTE_SIGMOID, ROUTE_GROUPED_SIGMOID_BIAS = 0, 1, 2
WDT_BF16, WDT_FP8, WDT_INT4 = 0, 2, 3

_ROWS_PER_BLOCK = 64
_T_HIDDEN, _T_LOGITS, _T_BIAS, _T_W13, _T_W2, _T_PERM, _T_GUMBEL = range(7)


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    E: int
    k: int
    H: int
    I: int
    route_kind: int
    renormalize: bool
    wdtype: int
    seed: int
    t_sweep: tuple
    n_group: int = 1
    topk_group: int = 1
    routed_scaling: float = 1.0
    logit_var: float = 1.0
    bias_var: float = 0.0       # > 0: a correction bias ~ N(0, bias_var) is drawn
    zipf_s: float = 0.0         # > 0: router logits skewed to Zipf(zipf_s) popularity

    @property
    def t_max(self):
        return max(self.t_sweep)

    def with_shape(self, **kw):
        return dataclasses.replace(self, **kw)


def _pow2(lo, hi):
    return tuple(2 ** i for i in range(int(math.log2(lo)), int(math.log2(hi)) + 1))


CONFIGS = {
    "tiny": LayerConfig("tiny", E=8, k=2, H=128, I=256, route_kind=ROUTE_SOFTMAX, renormalize=True,
                        wdtype=WDT_BF16, seed=1001, t_sweep=(16,)),
    "mixtral": LayerConfig("mixtral", E=8, k=2, H=4096, I=7168, route_kind=ROUTE_SOFTMAX,
                           renormalize=True, wdtype=WDT_BF16, seed=1002, t_sweep=_pow2(1, 4096),
                           logit_var=1.5),
    "qwen2": LayerConfig("qwen2", E=64, k=8, H=3584, I=640, route_kind=ROUTE_SOFTMAX,
                         renormalize=False, wdtype=WDT_FP8, seed=1003, t_sweep=_pow2(1, 4096)),
    "deepseek": LayerConfig("deepseek", E=256, k=8, H=7168, I=2048,
                            route_kind=ROUTE_GROUPED_SIGMOID_BIAS, renormalize=True, wdtype=WDT_INT4,
                            seed=1004, t_sweep=_pow2(1, 512), n_group=8, topk_group=4,
                            routed_scaling=2.5, bias_var=0.01),
    "scout": LayerConfig("scout", E=16, k=1, H=5120, I=8192, route_kind=ROUTE_SIGMOID,
                         renormalize=False, wdtype=WDT_BF16, seed=1005, t_sweep=_pow2(1, 8192),
                         zipf_s=1.2),
}


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _normal_rows(cfg, tensor_id, T, cols, std):
    """[T, cols] fp32 ~ N(0, std^2), drawn in 64-row blocks (T-prefix property)."""
    out = np.empty((T, cols), np.float32)
    for b in range((T + _ROWS_PER_BLOCK - 1) // _ROWS_PER_BLOCK):
        r0, r1 = b * _ROWS_PER_BLOCK, min(T, (b + 1) * _ROWS_PER_BLOCK)
        blk = _rng(cfg.seed, tensor_id, b).standard_normal((_ROWS_PER_BLOCK, cols), dtype=np.float32)
        out[r0:r1] = blk[: r1 - r0] * np.float32(std)
    return out


def _bf16(a32: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a32)).to(torch.bfloat16)


def hidden_states(cfg: LayerConfig, T: int) -> torch.Tensor:
    """bf16 [T, H] ~ N(0, 1)."""
    return _bf16(_normal_rows(cfg, _T_HIDDEN, T, cfg.H, 1.0))


def zipf_popularity(cfg: LayerConfig) -> np.ndarray:
    """Per-expert probability p_e: ranks r = 1..E with p_r proportional to r^-s, assigned to
    experts by a seeded permutation.  (Gumbel-max sampling with logits ln p_e + Gumbel noise
    picks expert e with probability p_e.)"""
    ranks = np.arange(1, cfg.E + 1, dtype=np.float64)
    p = ranks ** (-cfg.zipf_s)
    p /= p.sum()
    perm = _rng(cfg.seed, _T_PERM, 0).permutation(cfg.E)
    return p[perm]


def router_logits(cfg: LayerConfig, T: int) -> torch.Tensor:
    """bf16 [T, E]: N(0, logit_var), or for a Zipf-skewed layer ln p_e + Gumbel(0, 1)."""
    if cfg.zipf_s > 0:
        lp = np.log(zipf_popularity(cfg)).astype(np.float32)
        out = np.empty((T, cfg.E), np.float32)
        for b in range((T + _ROWS_PER_BLOCK - 1) // _ROWS_PER_BLOCK):
            r0, r1 = b * _ROWS_PER_BLOCK, min(T, (b + 1) * _ROWS_PER_BLOCK)
            g = _rng(cfg.seed, _T_GUMBEL, b).gumbel(size=(_ROWS_PER_BLOCK, cfg.E)).astype(np.float32)
            out[r0:r1] = (lp[None, :] + g)[: r1 - r0]
        return _bf16(out)
    return _bf16(_normal_rows(cfg, _T_LOGITS, T, cfg.E, math.sqrt(cfg.logit_var)))


def correction_bias(cfg: LayerConfig):
    """fp32 [E] ~ N(0, bias_var), or None."""
    if cfg.bias_var <= 0:
        return None
    b = _rng(cfg.seed, _T_BIAS, 0).standard_normal(cfg.E, dtype=np.float32) * np.float32(math.sqrt(cfg.bias_var))
    return torch.from_numpy(b)


def _expert_matrix(cfg, tensor_id, e, rows, cols, device="cpu"):
    """fp32 [rows, cols] ~ N(0, 1/cols) for expert e (numpy array on the host, or a torch
    tensor drawn on the given CUDA device)."""
    if device == "cpu":
        return _rng(cfg.seed, tensor_id, e).standard_normal((rows, cols), dtype=np.float32) * np.float32(
            1.0 / math.sqrt(cols))
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([cfg.seed, tensor_id, e]).generate_state(1, np.uint64)[0] >> 1))
    return torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32) * (1.0 / math.sqrt(cols))


def _fp8_encode(w32):
    """Per-tensor E4M3 storage of one expert matrix: scale = amax / 448, codes = the
    nearest E4M3 value of w / scale (torch's float8_e4m3fn cast)."""
    w = torch.from_numpy(w32) if isinstance(w32, np.ndarray) else w32
    amax = float(w.abs().max())
    scale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    q = torch.clamp(w / scale, -448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale


def _int4_encode(w32):
    """Asymmetric int4 with group size 128 along the row: per (row, group) an fp16 scale
    s = (max - min) / 15 and an integer-valued fp16 zero point z = clamp(rint(-min / s),
    0, 15); nibble q = clamp(rint(w / s + z), 0, 15) (rint: round half to even).  Column c
    goes to byte c/2, the low nibble when c is even.  Returns torch tensors (packed uint8
    [rows, cols/2], s fp16, z fp16) on the input's device."""
    w = torch.from_numpy(w32) if isinstance(w32, np.ndarray) else w32
    rows, cols = w.shape
    g = w.reshape(rows, cols // 128, 128)
    lo, hi = g.amin(dim=2), g.amax(dim=2)
    s = ((hi - lo) / 15.0).to(torch.float16)
    s = torch.where(s == 0, torch.ones_like(s), s)
    s32 = s.float()
    z = torch.clamp(torch.round(-lo / s32), 0, 15).to(torch.float16)
    q = torch.clamp(torch.round(g / s32[..., None] + z.float()[..., None]), 0, 15).to(torch.uint8)
    q = q.reshape(rows, cols)
    packed = q[:, 0::2] | (q[:, 1::2] << 4)
    return packed, s, z


@dataclasses.dataclass
class ExpertWeights:
    """Stacked expert weights on the host, in the layer's storage format.
    bf16: w13 bf16 [E,2I,H], w2 bf16 [E,H,I].
    fp8:  w13/w2 uint8 E4M3 codes (same shapes), w13_scale/w2_scale fp32 [E].
    int4: w13 uint8 [E,2I,H/2], w2 uint8 [E,H,I/2], *_s/*_z fp16 [E,K/128,N] (group-major)."""
    wdtype: int
    w13: torch.Tensor
    w2: torch.Tensor
    w13_scale: torch.Tensor = None
    w2_scale: torch.Tensor = None
    w13_s: torch.Tensor = None
    w13_z: torch.Tensor = None
    w2_s: torch.Tensor = None
    w2_z: torch.Tensor = None

    def tensors(self):
        return {f.name: getattr(self, f.name) for f in dataclasses.fields(self)
                if isinstance(getattr(self, f.name), torch.Tensor)}


def expert_weights(cfg: LayerConfig, device: str = "cpu") -> ExpertWeights:
    """All E experts' weights, drawn expert by expert (one expert in fp32 at a time), stored
    on `device` ("cpu": numpy stream; a CUDA device: torch's Philox stream, drawn there)."""
    E, H, I = cfg.E, cfg.H, cfg.I
    mat = lambda tid, e, r, c: _expert_matrix(cfg, tid, e, r, c, device)  # noqa: E731
    to_bf16 = (lambda a: _bf16(a)) if device == "cpu" else (lambda a: a.to(torch.bfloat16))
    if cfg.wdtype == WDT_BF16:
        w13 = torch.empty((E, 2 * I, H), dtype=torch.bfloat16, device=device)
        w2 = torch.empty((E, H, I), dtype=torch.bfloat16, device=device)
        for e in range(E):
            w13[e] = to_bf16(mat(_T_W13, e, 2 * I, H))
            w2[e] = to_bf16(mat(_T_W2, e, H, I))
        return ExpertWeights(WDT_BF16, w13, w2)
    if cfg.wdtype == WDT_FP8:
        w13 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device=device)
        w2 = torch.empty((E, H, I), dtype=torch.uint8, device=device)
        s13 = torch.empty(E, dtype=torch.float32)
        s2 = torch.empty(E, dtype=torch.float32)
        for e in range(E):
            w13[e], s13[e] = _fp8_encode(mat(_T_W13, e, 2 * I, H))
            w2[e], s2[e] = _fp8_encode(mat(_T_W2, e, H, I))
        return ExpertWeights(WDT_FP8, w13, w2, w13_scale=s13.to(device), w2_scale=s2.to(device))
    if cfg.wdtype == WDT_INT4:
        w13 = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=device)
        w2 = torch.empty((E, H, I // 2), dtype=torch.uint8, device=device)
        # scales and zero points group-major: [E, K/128, N]
        s13 = torch.empty((E, H // 128, 2 * I), dtype=torch.float16, device=device)
        z13 = torch.empty_like(s13)
        s2 = torch.empty((E, I // 128, H), dtype=torch.float16, device=device)
        z2 = torch.empty_like(s2)
        for e in range(E):
            w13[e], s, z = _int4_encode(mat(_T_W13, e, 2 * I, H))
            s13[e], z13[e] = s.t(), z.t()
            w2[e], s, z = _int4_encode(mat(_T_W2, e, H, I))
            s2[e], z2[e] = s.t(), z.t()
        return ExpertWeights(WDT_INT4, w13, w2, w13_s=s13, w13_z=z13, w2_s=s2, w2_z=z2)
    raise ValueError("unknown weight dtype")


_T_GG_X, _T_GG_SIZES = 20, 21


def grouped_gemm_inputs(cfg: LayerConfig, T: int):
    """Inputs of the EP-MoE grouped GEMM on a layer's w13 (W [E, 2I, H]: N = 2I, K = H):
    M = T*k rows grouped by expert in contiguous segments, the sizes counted from T*k
    expert draws (the config's Zipf popularity, else uniform); X [M, H] ~ N(0, 1) -- bf16,
    or for fp8 weights E4M3 codes of X / s with the per-tensor scale s = amax / 448.
    Returns (x on the host, x_scale fp32 [1] or None, m_sizes int32 [E])."""
    M = T * cfg.k
    rng = _rng(cfg.seed, _T_GG_SIZES, T)
    p = zipf_popularity(cfg) if cfg.zipf_s > 0 else np.full(cfg.E, 1.0 / cfg.E)
    sizes = np.bincount(rng.choice(cfg.E, size=M, p=p), minlength=cfg.E).astype(np.int32)
    x32 = _rng(cfg.seed, _T_GG_X, T).standard_normal((M, cfg.H), dtype=np.float32)
    if cfg.wdtype == WDT_FP8:
        codes, scale = _fp8_encode(x32)
        return codes, torch.tensor([scale], dtype=torch.float32), torch.from_numpy(sizes)
    return _bf16(x32), None, torch.from_numpy(sizes)
