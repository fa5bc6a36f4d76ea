"""ctypes binding of libmoe.so (the C ABI in include/moe.h).

Argument marshalling only: torch tensors become device pointers, the current torch stream
becomes the HIP stream; every step of the layer runs in the library's HIP kernels.  There
is no fallback: if libmoe.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = range(5)
ROUTE_SOFTMAX, ROUTE_SIGMOID, ROUTE_GROUPED_SIGMOID_BIAS = 0, 1, 2
DT_BF16, DT_FP32, DT_FP8_E4M3, DT_INT4_G128 = 0, 1, 2, 3
STAGES = ("route", "align", "act_quant", "gemm1", "h_quant", "gemm2", "reduce", "prologue", "gemm1_finish")
STAGE_COUNT = len(STAGES)
WS_REGIONS = ("topk_ids", "topk_weights", "sorted_ids", "expert_ids", "num_post_pad", "expert_counts",
              "inv_pos", "scalars", "x_q", "h", "h_q", "y", "align_scratch", "gemm1_partials", "gemm2_tail",
              "gemm1_tail", "block_start")

# every function include/moe.h declares (checked against the header by the tests)
EXPORTS = ("moe_status_str", "moe_align_capacity", "moe_route", "moe_align", "moe_default_plan",
           "moe_workspace_bytes", "moe_forward", "moe_forward_profiled", "moe_plan_describe",
           "moe_workspace_offsets", "moe_grouped_gemm_default_tile", "moe_grouped_gemm_workspace_bytes",
           "moe_grouped_gemm", "moe_forward_static")
STATIC_WORKSPACE_BYTES = 128 << 20   # MOE_STATIC_WORKSPACE_BYTES


class MoEError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s: %s (status %d)" % (what, status_str(status), status))
        self.status = status


class RouteCfg(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float), ("logits_dtype", ctypes.c_int32)]


class Layer(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("route", RouteCfg),
                ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("w13_s", ctypes.c_void_p), ("w13_z", ctypes.c_void_p),
                ("w2_s", ctypes.c_void_p), ("w2_z", ctypes.c_void_p),
                ("correction_bias", ctypes.c_void_p)]


class GroupedGemmDesc(ctypes.Structure):
    _fields_ = [("num_groups", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("w", ctypes.c_void_p), ("w_scale", ctypes.c_void_p)]


class Plan(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("gemm1_tile", ctypes.c_int32), ("gemm2_tile", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("split_k1", ctypes.c_int32), ("split_tail", ctypes.c_int32),
                ("max_workgroups", ctypes.c_int32), ("split_tail1", ctypes.c_int32), ("ragged", ctypes.c_int32)]

    def as_tuple(self):
        """(block_m, gemm1_tile, gemm2_tile, split_k[, split_k1[, split_tail[, max_workgroups[,
        split_tail1[, ragged]]]]]), trailing defaults left out."""
        t = (self.block_m, self.gemm1_tile, self.gemm2_tile, self.split_k, self.split_k1, self.split_tail,
             self.max_workgroups, self.split_tail1, self.ragged)
        n = 4
        for i in range(4, 9):
            if t[i] > (0 if i in (6, 8) else 1):
                n = i + 1
        return t[:n]


_lib = None


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.moe_status_str.argtypes, L.moe_status_str.restype = [ctypes.c_int], ctypes.c_char_p
        L.moe_align_capacity.argtypes, L.moe_align_capacity.restype = [I32, I32, I32, I32], I64
        L.moe_route.argtypes = [ctypes.POINTER(RouteCfg), I32, P, P, P, P, P]
        L.moe_align.argtypes = [I32, I32, I32, I32, P, P, P, P, P, P, P]
        L.moe_default_plan.argtypes = [ctypes.POINTER(Layer), I32, ctypes.POINTER(Plan)]
        L.moe_workspace_bytes.argtypes = [ctypes.POINTER(Layer), I32, ctypes.POINTER(Plan), ctypes.POINTER(SZ)]
        L.moe_forward.argtypes = [ctypes.POINTER(Layer), I32, P, P, P, P, SZ, ctypes.POINTER(Plan), P]
        L.moe_forward_static.argtypes = [ctypes.POINTER(Layer), I32, P, P, P, ctypes.POINTER(Plan), P]
        L.moe_forward_profiled.argtypes = [ctypes.POINTER(Layer), I32, P, P, P, P, SZ, ctypes.POINTER(Plan), P,
                                           ctypes.POINTER(P), I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]
        L.moe_plan_describe.argtypes = [ctypes.POINTER(Layer), I32, ctypes.POINTER(Plan), ctypes.c_char_p, SZ]
        L.moe_workspace_offsets.argtypes = [ctypes.POINTER(Layer), I32, ctypes.POINTER(Plan), ctypes.POINTER(I64)]
        G = ctypes.POINTER(GroupedGemmDesc)
        L.moe_grouped_gemm_default_tile.argtypes = [G, I32, ctypes.POINTER(I32)]
        L.moe_grouped_gemm_workspace_bytes.argtypes = [G, I32, I32, ctypes.POINTER(SZ)]
        L.moe_grouped_gemm.argtypes = [G, I32, P, P, P, P, P, SZ, I32, P]
        for f in ("moe_route", "moe_align", "moe_default_plan", "moe_workspace_bytes", "moe_forward",
                  "moe_forward_profiled", "moe_plan_describe", "moe_workspace_offsets",
                  "moe_grouped_gemm_default_tile", "moe_grouped_gemm_workspace_bytes", "moe_grouped_gemm",
                  "moe_forward_static"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def _check(status, what):
    if status != MOE_OK:
        raise MoEError(status, what)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return ctypes.c_void_p(t.data_ptr())
    return ctypes.c_void_p(int(t))


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def route_cfg(E, k, kind, renormalize=True, n_group=1, topk_group=1, routed_scaling=1.0, logits_dtype=DT_BF16):
    return RouteCfg(E, k, kind, int(bool(renormalize)), n_group, topk_group, routed_scaling, logits_dtype)


# ---- the C functions, one wrapper each ---------------------------------------------------

def moe_align_capacity(T, k, E, block_m) -> int:
    return int(lib().moe_align_capacity(T, k, E, block_m))


def moe_route(cfg: RouteCfg, T, logits, bias, topk_ids, topk_weights, stream=None):
    _check(lib().moe_route(ctypes.byref(cfg), T, _ptr(logits), _ptr(bias), _ptr(topk_ids), _ptr(topk_weights),
                           _stream(stream)), "moe_route")


def moe_align(T, k, E, block_m, topk_ids, sorted_token_ids, expert_ids, num_tokens_post_padded, expert_counts,
              inv_pos, stream=None):
    _check(lib().moe_align(T, k, E, block_m, _ptr(topk_ids), _ptr(sorted_token_ids), _ptr(expert_ids),
                           _ptr(num_tokens_post_padded), _ptr(expert_counts), _ptr(inv_pos), _stream(stream)),
           "moe_align")


def moe_default_plan(layer: Layer, T) -> Plan:
    p = Plan()
    _check(lib().moe_default_plan(ctypes.byref(layer), T, ctypes.byref(p)), "moe_default_plan")
    return p


def moe_workspace_bytes(layer: Layer, T, plan: Plan = None) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_bytes(ctypes.byref(layer), T, ctypes.byref(plan) if plan else None,
                                     ctypes.byref(n)), "moe_workspace_bytes")
    return n.value


def moe_forward(layer: Layer, T, hidden, logits, out, workspace, plan: Plan = None, stream=None):
    _check(lib().moe_forward(ctypes.byref(layer), T, _ptr(hidden), _ptr(logits), _ptr(out), _ptr(workspace),
                             workspace.numel() * workspace.element_size(),
                             ctypes.byref(plan) if plan else None, _stream(stream)), "moe_forward")


def moe_forward_static(layer: Layer, T, hidden, logits, out, plan: Plan = None, stream=None):
    """moe_forward on the library's own static device workspace (no allocation anywhere)."""
    _check(lib().moe_forward_static(ctypes.byref(layer), T, _ptr(hidden), _ptr(logits), _ptr(out),
                                    ctypes.byref(plan) if plan else None, _stream(stream)), "moe_forward_static")


def moe_forward_profiled(layer: Layer, T, hidden, logits, out, workspace, events, plan: Plan = None, stream=None):
    """events: STAGE_COUNT + 1 torch.cuda.Event(enable_timing=True).  Returns the stage names
    launched; events[0..n] bracket them."""
    for ev in events:   # make sure each event exists on the device before taking its handle
        if ev.cuda_event == 0:
            ev.record()
    handles = (ctypes.c_void_p * len(events))(*[ev.cuda_event for ev in events])
    stages = (ctypes.c_int32 * STAGE_COUNT)()
    n = ctypes.c_int32()
    _check(lib().moe_forward_profiled(ctypes.byref(layer), T, _ptr(hidden), _ptr(logits), _ptr(out),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      ctypes.byref(plan) if plan else None, _stream(stream), handles, len(events),
                                      stages, ctypes.byref(n)), "moe_forward_profiled")
    return [STAGES[stages[i]] for i in range(n.value)]


def moe_plan_describe(layer: Layer, T, plan: Plan) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().moe_plan_describe(ctypes.byref(layer), T, ctypes.byref(plan), buf, 256), "moe_plan_describe")
    return buf.value.decode()


def moe_workspace_offsets(layer: Layer, T, plan: Plan = None) -> dict:
    off = (ctypes.c_int64 * len(WS_REGIONS))()
    _check(lib().moe_workspace_offsets(ctypes.byref(layer), T, ctypes.byref(plan) if plan else None, off),
           "moe_workspace_offsets")
    return {name: int(off[i]) for i, name in enumerate(WS_REGIONS)}


def grouped_gemm_desc(w, dtype, w_scale=None) -> GroupedGemmDesc:
    """Descriptor of a grouped GEMM over the device weights w [E, N, K] (bf16, or E4M3 codes
    as uint8 with per-expert fp32 scales w_scale [E])."""
    E, N, K = w.shape
    return GroupedGemmDesc(E, N, K, dtype, _ptr(w), _ptr(w_scale))


def moe_grouped_gemm_default_tile(desc: GroupedGemmDesc, M) -> int:
    t = ctypes.c_int32()
    _check(lib().moe_grouped_gemm_default_tile(ctypes.byref(desc), M, ctypes.byref(t)), "moe_grouped_gemm_default_tile")
    return t.value


def moe_grouped_gemm_workspace_bytes(desc: GroupedGemmDesc, M, tile=-1) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_grouped_gemm_workspace_bytes(ctypes.byref(desc), M, tile, ctypes.byref(n)),
           "moe_grouped_gemm_workspace_bytes")
    return n.value


def moe_grouped_gemm(desc: GroupedGemmDesc, x, m_sizes, y, workspace, x_scale=None, tile=-1, stream=None):
    """Y[r] = X[r] W[e]^T over the contiguous segments of m_sizes (device int32 [E])."""
    M = x.shape[0]
    _check(lib().moe_grouped_gemm(ctypes.byref(desc), M, _ptr(x), _ptr(x_scale), _ptr(m_sizes), _ptr(y),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), tile,
                                  _stream(stream)), "moe_grouped_gemm")


# ---- a layer object over device tensors ----------------------------------------------------

@dataclasses.dataclass
class MoELayer:
    """A layer's device tensors and its C descriptor (the tensors are kept alive here)."""
    struct: Layer
    tensors: dict

    @staticmethod
    def create(E, H, I, k, route_kind, weight_dtype, w13, w2, renormalize=True, n_group=1, topk_group=1,
               routed_scaling=1.0, logits_dtype=DT_BF16, w13_scale=None, w2_scale=None, w13_s=None,
               w13_z=None, w2_s=None, w2_z=None, correction_bias=None):
        t = dict(w13=w13, w2=w2, w13_scale=w13_scale, w2_scale=w2_scale, w13_s=w13_s, w13_z=w13_z,
                 w2_s=w2_s, w2_z=w2_z, correction_bias=correction_bias)
        for name, v in t.items():
            if v is not None and (not v.is_cuda or not v.is_contiguous()):
                raise ValueError("%s must be a contiguous CUDA tensor" % name)
        cfg = route_cfg(E, k, route_kind, renormalize, n_group, topk_group, routed_scaling, logits_dtype)
        ptr = lambda v: None if v is None else v.data_ptr()  # noqa: E731
        s = Layer(E, H, I, weight_dtype, cfg, *[ptr(t[n]) for n in
                  ("w13", "w2", "w13_scale", "w2_scale", "w13_s", "w13_z", "w2_s", "w2_z", "correction_bias")])
        return MoELayer(s, t)

    @property
    def H(self):
        return self.struct.H

    def plan(self, T) -> Plan:
        return moe_default_plan(self.struct, T)

    def workspace(self, T, plan: Plan = None, device="cuda"):
        n = moe_workspace_bytes(self.struct, T, plan)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)

    def forward(self, hidden, logits, out=None, workspace=None, plan: Plan = None, stream=None):
        T = hidden.shape[0]
        if out is None:
            out = torch.empty((T, self.struct.H), dtype=torch.bfloat16, device=hidden.device)
        if workspace is None:
            workspace = self.workspace(T, plan, hidden.device)
        moe_forward(self.struct, T, hidden, logits, out, workspace, plan, stream)
        return out
