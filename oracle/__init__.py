"""CPU oracle of the fused-MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product library never loads it.

This module is a thin ctypes wrapper over ``moe_oracle.c`` (plain C, fp64 accumulation,
tokens optionally spread over threads with results identical to one thread); every formula
lives there, with its citation.  Arrays are numpy; bf16 tensors travel as
their uint16 bit patterns, fp8 and packed int4 weights as uint8, fp16 scales and zero
points as uint16 bit patterns.

Parity status of each function (what pins it; see tests/test_oracle_pins.py):
  codecs          exhaustive / midpoint comparison with torch's casts
  route           brute-force full sort on tiny inputs, forced ties, closed forms
  align           brute-force stable argsort, invariants, permute/unpermute identity
  forward (bf16)  E=1,k=1 dense FFN via torch matmul; per-slot sums of dense FFNs
  forward (int4)  dense FFN on weights dequantised by the test from (q, z, s) triples
  forward (fp8)   codec pins, scale invariants, exact case with identity down projection
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ROUTE_SOFTMAX, ROUTE_SIGMOID, ROUTE_GROUPED_SIGMOID_BIAS = 0, 1, 2
BF16, FP32, FP8_E4M3, INT4_G128 = 0, 1, 2, 3


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so (in-tree).  MOE_ORACLE_LIB
    names a prebuilt copy instead (the mutation test loads deliberately broken copies)."""
    if os.environ.get("MOE_ORACLE_LIB"):
        return os.environ["MOE_ORACLE_LIB"]
    stale = not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "moe_oracle.h")))
    if force or stale:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-pthread", "-fPIC", "-shared",
                               _SRC, "-lm", "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Weights(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int),
                ("wdtype", ctypes.c_int),
                ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("w13_s", ctypes.c_void_p), ("w13_z", ctypes.c_void_p),
                ("w2_s", ctypes.c_void_p), ("w2_z", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        P, I, F, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
        L.orc_bf16_to_f32.argtypes, L.orc_bf16_to_f32.restype = [ctypes.c_uint16], F
        L.orc_f32_to_bf16.argtypes, L.orc_f32_to_bf16.restype = [F], ctypes.c_uint16
        L.orc_f16_to_f32.argtypes, L.orc_f16_to_f32.restype = [ctypes.c_uint16], F
        L.orc_e4m3_to_f32.argtypes, L.orc_e4m3_to_f32.restype = [ctypes.c_uint8], F
        L.orc_f32_to_e4m3.argtypes, L.orc_f32_to_e4m3.restype = [F], ctypes.c_uint8
        L.orc_sigmoid.argtypes, L.orc_sigmoid.restype = [F], F
        L.orc_route.argtypes = [I, I, I, I, I, I, F, I, P, P, I, P, P]
        L.orc_route.restype = I
        L.orc_align_capacity.argtypes, L.orc_align_capacity.restype = [I, I, I, I], ctypes.c_int64
        L.orc_align.argtypes, L.orc_align.restype = [I, I, I, I, P, P, P, P, P, P], I
        L.orc_weight.argtypes = [ctypes.POINTER(_Weights), I, I, ctypes.c_int64, ctypes.c_int64]
        L.orc_weight.restype = D
        L.orc_forward.argtypes = [ctypes.POINTER(_Weights), I, I, P, P, P, I, P, P, P]
        L.orc_forward.restype = I
        L.orc_forward_ex.argtypes = [ctypes.POINTER(_Weights), I, I, P, P, P, I, P, P, P, I, I]
        L.orc_forward_ex.restype = I
        L.orc_fp8_intermediate.argtypes = [ctypes.POINTER(_Weights), I, I, P, P, P, P, P]
        L.orc_fp8_intermediate.restype = I
        L.orc_grouped_gemm.argtypes = [I, I, I, I, I, P, F, P, P, P, P]
        L.orc_grouped_gemm.restype = I
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---- codecs (scalar C functions mapped over arrays) ----------------------------------

def bf16_to_f32(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([lib().orc_bf16_to_f32(int(v)) for v in b.ravel()], np.float32).reshape(b.shape)


def f32_to_bf16(x):
    a = np.asarray(x, dtype=np.float32)
    return np.array([lib().orc_f32_to_bf16(float(v)) for v in a.ravel()], np.uint16).reshape(a.shape)


def f16_to_f32(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([lib().orc_f16_to_f32(int(v)) for v in b.ravel()], np.float32).reshape(b.shape)


def e4m3_to_f32(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib().orc_e4m3_to_f32(int(v)) for v in c.ravel()], np.float32).reshape(c.shape)


def f32_to_e4m3(x):
    a = np.asarray(x, dtype=np.float32)
    return np.array([lib().orc_f32_to_e4m3(float(v)) for v in a.ravel()], np.uint8).reshape(a.shape)


def sigmoid(x):
    a = np.asarray(x, dtype=np.float32)
    return np.array([lib().orc_sigmoid(float(v)) for v in a.ravel()], np.float32).reshape(a.shape)


# ---- routing and align ---------------------------------------------------------------

def route(kind, E, k, logits, renormalize=True, n_group=1, topk_group=1, routed_scaling=1.0,
          bias=None):
    """logits: [T,E] uint16 (bf16 bits) or float32.  Returns (ids int32 [T,k], w float32 [T,k])."""
    logits = np.ascontiguousarray(logits)
    if logits.dtype == np.uint16:
        ldt = BF16
    elif logits.dtype == np.float32:
        ldt = FP32
    else:
        raise TypeError("logits must be uint16 (bf16 bits) or float32")
    T = logits.shape[0]
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float32)
    bias = _c(bias, np.float32)
    rc = lib().orc_route(kind, E, k, int(renormalize), n_group, topk_group, float(routed_scaling),
                         ldt, _ptr(logits), _ptr(bias), T, _ptr(ids), _ptr(w))
    if rc:
        raise ValueError("orc_route rejected its arguments")
    return ids, w


def align_capacity(T, k, E, BM):
    return int(lib().orc_align_capacity(T, k, E, BM))


def align(ids, T, k, E, BM):
    ids = _c(ids, np.int32).reshape(-1)
    cap = align_capacity(T, k, E, BM)
    out = dict(sorted_token_ids=np.zeros(cap, np.int32), expert_ids=np.zeros(cap // BM, np.int32),
               num_tokens_post_padded=np.zeros(1, np.int32), expert_counts=np.zeros(E, np.int32),
               inv_pos=np.zeros(T * k, np.int32))
    rc = lib().orc_align(T, k, E, BM, _ptr(ids), _ptr(out["sorted_token_ids"]), _ptr(out["expert_ids"]),
                         _ptr(out["num_tokens_post_padded"]), _ptr(out["expert_counts"]),
                         _ptr(out["inv_pos"]))
    if rc:
        raise ValueError("orc_align rejected its arguments")
    return out


# ---- the layer -----------------------------------------------------------------------

class Weights:
    """Expert weights in the layouts the oracle reads (numpy arrays, kept alive here)."""

    def __init__(self, wdtype, E, H, I, w13, w2, w13_scale=None, w2_scale=None,
                 w13_s=None, w13_z=None, w2_s=None, w2_z=None):
        if wdtype == BF16:
            dt = np.uint16
        elif wdtype in (FP8_E4M3, INT4_G128):
            dt = np.uint8
        else:
            raise ValueError("unsupported weight dtype")
        self.arrays = dict(w13=_c(w13, dt), w2=_c(w2, dt), w13_scale=_c(w13_scale, np.float32),
                           w2_scale=_c(w2_scale, np.float32), w13_s=_c(w13_s, np.uint16),
                           w13_z=_c(w13_z, np.uint16), w2_s=_c(w2_s, np.uint16), w2_z=_c(w2_z, np.uint16))
        a = self.arrays
        self.c = _Weights(E, H, I, wdtype, *[_ptr(a[n]) for n in
                          ("w13", "w2", "w13_scale", "w2_scale", "w13_s", "w13_z", "w2_s", "w2_z")])
        self.E, self.H, self.I, self.wdtype = E, H, I, wdtype

    def value(self, m, e, n, c):
        return lib().orc_weight(ctypes.byref(self.c), m, e, n, c)


def default_threads() -> int:
    """Threads for the oracle's per-token work: the host's CPUs, at most 16 (MOE_ORACLE_THREADS
    overrides).  The results do not depend on it."""
    env = os.environ.get("MOE_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def forward(W: Weights, hidden_bits, ids, weights, tokens=None, return_scales=False, threads=None, acc32=False):
    """Layer output in fp64: [T,H], or [len(tokens),H] for the listed tokens.  threads: how
    many threads share the tokens (default: default_threads(); the result is the same for
    every count); acc32: accumulate in fp32 instead of fp64 (a cross-check of the fp64 run)."""
    hidden_bits = _c(hidden_bits, np.uint16)
    ids = _c(ids, np.int32)
    weights = _c(weights, np.float32)
    T, k = ids.shape
    assert hidden_bits.shape == (T, W.H)
    tok = _c(tokens, np.int32)
    n = T if tok is None else tok.size
    out = np.zeros((n, W.H), np.float64)
    dbg = np.zeros(2, np.float32)
    nth = default_threads() if threads is None else int(threads)
    rc = lib().orc_forward_ex(ctypes.byref(W.c), T, k, _ptr(hidden_bits), _ptr(ids), _ptr(weights),
                              0 if tok is None else tok.size, _ptr(tok), _ptr(out), _ptr(dbg), int(bool(acc32)), nth)
    if rc:
        raise ValueError("orc_forward rejected its arguments")
    return (out, dbg) if return_scales else out


def fp8_intermediate(W: Weights, hidden_bits, ids):
    """(h fp32 [T*k,I], h codes uint8 [T*k,I], scales [s1, s2]) of the w8a8 layer."""
    hidden_bits = _c(hidden_bits, np.uint16)
    ids = _c(ids, np.int32)
    T, k = ids.shape
    h = np.zeros((T * k, W.I), np.float32)
    hq = np.zeros((T * k, W.I), np.uint8)
    sc = np.zeros(2, np.float32)
    rc = lib().orc_fp8_intermediate(ctypes.byref(W.c), T, k, _ptr(hidden_bits), _ptr(ids),
                                    _ptr(h), _ptr(hq), _ptr(sc))
    if rc:
        raise ValueError("orc_fp8_intermediate rejected its arguments")
    return h, hq, sc


def to_bf16(out64):
    """Round the fp64 layer output to the layer's bf16 output (via fp32, RNE)."""
    return f32_to_bf16(np.asarray(out64, np.float64).astype(np.float32))


def grouped_gemm(dtype, E, N, K, x, w, m_sizes, x_scale=1.0, w_scale=None, M=None):
    """EP-MoE grouped GEMM over contiguous segments: y [M, N] fp64 (rows past the last
    segment are zero).  dtype BF16 (x, w as bf16 bits) or FP8_E4M3 (E4M3 codes, per-tensor
    x_scale and per-expert w_scale)."""
    x = _c(x, np.uint16 if dtype == BF16 else np.uint8)
    w = _c(w, np.uint16 if dtype == BF16 else np.uint8)
    m_sizes = _c(m_sizes, np.int32)
    M = x.shape[0] if M is None else M
    assert x.shape == (M, K) and w.shape == (E, N, K) and m_sizes.shape == (E,)
    y = np.zeros((M, N), np.float64)
    rc = lib().orc_grouped_gemm(E, N, K, dtype, M, _ptr(x), float(x_scale), _ptr(w), _ptr(_c(w_scale, np.float32)),
                                _ptr(m_sizes), _ptr(y))
    if rc != 0:
        raise ValueError("orc_grouped_gemm: invalid arguments")
    return y
