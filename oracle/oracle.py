"""ctypes wrapper of the fp64 CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build_lib(force: bool = False) -> str:
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11",
                               _SRC, "-o", _LIB_PATH + ".tmp", "-lm"])
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class Diag(ctypes.Structure):
    _fields_ = [("expert_margin", ctypes.c_double), ("group_margin", ctypes.c_double),
                ("flags", ctypes.c_int32), ("n_candidates", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        L = ctypes.CDLL(_LIB_PATH)
        p, i, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        L.oracle_f16_to_f64.restype = d
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = d
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_dequant.restype = None
        L.oracle_dequant.argtypes = [i, i, i, p, p, p]
        L.oracle_select.restype = i
        L.oracle_select.argtypes = [i, i, i, i, d, i, p, p, p, p, p, p]
        L.oracle_route.restype = i
        L.oracle_route.argtypes = [i, i, i, i, i, i, d, i, i, p, p, p, p, p, p, p]
        L.oracle_expert_ffn.restype = None
        L.oracle_expert_ffn.argtypes = [i, i, i, p, p, p, p, p, p, p, p, p]
        L.oracle_moe_ffn.restype = i
        L.oracle_moe_ffn.argtypes = [i] * 8 + [p] * 10
        L.oracle_dequant_fmt.restype = None
        L.oracle_dequant_fmt.argtypes = [i, i, i, i, p, p, p]
        L.oracle_expert_ffn_fmt.restype = None
        L.oracle_expert_ffn_fmt.argtypes = [i, i, i, i, p, p, p, p, p, p, p, p, p]
        L.oracle_moe_ffn_fmt.restype = i
        L.oracle_moe_ffn_fmt.argtypes = [i] * 9 + [p] * 10
        L.oracle_moe_ffn_mode.restype = i
        L.oracle_moe_ffn_mode.argtypes = [i] * 10 + [p] * 10
        L.oracle_moe_ffn_mask.restype = i
        L.oracle_moe_ffn_mask.argtypes = [i] * 10 + [p] * 11
        L.oracle_bf16_round.restype = ctypes.c_float
        L.oracle_bf16_round.argtypes = [ctypes.c_float]
        L.oracle_quant_row.restype = ctypes.c_float
        L.oracle_quant_row.argtypes = [i, p, p, p]
        L.oracle_expert_ffn_int8act.restype = None
        L.oracle_expert_ffn_int8act.argtypes = [i, i, i, i, p, p, p, p, p, p, p, p, p]
        L.oracle_num_threads.restype = i
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [i]
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def f16_to_f64(h: int) -> float:
    return lib().oracle_f16_to_f64(h)


def bf16_to_f64(b: int) -> float:
    return lib().oracle_bf16_to_f64(b)


def dequant(q: np.ndarray, s: np.ndarray, gsz: int = 32) -> np.ndarray:
    R = q.shape[0]
    K = q.shape[1] * 2
    out = np.empty((R, K), np.float64)
    lib().oracle_dequant(R, K, gsz, _p(np.ascontiguousarray(q)), _p(np.ascontiguousarray(s)), _p(out))
    return out


def dequant_fmt(fmt: int, q: np.ndarray, s: np.ndarray, gsz: int = 32) -> np.ndarray:
    """[R, K] fp64 weights of a matrix in weight format ``fmt`` (0: int4 + fp16 per
    ``gsz``; 1: int4 + fp32 per row; 2: int8 + fp32 per row)."""
    R = q.shape[0]
    K = q.shape[1] if fmt == 2 else q.shape[1] * 2
    out = np.empty((R, K), np.float64)
    lib().oracle_dequant_fmt(fmt, R, K, gsz, _p(np.ascontiguousarray(q)), _p(np.ascontiguousarray(s)), _p(out))
    return out


def quant_row(v: np.ndarray):
    """int8 activation quantisation of one fp32 row: (q int8[n], d fp32, q * d fp64[n])."""
    v = np.ascontiguousarray(v, np.float32)
    q = np.empty(v.size, np.int8)
    out = np.empty(v.size, np.float64)
    d = lib().oracle_quant_row(v.size, _p(v), _p(q), _p(out))
    return q, np.float32(d), out


def expert_ffn_int8act(ex, x: np.ndarray, H: int, gsz: int = 32, return_h: bool = False):
    """One expert on one fp32 token in int8-activation mode: x and h are quantised per row."""
    x = np.ascontiguousarray(x, np.float32)
    y = np.empty(H, np.float64)
    h = np.empty(ex.inter, np.float64)
    lib().oracle_expert_ffn_int8act(ex.fmt, H, ex.inter, gsz, *[_p(np.ascontiguousarray(a)) for a in ex.parts()],
                                    _p(x), _p(y), _p(h))
    return (y, h) if return_h else y


def select(cfg, logits: np.ndarray, bias: np.ndarray):
    """Selection for one token from fp64 logits: (idx[k], w[k] fp64, s[E] fp64, Diag)."""
    E, k = cfg.n_experts, cfg.top_k
    l = np.ascontiguousarray(logits, np.float64)
    b = np.ascontiguousarray(bias, np.float32)
    idx = np.empty(k, np.int32)
    w = np.empty(k, np.float64)
    s = np.empty(E, np.float64)
    dg = Diag()
    rc = lib().oracle_select(E, cfg.n_group, cfg.topk_group, k, cfg.routed_scaling_factor, cfg.norm_topk_prob,
                             _p(l), _p(b), _p(idx), _p(w), _p(s), ctypes.addressof(dg))
    if rc:
        raise ValueError("oracle_select rejected the configuration")
    return idx, w, s, dg


def route(cfg, x: np.ndarray, W: np.ndarray, bias: np.ndarray, x_is_bf16: bool = False):
    """Router for S tokens: (idx[S,k] int32, w[S,k] fp64, logits[S,E] fp64, flags[S], margins[S,2])."""
    S, H = x.shape
    E, k = cfg.n_experts, cfg.top_k
    x = np.ascontiguousarray(x)
    W = np.ascontiguousarray(W, np.float32)
    b = np.ascontiguousarray(bias, np.float32)
    idx = np.empty((S, k), np.int32)
    w = np.empty((S, k), np.float64)
    logits = np.empty((S, E), np.float64)
    dg = (Diag * max(S, 1))()
    rc = lib().oracle_route(S, H, E, cfg.n_group, cfg.topk_group, k, cfg.routed_scaling_factor, cfg.norm_topk_prob,
                            int(x_is_bf16), _p(x), _p(W), _p(b), _p(idx), _p(w), _p(logits), ctypes.addressof(dg))
    if rc:
        raise ValueError("oracle_route rejected the configuration")
    flags = np.array([dg[t].flags for t in range(S)], np.int32)
    margins = np.array([[dg[t].expert_margin, dg[t].group_margin] for t in range(S)], np.float64).reshape(S, 2)
    return idx, w, logits, flags, margins


def expert_ffn(ex, x: np.ndarray, H: int, gsz: int = 32, return_h: bool = False):
    """One expert on one fp64 token: y[H] (and h[I])."""
    I = ex.inter
    x = np.ascontiguousarray(x, np.float64)
    y = np.empty(H, np.float64)
    h = np.empty(I, np.float64)
    lib().oracle_expert_ffn_fmt(ex.fmt, H, I, gsz, *[_p(np.ascontiguousarray(a)) for a in ex.parts()], _p(x), _p(y),
                                _p(h))
    return (y, h) if return_h else y


def bf16_round(v: float) -> float:
    """R8's rounding of one fp32 value to the nearest bf16 (ties to even)."""
    return float(lib().oracle_bf16_round(float(v)))


def moe_ffn(cfg, x: np.ndarray, idx: np.ndarray, w: np.ndarray, experts: dict, x_is_bf16: bool = False,
            act_int8: bool = False, bf16_experts=()):
    """The layer's FFN for S tokens given routing; ``experts`` maps expert id -> ExpertWeights
    (id ``n_experts`` is the shared expert).  act_int8: x and every h are quantised to int8 per
    row before their matmuls.  bf16_experts: ids (``n_experts`` for the shared expert) computed
    with bf16 operands (R8).  Returns y[S,H] fp64."""
    S, H = x.shape
    E, k = cfg.n_experts, cfg.top_k
    arrs = [[None] * (E + 1) for _ in range(6)]
    fmts = {ex.fmt for ex in experts.values()}
    if len(fmts) > 1:
        raise ValueError("oracle_moe_ffn: experts in mixed weight formats")
    fmt = fmts.pop() if fmts else 0
    for e, ex in experts.items():
        for j, a in enumerate(ex.parts()):
            arrs[j][e] = _p(np.ascontiguousarray(a))
    ptrs = [(ctypes.c_void_p * (E + 1))(*arrs[j]) for j in range(6)]
    y = np.empty((S, H), np.float64)
    x = np.ascontiguousarray(x)
    idx = np.ascontiguousarray(idx, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    mask = np.zeros(E + 1, np.uint8)
    for e in bf16_experts:
        mask[int(e)] = 1
    rc = lib().oracle_moe_ffn_mask(fmt, int(act_int8), S, H, E, k, cfg.moe_inter, cfg.shared_inter, cfg.group_size,
                                   int(x_is_bf16), _p(x), _p(idx), _p(w),
                                   *[ctypes.cast(pp, ctypes.c_void_p) for pp in ptrs], _p(mask), _p(y))
    if rc == -2:
        raise ValueError("oracle_moe_ffn: bf16 operands are not combined with int8 activations")
    if rc:
        raise ValueError("oracle_moe_ffn: routing names an expert without weights")
    return y


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(n)
