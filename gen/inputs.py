"""Seeded synthetic inputs for one GLM-5.2-style MoE layer (and a stack of them).

Shared by the CPU oracle's tests and the GPU library's tests and benchmark.  It
draws random numbers and encodes them; it computes nothing of the layer itself.

Interchange format of one expert matrix with R rows and K columns (K along the
contraction, groups of 32 along K):
  * ``q``: uint8 ``[R, K/2]``; element ``(r, 2j)`` is the low nibble of byte
    ``(r, j)`` and ``(r, 2j+1)`` the high nibble.  Nibbles are offset-binary: the
    int4 value is ``nibble - 8`` (the Colibri container's Q4 convention, described
    in the port design's G2 implementation status).
  * ``s``: uint16 ``[R, K/32]`` holding IEEE fp16 bits, one scale per 32
    consecutive elements of a row.
An expert has gate ``[I, H]``, up ``[I, H]`` and down ``[H, I]`` matrices.

Row-scaled formats (``LayerConfig.weight_format``): 1 = the same int4 bytes with
``s`` float32 ``[R]``, one scale per row (the production container's whole-row
group); 2 = ``q`` int8 ``[R, K]`` (two's complement, element ``(r, c)`` at byte
``(r, c)``) with ``s`` float32 ``[R]`` (the MTP layer's signed int8 experts).

Distributions (N(0, v) names the variance v; the scale recipe's 0.02 is a
standard deviation, the usual weight-init convention):
  x ~ N(0, 1) in fp32 (prefill: fp32 draw rounded RNE to bf16);
  router W ~ N(0, 1/H) fp32; bias ~ U(-0.1, 0.1) plus a workload skew;
  int4 values uniform on [-8, 7]; scales |N(0, 0.02^2)| rounded RNE to fp16;
  row-scaled int4: the same nibbles, scales |N(0, 0.02^2)| in fp32; int8 values
  uniform on [-128, 127], scales |N(0, (0.02/16)^2)| in fp32 (about the int4
  experts' output magnitude).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

KIND_ROUTER_W = 1
KIND_BIAS = 2
KIND_SKEW = 3
KIND_X = 4
KIND_EXPERT = 5
KIND_PERM = 6

# Bias skews (calibrated against the realised routing statistics that
# tests/test_workload_stats.py measures with the oracle).
BETA_SHARED = 0.28   # verify batch: about 40% of the union experts chosen by >= 2 of 4 tokens (union ~20)
BETA_ZIPF = 0.16     # prefill: per-expert token counts Zipf-like, log-log slope about -1.1
BETA_HOT = 0.20      # stack: a random 20% of experts receive about 80% of selections


def build_lib(force: bool = False) -> str:
    """Compile ``libsynth.so`` with gcc (OpenMP, IEEE semantics)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                               "-std=c11", src, "-o", _LIB_PATH + ".tmp", "-lm"])
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        L = ctypes.CDLL(_LIB_PATH)
        u64, p = ctypes.c_uint64, ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64] * 5
        for name, args in {
            "synth_fill_bytes": [u64, u64, p],
            "synth_fill_normal_f32": [u64, u64, ctypes.c_double, p],
            "synth_fill_normal_bf16": [u64, u64, ctypes.c_double, p],
            "synth_fill_absnormal_f16": [u64, u64, ctypes.c_double, p],
            "synth_fill_normal_f64": [u64, u64, p],
            "synth_fill_uniform_f64": [u64, u64, ctypes.c_double, ctypes.c_double, p],
            "synth_permutation": [u64, ctypes.c_int32, p],
            "synth_encode_f16": [u64, p, p],
            "synth_encode_bf16": [u64, p, p],
        }.items():
            getattr(L, name).restype = None
            getattr(L, name).argtypes = args
        _lib = L
    return _lib


def key(seed: int, a: int = 0, b: int = 0, c: int = 0, d: int = 0) -> int:
    return lib().synth_key(seed & (2**64 - 1), a, b, c, d)


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def fill_bytes(k: int, out: np.ndarray) -> np.ndarray:
    lib().synth_fill_bytes(k, out.nbytes, _ptr(out))
    return out


def normal_f32(k: int, n: int, sigma: float) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_fill_normal_f32(k, n, sigma, _ptr(out))
    return out


def normal_bf16_bits(k: int, n: int, sigma: float) -> np.ndarray:
    out = np.empty(n, np.uint16)
    lib().synth_fill_normal_bf16(k, n, sigma, _ptr(out))
    return out


def absnormal_f16_bits(k: int, out: np.ndarray, sigma: float) -> np.ndarray:
    assert out.dtype == np.uint16
    lib().synth_fill_absnormal_f16(k, out.size, sigma, _ptr(out))
    return out


def normal_f64(k: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_fill_normal_f64(k, n, _ptr(out))
    return out


def uniform_f64(k: int, n: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_fill_uniform_f64(k, n, lo, hi, _ptr(out))
    return out


def permutation(k: int, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_permutation(k, n, _ptr(out))
    return out


def encode_f16(values: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(values, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().synth_encode_f16(v.size, _ptr(v), _ptr(out))
    return out


def encode_bf16(values: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(values, np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().synth_encode_bf16(v.size, _ptr(v), _ptr(out))
    return out


@dataclass(frozen=True)
class LayerConfig:
    """Shape and routing constants of one MoE layer."""
    hidden: int
    n_experts: int
    n_group: int
    topk_group: int
    top_k: int
    moe_inter: int
    shared_inter: int
    group_size: int = 32
    routed_scaling_factor: float = 2.5
    norm_topk_prob: int = 1
    weight_format: int = 0        # 0: int4 + fp16 per 32; 1: int4 + fp32 per row; 2: int8 + fp32 per row


@dataclass(frozen=True)
class Workload:
    """A seeded synthetic workload: layer shape, token count and input recipe."""
    name: str
    cfg: LayerConfig
    tokens: int
    x_dtype: str = "f32"          # "f32" or "bf16"
    bias_recipe: str = "uniform"  # "uniform", "shared", "zipf", "hotset"
    layers: int = 1
    steps: int = 1
    seed: int = 0
    n_blobs: int = 0              # >0: logical experts alias onto this many distinct weight blobs

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = LayerConfig(hidden=256, n_experts=16, n_group=4, topk_group=2, top_k=2, moe_inter=128, shared_inter=128)
GLM52 = LayerConfig(hidden=6144, n_experts=256, n_group=8, topk_group=4, top_k=8, moe_inter=2048, shared_inter=2048)

WORKLOADS = {
    "tiny": Workload("tiny", TINY, tokens=1, seed=0),
    "decode": Workload("decode", GLM52, tokens=1, seed=1),
    "verify": Workload("verify", GLM52, tokens=4, bias_recipe="shared", seed=2),
    "prefill": Workload("prefill", GLM52, tokens=2048, x_dtype="bf16", bias_recipe="zipf", seed=3),
    "stack": Workload("stack", GLM52, tokens=1, bias_recipe="hotset", layers=75, steps=64, seed=4, n_blobs=1024),
}


def router_weights(w: Workload, layer: int = 0) -> np.ndarray:
    c = w.cfg
    W = normal_f32(key(w.seed, KIND_ROUTER_W, layer), c.n_experts * c.hidden, 1.0 / math.sqrt(c.hidden))
    return W.reshape(c.n_experts, c.hidden)


def router_bias(w: Workload, layer: int = 0) -> np.ndarray:
    c = w.cfg
    E = c.n_experts
    b = uniform_f64(key(w.seed, KIND_BIAS, layer), E, -0.1, 0.1)
    if w.bias_recipe == "shared":
        b = b + BETA_SHARED * normal_f64(key(w.seed, KIND_SKEW, layer), E)
    elif w.bias_recipe == "zipf":
        rank = permutation(key(w.seed, KIND_PERM, layer), E).astype(np.float64) + 1.0
        b = b + BETA_ZIPF * (-np.log(rank))
    elif w.bias_recipe == "hotset":
        hot = permutation(key(w.seed, KIND_PERM, layer), E)[: int(round(0.2 * E))]
        b[hot] += BETA_HOT
    elif w.bias_recipe != "uniform":
        raise ValueError(w.bias_recipe)
    return b.astype(np.float32)


def hot_set(w: Workload, layer: int = 0) -> np.ndarray:
    E = w.cfg.n_experts
    return np.sort(permutation(key(w.seed, KIND_PERM, layer), E)[: int(round(0.2 * E))])


def tokens(w: Workload, layer: int = 0, step: int = 0, S: int | None = None, offset: int = 0) -> np.ndarray:
    """x for (layer, step): fp32 [S, H], or bf16 bits uint16 [S, H] for bf16 workloads.

    Token ``t`` of a call with ``offset`` is token ``offset + t`` of the (layer, step) stream,
    so any subset of a batch can be regenerated on its own."""
    c = w.cfg
    S = w.tokens if S is None else S
    out = []
    for t in range(offset, offset + S):
        k = key(w.seed, KIND_X, layer, step, t)
        if w.x_dtype == "bf16":
            out.append(normal_bf16_bits(k, c.hidden, 1.0))
        else:
            out.append(normal_f32(k, c.hidden, 1.0))
    if not out:
        return np.zeros((0, c.hidden), np.uint16 if w.x_dtype == "bf16" else np.float32)
    return np.stack(out)


@dataclass
class ExpertWeights:
    inter: int
    qg: np.ndarray
    sg: np.ndarray
    qu: np.ndarray
    su: np.ndarray
    qd: np.ndarray
    sd: np.ndarray
    fmt: int = 0

    def parts(self):
        return (self.qg, self.sg, self.qu, self.su, self.qd, self.sd)


def empty_expert(cfg: LayerConfig, inter: int) -> ExpertWeights:
    H, g, f = cfg.hidden, cfg.group_size, cfg.weight_format
    if f == 0:
        return ExpertWeights(
            inter,
            np.empty((inter, H // 2), np.uint8), np.empty((inter, H // g), np.uint16),
            np.empty((inter, H // 2), np.uint8), np.empty((inter, H // g), np.uint16),
            np.empty((H, inter // 2), np.uint8), np.empty((H, inter // g), np.uint16),
        )
    qt, d = (np.uint8, 2) if f == 1 else (np.int8, 1)
    return ExpertWeights(
        inter,
        np.empty((inter, H // d), qt), np.empty(inter, np.float32),
        np.empty((inter, H // d), qt), np.empty(inter, np.float32),
        np.empty((H, inter // d), qt), np.empty(H, np.float32),
        f,
    )


def blob_of(w: Workload, layer: int, e: int) -> tuple[int, int]:
    """Generator identity of logical expert (layer, e); the stack workload aliases
    logical experts onto ``n_blobs`` distinct weight blobs (the shared expert of
    each layer is never aliased)."""
    E = w.cfg.n_experts
    if w.n_blobs and e < E:
        return (0, (layer * E + e) % w.n_blobs)
    return (layer, e)


def expert_weights(w: Workload, layer: int, e: int, out: ExpertWeights | None = None) -> ExpertWeights:
    """Weights of routed expert ``e`` of ``layer``; ``e == n_experts`` is the shared expert."""
    c = w.cfg
    inter = c.shared_inter if e == c.n_experts else c.moe_inter
    ex = out if out is not None else empty_expert(c, inter)
    assert ex.inter == inter
    bl, be = blob_of(w, layer, e)
    for part, arr in enumerate(ex.parts()):
        k = key(w.seed, KIND_EXPERT, bl, be, part)
        if arr.dtype in (np.uint8, np.int8):
            fill_bytes(k, arr.view(np.uint8))
        elif arr.dtype == np.uint16:
            absnormal_f16_bits(k, arr, 0.02)
        else:  # fp32 row scales
            lib().synth_fill_normal_f32(k, arr.size, 0.02 / 16 if c.weight_format == 2 else 0.02, _ptr(arr))
            np.abs(arr, out=arr)
    return ex
