"""Helpers for GPU tests: put a seeded synthetic layer into HBM through the C ABI
(device-side packer) and run moe_route / moe_ffn on it."""
from __future__ import annotations

import numpy as np
import torch

from gen import inputs as gen
from int4_routed_expert_amd import moe as M


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


class DeviceLayer:
    """Routed experts of one layer packed into one slab (table[e] = e), the shared
    expert in its own buffer, router weights on the device."""

    def __init__(self, w: gen.Workload, layer: int = 0, experts=None, host_experts: bool = False,
                 mfma_min_tokens: int = M.MFMA_MIN_TOKENS, act_int8: int = 0):
        self.w = w
        c = w.cfg
        self.c = c
        self.act_int8 = act_int8
        self.cfg = M.make_cfg(c, mfma_min_tokens, act_int8)
        E = c.n_experts
        self.slot_bytes = M.moe_expert_bytes(self.cfg, c.moe_inter)
        self.experts = list(range(E)) if experts is None else sorted(set(experts))
        self.slab = torch.zeros(E * self.slot_bytes, dtype=torch.uint8, device="cuda")
        self.table = torch.arange(E, dtype=torch.int32, device="cuda")
        self.host = {}
        stage = gen.empty_expert(c, c.moe_inter)
        for e in self.experts:
            gen.expert_weights(w, layer, e, out=stage)
            self._pack(stage, c.moe_inter, self.slab[e * self.slot_bytes:(e + 1) * self.slot_bytes])
            if host_experts:
                self.host[e] = gen.ExpertWeights(stage.inter, *[a.copy() for a in stage.parts()], stage.fmt)
        self.shared = None
        if c.shared_inter > 0:
            sb = M.moe_expert_bytes(self.cfg, c.shared_inter)
            self.shared = torch.zeros(sb, dtype=torch.uint8, device="cuda")
            sh = gen.expert_weights(w, layer, E)
            self._pack(sh, c.shared_inter, self.shared)
            self.host[E] = sh
        self.W_host = gen.router_weights(w, layer)
        self.bias_host = gen.router_bias(w, layer)
        self.W = dev(self.W_host)
        self.bias = dev(self.bias_host)
        torch.cuda.synchronize()

    def _pack(self, ex: gen.ExpertWeights, inter: int, dst: torch.Tensor) -> None:
        parts = [dev(a) for a in ex.parts()]
        M.pack_expert(self.cfg, inter, *parts, dst, 1)
        torch.cuda.current_stream().synchronize()

    def host_expert(self, e: int, layer: int = 0) -> gen.ExpertWeights:
        if e not in self.host:
            self.host[e] = gen.expert_weights(self.w, layer, e)
        return self.host[e]

    def view(self, table: torch.Tensor | None = None) -> M.moe_slot_view:
        t = self.table if table is None else table
        return M.slot_view(self.slab, self.slot_bytes, t, self.c.n_experts)

    def workspace(self, S: int) -> torch.Tensor:
        return M.workspace(self.cfg, S)

    def route(self, x: torch.Tensor, x_dtype: int, ws: torch.Tensor | None = None):
        S = x.shape[0]
        ws = self.workspace(S) if ws is None else ws
        idx = torch.full((S, self.c.top_k), -1, dtype=torch.int32, device="cuda")
        wt = torch.full((S, self.c.top_k), float("nan"), dtype=torch.float32, device="cuda")
        M.moe_route(self.cfg, x, x_dtype, S, self.W, self.bias, idx, wt, ws, ws.numel())
        return idx, wt

    def ffn(self, x: torch.Tensor, x_dtype: int, idx: torch.Tensor, wt: torch.Tensor, table=None, ws=None,
            mfma_min_tokens: int | None = None):
        """moe_ffn; mfma_min_tokens overrides the layer's threshold of the matrix-core path."""
        S = x.shape[0]
        ws = self.workspace(S) if ws is None else ws
        cfg = self.cfg if mfma_min_tokens is None else M.make_cfg(self.c, mfma_min_tokens, self.act_int8)
        y = torch.full((S, self.c.hidden), float("nan"), dtype=torch.float32, device="cuda")
        M.moe_ffn(cfg, x, x_dtype, S, idx, wt, self.view(table), self.shared, y, ws, ws.numel())
        return y


    def layer(self, x: torch.Tensor, x_dtype: int, table=None, ws=None):
        """moe_layer: (idx, w, y)."""
        S = x.shape[0]
        ws = self.workspace(S) if ws is None else ws
        idx = torch.full((S, self.c.top_k), -7, dtype=torch.int32, device="cuda")
        wt = torch.full((S, self.c.top_k), float("nan"), dtype=torch.float32, device="cuda")
        y = torch.full((S, self.c.hidden), float("nan"), dtype=torch.float32, device="cuda")
        M.moe_layer(self.cfg, x, x_dtype, S, self.W, self.bias, idx, wt, self.view(table), self.shared, y, ws,
                    ws.numel())
        return idx, wt, y


def x_device(w: gen.Workload, x_host: np.ndarray):
    """(tensor, dtype code) for generator activations (fp32, or bf16 bits)."""
    if w.x_dtype == "bf16":
        return dev(x_host.view(np.int16)).view(torch.bfloat16), M.MOE_BF16
    return dev(x_host), M.MOE_F32


def matrix_core_experts(ridx: np.ndarray, n_experts: int, shared_inter: int, mfma_min_tokens: int) -> list:
    """The experts (``n_experts`` for the shared one) that a batch with routing ridx
    sends to the bf16 matrix cores (moe_cfg.mfma_min_tokens): in batches of more
    than 4 tokens, every expert chosen by at least that many tokens, and the shared
    expert when the batch has at least that many tokens."""
    S = ridx.shape[0]
    if mfma_min_tokens <= 0 or S <= 4:
        return []
    counts = np.bincount(ridx.ravel(), minlength=n_experts)
    out = [int(e) for e in np.where(counts >= mfma_min_tokens)[0]]
    if shared_inter > 0 and S >= mfma_min_tokens:
        out.append(n_experts)
    return out


def max_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max over tokens of max_i |y - ref| / max_i |ref| (0 when both are exactly zero)."""
    worst = 0.0
    for t in range(ref.shape[0]):
        den = np.abs(ref[t]).max()
        num = np.abs(y[t].astype(np.float64) - ref[t]).max()
        if den == 0.0:
            if num != 0.0:
                return float("inf")
            continue
        worst = max(worst, num / den)
    return worst


def tile_cover(ridx: np.ndarray, n_experts: int, mfma_min_tokens: int, tile_rows: int = 256, item_rows: int = 4,
               extra: int = 0, seed: int = 0) -> np.ndarray:
    """Tokens of a batch such that every unit of work of the large-batch path holds
    at least one of them: each matrix-core tile (tile_rows consecutive entries of
    an expert's token list, which is in token order; the shared expert's tiles
    are consecutive tokens) and each GEMV item (item_rows consecutive entries of
    an expert below the threshold, or of the shared expert when the batch is).
    Greedy set cover (a token sits in up to top_k + 1 units), plus `extra`
    random tokens."""
    from collections import Counter
    S = ridx.shape[0]
    units = []
    for e in range(n_experts):
        toks = np.where((ridx == e).any(axis=1))[0]
        if toks.size == 0:
            continue
        step = tile_rows if mfma_min_tokens > 0 and toks.size >= mfma_min_tokens else item_rows
        units += [set(toks[i:i + step].tolist()) for i in range(0, toks.size, step)]
    step = tile_rows if mfma_min_tokens > 0 and S >= mfma_min_tokens else item_rows
    units += [set(range(i, min(S, i + step))) for i in range(0, S, step)]
    chosen = []
    while units:
        cnt = Counter(t for u in units for t in u)
        best = max(cnt.items(), key=lambda kv: (kv[1], -kv[0]))[0]
        chosen.append(best)
        units = [u for u in units if best not in u]
    rng = np.random.default_rng(seed)
    chosen = set(chosen) | set(rng.choice(S, size=min(extra, S), replace=False).tolist())
    return np.array(sorted(chosen))
