"""Python binding of ``libmoe.so`` (include/moe.h): argument marshalling only.

Every function with a ``moe_`` name calls the C entry point of the same name.
Tensors are passed as raw pointers (``torch.Tensor.data_ptr()`` for device
memory, numpy arrays for host memory); streams as ``torch.cuda.Stream`` handles.
The library does all the work; if it is missing this module raises on import.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

MOE_OK, MOE_EINVAL, MOE_ENULL, MOE_EDTYPE, MOE_EWORKSPACE, MOE_ENOSLOT, MOE_ESTALE, MOE_EHIP, MOE_ELEASE = \
    0, -1, -2, -3, -4, -5, -6, -7, -8
MOE_F32, MOE_BF16 = 0, 1
MOE_WF_Q4_G32, MOE_WF_Q4_ROW, MOE_WF_Q8_ROW = 0, 1, 2


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.moe_status_string(status).decode()
        if status == MOE_EHIP:
            msg += ": " + _lib.moe_last_hip_error().decode()
        super().__init__(f"{where}: {msg} ({status})")


class moe_cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("top_k", ctypes.c_int32), ("moe_inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("norm_topk_prob", ctypes.c_int32),
                ("mfma_min_tokens", ctypes.c_int32), ("weight_format", ctypes.c_int32), ("act_int8", ctypes.c_int32)]


class moe_slot_view(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("slot_bytes", ctypes.c_int64), ("table", ctypes.c_void_p),
                ("n_slots", ctypes.c_int32), ("gen", ctypes.c_void_p), ("slot_gen", ctypes.c_void_p),
                ("lease", ctypes.c_uint64)]


class moe_layer_call(ctypes.Structure):
    _fields_ = [("cfg", ctypes.POINTER(moe_cfg)), ("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int32),
                ("S", ctypes.c_int32), ("W_gate", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("idx", ctypes.c_void_p), ("w", ctypes.c_void_p), ("experts", ctypes.POINTER(moe_slot_view)),
                ("shared", ctypes.c_void_p), ("y", ctypes.c_void_p), ("ws", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_size_t)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc for gfx950)")
    # torch ships its own HIP runtime and loads it by path.  Loaded first, the
    # library would resolve libamdhip64.so.7 through its run path to a second
    # runtime in the same process, which sees no device and knows none of
    # torch's streams; with torch loaded first, the soname binds to torch's copy.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cp = ctypes.POINTER(moe_cfg)
    sigs = {
        "moe_validate_cfg": (ctypes.c_int, [cp]),
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_last_hip_error": (ctypes.c_char_p, []),
        "moe_expert_bytes": (i64, [cp, i32]),
        "moe_workspace_bytes": (sz, [cp, i32]),
        "moe_workspace_init": (ctypes.c_int, [p, sz, p]),
        "moe_pack_expert": (ctypes.c_int, [cp, i32, p, p, p, p, p, p, p, i32, p]),
        "moe_unpack_expert": (ctypes.c_int, [cp, i32, p, p, p, p, p, p, p]),
        "moe_pack_expert_rows": (ctypes.c_int, [cp, i32, p, p, p, p, p, p, p, i32, p]),
        "moe_unpack_expert_rows": (ctypes.c_int, [cp, i32, p, p, p, p, p, p, p]),
        "moe_route": (ctypes.c_int, [cp, p, i32, i32, p, p, p, p, p, sz, p]),
        "moe_ffn": (ctypes.c_int, [cp, p, i32, i32, p, p, ctypes.POINTER(moe_slot_view), p, p, p, sz, p]),
        "moe_layer": (ctypes.c_int, [cp, p, i32, i32, p, p, p, p, ctypes.POINTER(moe_slot_view), p, p, p, sz, p]),
        "moe_layer_noalloc": (ctypes.c_int, [cp, p, i32, i32, p, p, p, p, ctypes.POINTER(moe_slot_view), p, p, p]),
        "moe_chain_create": (ctypes.c_int, [ctypes.POINTER(moe_layer_call), i32, ctypes.POINTER(p)]),
        "moe_chain_launch": (ctypes.c_int, [p, p]),
        "moe_chain_destroy": (None, [p]),
        "moe_pool_create": (ctypes.c_int, [cp, i32, i32, i32, ctypes.POINTER(p)]),
        "moe_pool_destroy": (None, [p]),
        "moe_pool_register_host": (ctypes.c_int, [p, i32, i32, p]),
        "moe_pool_acquire": (ctypes.c_int, [p, i32, p, i32, ctypes.POINTER(moe_slot_view), ctypes.POINTER(i32), p, p]),
        "moe_pool_release": (ctypes.c_int, [p, i32, p]),
        "moe_pool_prefetch": (ctypes.c_int, [p, i32, p, i32, ctypes.POINTER(i32), p]),
        "moe_pool_trace": (ctypes.c_int, [p, p, i32]),
        "moe_pool_stats": (ctypes.c_int, [p, ctypes.c_char_p, sz]),
        "moe_pool_check_view": (ctypes.c_int, [p, i32, ctypes.POINTER(moe_slot_view)]),
        "moe_profile_enable": (ctypes.c_int, [ctypes.c_int]),
        "moe_profile_report": (ctypes.c_int, [ctypes.c_char_p, sz]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


_lib = _load()


def header_functions() -> list[str]:
    """Names of the functions include/moe.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    return _lib


MFMA_MIN_TOKENS = 3  # default threshold of the matrix-core path (tokens per expert)


def make_cfg(c, mfma_min_tokens: int = MFMA_MIN_TOKENS, act_int8: int = 0) -> moe_cfg:
    """moe_cfg from any object with the LayerConfig field names."""
    return moe_cfg(c.hidden, c.n_experts, c.n_group, c.topk_group, c.top_k, c.moe_inter, c.shared_inter,
                   c.group_size, c.routed_scaling_factor, c.norm_topk_prob, mfma_min_tokens,
                   getattr(c, "weight_format", MOE_WF_Q4_G32), act_int8)


def ptr(t) -> int | None:
    """Raw address of a torch tensor or numpy array, or an address given as an int (None passes NULL)."""
    if t is None or isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    return t.ctypes.data


def stream_handle(stream=None) -> int | None:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(rc: int, where: str) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, where)


def moe_validate_cfg(cfg: moe_cfg) -> int:
    return _lib.moe_validate_cfg(ctypes.byref(cfg))


def moe_expert_bytes(cfg: moe_cfg, inter: int) -> int:
    return _lib.moe_expert_bytes(ctypes.byref(cfg), inter)


def moe_workspace_bytes(cfg: moe_cfg, max_S: int) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(cfg), max_S)


def moe_workspace_init(ws, ws_bytes: int | None = None, stream=None) -> None:
    """Write the workspace header (magic words, zeroed counters) on `stream`."""
    n = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(_lib.moe_workspace_init(ptr(ws), n, stream_handle(stream)), "moe_workspace_init")


def workspace(cfg: moe_cfg, max_S: int, device="cuda", stream=None):
    """A device workspace for up to max_S tokens, initialised (torch uint8 tensor)."""
    import torch
    ws = torch.empty(moe_workspace_bytes(cfg, max_S), dtype=torch.uint8, device=device)
    moe_workspace_init(ws, stream=stream)
    return ws


def moe_pack_expert(cfg: moe_cfg, inter: int, qg, sg, qu, su, qd, sd, dst, where: int, stream=None) -> None:
    st = stream_handle(stream) if where == 1 else None
    _check(_lib.moe_pack_expert(ctypes.byref(cfg), inter, ptr(qg), ptr(sg), ptr(qu), ptr(su), ptr(qd), ptr(sd),
                                ptr(dst), where, st), "moe_pack_expert")


def moe_unpack_expert(cfg: moe_cfg, inter: int, src, qg, sg, qu, su, qd, sd) -> None:
    _check(_lib.moe_unpack_expert(ctypes.byref(cfg), inter, ptr(src), ptr(qg), ptr(sg), ptr(qu), ptr(su), ptr(qd),
                                  ptr(sd)), "moe_unpack_expert")


def moe_pack_expert_rows(cfg: moe_cfg, inter: int, qg, sg, qu, su, qd, sd, dst, where: int, stream=None) -> None:
    st = stream_handle(stream) if where == 1 else None
    _check(_lib.moe_pack_expert_rows(ctypes.byref(cfg), inter, ptr(qg), ptr(sg), ptr(qu), ptr(su), ptr(qd), ptr(sd),
                                     ptr(dst), where, st), "moe_pack_expert_rows")


def moe_unpack_expert_rows(cfg: moe_cfg, inter: int, src, qg, sg, qu, su, qd, sd) -> None:
    _check(_lib.moe_unpack_expert_rows(ctypes.byref(cfg), inter, ptr(src), ptr(qg), ptr(sg), ptr(qu), ptr(su),
                                       ptr(qd), ptr(sd)), "moe_unpack_expert_rows")


def pack_expert(cfg: moe_cfg, inter: int, qg, sg, qu, su, qd, sd, dst, where: int, stream=None) -> None:
    """moe_pack_expert or moe_pack_expert_rows, by cfg.weight_format."""
    f = moe_pack_expert if cfg.weight_format == MOE_WF_Q4_G32 else moe_pack_expert_rows
    f(cfg, inter, qg, sg, qu, su, qd, sd, dst, where, stream)


def moe_route(cfg: moe_cfg, x, x_dtype: int, S: int, W, bias, idx, w, ws, ws_bytes: int, stream=None) -> None:
    _check(_lib.moe_route(ctypes.byref(cfg), ptr(x), x_dtype, S, ptr(W), ptr(bias), ptr(idx), ptr(w), ptr(ws),
                          ws_bytes, stream_handle(stream)), "moe_route")


def moe_ffn(cfg: moe_cfg, x, x_dtype: int, S: int, idx, w, view: moe_slot_view, shared, y, ws, ws_bytes: int,
            stream=None) -> None:
    _check(_lib.moe_ffn(ctypes.byref(cfg), ptr(x), x_dtype, S, ptr(idx), ptr(w), ctypes.byref(view), ptr(shared),
                        ptr(y), ptr(ws), ws_bytes, stream_handle(stream)), "moe_ffn")


def moe_layer(cfg: moe_cfg, x, x_dtype: int, S: int, W, bias, idx, w, view: moe_slot_view, shared, y, ws,
              ws_bytes: int, stream=None) -> None:
    _check(_lib.moe_layer(ctypes.byref(cfg), ptr(x), x_dtype, S, ptr(W), ptr(bias), ptr(idx), ptr(w),
                          ctypes.byref(view), ptr(shared), ptr(y), ptr(ws), ws_bytes, stream_handle(stream)),
           "moe_layer")


def moe_layer_noalloc(cfg: moe_cfg, x, x_dtype: int, S: int, W, bias, idx, w, view: moe_slot_view, shared, y,
                      stream=None) -> None:
    _check(_lib.moe_layer_noalloc(ctypes.byref(cfg), ptr(x), x_dtype, S, ptr(W), ptr(bias), ptr(idx), ptr(w),
                                  ctypes.byref(view), ptr(shared), ptr(y), stream_handle(stream)), "moe_layer_noalloc")


MOE_SCRATCH_BYTES = 8 << 20  # the library's per-device workspace of moe_layer_noalloc


def _x_dtype(x, cfg: moe_cfg) -> int:
    """dtype code of the activations x, which must be a contiguous [S, hidden] fp32 or bf16 tensor."""
    import torch
    if x.dim() != 2 or x.shape[1] != cfg.hidden or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous [S, {cfg.hidden}] tensor, not {tuple(x.shape)} "
                         f"with strides {tuple(x.stride())}")
    if x.dtype == torch.float32:
        return MOE_F32
    if x.dtype == torch.bfloat16:
        return MOE_BF16
    raise ValueError(f"x must be float32 or bfloat16, not {x.dtype}")


def _check_routing(idx, w, S: int, cfg: moe_cfg) -> None:
    import torch
    for name, t, dtype in (("idx", idx, torch.int32), ("w", w, torch.float32)):
        if tuple(t.shape) != (S, cfg.top_k) or t.dtype != dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [{S}, {cfg.top_k}] {dtype} tensor")


def route(x, W, bias, cfg: moe_cfg, ws=None, stream=None):
    """(idx [S, k] int32, w [S, k] fp32) for the tokens x ([S, H] fp32 or bf16 device tensor): moe_route with
    its outputs (and, when ws is None, an initialised workspace) allocated on x's device."""
    import torch
    dt = _x_dtype(x, cfg)
    S = x.shape[0]
    ws = workspace(cfg, S, device=x.device, stream=stream) if ws is None else ws
    idx = torch.empty((S, cfg.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((S, cfg.top_k), dtype=torch.float32, device=x.device)
    moe_route(cfg, x, dt, S, W, bias, idx, w, ws, ws.numel(), stream)
    return idx, w


def ffn(x, idx, w, view: moe_slot_view, shared, cfg: moe_cfg, ws=None, stream=None):
    """y [S, H] fp32: moe_ffn with its output (and, when ws is None, a workspace) allocated on x's device."""
    import torch
    dt = _x_dtype(x, cfg)
    S = x.shape[0]
    _check_routing(idx, w, S, cfg)
    ws = workspace(cfg, S, device=x.device, stream=stream) if ws is None else ws
    y = torch.empty((S, cfg.hidden), dtype=torch.float32, device=x.device)
    moe_ffn(cfg, x, dt, S, idx, w, view, shared, y, ws, ws.numel(), stream)
    return y


def layer(x, W, bias, view: moe_slot_view, shared, cfg: moe_cfg, ws=None, stream=None):
    """(idx, w, y): moe_layer with its outputs (and, when ws is None, a workspace) allocated on x's device."""
    import torch
    dt = _x_dtype(x, cfg)
    S = x.shape[0]
    ws = workspace(cfg, S, device=x.device, stream=stream) if ws is None else ws
    idx = torch.empty((S, cfg.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((S, cfg.top_k), dtype=torch.float32, device=x.device)
    y = torch.empty((S, cfg.hidden), dtype=torch.float32, device=x.device)
    moe_layer(cfg, x, dt, S, W, bias, idx, w, view, shared, y, ws, ws.numel(), stream)
    return idx, w, y


def layer_call(cfg: moe_cfg, x, x_dtype: int, S: int, W, bias, idx, w, view: moe_slot_view, shared, y, ws,
               ws_bytes: int) -> moe_layer_call:
    """The arguments of one moe_layer call, for moe_chain_create (raw addresses; the struct keeps
    references to the cfg and view it points to)."""
    return moe_layer_call(ctypes.pointer(cfg), ptr(x), x_dtype, S, ptr(W), ptr(bias), ptr(idx), ptr(w),
                          ctypes.pointer(view), ptr(shared), ptr(y), ptr(ws), ws_bytes)


def moe_chain_create(calls) -> int:
    """Records the moe_layer calls (a sequence of layer_call results) as one graph; returns the chain handle."""
    arr = (moe_layer_call * len(calls))(*calls) if len(calls) else None
    out = ctypes.c_void_p()
    _check(_lib.moe_chain_create(arr, len(calls), ctypes.byref(out)), "moe_chain_create")
    return out.value


def moe_chain_launch(chain: int, stream=None) -> None:
    _check(_lib.moe_chain_launch(chain, stream_handle(stream)), "moe_chain_launch")


def moe_chain_destroy(chain: int | None) -> None:
    _lib.moe_chain_destroy(chain)


def moe_profile_enable(on: bool) -> None:
    _check(_lib.moe_profile_enable(int(on)), "moe_profile_enable")


def moe_profile_report() -> dict:
    """{kernel: (total_ms, launches)} since the last report."""
    import json
    buf = ctypes.create_string_buffer(1 << 16)
    _check(_lib.moe_profile_report(buf, len(buf)), "moe_profile_report")
    return {k: (v[0], v[1]) for k, v in json.loads(buf.value.decode()).items()}


MOE_POOL_NO_DEVICE, MOE_POOL_POISON = 1, 2


class Pool:
    """Owner of a moe_pool handle (the C calls, with errors raised as MoeError)."""

    def __init__(self, cfg: moe_cfg, n_layers: int, slots_per_layer: int, flags: int = 0):
        self.h = ctypes.c_void_p()
        self._src = {}  # (layer, expert) -> registered host buffer, kept alive while the pool may copy from it
        _check(_lib.moe_pool_create(ctypes.byref(cfg), n_layers, slots_per_layer, flags, ctypes.byref(self.h)),
               "moe_pool_create")

    def register_host(self, layer: int, expert: int, src) -> None:
        _check(_lib.moe_pool_register_host(self.h, layer, expert, ptr(src)), "moe_pool_register_host")
        self._src[(layer, expert)] = src

    def acquire(self, layer: int, idx_host, compute=None, side=None):
        """-> (moe_slot_view, n_miss); idx_host: int32 numpy array."""
        import numpy as np
        idx = np.ascontiguousarray(idx_host, np.int32).ravel()
        view = moe_slot_view()
        n_miss = ctypes.c_int32(0)
        c = stream_handle(compute) if compute is not None or side is not None else None
        s_ = stream_handle(side) if side is not None else c
        _check(_lib.moe_pool_acquire(self.h, layer, idx.ctypes.data, idx.size, ctypes.byref(view), ctypes.byref(n_miss),
                                     c, s_), "moe_pool_acquire")
        return view, n_miss.value

    def prefetch(self, layer: int, idx_host, side=None) -> int:
        """Predicted routing idx_host (int32 numpy array) of `layer`; -> copies enqueued."""
        import numpy as np
        idx = np.ascontiguousarray(idx_host, np.int32).ravel()
        n_fill = ctypes.c_int32(0)
        _check(_lib.moe_pool_prefetch(self.h, layer, idx.ctypes.data, idx.size, ctypes.byref(n_fill),
                                      stream_handle(side) if side is not None else None), "moe_pool_prefetch")
        return n_fill.value

    def release(self, layer: int, compute=None) -> None:
        c = stream_handle(compute) if compute is not None else None
        _check(_lib.moe_pool_release(self.h, layer, c), "moe_pool_release")

    def trace(self):
        import numpy as np
        out = np.zeros(3 * 4096, np.int32)
        n = _lib.moe_pool_trace(self.h, out.ctypes.data, out.size)
        if n < 0:
            raise MoeError(n, "moe_pool_trace")
        return [tuple(out[3 * i:3 * i + 3]) for i in range(n)]

    def stats(self) -> dict:
        import json
        buf = ctypes.create_string_buffer(1024)
        _check(_lib.moe_pool_stats(self.h, buf, len(buf)), "moe_pool_stats")
        return json.loads(buf.value.decode())

    def check_view(self, layer: int, view: moe_slot_view) -> int:
        """moe_pool_check_view: MOE_OK or MOE_ESTALE (other statuses raise)."""
        rc = _lib.moe_pool_check_view(self.h, layer, ctypes.byref(view))
        if rc not in (MOE_OK, MOE_ESTALE):
            raise MoeError(rc, "moe_pool_check_view")
        return rc

    def close(self) -> None:
        if self.h:
            _lib.moe_pool_destroy(self.h)
            self.h = ctypes.c_void_p()
        self._src = {}

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def slot_view(base, slot_bytes: int, table, n_slots: int, gen=None, slot_gen=None) -> moe_slot_view:
    """A view of caller-owned slots (generation tags optional: gen [E] and slot_gen [n_slots] uint32).
    The view stores raw addresses; it also holds references to the objects given, so that
    a table built inline is not freed (and its memory reused) while the view is alive."""
    v = moe_slot_view(ptr(base), slot_bytes, ptr(table), n_slots, ptr(gen), ptr(slot_gen), 0)
    v._refs = (base, table, gen, slot_gen)
    return v
