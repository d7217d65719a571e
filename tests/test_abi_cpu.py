"""C ABI checks that need no GPU: the library loads and exports every declared
symbol, configurations are validated, sizes are as documented, the host packer
round-trips and lays bytes out as documented, and argument errors return the
documented codes before anything is enqueued."""
import ctypes
import os

import numpy as np
import pytest

from gen import inputs as gen
from int4_routed_expert_amd import moe as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    names = M.header_functions()
    assert {"moe_route", "moe_ffn", "moe_pack_expert", "moe_workspace_bytes", "moe_expert_bytes"} <= set(names)
    for n in names:
        assert hasattr(M.lib(), n), n
        assert callable(getattr(M, n, None) or getattr(M.lib(), n))


def test_validate_cfg():
    assert M.moe_validate_cfg(M.make_cfg(gen.GLM52)) == M.MOE_OK
    assert M.moe_validate_cfg(M.make_cfg(gen.TINY)) == M.MOE_OK
    bad = [
        dict(hidden=100), dict(hidden=0), dict(hidden=8224), dict(moe_inter=48), dict(shared_inter=16),
        dict(n_group=3), dict(topk_group=9), dict(topk_group=0), dict(top_k=0), dict(top_k=17),
        dict(n_experts=2048, n_group=8), dict(group_size=64), dict(norm_topk_prob=2),
        dict(n_experts=16, n_group=4, topk_group=1, top_k=5),
    ]
    for b in bad:
        c = gen.LayerConfig(**{**gen.GLM52.__dict__, **b})
        assert M.moe_validate_cfg(M.make_cfg(c)) == M.MOE_EINVAL, b
    c = M.make_cfg(gen.GLM52)
    c.routed_scaling_factor = float("nan")
    assert M.moe_validate_cfg(c) == M.MOE_EINVAL
    assert M.lib().moe_validate_cfg(None) == M.MOE_ENULL
    ok_no_shared = gen.LayerConfig(**{**gen.GLM52.__dict__, "shared_inter": 0})
    assert M.moe_validate_cfg(M.make_cfg(ok_no_shared)) == M.MOE_OK


def test_expert_bytes_glm_shape():
    # 3 * 6144 * 2048 nibbles (18,874,368 B) + fp16 scale per 32 (2,359,296 B)
    c = M.make_cfg(gen.GLM52)
    assert M.moe_expert_bytes(c, 2048) == 21_233_664
    assert M.moe_expert_bytes(c, 48) == M.MOE_EINVAL
    t = M.make_cfg(gen.TINY)
    payload = 3 * 256 * 128 // 2 + 3 * 256 * 128 // 32 * 2
    assert M.moe_expert_bytes(t, 128) == (payload + 4095) // 4096 * 4096


def test_workspace_sizes():
    c = M.make_cfg(gen.GLM52)
    sizes = [M.moe_workspace_bytes(c, s) for s in (0, 1, 4, 5, 64, 2048)]
    assert all(s >= 256 and s % 256 == 0 for s in sizes)
    assert sizes == sorted(sizes)
    bad = M.make_cfg(gen.GLM52)
    bad.hidden = 100
    assert M.moe_workspace_bytes(bad, 4) == 0


def _expert_host(shape_cfg, inter, seed=0):
    w = gen.Workload("t", shape_cfg, tokens=1, seed=seed)
    e = shape_cfg.n_experts if inter == shape_cfg.shared_inter and inter != shape_cfg.moe_inter else 1
    return gen.expert_weights(w, 0, e)


@pytest.mark.parametrize("shape", [gen.TINY, gen.LayerConfig(hidden=96, n_experts=4, n_group=2, topk_group=1,
                                                                 top_k=2, moe_inter=64, shared_inter=32)])
def test_host_pack_round_trip_and_layout(shape):
    c = M.make_cfg(shape)
    ex = _expert_host(shape, shape.moe_inter)
    nb = M.moe_expert_bytes(c, shape.moe_inter)
    dst = np.full(nb, 0xAB, np.uint8)
    M.moe_pack_expert(c, shape.moe_inter, *ex.parts(), dst, 0)
    out = gen.empty_expert(shape, shape.moe_inter)
    M.moe_unpack_expert(c, shape.moe_inter, dst, *out.parts())
    for a, b in zip(ex.parts(), out.parts()):
        assert np.array_equal(a, b)
    # documented layout, re-derived: gate/up tiles of 8 rows (g r, u r for 4 r), then scales [group][8];
    # nibbles hold the int4 value in two's complement (interchange nibble with its top bit flipped)
    H, I = shape.hidden, shape.moe_inter
    tw = lambda q: q ^ np.uint8(0x88)
    tile = 8 * (H // 2) + (H // 32) * 8 * 2
    for t in range(I // 4):
        base = t * tile
        for i in range(8):
            src = ex.qu if i % 2 else ex.qg
            r = 4 * t + i // 2
            assert np.array_equal(dst[base + i * (H // 2): base + (i + 1) * (H // 2)], tw(src[r]))
        scl = dst[base + 8 * (H // 2): base + tile].view(np.uint16).reshape(H // 32, 8)
        for i in range(8):
            s = ex.su if i % 2 else ex.sg
            assert np.array_equal(scl[:, i], s[4 * t + i // 2])
    dtile = 8 * (I // 2) + (I // 32) * 8 * 2
    d0 = (I // 4) * tile
    for t in range(H // 8):
        base = d0 + t * dtile
        for i in range(8):
            assert np.array_equal(dst[base + i * (I // 2): base + (i + 1) * (I // 2)], tw(ex.qd[8 * t + i]))
        scl = dst[base + 8 * (I // 2): base + dtile].view(np.uint16).reshape(I // 32, 8)
        assert np.array_equal(scl.T, ex.sd[8 * t: 8 * t + 8])
    assert np.all(dst[d0 + (H // 8) * dtile:] == 0)


def test_expert_bytes_row_formats():
    # int4 nibbles or int8 bytes of the three matrices plus one fp32 scale per row
    # (tiles of 8 rows carry 32 B of scales); 40,960 B of scales for GLM-5.2
    for fmt, per_w in ((M.MOE_WF_Q4_ROW, 0.5), (M.MOE_WF_Q8_ROW, 1.0)):
        c = M.make_cfg(gen.LayerConfig(**{**gen.GLM52.__dict__, "weight_format": fmt}))
        payload = int(3 * 6144 * 2048 * per_w) + (2048 // 4 + 6144 // 8) * 32
        assert M.moe_expert_bytes(c, 2048) == (payload + 4095) // 4096 * 4096
    assert M.moe_expert_bytes(M.make_cfg(gen.LayerConfig(**{**gen.GLM52.__dict__, "weight_format": 1})),
                              2048) == 18_915_328
    bad = M.make_cfg(gen.GLM52)
    bad.weight_format = 3
    assert M.moe_validate_cfg(bad) == M.MOE_EINVAL


def test_int8_activation_flag_and_workspace():
    c = M.make_cfg(gen.GLM52, act_int8=1)
    assert M.moe_validate_cfg(c) == M.MOE_OK
    for v in (2, -1):
        c.act_int8 = v
        assert M.moe_validate_cfg(c) == M.MOE_EINVAL
    # the quantised rows (S*H + S*(k+1)*Imax bytes) and their scales come on top of the exact-mode workspace
    for S in (1, 4, 2048):
        extra = M.moe_workspace_bytes(M.make_cfg(gen.GLM52, act_int8=1), S) - M.moe_workspace_bytes(M.make_cfg(gen.GLM52), S)
        assert extra >= S * 6144 + S * 9 * 2048 + S * 4 + S * 9 * 4


@pytest.mark.parametrize("fmt", [M.MOE_WF_Q4_ROW, M.MOE_WF_Q8_ROW])
@pytest.mark.parametrize("base", [gen.TINY, gen.LayerConfig(hidden=96, n_experts=4, n_group=2, topk_group=1,
                                                                top_k=2, moe_inter=64, shared_inter=32)])
def test_host_pack_rows_round_trip_and_layout(fmt, base):
    shape = gen.LayerConfig(**{**base.__dict__, "weight_format": fmt})
    c = M.make_cfg(shape)
    ex = _expert_host(shape, shape.moe_inter)
    nb = M.moe_expert_bytes(c, shape.moe_inter)
    dst = np.full(nb, 0xAB, np.uint8)
    M.moe_pack_expert_rows(c, shape.moe_inter, *ex.parts(), dst, 0)
    out = gen.empty_expert(shape, shape.moe_inter)
    M.moe_unpack_expert_rows(c, shape.moe_inter, dst, *out.parts())
    for a, b in zip(ex.parts(), out.parts()):
        assert np.array_equal(a, b)
    # documented layout, re-derived: 8 rows per tile (gate/up interleaved), then 8 fp32 scales
    H, I = shape.hidden, shape.moe_inter
    rb = (lambda K: K) if fmt == M.MOE_WF_Q8_ROW else (lambda K: K // 2)
    conv = (lambda q: q.view(np.uint8)) if fmt == M.MOE_WF_Q8_ROW else (lambda q: q ^ np.uint8(0x88))
    tile = 8 * rb(H) + 32
    for t in range(I // 4):
        base_ = t * tile
        for i in range(8):
            src = ex.qu if i % 2 else ex.qg
            assert np.array_equal(dst[base_ + i * rb(H): base_ + (i + 1) * rb(H)], conv(src[4 * t + i // 2]))
        scl = dst[base_ + 8 * rb(H): base_ + tile].view(np.float32)
        assert np.array_equal(scl[0::2], ex.sg[4 * t: 4 * t + 4]) and np.array_equal(scl[1::2], ex.su[4 * t: 4 * t + 4])
    dtile = 8 * rb(I) + 32
    d0 = (I // 4) * tile
    for t in range(H // 8):
        base_ = d0 + t * dtile
        for i in range(8):
            assert np.array_equal(dst[base_ + i * rb(I): base_ + (i + 1) * rb(I)], conv(ex.qd[8 * t + i]))
        assert np.array_equal(dst[base_ + 8 * rb(I): base_ + dtile].view(np.float32), ex.sd[8 * t: 8 * t + 8])
    assert np.all(dst[d0 + (H // 8) * dtile:] == 0)


def test_pack_entry_points_reject_the_other_formats():
    L = M.lib()
    g = M.make_cfg(gen.TINY)
    r = M.make_cfg(gen.LayerConfig(**{**gen.TINY.__dict__, "weight_format": 1}))
    exg, exr = _expert_host(gen.TINY, 128), _expert_host(gen.LayerConfig(**{**gen.TINY.__dict__, "weight_format": 1}), 128)
    dst = np.zeros(max(M.moe_expert_bytes(g, 128), M.moe_expert_bytes(r, 128)), np.uint8)
    pg = [M.ptr(a) for a in exg.parts()]
    pr = [M.ptr(a) for a in exr.parts()]
    assert L.moe_pack_expert(ctypes.byref(r), 128, *pg, M.ptr(dst), 0, None) == M.MOE_EINVAL
    assert L.moe_pack_expert_rows(ctypes.byref(g), 128, *pr, M.ptr(dst), 0, None) == M.MOE_EINVAL
    assert L.moe_unpack_expert(ctypes.byref(r), 128, M.ptr(dst), *pg) == M.MOE_EINVAL
    assert L.moe_unpack_expert_rows(ctypes.byref(g), 128, M.ptr(dst), *pr) == M.MOE_EINVAL
    assert L.moe_pack_expert_rows(ctypes.byref(r), 128, *pr[:5], None, M.ptr(dst), 0, None) == M.MOE_ENULL


def test_pack_argument_errors():
    c = M.make_cfg(gen.TINY)
    ex = _expert_host(gen.TINY, 128)
    dst = np.zeros(M.moe_expert_bytes(c, 128), np.uint8)
    L = M.lib()
    p = [M.ptr(a) for a in ex.parts()]
    assert L.moe_pack_expert(ctypes.byref(c), 128, *p, None, 0, None) == M.MOE_ENULL
    assert L.moe_pack_expert(ctypes.byref(c), 128, None, *p[1:], M.ptr(dst), 0, None) == M.MOE_ENULL
    assert L.moe_pack_expert(ctypes.byref(c), 100, *p, M.ptr(dst), 0, None) == M.MOE_EINVAL
    assert L.moe_pack_expert(ctypes.byref(c), 128, *p, M.ptr(dst), 2, None) == M.MOE_EINVAL


def test_route_and_ffn_argument_errors_before_any_launch():
    """These return before touching the GPU, so they run without one."""
    c = M.make_cfg(gen.TINY)
    L = M.lib()
    fake = ctypes.c_void_p(4096)  # never dereferenced: every call below fails validation first
    ws_need = M.moe_workspace_bytes(c, 4)
    R = lambda **kw: L.moe_route(ctypes.byref(kw.get("cfg", c)), kw.get("x", fake), kw.get("dt", M.MOE_F32),
                                 kw.get("S", 4), kw.get("W", fake), kw.get("b", fake), kw.get("idx", fake),
                                 kw.get("w", fake), kw.get("ws", fake), kw.get("wsb", ws_need), None)
    assert R(x=None) == M.MOE_ENULL
    assert R(W=None) == M.MOE_ENULL
    assert R(dt=7) == M.MOE_EDTYPE
    assert R(wsb=ws_need - 1) == M.MOE_EWORKSPACE
    assert R(S=-1) == M.MOE_EINVAL
    assert R(S=0, x=None) == M.MOE_OK  # empty batch: a no-op
    bad = M.make_cfg(gen.TINY)
    bad.n_group = 3
    assert R(cfg=bad) == M.MOE_EINVAL

    sb = M.moe_expert_bytes(c, 128)
    view = M.moe_slot_view(4096, sb, 4096, 16)
    F = lambda **kw: L.moe_ffn(ctypes.byref(kw.get("cfg", c)), kw.get("x", fake), kw.get("dt", M.MOE_F32),
                               kw.get("S", 4), kw.get("idx", fake), kw.get("w", fake),
                               ctypes.byref(kw.get("view", view)), kw.get("shared", fake), kw.get("y", fake),
                               kw.get("ws", fake), kw.get("wsb", ws_need), None)
    assert F(shared=None) == M.MOE_ENULL
    assert F(y=None) == M.MOE_ENULL
    assert F(dt=-1) == M.MOE_EDTYPE
    assert F(wsb=10) == M.MOE_EWORKSPACE
    assert F(view=M.moe_slot_view(4096, sb - 256, 4096, 16)) == M.MOE_EINVAL
    assert F(view=M.moe_slot_view(4096, sb + 1, 4096, 16)) == M.MOE_EINVAL
    assert F(view=M.moe_slot_view(4096, sb, 4096, 0)) == M.MOE_EINVAL
    assert F(view=M.moe_slot_view(None, sb, 4096, 16)) == M.MOE_ENULL
    assert F(S=0, x=None) == M.MOE_OK
    noshared = M.make_cfg(gen.TINY)
    noshared.shared_inter = 0
    # without a shared expert a NULL shared pointer is fine; validation then passes and the call
    # would launch, so only check that the NULL-shared rule is not applied (use a bad workspace)
    assert F(cfg=noshared, shared=None, wsb=10) == M.MOE_EWORKSPACE


def test_chain_argument_errors_before_any_recording():
    """moe_chain_create checks every call before it records anything, so its errors need no GPU;
    on any error the out handle is NULL."""
    c = M.make_cfg(gen.TINY)
    L = M.lib()
    fake = 4096  # never dereferenced: every call below fails validation first
    ws_need = M.moe_workspace_bytes(c, 1)
    view = M.moe_slot_view(4096, M.moe_expert_bytes(c, 128), 4096, 16)

    def call(**kw):
        a = dict(cfg=c, x=fake, x_dtype=M.MOE_F32, S=1, W=fake, bias=fake, idx=fake, w=fake, view=view,
                 shared=fake, y=fake, ws=fake, ws_bytes=ws_need)
        a.update(kw)
        return M.layer_call(a["cfg"], a["x"], a["x_dtype"], a["S"], a["W"], a["bias"], a["idx"], a["w"], a["view"],
                            a["shared"], a["y"], a["ws"], a["ws_bytes"])

    def create(calls, n=None):
        arr = (M.moe_layer_call * len(calls))(*calls) if calls else None
        out = ctypes.c_void_p(1234)
        rc = L.moe_chain_create(arr, len(calls) if n is None else n, ctypes.byref(out))
        assert out.value is None, "the handle must be NULL after an error"
        return rc

    assert create([]) == M.MOE_EINVAL
    assert create([call()], n=0) == M.MOE_EINVAL
    assert L.moe_chain_create(None, 1, ctypes.byref(ctypes.c_void_p())) == M.MOE_ENULL
    assert L.moe_chain_create((M.moe_layer_call * 1)(call()), 1, None) == M.MOE_ENULL
    nocfg = call()
    nocfg.cfg = ctypes.POINTER(M.moe_cfg)()
    assert create([nocfg]) == M.MOE_ENULL
    bad = M.make_cfg(gen.TINY)
    bad.n_group = 3
    assert create([call(cfg=bad)]) == M.MOE_EINVAL
    # the first failing call's status is returned, whichever position it has
    assert create([call(y=None), call(x_dtype=9)]) == M.MOE_ENULL
    assert create([call(x_dtype=9), call(y=None)]) == M.MOE_EDTYPE
    assert create([call(S=4, x=None, ws_bytes=ws_need)]) == M.MOE_ENULL
    assert create([call(S=4, ws_bytes=ws_need)]) == M.MOE_EWORKSPACE
    assert create([call(), call(S=-2)]) == M.MOE_EINVAL
    assert L.moe_chain_launch(None, None) == M.MOE_ENULL
    M.moe_chain_destroy(None)  # a no-op


def test_status_strings():
    for s in range(0, -8, -1):
        assert M.lib().moe_status_string(s)
    assert M.lib().moe_status_string(-99) == b"unknown status"


def test_library_shares_torchs_hip_runtime():
    """Importing the binding first must still leave one HIP runtime in the process
    (the library binds to the copy torch loads; a second copy sees no device)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from int4_routed_expert_amd import moe\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "print(sorted({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    import ast
    libs = ast.literal_eval(out.stdout.strip().splitlines()[-1])
    assert len(libs) == 1, libs


def test_slot_view_keeps_its_tensors_alive():
    """A view holds references to the tensors whose addresses it stores: a table
    built inline stays allocated (its address unchanged) while the view lives."""
    import gc
    import torch
    base = torch.zeros(64, dtype=torch.uint8)
    v = M.slot_view(base, 16, torch.arange(4, dtype=torch.int32), 4)
    gc.collect()
    table = v._refs[1]
    assert v.table == table.data_ptr() and v.base == base.data_ptr() and v.n_slots == 4
    assert table.tolist() == [0, 1, 2, 3]


def test_header_is_c11_and_links_from_c(tmp_path):
    """include/moe.h compiles as strict C11 (-pedantic, warnings as errors) and a C
    program links against libmoe.so and calls its host entry points."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib_dir = os.path.join(root, "int4_routed_expert_amd")
    src = tmp_path / "abi_check.c"
    src.write_text(r"""
#include <stdio.h>
#include "moe.h"
int main(void) {
  moe_cfg c = {0};
  c.hidden = 6144; c.n_experts = 256; c.n_group = 8; c.topk_group = 4; c.top_k = 8;
  c.moe_inter = 2048; c.shared_inter = 2048; c.group_size = 32; c.routed_scaling_factor = 2.5f;
  c.norm_topk_prob = 1; c.mfma_min_tokens = 3; c.weight_format = MOE_WF_Q4_G32; c.act_int8 = 0;
  printf("%d %lld\n", moe_validate_cfg(&c), (long long)moe_expert_bytes(&c, 2048));
  c.top_k = 99;
  printf("%d %s\n", moe_validate_cfg(&c), moe_status_string(moe_validate_cfg(&c)));
  return 0;
}
""")
    exe = tmp_path / "abi_check"
    subprocess.check_call([gcc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(root, "include"),
                           str(src), "-L", lib_dir, "-lmoe", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60, check=True).stdout.split("\n")
    assert out[0] == "0 21233664"
    assert out[1].startswith(f"{M.MOE_EINVAL} ")


def test_allocating_calls_check_shapes_first():
    """M.route / M.ffn / M.layer refuse activations of the wrong dtype, width or layout, and routing tensors of
    the wrong shape, before anything is allocated or launched (so these run without a GPU)."""
    import torch
    c = M.make_cfg(gen.TINY)
    H, k = c.hidden, c.top_k
    view = M.moe_slot_view(4096, M.moe_expert_bytes(c, 128), 4096, 16)
    bad_x = [torch.zeros((2, H), dtype=torch.float64), torch.zeros((2, H - 32)), torch.zeros((2, 2 * H))[:, ::2],
             torch.zeros((H, 1)).t().t(), torch.zeros((1, H)).t(), torch.zeros(H)]
    for x in bad_x:
        with pytest.raises(ValueError):
            M.route(x, None, None, c)
        with pytest.raises(ValueError):
            M.layer(x, None, None, view, None, c)
    x = torch.zeros((2, H))
    for idx, w in [(torch.zeros((2, k + 1), dtype=torch.int32), torch.zeros((2, k))),
                   (torch.zeros((2, k), dtype=torch.int64), torch.zeros((2, k))),
                   (torch.zeros((2, k), dtype=torch.int32), torch.zeros((3, k)))]:
        with pytest.raises(ValueError):
            M.ffn(x, idx, w, view, None, c)
