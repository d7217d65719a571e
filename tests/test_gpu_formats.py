"""Row-scaled weight formats on the GPU, through the C ABI, against the fp64
oracle: int4 with one fp32 scale per row (the production container's format)
and signed int8 with one fp32 scale per row (the MTP layer's experts).  Same
bars as the grouped format: indices exact, outputs within 2e-3 on the exact
path and 1e-2 on the bf16 matrix-core path (max relative error per token)."""
import numpy as np
import pytest
import torch

from gen import inputs as gen
from int4_routed_expert_amd import moe as M
from tests.devlayer import DeviceLayer, tile_cover, x_device
from tests.test_gpu_parity import MID, TOL_BF16, TOL_FP32, check_ffn, check_route, run_gpu, say

pytestmark = pytest.mark.gpu

FORMATS = {"q4row": M.MOE_WF_Q4_ROW, "q8row": M.MOE_WF_Q8_ROW}


def fmt_workload(w: gen.Workload, fmt: int) -> gen.Workload:
    return w.with_(cfg=gen.LayerConfig(**{**w.cfg.__dict__, "weight_format": fmt}))


@pytest.fixture(scope="module", params=list(FORMATS))
def tiny_f(request):
    return DeviceLayer(fmt_workload(gen.WORKLOADS["tiny"], FORMATS[request.param]), host_experts=True,
                       mfma_min_tokens=0)


@pytest.fixture(scope="module", params=list(FORMATS))
def mid_f(request):
    w = gen.Workload("mid", MID, tokens=67, seed=11)
    return DeviceLayer(fmt_workload(w, FORMATS[request.param]), host_experts=True, mfma_min_tokens=0)


def test_device_pack_equals_host_pack(tiny_f):
    c = tiny_f.cfg
    for e in (0, 7, 15):
        ex = tiny_f.host_expert(e)
        host = np.zeros(tiny_f.slot_bytes, np.uint8)
        M.moe_pack_expert_rows(c, 128, *ex.parts(), host, 0)
        devb = tiny_f.slab[e * tiny_f.slot_bytes:(e + 1) * tiny_f.slot_bytes].cpu().numpy()
        used = M.moe_expert_bytes(c, 128)
        assert np.array_equal(host[:used], devb[:used])


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 37])
def test_tiny_layer(tiny_f, S):
    w = tiny_f.w.with_(tokens=S)
    x = gen.tokens(w, step=S)
    idx, wt, y = run_gpu(tiny_f, x)
    ridx, rw = check_route(tiny_f, x, idx, wt)
    check_ffn(tiny_f, x, ridx, rw, y, np.arange(S), TOL_FP32)


@pytest.mark.parametrize("S", [1, 4, 67])
def test_mid_layer(mid_f, S):
    x = gen.tokens(mid_f.w.with_(tokens=S), step=100 + S)
    idx, wt, y = run_gpu(mid_f, x)
    ridx, rw = check_route(mid_f, x, idx, wt)
    check_ffn(mid_f, x, ridx, rw, y, np.arange(S), TOL_FP32)


def matrix_core_case(dl, S, thr):
    """Experts over the threshold run the bf16 grouped GEMM on the format's
    dequantised weights: within the bf16 bar, and different from the exact path."""
    w = dl.w.with_(tokens=S)
    x = gen.tokens(w, step=900 + S)
    xt, dt = x_device(w, x)
    idx, wt = dl.route(xt, dt)
    y_mfma = dl.ffn(xt, dt, idx, wt, mfma_min_tokens=thr).cpu().numpy()
    y_exact = dl.ffn(xt, dt, idx, wt, mfma_min_tokens=0).cpu().numpy()
    ridx, rw = check_route(dl, x, idx.cpu().numpy(), wt.cpu().numpy())
    assert (np.bincount(ridx.ravel(), minlength=dl.c.n_experts) >= thr).any()
    check_ffn(dl, x, ridx, rw, y_mfma, np.arange(S), TOL_BF16, mfma_min_tokens=thr)
    check_ffn(dl, x, ridx, rw, y_exact, np.arange(S), TOL_FP32)
    assert not np.array_equal(y_mfma, y_exact)


def test_matrix_core_path_tiny(tiny_f):
    matrix_core_case(tiny_f, 37, 4)


@pytest.mark.parametrize("S,thr", [(67, 4), (300, 16)])
def test_matrix_core_path_mid(mid_f, S, thr):
    matrix_core_case(mid_f, S, thr)


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_matrix_core_odd_group_count(fmt):
    """H = 544 (17 groups), I = 96 (3 groups), shared 64, bf16 input: the bf16
    grouped GEMM skips the group past the end of each row's last stage."""
    from tests.test_gpu_parity import RAGGED
    w = fmt_workload(gen.Workload("ragged", RAGGED, tokens=40, seed=31, x_dtype="bf16"), FORMATS[fmt])
    dl = DeviceLayer(w, host_experts=True, mfma_min_tokens=0)
    matrix_core_case(dl, 40, 2)


@pytest.mark.parametrize("S", [1, 3, 8])
def test_unresident_slot_poisons_only_its_tokens(tiny_f, S):
    w = tiny_f.w.with_(tokens=S)
    x = gen.tokens(w, step=77 + S)
    xt, dt = x_device(w, x)
    idx, wt = tiny_f.route(xt, dt)
    ih = idx.cpu().numpy()
    victim = int(ih[0, 0])
    table = tiny_f.table.clone()
    table[victim] = -1
    y = tiny_f.ffn(xt, dt, idx, wt, table=table).cpu().numpy()
    hit = (ih == victim).any(axis=1)
    assert np.isnan(y[hit]).all(axis=1).all() and np.isfinite(y[~hit]).all()


def test_layer_call_matches_route_then_ffn(tiny_f):
    x = gen.tokens(tiny_f.w, step=5)
    xt, dt = x_device(tiny_f.w, x)
    idx, wt, y = tiny_f.layer(xt, dt)
    idx2, wt2 = tiny_f.route(xt, dt)
    y2 = tiny_f.ffn(xt, dt, idx2, wt2)
    assert torch.equal(idx, idx2) and torch.equal(wt, wt2) and torch.equal(y, y2)


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_glm_shape_decode_verify_prefill(fmt):
    """GLM-5.2 shape (256 routed experts of 6144 x 2048 and the shared expert):
    decode (moe_layer, one token), a verify batch of 4 and a 2048-token bf16
    batch (outputs on one token of every matrix-core tile and GEMV item), all
    with the same experts and router."""
    say(f"packing 257 GLM-5.2-shaped experts in format {fmt}")
    dl = DeviceLayer(fmt_workload(gen.WORKLOADS["decode"], FORMATS[fmt]))
    for step in range(3):
        x = gen.tokens(dl.w, step=step)
        xt, dt = x_device(dl.w, x)
        idx, wt, y = dl.layer(xt, dt)
        ridx, rw = check_route(dl, x, idx.cpu().numpy(), wt.cpu().numpy())
        check_ffn(dl, x, ridx, rw, y.cpu().numpy(), np.arange(1), TOL_FP32)
    x = gen.tokens(dl.w.with_(tokens=4), step=50)  # a verify batch
    idx, wt, y = run_gpu(dl, x)
    ridx, rw = check_route(dl, x, idx, wt)
    check_ffn(dl, x, ridx, rw, y, np.arange(4), TOL_FP32)
    dl.w = dl.w.with_(x_dtype="bf16", tokens=2048)  # same seed: the same experts and router
    x = gen.tokens(dl.w)
    idx, wt, y = run_gpu(dl, x)
    ridx, rw = check_route(dl, x, idx, wt)
    counts = np.bincount(ridx.ravel(), minlength=dl.c.n_experts)
    say(f"prefill: experts with >= 16 tokens {(counts >= 16).sum()}")
    tokens = np.union1d(tile_cover(ridx, dl.c.n_experts, dl.cfg.mfma_min_tokens), [0, 2047])
    check_ffn(dl, x, ridx, rw, y, tokens, TOL_BF16, mfma_min_tokens=dl.cfg.mfma_min_tokens)
    assert np.isfinite(y).all()
