"""int8-activation mode (moe_cfg.act_int8 = 1) on the GPU, through the C ABI,
against the oracle's int8-activation mode: each token's x and each expert's
hidden row h are quantised per row (d = amax / 127, q = rint(v / d)) before their
matmuls.  The quantisation of x is decided in fp32 on both sides, so it agrees
exactly; h is the GPU's fp32 result, which differs from the oracle's fp64 h
rounded to fp32 by a few ulps, so an element of h that sits on a rounding tie of
the int8 grid may land one step apart (a change of about d_h * |w| in the
affected outputs: up to about d_h * max|Wd| / max|y|, a few 1e-3).  Bar: max
relative error per token 5e-3, and the median over tokens below 1e-5 (the fp32
level of the exact path)."""
import numpy as np
import pytest
import torch

from gen import inputs as gen
from int4_routed_expert_amd import moe as M
from oracle import oracle as O
from tests.devlayer import DeviceLayer, max_rel_err, tile_cover, x_device
from tests.test_gpu_parity import MID, check_route, run_gpu, say

pytestmark = pytest.mark.gpu

TOL_MAX = 5e-3
TOL_MEDIAN = 1e-5


def fmt_workload(w: gen.Workload, fmt: int) -> gen.Workload:
    return w.with_(cfg=gen.LayerConfig(**{**w.cfg.__dict__, "weight_format": fmt}))


def check_int8act(dl: DeviceLayer, x_host, ridx, rw, y, tokens):
    c = dl.c
    need = set(ridx[tokens].ravel().tolist())
    experts = {e: dl.host_expert(e) for e in need}
    if c.shared_inter > 0:
        experts[c.n_experts] = dl.host[c.n_experts]
    bf = dl.w.x_dtype == "bf16"
    xs = np.ascontiguousarray(x_host[tokens])
    ref = O.moe_ffn(c, xs, ridx[tokens], rw[tokens], experts, x_is_bf16=bf, act_int8=True)
    errs = [max_rel_err(y[t:t + 1], ref[i:i + 1]) for i, t in enumerate(tokens)]
    exact = O.moe_ffn(c, xs, ridx[tokens], rw[tokens], experts, x_is_bf16=bf)
    dev_from_exact = max_rel_err(ref, exact)
    say(f"  int8-act: max rel err {max(errs):.3e}, median {np.median(errs):.3e} over {len(tokens)} tokens; "
        f"oracle int8-act vs exact {dev_from_exact:.3e}")
    assert max(errs) <= TOL_MAX and np.median(errs) <= TOL_MEDIAN
    assert dev_from_exact > 10 * TOL_MEDIAN  # the mode really quantises


@pytest.fixture(scope="module", params=[0, 1, 2], ids=["q4g32", "q4row", "q8row"])
def tiny_q(request):
    return DeviceLayer(fmt_workload(gen.WORKLOADS["tiny"], request.param), host_experts=True, mfma_min_tokens=0,
                       act_int8=1)


@pytest.mark.parametrize("S", [1, 2, 4, 5, 37])
def test_tiny_layer(tiny_q, S):
    x = gen.tokens(tiny_q.w.with_(tokens=S), step=300 + S)
    idx, wt, y = run_gpu(tiny_q, x)
    ridx, rw = check_route(tiny_q, x, idx, wt)
    check_int8act(tiny_q, x, ridx, rw, y, np.arange(S))


@pytest.mark.parametrize("fmt", [0, 2], ids=["q4g32", "q8row"])
def test_mid_layer(fmt):
    dl = DeviceLayer(fmt_workload(gen.Workload("mid", MID, tokens=67, seed=11), fmt), host_experts=True, act_int8=1)
    for S in (1, 4, 67):
        x = gen.tokens(dl.w.with_(tokens=S), step=500 + S)
        idx, wt, y = run_gpu(dl, x)
        ridx, rw = check_route(dl, x, idx, wt)
        check_int8act(dl, x, ridx, rw, y, np.arange(S))


def test_layer_call_and_poison(tiny_q):
    x = gen.tokens(tiny_q.w.with_(tokens=3), step=9)
    xt, dt = x_device(tiny_q.w, x)
    idx, wt, y = tiny_q.layer(xt[:1], dt)
    idx2, wt2 = tiny_q.route(xt[:1], dt)
    assert torch.equal(y, tiny_q.ffn(xt[:1], dt, idx2, wt2))
    idx3, wt3 = tiny_q.route(xt, dt)
    ih = idx3.cpu().numpy()
    table = tiny_q.table.clone()
    table[int(ih[0, 0])] = -1
    y3 = tiny_q.ffn(xt, dt, idx3, wt3, table=table).cpu().numpy()
    hit = (ih == ih[0, 0]).any(axis=1)
    assert np.isnan(y3[hit]).all(axis=1).all() and np.isfinite(y3[~hit]).all()


@pytest.mark.parametrize("fmt", [0, 1], ids=["q4g32", "q4row"])
def test_glm_shape_decode_and_verify(fmt):
    say(f"packing 257 GLM-5.2-shaped experts (format {fmt})")
    dl = DeviceLayer(fmt_workload(gen.WORKLOADS["decode"], fmt), act_int8=1)
    for step in range(3):
        x = gen.tokens(dl.w, step=step)
        xt, dt = x_device(dl.w, x)
        idx, wt, y = dl.layer(xt, dt)
        ridx, rw = check_route(dl, x, idx.cpu().numpy(), wt.cpu().numpy())
        check_int8act(dl, x, ridx, rw, y.cpu().numpy(), np.arange(1))
    x = gen.tokens(dl.w.with_(tokens=4), step=60)
    idx, wt, y = run_gpu(dl, x)
    ridx, rw = check_route(dl, x, idx, wt)
    check_int8act(dl, x, ridx, rw, y, np.arange(4))


@pytest.mark.parametrize("fmt", [0, 1, 2], ids=["q4g32", "q4row", "q8row"])
@pytest.mark.parametrize("S,thr", [(37, 4), (67, 4), (300, 16)])
def test_matrix_core_path(fmt, S, thr):
    """int8 activations: experts over the threshold run the matrix cores (row-scaled
    weights: the integer GEMM, exact int32 sums scaled once; fp16 group scales:
    one exact integer group dot per MFMA, scaled per group in fp32), the others
    the GEMV items.  Both against the oracle's int8-activation mode."""
    base = gen.WORKLOADS["tiny"] if S == 37 else gen.Workload("mid", MID, tokens=S, seed=11)
    dl = DeviceLayer(fmt_workload(base, fmt), host_experts=True, mfma_min_tokens=thr, act_int8=1)
    w = dl.w.with_(tokens=S)
    x = gen.tokens(w, step=700 + S)
    xt, dt = x_device(w, x)
    idx, wt = dl.route(xt, dt)
    y_mfma = dl.ffn(xt, dt, idx, wt).cpu().numpy()
    y_gemv = dl.ffn(xt, dt, idx, wt, mfma_min_tokens=0).cpu().numpy()
    ridx, rw = check_route(dl, x, idx.cpu().numpy(), wt.cpu().numpy())
    counts = np.bincount(ridx.ravel(), minlength=dl.c.n_experts)
    say(f"S={S}: {(counts >= thr).sum()} experts at or over {thr} tokens")
    assert (counts >= thr).any()
    check_int8act(dl, x, ridx, rw, y_mfma, np.arange(S))
    check_int8act(dl, x, ridx, rw, y_gemv, np.arange(S))
    assert not np.array_equal(y_mfma, y_gemv)


@pytest.mark.parametrize("fmt", [0, 1, 2], ids=["q4g32", "q4row", "q8row"])
def test_matrix_core_odd_group_count(fmt):
    """H = 544 (17 groups: the integer GEMM's last stage has one live group and
    lanes of the other are masked), I = 96, shared 64, bf16 input."""
    from tests.test_gpu_parity import RAGGED
    w = fmt_workload(gen.Workload("ragged", RAGGED, tokens=40, seed=31, x_dtype="bf16"), fmt)
    dl = DeviceLayer(w, host_experts=True, mfma_min_tokens=2, act_int8=1)
    x = gen.tokens(w, step=41)
    xt, dt = x_device(w, x)
    idx, wt = dl.route(xt, dt)
    y = dl.ffn(xt, dt, idx, wt).cpu().numpy()
    ridx, rw = check_route(dl, x, idx.cpu().numpy(), wt.cpu().numpy())
    assert (np.bincount(ridx.ravel(), minlength=dl.c.n_experts) >= 2).any()
    check_int8act(dl, x, ridx, rw, y, np.arange(40))


@pytest.mark.parametrize("fmt", [1, 0], ids=["q4row", "q4g32"])
def test_glm_shape_batch(fmt):
    """2048 bf16 tokens, GLM-5.2 shape, int8 activations: the matrix-core path for
    the many-token experts (integer tiles for row scales, per-group scaled integer
    group dots for fp16 group scales); outputs on one token of every matrix-core
    tile and GEMV item."""
    w = fmt_workload(gen.WORKLOADS["decode"], fmt).with_(x_dtype="bf16", tokens=2048)
    dl = DeviceLayer(w, act_int8=1)
    x = gen.tokens(w)
    idx, wt, y = run_gpu(dl, x)
    ridx, rw = check_route(dl, x, idx, wt)
    counts = np.bincount(ridx.ravel(), minlength=w.cfg.n_experts)
    say(f"experts with >= 16 tokens: {(counts >= 16).sum()}")
    tokens = np.union1d(tile_cover(ridx, w.cfg.n_experts, dl.cfg.mfma_min_tokens), [0, 2047])
    check_int8act(dl, x, ridx, rw, y, tokens)
    assert np.isfinite(y).all()


@pytest.mark.parametrize("S", [1, 3])
def test_layer_call_graph_replays(tiny_q, S):
    """moe_layer with int8 activations captured in a HIP graph (the quantisation
    kernels included): replays with new inputs, each bitwise equal to the eager
    call on the same input and workspace."""
    dl = tiny_q
    c = dl.c
    ws = dl.workspace(S)
    xbuf = torch.empty((S, c.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((S, c.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((S, c.top_k), dtype=torch.float32, device="cuda")
    y = torch.empty((S, c.hidden), dtype=torch.float32, device="cuda")
    view = dl.view()

    def call():
        M.moe_layer(dl.cfg, xbuf, M.MOE_F32, S, dl.W, dl.bias, idx, wt, view, dl.shared, y, ws, ws.numel())

    xs = [torch.from_numpy(gen.tokens(dl.w.with_(tokens=S), step=950 + i)).cuda() for i in range(4)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        xbuf.copy_(xs[0])
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for i in range(1, 4):
        xbuf.copy_(xs[i])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (idx.clone(), wt.clone(), y.clone())
        i_e, w_e, y_e = dl.layer(xs[i], M.MOE_F32, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(got[0], i_e) and torch.equal(got[1], w_e) and torch.equal(got[2], y_e), i
        assert torch.isfinite(y_e).all()


@pytest.mark.parametrize("thr", [0, 2], ids=["gemv", "matrix_cores"])
def test_zero_and_nan_rows(tiny_q, thr):
    """An all-zero token quantises to zeros (d = 0) and gives exactly zero output;
    a token holding a NaN gets d = NaN and NaN outputs, and the other tokens of
    the batch are untouched (int8 activations, decode and batch paths; with the
    threshold at 2 tokens the 9-token batch sends the shared expert and every
    expert chosen twice, zero and NaN rows included, to the matrix cores)."""
    for S in (3, 9):
        x = gen.tokens(tiny_q.w.with_(tokens=S), step=1234 + S).copy()
        x[0] = 0.0
        x[1, 7] = np.nan
        xt, dt = x_device(tiny_q.w, x)
        # route the finite tokens on a clean copy (a NaN logit has no defined selection)
        xr = x.copy()
        xr[1] = xr[2]
        idx, wt = tiny_q.route(x_device(tiny_q.w, xr)[0], dt)
        y = tiny_q.ffn(xt, dt, idx, wt, mfma_min_tokens=thr).cpu().numpy()
        assert np.all(y[0] == 0.0), S
        assert np.isnan(y[1]).all(), S
        ridx, rw = check_route(tiny_q, xr, idx.cpu().numpy(), wt.cpu().numpy())
        check_int8act(tiny_q, x, ridx, rw, y, np.arange(2, S))
