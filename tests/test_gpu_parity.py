"""HIP path vs the fp64 CPU oracle, through the C ABI, on seeded synthetic inputs.

Bars (from the layer's contract): router indices identical (rank order), weights
within 1e-6 * rsf, outputs within max relative error 2e-3 where every expert is
contracted in fp32 (decode batches and the large-batch fp32 path) and 1e-2 where
bf16 MFMA is used (prefill).  Per token: max_i |y - y_ref| / max_i |y_ref|.
"""
import os

import numpy as np
import pytest
import torch

from gen import inputs as gen
from int4_routed_expert_amd import moe as M
from oracle import oracle as O
from tests.devlayer import matrix_core_experts, DeviceLayer, dev, max_rel_err, tile_cover, x_device

pytestmark = pytest.mark.gpu

TOL_FP32 = 2e-3
TOL_BF16 = 1e-2
# against the oracle with the same bf16 operands: only accumulation order and
# the odd element of h on the other side of a bf16 rounding boundary differ
TOL_BF16_OPS = 2e-3

MID = gen.LayerConfig(hidden=512, n_experts=32, n_group=4, topk_group=2, top_k=4, moe_inter=256, shared_inter=192)


def say(*a):
    print(*a, flush=True)


def run_gpu(dl: DeviceLayer, x_host: np.ndarray, table=None):
    x, dt = x_device(dl.w, x_host)
    idx, wt = dl.route(x, dt)
    y = dl.ffn(x, dt, idx, wt, table=table)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), wt.cpu().numpy(), y.cpu().numpy()


def check_route(dl: DeviceLayer, x_host, idx, wt):
    c = dl.c
    ridx, rw, _, flags, margins = O.route(c, x_host, dl.W_host, dl.bias_host, x_is_bf16=dl.w.x_dtype == "bf16")
    ok = flags == 0
    assert ok.sum() == len(ok), f"{(~ok).sum()} tokens sit on an fp32 rounding boundary"
    mism = np.where((idx != ridx).any(axis=1))[0]
    assert len(mism) == 0, f"idx mismatch on tokens {mism[:10]}: gpu {idx[mism[:3]]} oracle {ridx[mism[:3]]}"
    assert np.abs(wt - rw).max() <= 1e-6 * c.routed_scaling_factor
    return ridx, rw


def check_ffn(dl: DeviceLayer, x_host, ridx, rw, y, tokens, tol, mfma_min_tokens: int | None = None):
    """y on `tokens` against the exact oracle within tol; with mfma_min_tokens, also
    against the oracle with bf16 operands for the experts the whole batch (ridx)
    sends to the matrix cores, within TOL_BF16_OPS."""
    c = dl.c
    xs = np.ascontiguousarray(x_host[tokens])
    need = set(ridx[tokens].ravel().tolist())
    experts = {e: dl.host_expert(e) for e in need}
    if c.shared_inter > 0:
        experts[c.n_experts] = dl.host[c.n_experts]
    bf = dl.w.x_dtype == "bf16"
    ref = O.moe_ffn(c, xs, ridx[tokens], rw[tokens], experts, x_is_bf16=bf)
    err = max_rel_err(y[tokens], ref)
    msg = f"  max rel err over {len(tokens)} tokens: {err:.3e}"
    err_b = None
    if mfma_min_tokens is not None:
        mc = matrix_core_experts(ridx, c.n_experts, c.shared_inter, mfma_min_tokens)
        ref_b = O.moe_ffn(c, xs, ridx[tokens], rw[tokens], experts, x_is_bf16=bf, bf16_experts=mc)
        err_b = max_rel_err(y[tokens], ref_b)
        msg += f"; against bf16 operands on the {len(mc)} matrix-core experts: {err_b:.3e}"
    say(msg)
    assert err <= tol
    if err_b is not None:
        assert err_b <= TOL_BF16_OPS
    return err


@pytest.fixture(scope="module")
def tiny():
    # exact fp32 path at every batch size; the matrix-core path is tested with explicit thresholds
    return DeviceLayer(gen.WORKLOADS["tiny"], host_experts=True, mfma_min_tokens=0)


@pytest.fixture(scope="module")
def mid():
    return DeviceLayer(gen.Workload("mid", MID, tokens=67, seed=11), host_experts=True, mfma_min_tokens=0)


@pytest.fixture(scope="module")
def glm():
    say("packing 256 + 1 GLM-5.2-shaped experts into HBM")
    return DeviceLayer(gen.WORKLOADS["decode"])


def test_device_pack_equals_host_pack(tiny):
    c = tiny.cfg
    for e in (0, 5, 15):
        ex = tiny.host_expert(e)
        host = np.zeros(tiny.slot_bytes, np.uint8)
        M.moe_pack_expert(c, 128, *ex.parts(), host, 0)
        devb = tiny.slab[e * tiny.slot_bytes:(e + 1) * tiny.slot_bytes].cpu().numpy()
        assert np.array_equal(host, devb)


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 9, 37])
def test_tiny_layer(tiny, S):
    w = tiny.w.with_(tokens=S)
    x = gen.tokens(w, step=S)
    idx, wt, y = run_gpu(tiny, x)
    ridx, rw = check_route(tiny, x, idx, wt)
    check_ffn(tiny, x, ridx, rw, y, np.arange(S), TOL_FP32)


@pytest.mark.parametrize("S", [1, 4, 67])
def test_mid_layer(mid, S):
    x = gen.tokens(mid.w.with_(tokens=S), step=100 + S)
    idx, wt, y = run_gpu(mid, x)
    ridx, rw = check_route(mid, x, idx, wt)
    check_ffn(mid, x, ridx, rw, y, np.arange(S), TOL_FP32)


def test_decode_full_size(glm):
    """GLM-5.2 shape, one token per call (the decode launch configuration)."""
    w = glm.w
    errs = []
    for step in range(6):
        x = gen.tokens(w, step=step)
        idx, wt, y = run_gpu(glm, x)
        ridx, rw = check_route(glm, x, idx, wt)
        say(f"step {step}: experts {ridx[0].tolist()}")
        errs.append(check_ffn(glm, x, ridx, rw, y, np.arange(1), TOL_FP32))
    say("decode worst", max(errs))


@pytest.mark.parametrize("layer", ["tiny", "mid", "glm"])
def test_router_reused_workspace_all_sizes(tiny, mid, glm, layer):
    """One workspace for a run of calls with S = 1..8 (single fused launch whose
    last workgroup selects) and S = 9, 13 (logits + per-token select kernels),
    fp32 and bf16 inputs: indices exact and weights within 1e-6 * rsf on every
    call, so the completion counter is back at zero after each call."""
    dl = {"tiny": tiny, "mid": mid, "glm": glm}[layer]
    ws = dl.workspace(16)
    sizes = [1, 2, 3, 4, 5, 6, 7, 8, 9, 1, 8, 13, 1]
    for n, S in enumerate(sizes):
        for bf16 in (False, True):
            w = dl.w.with_(tokens=S, x_dtype="bf16" if bf16 else "f32")
            x = gen.tokens(w, step=500 + n)
            xt, dt = x_device(w, x)
            idx = torch.empty((S, dl.c.top_k), dtype=torch.int32, device="cuda")
            wt = torch.empty((S, dl.c.top_k), dtype=torch.float32, device="cuda")
            M.moe_route(dl.cfg, xt, dt, S, dl.W, dl.bias, idx, wt, ws, ws.numel())
            torch.cuda.synchronize()
            ridx, rw, _, flags, _ = O.route(dl.c, x, dl.W_host, dl.bias_host, x_is_bf16=bf16)
            assert not flags.any()
            assert np.array_equal(idx.cpu().numpy(), ridx), (layer, S, bf16)
            assert np.abs(wt.cpu().numpy() - rw).max() <= 1e-6 * dl.c.routed_scaling_factor


def tied_router(c, W, bias, variant):
    """Router weights with exact ties: 'all' gives every expert the same row and
    bias (every key and every group score tied); 'groups' copies group 1 into the
    last group (whole-group score tie) with groups boosted so that exactly one of
    the two fits in the kept set, and copies an expert inside group 0 (key tie
    inside a group)."""
    W = W.copy()
    b = bias.copy()
    E, G = c.n_experts, c.n_group
    per = E // G
    if variant == "all":
        W[:] = W[0]
        b[:] = b[0]
        return W, b
    boost = np.zeros(G, np.float32)
    boost[: c.topk_group - 1] = 1.0  # these groups are kept outright
    boost[1] = 0.5                   # group 1 and its copy contest the last kept slot
    boost[G - 1] = 0.5
    for g in range(G):
        b[g * per:(g + 1) * per] += boost[g]
    W[(G - 1) * per:] = W[per:2 * per]
    b[(G - 1) * per:] = b[per:2 * per]
    if per >= 2:
        W[1] = W[0]
        b[1] = b[0]
    return W, b


@pytest.mark.parametrize("variant", ["all", "groups"])
@pytest.mark.parametrize("layer", ["tiny", "glm"])
def test_router_exact_ties(tiny, glm, layer, variant):
    """Exactly equal keys and group scores: the lower expert index (group index)
    wins, on the one-launch router (S <= 8) and the many-token kernels."""
    dl = {"tiny": tiny, "glm": glm}[layer]
    c = dl.c
    Wt, bt = tied_router(c, dl.W_host, dl.bias_host, variant)
    Wd, bd = dev(Wt), dev(bt)
    ws = dl.workspace(13)
    for S in (1, 3, 8, 13):
        x = gen.tokens(dl.w.with_(tokens=S), step=900 + S)
        xt, dt = x_device(dl.w, x)
        idx = torch.empty((S, c.top_k), dtype=torch.int32, device="cuda")
        wt = torch.empty((S, c.top_k), dtype=torch.float32, device="cuda")
        M.moe_route(dl.cfg, xt, dt, S, Wd, bd, idx, wt, ws, ws.numel())
        torch.cuda.synchronize()
        # (the oracle's near-midpoint flag is not asserted here: an exactly tied pair of
        # group scores is the fp32 rounding of an exact fp64 sum of two fp32 keys, the
        # same on both sides even when that sum sits on a midpoint)
        ridx, rw, _, _, _ = O.route(c, x, Wt, bt, x_is_bf16=dl.w.x_dtype == "bf16")
        if variant == "all":
            assert (ridx == np.arange(c.top_k)).all()  # lowest indices of the lowest kept groups
        assert np.array_equal(idx.cpu().numpy(), ridx), (layer, variant, S)
        assert np.abs(wt.cpu().numpy() - rw).max() <= 1e-6 * c.routed_scaling_factor


@pytest.mark.parametrize("layer", ["tiny", "mid", "glm"])
def test_layer_call_matches_route_then_ffn(tiny, mid, glm, layer):
    """moe_layer (for one token: scores-only router kernel, selection inside the
    gate/up kernel) gives idx, w and y bit-identical to moe_route then moe_ffn,
    over a run of calls on one workspace (fp32 and bf16 inputs, S = 1 and the
    S > 1 fallback), and matches the oracle."""
    dl = {"tiny": tiny, "mid": mid, "glm": glm}[layer]
    c = dl.c
    ws = dl.workspace(5)
    for n, S in enumerate([1, 1, 3, 1, 5, 1]):
        for bf16 in (False, True):
            w = dl.w.with_(tokens=S, x_dtype="bf16" if bf16 else "f32")
            x = gen.tokens(w, step=700 + 10 * n)
            xt, dt = x_device(w, x)
            idx_l, wt_l, y_l = dl.layer(xt, dt, ws=ws)
            idx_r, wt_r = dl.route(xt, dt, ws=ws)
            y_r = dl.ffn(xt, dt, idx_r, wt_r, ws=ws)
            torch.cuda.synchronize()
            assert np.array_equal(idx_l.cpu().numpy(), idx_r.cpu().numpy()), (layer, S, bf16)
            assert np.array_equal(wt_l.cpu().numpy(), wt_r.cpu().numpy()), (layer, S, bf16)
            assert np.array_equal(y_l.cpu().numpy(), y_r.cpu().numpy()), (layer, S, bf16)
            if n < 2:
                ridx, rw, _, flags, _ = O.route(c, x, dl.W_host, dl.bias_host, x_is_bf16=bf16)
                assert not flags.any()
                assert np.array_equal(idx_l.cpu().numpy(), ridx)
                assert np.abs(wt_l.cpu().numpy() - rw).max() <= 1e-6 * c.routed_scaling_factor
                xs = np.ascontiguousarray(x)
                experts = {e: dl.host_expert(e) for e in set(ridx.ravel().tolist())}
                experts[c.n_experts] = dl.host[c.n_experts]
                ref = O.moe_ffn(c, xs, ridx, rw, experts, x_is_bf16=bf16)
                assert max_rel_err(y_l.cpu().numpy(), ref) <= TOL_FP32


@pytest.mark.parametrize("layer", ["tiny", "glm"])
def test_layer_call_graph_replays(tiny, glm, layer):
    """The one-token moe_layer captured in a HIP graph: replays with new inputs
    written between them, interleaved with eager calls on the same workspace,
    each bitwise equal to the eager call on the same input."""
    dl = {"tiny": tiny, "glm": glm}[layer]
    c = dl.c
    ws = dl.workspace(1)
    xbuf = torch.empty((1, c.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, c.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((1, c.top_k), dtype=torch.float32, device="cuda")
    y = torch.empty((1, c.hidden), dtype=torch.float32, device="cuda")
    view = dl.view()

    def call():
        M.moe_layer(dl.cfg, xbuf, M.MOE_F32, 1, dl.W, dl.bias, idx, wt, view, dl.shared, y, ws, ws.numel())

    xs = [dev(gen.tokens(dl.w.with_(tokens=1), step=900 + i)) for i in range(4)]
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
        i_e, w_e, y_e = dl.layer(xs[i], M.MOE_F32, ws=ws)  # eager call on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(got[0], i_e) and torch.equal(got[1], w_e), (layer, i)
        assert torch.equal(got[2], y_e), (layer, i)
        assert not torch.isnan(y_e).any(), (layer, i)


def test_layer_call_unresident_and_tied(tiny):
    """moe_layer for one token with an unresident selected expert (its row is
    NaN, as from moe_ffn) and with exactly tied router rows (lowest indices)."""
    c = tiny.c
    x = gen.tokens(tiny.w.with_(tokens=1), step=31)
    xt, dt = x_device(tiny.w, x)
    idx_r, _ = tiny.route(xt, dt)
    table = tiny.table.clone()
    table[int(idx_r[0, 1])] = -1
    idx_l, wt_l, y_l = tiny.layer(xt, dt, table=table)
    torch.cuda.synchronize()
    assert np.isnan(y_l.cpu().numpy()).all()
    assert np.array_equal(idx_l.cpu().numpy(), idx_r.cpu().numpy())
    Wt, bt = tied_router(c, tiny.W_host, tiny.bias_host, "all")
    W0, b0 = tiny.W, tiny.bias
    try:
        tiny.W, tiny.bias = dev(Wt), dev(bt)
        idx_l, wt_l, y_l = tiny.layer(xt, dt)
        torch.cuda.synchronize()
    finally:
        tiny.W, tiny.bias = W0, b0
    assert (idx_l.cpu().numpy() == np.arange(c.top_k)).all()
    assert np.allclose(wt_l.cpu().numpy(), c.routed_scaling_factor / c.top_k, rtol=1e-6)


@pytest.mark.parametrize("S", [1, 5, 8])
def test_router_uninitialised_workspace_is_poisoned(tiny, S):
    """A workspace whose header was never written gives idx -1 and w NaN for
    every token (and then NaN rows from moe_ffn), not a silent selection;
    after moe_workspace_init the same buffer routes correctly."""
    c = tiny.c
    ws = torch.full((M.moe_workspace_bytes(tiny.cfg, S),), 0xAB, dtype=torch.uint8, device="cuda")
    x = gen.tokens(tiny.w.with_(tokens=S), step=77)
    xt = dev(x)
    idx = torch.zeros((S, c.top_k), dtype=torch.int32, device="cuda")
    wt = torch.zeros((S, c.top_k), dtype=torch.float32, device="cuda")
    M.moe_route(tiny.cfg, xt, M.MOE_F32, S, tiny.W, tiny.bias, idx, wt, ws, ws.numel())
    y = tiny.ffn(xt, M.MOE_F32, idx, wt)
    torch.cuda.synchronize()
    assert (idx.cpu().numpy() == -1).all()
    assert np.isnan(wt.cpu().numpy()).all()
    assert np.isnan(y.cpu().numpy()).all()
    M.moe_workspace_init(ws)
    M.moe_route(tiny.cfg, xt, M.MOE_F32, S, tiny.W, tiny.bias, idx, wt, ws, ws.numel())
    torch.cuda.synchronize()
    ridx, rw, _, _, _ = O.route(c, x, tiny.W_host, tiny.bias_host)
    assert np.array_equal(idx.cpu().numpy(), ridx)


def test_decode_bf16_input(glm):
    w = glm.w.with_(x_dtype="bf16")
    x = gen.tokens(w, step=3)
    xt = dev(x.view(np.int16)).view(torch.bfloat16)
    idx, wt = glm.route(xt, M.MOE_BF16)
    y = glm.ffn(xt, M.MOE_BF16, idx, wt)
    torch.cuda.synchronize()
    dl = glm
    ridx, rw, _, flags, _ = O.route(dl.c, x, dl.W_host, dl.bias_host, x_is_bf16=True)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    experts = {e: dl.host_expert(e) for e in ridx.ravel().tolist()}
    experts[dl.c.n_experts] = dl.host[dl.c.n_experts]
    ref = O.moe_ffn(dl.c, x, ridx, rw, experts, x_is_bf16=True)
    assert max_rel_err(y.cpu().numpy(), ref) <= TOL_FP32


def test_verify_batch_full_size():
    """S = 4 verify batch with the skewed bias: the union is streamed once."""
    w = gen.WORKLOADS["verify"]
    dl = DeviceLayer(w)
    for step in range(2):
        x = gen.tokens(w, step=step)
        idx, wt, y = run_gpu(dl, x)
        ridx, rw = check_route(dl, x, idx, wt)
        U = len(set(ridx.ravel().tolist()))
        say(f"verify step {step}: union {U}")
        check_ffn(dl, x, ridx, rw, y, np.arange(4), TOL_FP32)


def test_row_stability_decode_family(tiny, glm):
    """A token's output in a 4-token batch is bitwise equal to its 1-token result."""
    for dl in (tiny, glm):
        x4 = gen.tokens(dl.w.with_(tokens=4), step=77)
        _, _, y4 = run_gpu(dl, x4)
        for t in range(4):
            _, _, y1 = run_gpu(dl, x4[t:t + 1])
            assert np.array_equal(y1[0], y4[t])


def test_zero_input(tiny, glm):
    for dl in (tiny, glm):
        c = dl.c
        for S in (1, 6):
            x = np.zeros((S, c.hidden), np.float32)
            idx, wt, y = run_gpu(dl, x)
            assert np.all(wt == np.float32(c.routed_scaling_factor / c.top_k))
            ridx, _ = check_route(dl, x, idx, wt)
            assert np.all(y == 0.0)


def test_empty_batch(tiny):
    x = torch.zeros((0, tiny.c.hidden), device="cuda")
    idx = torch.full((1, 2), 7, dtype=torch.int32, device="cuda")
    wt = torch.zeros((1, 2), device="cuda")
    ws = tiny.workspace(1)
    M.moe_route(tiny.cfg, x, M.MOE_F32, 0, tiny.W, tiny.bias, idx, wt, ws, ws.numel())
    y = torch.full((1, tiny.c.hidden), 3.0, device="cuda")
    M.moe_ffn(tiny.cfg, x, M.MOE_F32, 0, idx, wt, tiny.view(), tiny.shared, y, ws, ws.numel())
    torch.cuda.synchronize()
    assert torch.all(idx == 7) and torch.all(y == 3.0)


@pytest.mark.parametrize("S", [1, 3, 8])
def test_unresident_slot_poisons_only_its_tokens(tiny, S):
    x = gen.tokens(tiny.w.with_(tokens=S), step=500 + S)
    idx, wt, y_ok = run_gpu(tiny, x)
    victim = int(idx[0, 0])
    table = tiny.table.clone()
    table[victim] = -1
    xt = dev(x)
    y = tiny.ffn(xt, M.MOE_F32, dev(idx), dev(wt), table=table).cpu().numpy()
    uses = (idx == victim).any(axis=1)
    assert np.all(np.isnan(y[uses]).all(axis=1))
    assert np.array_equal(y[~uses], y_ok[~uses])
    table[victim] = 10 ** 6
    y = tiny.ffn(xt, M.MOE_F32, dev(idx), dev(wt), table=table).cpu().numpy()
    assert np.all(np.isnan(y[uses]).all(axis=1))


@pytest.mark.parametrize("S", [1, 2, 6])
@pytest.mark.parametrize("mode", ["out_of_range", "negative", "repeated"])
def test_invalid_idx_poisons_only_its_token(tiny, S, mode):
    x = gen.tokens(tiny.w.with_(tokens=S), step=900 + S)
    idx, wt, y_ok = run_gpu(tiny, x)
    bad = idx.copy()
    t = min(1, S - 1)  # the poisoned token
    bad[t, 1] = {"out_of_range": 12345, "negative": -3, "repeated": bad[t, 0]}[mode]
    y = tiny.ffn(dev(x), M.MOE_F32, dev(bad), dev(wt)).cpu().numpy()
    assert np.all(np.isnan(y[t]))
    keep = np.ones(S, bool)
    keep[t] = False
    # each token's arithmetic does not depend on the others: the rest is bitwise unchanged
    assert np.array_equal(y[keep], y_ok[keep])


def test_largest_shapes():
    """H = I = Is = 8192 (the largest supported): one token, three tokens (the few-token kernels with h
    converted in registers) and the large-batch path."""
    cfg = gen.LayerConfig(hidden=8192, n_experts=8, n_group=2, topk_group=1, top_k=2, moe_inter=8192,
                          shared_inter=8192)
    w = gen.Workload("max", cfg, tokens=5, seed=21)
    dl = DeviceLayer(w, mfma_min_tokens=0)
    for S in (1, 3, 5):
        x = gen.tokens(w.with_(tokens=S), step=S)
        idx, wt, y = run_gpu(dl, x)
        ridx, rw = check_route(dl, x, idx, wt)
        check_ffn(dl, x, ridx, rw, y, np.arange(min(S, 2)), TOL_FP32)


RAGGED = gen.LayerConfig(hidden=544, n_experts=8, n_group=2, topk_group=1, top_k=2, moe_inter=96, shared_inter=64)


@pytest.mark.parametrize("case", ["tiny_S37_t4", "mid_S67_t4", "mid_S300_t16", "ragged_S40_t4", "ragged_bf16_S40_t2"])
def test_matrix_core_path(tiny, mid, case):
    """Experts with at least the threshold's tokens run the bf16 grouped GEMM
    (several and ragged 128-row tiles, 64-column tiles that overhang H = 544,
    shared expert included): every token within the bf16 bar of the oracle;
    the same call with the threshold at 0 (exact path) stays within the fp32
    bar and differs from the matrix-core result, so the tiles really ran."""
    name, S, thr = case.rsplit("_", 2)[0], int(case.rsplit("_", 2)[1][1:]), int(case.rsplit("_", 1)[1][1:])
    if name == "tiny":
        dl = tiny
    elif name == "mid":
        dl = mid
    else:
        wl = gen.Workload("ragged", RAGGED, tokens=S, seed=31, x_dtype="bf16" if "bf16" in name else "f32")
        dl = DeviceLayer(wl, host_experts=True)
    w = dl.w.with_(tokens=S)
    x = gen.tokens(w, step=900 + S)
    xt, dt = x_device(w, x)
    idx, wt = dl.route(xt, dt)
    y_mfma = dl.ffn(xt, dt, idx, wt, mfma_min_tokens=thr)
    y_exact = dl.ffn(xt, dt, idx, wt, mfma_min_tokens=0)
    torch.cuda.synchronize()
    ridx, rw = check_route(dl, x, idx.cpu().numpy(), wt.cpu().numpy())
    counts = np.bincount(ridx.ravel(), minlength=dl.c.n_experts)
    say(f"{case}: tokens per expert max {counts.max()}, experts at or over {thr}: {(counts >= thr).sum()}")
    assert (counts >= thr).any() or S >= thr
    ym, ye = y_mfma.cpu().numpy(), y_exact.cpu().numpy()
    check_ffn(dl, x, ridx, rw, ym, np.arange(S), TOL_BF16, mfma_min_tokens=thr)
    check_ffn(dl, x, ridx, rw, ye, np.arange(S), TOL_FP32)
    assert not np.array_equal(ym, ye)


# Tokens per expert chosen so that the matrix-core tiles take every height that
# changes which waves multiply (1 to 16 row blocks of 16, partial last blocks),
# a full 256-row tile and experts of two tiles, beside GEMV-item experts.
TILE_COUNTS = [8, 9, 16, 17, 24, 31, 32, 33, 48, 63, 64, 65, 80, 100, 127, 128, 129, 143, 200, 255, 256, 257, 300,
               400]


def crafted_routing(counts, n_experts: int, k: int, S: int, seed: int):
    """idx (S x k) in which expert e is chosen by counts[e] tokens: expert e takes
    the next counts[e] places of the (slot, token) order, so its tokens are
    distinct whenever counts[e] <= S; weights uniform in [0.5, 1.5) / k."""
    assert sum(counts) == S * k and max(counts) <= S and len(counts) <= n_experts
    place = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(counts)])
    idx = place.reshape(k, S).T.copy()
    assert all(len(set(r)) == k for r in idx.tolist())
    rng = np.random.default_rng(seed)
    return idx, (rng.random((S, k)) + 0.5).astype(np.float32) / k


def test_matrix_core_every_tile_height(mid):
    """Crafted routing at the mid shape: experts with 8 to 400 tokens (tiles of
    every height, partial blocks, one and two tiles per expert), the rest on the
    GEMV path; all 800 tokens within the bf16 bar of the oracle."""
    c = mid.c
    k, S = c.top_k, 800
    counts = list(TILE_COUNTS)
    rest = S * k - sum(counts)
    small = [7, 5, 3, 1, 6, 4, 2, 7]
    counts += small
    counts[-1] += rest - sum(small)  # one more expert of two tiles
    assert counts[-1] <= S and len(counts) == c.n_experts, (counts[-1], len(counts))
    idx, wt = crafted_routing(counts, c.n_experts, k, S, seed=5)
    w = mid.w.with_(tokens=S)
    x = gen.tokens(w, step=77)
    xt, dt = x_device(w, x)
    y = mid.ffn(xt, dt, dev(idx), dev(wt), mfma_min_tokens=8).cpu().numpy()
    say(f"tokens per expert: {sorted(np.bincount(idx.ravel(), minlength=c.n_experts).tolist())}")
    check_ffn(mid, x, idx, wt, y, np.arange(S), TOL_BF16, mfma_min_tokens=8)


def test_matrix_core_zero_and_nan_rows(mid):
    """The bf16 matrix-core tiles are row-local: in a 40-token batch with the
    threshold at 2 tokens (every expert chosen twice, and the shared expert, on
    the matrix cores), an all-zero token gives exactly zero output, a token with
    one NaN activation gives NaN outputs, and every other token matches the
    oracle."""
    S = 40
    w = mid.w.with_(tokens=S)
    x = gen.tokens(w, step=4321).copy()
    x[0] = 0.0
    x[1, 7] = np.nan
    xt, dt = x_device(w, x)
    xr = x.copy()
    xr[1] = xr[2]  # route the finite tokens on a clean copy (a NaN logit has no defined selection)
    idx, wt = mid.route(x_device(w, xr)[0], dt)
    ridx, rw = check_route(mid, xr, idx.cpu().numpy(), wt.cpu().numpy())
    assert (np.bincount(ridx.ravel(), minlength=mid.c.n_experts) >= 2).any()
    y = mid.ffn(xt, dt, idx, wt, mfma_min_tokens=2).cpu().numpy()
    assert np.all(y[0] == 0.0)
    assert np.isnan(y[1]).all()
    check_ffn(mid, x, ridx, rw, y, np.arange(2, S), TOL_BF16, mfma_min_tokens=2)


def test_matrix_core_unresident_slot_poisons_only_its_tokens(mid):
    S, thr = 67, 4
    w = mid.w.with_(tokens=S)
    x = gen.tokens(w, step=4242)
    xt, dt = x_device(w, x)
    idx, wt = mid.route(xt, dt)
    ih = idx.cpu().numpy()
    counts = np.bincount(ih.ravel(), minlength=mid.c.n_experts)
    victim = int(np.argmax(counts))  # a matrix-core expert
    assert counts[victim] >= thr
    table = mid.table.clone()
    table[victim] = 1 << 20  # outside [0, n_slots)
    y = mid.ffn(xt, dt, idx, wt, table=table, mfma_min_tokens=thr).cpu().numpy()
    hit = (ih == victim).any(axis=1)
    assert np.isnan(y[hit]).all(axis=1).all()
    assert np.isfinite(y[~hit]).all()
    ridx, rw = check_route(mid, x, ih, wt.cpu().numpy())
    check_ffn(mid, x, ridx, rw, y, np.where(~hit)[0], TOL_BF16, mfma_min_tokens=thr)


def test_prefill_full_size():
    """2048 tokens, bf16 activations, Zipf-skewed routing, in the launch
    configuration the prefill benchmark times: every token's indices and weights
    are checked; outputs on a set of tokens that holds at least one token of
    every 256-row matrix-core tile of every expert (and of the shared expert) and
    of every 4-token GEMV item (the oracle runs one token at a time), plus the
    batch's first and last token and a few random ones."""
    w = gen.WORKLOADS["prefill"]
    dl = DeviceLayer(w)
    x = gen.tokens(w)
    say("prefill: running GPU path")
    idx, wt, y = run_gpu(dl, x)
    ridx, rw = check_route(dl, x, idx, wt)
    counts = np.bincount(ridx.ravel(), minlength=w.cfg.n_experts)
    say(f"prefill: max tokens per expert {counts.max()}, experts with >= 16 tokens {(counts >= 16).sum()}")
    tokens = np.union1d(tile_cover(ridx, w.cfg.n_experts, dl.cfg.mfma_min_tokens, extra=6), [0, 2047])
    say(f"prefill: comparing {tokens.size} tokens")
    check_ffn(dl, x, ridx, rw, y, tokens, TOL_BF16, mfma_min_tokens=dl.cfg.mfma_min_tokens)
    assert np.isfinite(y).all()


def scaled_rows(x: np.ndarray, kind: str, seed: int) -> np.ndarray:
    """x rows rescaled: 'wide' multiplies each 32-element group by 2^a and each
    element by 2^b more (a, b uniform integers in [-20, 20]: values within a group
    and across the row span about 2^40); 'big' by 2^58 and 'small' by 2^-64 (the
    outputs then lie near the top and the bottom of the fp32 range: SwiGLU
    squares the activations' scale)."""
    rng = np.random.default_rng(seed)
    x = x.astype(np.float64)
    if kind == "wide":
        a = rng.integers(-20, 21, size=(x.shape[0], x.shape[1] // 32, 1))
        b = rng.integers(-20, 21, size=(x.shape[0], x.shape[1] // 32, 32))
        x = (x.reshape(x.shape[0], -1, 32) * np.exp2(a + b)).reshape(x.shape)
    else:
        x = x * 2.0 ** (58 if kind == "big" else -64)
    return x.astype(np.float32)


@pytest.mark.parametrize("kind", ["wide", "big", "small"])
def test_decode_extreme_activations(glm, kind):
    """GLM-5.2 shape, the exact FFN paths (one token, a batch of four, a batch of
    six on the exact large-batch path) on activations whose groups span ~2^40, or
    whose outputs approach the largest (~1e37) or smallest (~1e-37) normal fp32
    values: every token within the fp32 bar of the oracle, and a token's row of
    the four-token batch bitwise equal to its one-token result.  The routing is
    that of the unscaled tokens, so only the FFN's arithmetic sees the extremes."""
    c = glm.c
    x0 = gen.tokens(glm.w.with_(tokens=6), step=4321)
    ridx, rw, _, flags, _ = O.route(c, x0, glm.W_host, glm.bias_host)
    assert not flags.any()
    x = scaled_rows(x0, kind, 17)
    experts = {e: glm.host_expert(e) for e in set(ridx.ravel().tolist())}
    experts[c.n_experts] = glm.host[c.n_experts]
    ref = O.moe_ffn(c, x, ridx, rw, experts)
    assert np.isfinite(ref).all() and np.abs(ref).max() > 0
    say(f"{kind}: |y_ref| in [{np.abs(ref).min():.3e}, {np.abs(ref).max():.3e}]")
    ys = {}
    for S in (1, 4, 6):
        y = glm.ffn(dev(x[:S]), M.MOE_F32, dev(ridx[:S]), dev(rw[:S].astype(np.float32)), mfma_min_tokens=0)
        torch.cuda.synchronize()
        ys[S] = y.cpu().numpy()
        err = max_rel_err(ys[S], ref[:S])
        say(f"  S={S}: max rel err {err:.3e}")
        assert err <= TOL_FP32, (kind, S, err)
    assert np.array_equal(ys[4][0], ys[1][0])


@pytest.mark.parametrize("S", [1, 4])
@pytest.mark.parametrize("layer", ["tiny", "glm"])
def test_layer_graph_replays_match_oracle(tiny, glm, layer, S):
    """moe_layer captured once in a HIP graph (one token: three kernels; four
    tokens: the router and the few-token kernels) and replayed over 8 distinct
    inputs written into its input buffer between replays: every replay's idx, w
    and y match the oracle (idx exactly, w within 1e-6 rsf, y within the fp32
    bar), with no eager call in between."""
    dl = {"tiny": tiny, "glm": glm}[layer]
    c = dl.c
    ws = dl.workspace(S)
    xbuf = torch.empty((S, c.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((S, c.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((S, c.top_k), dtype=torch.float32, device="cuda")
    y = torch.empty((S, c.hidden), dtype=torch.float32, device="cuda")
    view = dl.view()
    xs = [gen.tokens(dl.w.with_(tokens=S), step=1300 + 10 * i) for i in range(8)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up call outside the capture
        xbuf.copy_(dev(xs[0]))
        M.moe_layer(dl.cfg, xbuf, M.MOE_F32, S, dl.W, dl.bias, idx, wt, view, dl.shared, y, ws, ws.numel())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        M.moe_layer(dl.cfg, xbuf, M.MOE_F32, S, dl.W, dl.bias, idx, wt, view, dl.shared, y, ws, ws.numel())
    torch.cuda.synchronize()
    for i, xh in enumerate(xs):
        xbuf.copy_(dev(xh))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ridx, rw, _, flags, _ = O.route(c, xh, dl.W_host, dl.bias_host)
        assert not flags.any()
        assert np.array_equal(idx.cpu().numpy(), ridx), (layer, S, i)
        assert np.abs(wt.cpu().numpy() - rw).max() <= 1e-6 * c.routed_scaling_factor
        experts = {e: dl.host_expert(e) for e in set(ridx.ravel().tolist())}
        experts[c.n_experts] = dl.host[c.n_experts]
        ref = O.moe_ffn(c, xh, ridx, rw, experts)
        err = max_rel_err(y.cpu().numpy(), ref)
        assert err <= TOL_FP32, (layer, S, i, err)


@pytest.mark.parametrize("S", [1, 4, 9])
def test_allocating_binding_calls(tiny, S):
    """M.route / M.ffn / M.layer allocate their outputs (and a workspace) on x's device and give
    the same bits as the raw-pointer calls; routing and outputs against the oracle."""
    w = tiny.w.with_(tokens=S)
    xh = gen.tokens(w, step=4100 + S)
    x = dev(xh)
    view = tiny.view()
    idx, wt = M.route(x, tiny.W, tiny.bias, tiny.cfg)
    y = M.ffn(x, idx, wt, view, tiny.shared, tiny.cfg)
    li, lw, ly = M.layer(x, tiny.W, tiny.bias, view, tiny.shared, tiny.cfg)
    torch.cuda.synchronize()
    assert idx.dtype == torch.int32 and wt.dtype == torch.float32 and y.dtype == torch.float32
    assert tuple(y.shape) == (S, tiny.c.hidden) and y.device == x.device
    ridx, rw = check_route(tiny, xh, idx.cpu().numpy(), wt.cpu().numpy())
    check_ffn(tiny, xh, ridx, rw, y.cpu().numpy(), np.arange(S), TOL_FP32)
    e_idx, e_w, e_y = run_gpu(tiny, xh)
    assert np.array_equal(idx.cpu().numpy(), e_idx) and np.array_equal(wt.cpu().numpy(), e_w)
    assert np.array_equal(y.cpu().numpy(), e_y)
    assert np.array_equal(li.cpu().numpy(), e_idx) and np.array_equal(ly.cpu().numpy(), e_y)
    # wrong dtype, wrong width and a strided view are refused before anything is launched
    H = tiny.c.hidden
    for bad in (x.double(), x[:, : H - 32].contiguous(), torch.zeros((S, 2 * H), device="cuda")[:, ::2], x.t()):
        if bad.dim() == 2 and tuple(bad.shape) == (S, H) and bad.is_contiguous() and bad.dtype == torch.float32:
            continue  # x.t() of a single row is itself a valid [1, H] tensor
        with pytest.raises(ValueError):
            M.route(bad, tiny.W, tiny.bias, tiny.cfg)
    with pytest.raises(ValueError):
        M.ffn(x, idx[:, :1].contiguous(), wt, view, tiny.shared, tiny.cfg)
