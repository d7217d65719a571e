"""The decode benchmark's launch configuration, checked against the oracle:
GLM-5.2 shape, resident layers rotated step by step, one moe_layer call per
step for one token, 16 steps recorded per graph with one workspace shared by
all of them and each step writing its own rows of idx, w and y (as bench.py
does, here with 2 layers and 32 tokens).  The graphs are library chains
(moe_chain_create, the bench's default) or HIP graphs captured by torch over
the same calls (the bench's split-call mode uses those).  Every graph is replayed twice, with
the outputs poisoned before the second replays; then every step's indices are
exactly the oracle's, its weights within 1e-6 rsf and its output within the
fp32 bar."""
import numpy as np
import pytest
import torch

from gen import inputs as gen
from int4_routed_expert_amd import moe as M
from oracle import oracle as O
from tests.devlayer import DeviceLayer, dev, max_rel_err
from tests.test_gpu_parity import TOL_FP32, say

pytestmark = pytest.mark.gpu

CHUNK = 16
N_LAYERS = 2
N_TOKENS = 32


@pytest.mark.parametrize("mode", ["chain", "torch_graph"])
def test_decode_graphs_of_sixteen_steps(mode):
    w = gen.WORKLOADS["decode"]
    c = w.cfg
    layers = [DeviceLayer(w, layer=l) for l in range(N_LAYERS)]
    cfg = layers[0].cfg
    xh = np.concatenate([gen.tokens(w, layer=0, step=s) for s in range(N_TOKENS)])
    xs = dev(xh)
    ws = M.workspace(cfg, 1)
    idx = torch.full((N_TOKENS, c.top_k), -7, dtype=torch.int32, device="cuda")
    wt = torch.full((N_TOKENS, c.top_k), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((N_TOKENS, c.hidden), float("nan"), dtype=torch.float32, device="cuda")
    views = [L.view() for L in layers]

    def step(j: int) -> None:
        L = layers[j % N_LAYERS]
        t = o = j % N_TOKENS
        M.moe_layer(cfg, xs[t:t + 1], M.MOE_F32, 1, L.W, L.bias, idx[o:o + 1], wt[o:o + 1], views[j % N_LAYERS],
                    L.shared, y[o:o + 1], ws, ws.numel())

    period = int(np.lcm(N_TOKENS, N_LAYERS))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for j in range(CHUNK):
            step(j)
    torch.cuda.synchronize()
    launchers, chains = [], []
    for gi in range(period // CHUNK):
        if mode == "chain":
            calls = []
            for j in range(gi * CHUNK, (gi + 1) * CHUNK):
                L, t = layers[j % N_LAYERS], j % N_TOKENS
                calls.append(M.layer_call(cfg, xs[t:t + 1], M.MOE_F32, 1, L.W, L.bias, idx[t:t + 1], wt[t:t + 1],
                                          views[j % N_LAYERS], L.shared, y[t:t + 1], ws, ws.numel()))
            ch = M.moe_chain_create(calls)
            chains.append(ch)
            launchers.append(lambda ch=ch: M.moe_chain_launch(ch, s))
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for j in range(CHUNK):
                    step(gi * CHUNK + j)
            launchers.append(g.replay)
    torch.cuda.synchronize()
    for launch in launchers:
        launch()
    torch.cuda.synchronize()
    idx.fill_(-7)
    wt.fill_(float("nan"))
    y.fill_(float("nan"))
    torch.cuda.synchronize()
    for launch in launchers:
        launch()
    torch.cuda.synchronize()
    for ch in chains:
        M.moe_chain_destroy(ch)
    gi_, gw, gy = idx.cpu().numpy(), wt.cpu().numpy(), y.cpu().numpy()
    worst = 0.0
    for j in range(period):
        L, t = layers[j % N_LAYERS], j % N_TOKENS
        x1 = xh[t:t + 1]
        ridx, rw, _, flags, _ = O.route(c, x1, L.W_host, L.bias_host)
        assert not flags.any()
        assert np.array_equal(gi_[t:t + 1], ridx), j
        assert np.abs(gw[t:t + 1] - rw).max() <= 1e-6 * c.routed_scaling_factor, j
        experts = {e: L.host_expert(e, layer=j % N_LAYERS) for e in ridx[0].tolist()}
        experts[c.n_experts] = L.host[c.n_experts]
        err = max_rel_err(gy[t:t + 1], O.moe_ffn(c, x1, ridx, rw, experts))
        worst = max(worst, err)
        assert err <= TOL_FP32, (j, err)
    say(f"{mode}: {period} steps in {len(launchers)} graphs of {CHUNK}: worst max rel err {worst:.3e}")
