"""Recorded chains of layer calls (moe_chain_create / moe_chain_launch): one
library-owned HIP graph replays a sequence of moe_layer calls.  Each launch is
checked against the fp64 oracle call by call, on the inputs each call actually
received (a call's input may be the previous call's output), and against the
same moe_layer calls made one by one (bitwise)."""
import numpy as np
import pytest
import torch

from gen import inputs as gen
from int4_routed_expert_amd import moe as M
from oracle import oracle as O
from tests.devlayer import DeviceLayer, dev, max_rel_err

pytestmark = pytest.mark.gpu

TOL_FP32 = 2e-3


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def tiny():
    return DeviceLayer(gen.WORKLOADS["tiny"], host_experts=True, mfma_min_tokens=0)


@pytest.fixture(scope="module")
def glm():
    say("packing 256 + 1 GLM-5.2-shaped experts into HBM")
    return DeviceLayer(gen.WORKLOADS["decode"])


class Chain:
    """Buffers of n calls on one layer.  piped: call i reads call i - 1's y (y of
    one call is the next call's x); otherwise every call has its own input
    buffer.  Sizes S per call; one workspace (sized for the largest S) shared."""

    def __init__(self, dl: DeviceLayer, sizes, piped: bool):
        c = dl.c
        self.dl, self.sizes, self.piped = dl, list(sizes), piped
        f32 = dict(dtype=torch.float32, device="cuda")
        self.ws = dl.workspace(max(sizes))
        self.view = dl.view()
        self.x = [torch.zeros((S, c.hidden), **f32) for S in sizes]
        self.y = [torch.full((S, c.hidden), float("nan"), **f32) for S in sizes]
        self.idx = [torch.full((S, c.top_k), -1, dtype=torch.int32, device="cuda") for S in sizes]
        self.w = [torch.full((S, c.top_k), float("nan"), **f32) for S in sizes]
        self.calls = [M.layer_call(dl.cfg, self.input(i), M.MOE_F32, S, dl.W, dl.bias, self.idx[i], self.w[i],
                                   self.view, dl.shared, self.y[i], self.ws, self.ws.numel())
                      for i, S in enumerate(sizes)]

    def input(self, i):
        return self.y[i - 1] if self.piped and i > 0 else self.x[i]

    def eager(self, stream):
        dl = self.dl
        with torch.cuda.stream(stream):
            for i, S in enumerate(self.sizes):
                M.moe_layer(dl.cfg, self.input(i), M.MOE_F32, S, dl.W, dl.bias, self.idx[i], self.w[i], self.view,
                            dl.shared, self.y[i], self.ws, self.ws.numel(), stream)

    def outputs(self):
        return [(self.idx[i].cpu().numpy(), self.w[i].cpu().numpy(), self.y[i].cpu().numpy())
                for i in range(len(self.sizes))]


def check_against_oracle(ch: Chain, x_hosts, outs, tag):
    dl, c = ch.dl, ch.dl.c
    for i, S in enumerate(ch.sizes):
        xin = outs[i - 1][2] if ch.piped and i > 0 else x_hosts[i]
        idx, wt, y = outs[i]
        ridx, rw, _, flags, _ = O.route(c, xin, dl.W_host, dl.bias_host)
        assert not flags.any(), (tag, i, "a token sits on an fp32 rounding boundary")
        assert np.array_equal(idx, ridx), (tag, i)
        assert np.abs(wt - rw).max() <= 1e-6 * c.routed_scaling_factor, (tag, i)
        experts = {e: dl.host_expert(e) for e in set(ridx.ravel().tolist())}
        experts[c.n_experts] = dl.host[c.n_experts]
        ref = O.moe_ffn(c, np.ascontiguousarray(xin), ridx, rw, experts)
        err = max_rel_err(y, ref)
        assert err <= TOL_FP32, (tag, i, err)
        say(f"  {tag} call {i} (S={S}): idx exact, max rel err {err:.2e}")


@pytest.mark.parametrize("layer,sizes,piped", [
    ("tiny", (1, 1, 1), True),
    ("tiny", (4, 4), True),
    ("tiny", (1, 4, 2, 1), False),
    ("glm", (1, 1, 1), True),
    ("glm", (4, 1), False),
])
def test_chain_launches_match_oracle_and_eager_calls(tiny, glm, layer, sizes, piped):
    dl = {"tiny": tiny, "glm": glm}[layer]
    ch = Chain(dl, sizes, piped)
    chain = M.moe_chain_create(ch.calls)
    assert chain
    s = torch.cuda.Stream()
    try:
        for launch in range(4):
            x_hosts = [gen.tokens(dl.w.with_(tokens=S), step=5000 + 37 * launch + i) for i, S in enumerate(sizes)]
            for i in range(len(sizes)):
                if not piped or i == 0:
                    ch.x[i].copy_(dev(x_hosts[i]))
                ch.y[i].fill_(float("nan"))
            torch.cuda.synchronize()
            M.moe_chain_launch(chain, s)
            torch.cuda.synchronize()
            got = ch.outputs()
            check_against_oracle(ch, x_hosts, got, f"{layer} launch {launch}")
        # the same calls one by one on the same buffers: bitwise the same
        for i in range(len(sizes)):
            ch.y[i].fill_(float("nan"))
        torch.cuda.synchronize()
        ch.eager(s)
        torch.cuda.synchronize()
        for i, ((a0, a1, a2), (b0, b1, b2)) in enumerate(zip(got, ch.outputs())):
            assert np.array_equal(a0, b0) and np.array_equal(a1, b1) and np.array_equal(a2, b2), (layer, i)
    finally:
        M.moe_chain_destroy(chain)


def test_chain_reads_the_slot_table_at_every_launch(tiny):
    """Moving every expert to another slot (slab contents and table updated in
    place after recording) leaves the chain's results bitwise unchanged: the
    recorded graph reads the table and the slots when it runs."""
    dl = DeviceLayer(gen.WORKLOADS["tiny"], host_experts=True, mfma_min_tokens=0)
    E, sb = dl.c.n_experts, dl.slot_bytes
    ch = Chain(dl, (1, 3), False)
    chain = M.moe_chain_create(ch.calls)
    try:
        x_hosts = [gen.tokens(dl.w.with_(tokens=S), step=7100 + i) for i, S in enumerate(ch.sizes)]
        for i in range(2):
            ch.x[i].copy_(dev(x_hosts[i]))
        torch.cuda.synchronize()
        M.moe_chain_launch(chain)
        torch.cuda.synchronize()
        before = ch.outputs()
        check_against_oracle(ch, x_hosts, before, "before the move")
        perm = (torch.arange(E, device="cuda") * 5 + 3) % E  # a permutation of the slots (5 is coprime to 16)
        old = dl.slab.clone()
        for e in range(E):
            p = int(perm[e])
            dl.slab[p * sb:(p + 1) * sb].copy_(old[e * sb:(e + 1) * sb])
        dl.table.copy_(perm.to(torch.int32))
        for i in range(2):
            ch.y[i].fill_(float("nan"))
        torch.cuda.synchronize()
        M.moe_chain_launch(chain)
        torch.cuda.synchronize()
        after = ch.outputs()
        for (a0, a1, a2), (b0, b1, b2) in zip(before, after):
            assert np.array_equal(a0, b0) and np.array_equal(a1, b1) and np.array_equal(a2, b2)
    finally:
        M.moe_chain_destroy(chain)


def test_chain_refuses_while_profiling(tiny):
    ch = Chain(tiny, (1,), False)
    M.moe_profile_enable(True)
    try:
        with pytest.raises(M.MoeError) as ei:
            M.moe_chain_create(ch.calls)
        assert ei.value.status == M.MOE_EINVAL
    finally:
        M.moe_profile_enable(False)
        M.moe_profile_report()
