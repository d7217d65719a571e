"""moe_layer_noalloc (the entry point that takes no workspace and allocates
nothing) against moe_layer with a caller-owned workspace, through the C ABI:
router indices identical, weights and outputs bitwise equal (the same kernels
run on the library's per-device scratch array), on two calls in a row, the
second with fewer tokens, and a request larger than the scratch array refused
with nothing written."""
import numpy as np
import pytest
import torch

from gen import inputs as gen
from int4_routed_expert_amd import moe as M
from tests.devlayer import DeviceLayer, dev, max_rel_err

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def layers():
    return {"tiny": DeviceLayer(gen.WORKLOADS["tiny"]), "glm": DeviceLayer(gen.WORKLOADS["decode"])}


def outputs(dl, S):
    c = dl.c
    return (torch.full((S, c.top_k), -7, dtype=torch.int32, device="cuda"),
            torch.full((S, c.top_k), float("nan"), device="cuda"),
            torch.full((S, c.hidden), float("nan"), device="cuda"))


@pytest.mark.parametrize("layer,sizes", [("tiny", (4, 1)), ("tiny", (9, 2)), ("glm", (4, 1)), ("glm", (12, 3))])
def test_noalloc_matches_layer_call(layers, layer, sizes):
    dl = layers[layer]
    view = dl.view()
    for n, S in enumerate(sizes):
        say(f"{layer}: call {n} with S = {S}")
        x = dev(gen.tokens(dl.w.with_(tokens=S), step=600 + 7 * n))
        ws = dl.workspace(S)
        i_r, w_r, y_r = outputs(dl, S)
        M.moe_layer(dl.cfg, x, M.MOE_F32, S, dl.W, dl.bias, i_r, w_r, view, dl.shared, y_r, ws, ws.numel())
        i_n, w_n, y_n = outputs(dl, S)
        M.moe_layer_noalloc(dl.cfg, x, M.MOE_F32, S, dl.W, dl.bias, i_n, w_n, view, dl.shared, y_n)
        torch.cuda.synchronize()
        assert torch.equal(i_n, i_r), (layer, S)
        assert torch.equal(w_n, w_r), (layer, S)
        assert torch.equal(y_n, y_r), (layer, S)
        assert max_rel_err(y_n.cpu().numpy(), y_r.cpu().numpy().astype(np.float64)) <= 2e-3
        assert torch.isfinite(y_n).all()


def test_noalloc_refuses_more_than_its_scratch(layers):
    dl = layers["glm"]
    S = 64  # about 24 MB of workspace at this shape, over the 8 MiB array
    assert M.moe_workspace_bytes(dl.cfg, S) > M.MOE_SCRATCH_BYTES
    x = dev(gen.tokens(dl.w.with_(tokens=S), step=1))
    i_n, w_n, y_n = outputs(dl, S)
    with pytest.raises(M.MoeError) as e:
        M.moe_layer_noalloc(dl.cfg, x, M.MOE_F32, S, dl.W, dl.bias, i_n, w_n, dl.view(), dl.shared, y_n)
    assert e.value.status == M.MOE_EWORKSPACE
    torch.cuda.synchronize()
    assert (i_n == -7).all() and torch.isnan(y_n).all()
