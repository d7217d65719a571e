"""A sweep over layer configurations at the edges of what moe_validate_cfg accepts,
through the C ABI, against the fp64 oracle: up to 1024 experts in 64 groups, top_k
up to 16, a single group, no shared expert, norm_topk_prob = 0 with other scaling
factors, bf16 activations, hidden and intermediate sizes with an odd number of
32-element groups, H = 8192 on the few-token path, every weight format, and int8
activations; one token (moe_layer's fused selection), two to four tokens (the
batch-union path) and larger batches on both the exact items and the matrix cores.

Per case: router indices exactly those of the oracle and weights within 1e-6 rsf;
the FFN output within the bar of the path that ran (fp32 path 2e-3; bf16 matrix
cores 2e-3 against the oracle with the same bf16 operands, and 2.5e-2 against the
exact layer; int8 activations against the oracle's int8 mode: max 5e-3 and median
1e-5); and moe_layer bitwise equal to moe_route then moe_ffn on the same inputs.

The bf16 path's distance from the exact layer grows as the contractions shrink
(fewer independent roundings of x, W and h to average): a CPU evaluation of the
bf16 operands puts it at 1.1e-2 for H = 96, I = Is = 32 and one routed expert,
where the GEMM's 256-row tiles meet their smallest shapes; the check against the
oracle's bf16 operands is the tight one."""
import numpy as np
import pytest
import torch

from gen import inputs as gen
from tests.devlayer import DeviceLayer, matrix_core_experts, x_device
from tests.test_gpu_int8act import check_int8act
from tests.test_gpu_parity import TOL_FP32, check_ffn, check_route, say

TOL_BF16_SMALL = 2.5e-2  # bf16 path against the exact layer at these small shapes

pytestmark = pytest.mark.gpu

# name: (H, E, G, Gk, k, I, Is, norm, rsf, fmt, act_int8, S, threshold, x dtype)
CASES = {
    "e1024_g64_k16_S1": (256, 1024, 64, 8, 16, 64, 64, 1, 2.5, 0, 0, 1, 3, "f32"),
    "e1024_g64_k16_S3": (256, 1024, 64, 8, 16, 64, 64, 1, 2.5, 0, 0, 3, 3, "f32"),
    "e1024_g64_k16_S40_mfma": (256, 1024, 64, 8, 16, 64, 64, 1, 2.5, 0, 0, 40, 2, "f32"),
    "e512_g16_k12_noshared_S1": (512, 512, 16, 4, 12, 96, 0, 1, 2.5, 0, 0, 1, 3, "f32"),
    "e512_g16_k12_noshared_S4": (512, 512, 16, 4, 12, 96, 0, 1, 2.5, 0, 0, 4, 3, "f32"),
    "noshared_S70_mfma": (544, 32, 4, 2, 4, 160, 0, 1, 2.5, 0, 0, 70, 3, "f32"),
    "norm0_S1": (320, 64, 8, 3, 6, 128, 96, 0, 1.0, 0, 0, 1, 3, "f32"),
    "norm0_S9_mfma": (320, 64, 8, 3, 6, 128, 96, 0, 1.75, 0, 0, 9, 2, "f32"),
    "g1_k1_S1": (96, 8, 1, 1, 1, 32, 32, 1, 2.5, 0, 0, 1, 3, "f32"),
    "g1_k1_S33": (96, 8, 1, 1, 1, 32, 32, 1, 2.5, 0, 0, 33, 3, "f32"),
    "bf16_x_S1": (1024, 64, 8, 4, 8, 256, 256, 1, 2.5, 0, 0, 1, 3, "bf16"),
    "bf16_x_S4": (1024, 64, 8, 4, 8, 256, 256, 1, 2.5, 0, 0, 4, 3, "bf16"),
    "h8192_S2": (8192, 16, 4, 2, 4, 128, 64, 1, 2.5, 0, 0, 2, 3, "f32"),
    "q4row_k16_S5": (256, 128, 8, 4, 16, 96, 64, 1, 2.5, 1, 0, 5, 3, "f32"),
    "q8row_e1024_S1": (256, 1024, 32, 8, 8, 64, 32, 1, 2.5, 2, 0, 1, 3, "f32"),
    "q8row_odd_groups_S24_mfma": (224, 16, 4, 2, 4, 96, 160, 1, 2.5, 2, 0, 24, 2, "f32"),
    "int8_q4g32_k16_S40_mfma": (256, 128, 8, 4, 16, 96, 64, 1, 2.5, 0, 1, 40, 2, "f32"),
    "int8_q8row_noshared_S12_mfma": (288, 32, 4, 2, 4, 96, 0, 1, 2.5, 2, 1, 12, 3, "f32"),
    "int8_q4row_norm0_S1": (256, 64, 8, 4, 8, 64, 64, 0, 1.5, 1, 1, 1, 3, "f32"),
    # two to four tokens: the down kernel's h rows as limbs in LDS (I <= 2048) with shared rows narrower or wider
    # than the routed ones, int8 weights, int8 activations; and wider rows (the register path)
    "shared_narrow_S4": (512, 32, 4, 2, 4, 320, 192, 1, 2.5, 0, 0, 4, 3, "f32"),
    "shared_wide_S4": (256, 32, 4, 2, 4, 64, 160, 1, 2.5, 0, 0, 4, 3, "f32"),
    "q8row_S3": (256, 64, 8, 4, 8, 128, 64, 1, 2.5, 2, 0, 3, 3, "f32"),
    "int8_q4g32_S2": (256, 64, 8, 4, 8, 128, 128, 1, 2.5, 0, 1, 2, 3, "f32"),
    "i4096_S3": (1024, 16, 4, 2, 4, 4096, 2560, 1, 2.5, 0, 0, 3, 3, "f32"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_config(name):
    H, E, G, Gk, k, I, Is, norm, rsf, fmt, a8, S, thr, xdt = CASES[name]
    cfg = gen.LayerConfig(hidden=H, n_experts=E, n_group=G, topk_group=Gk, top_k=k, moe_inter=I, shared_inter=Is,
                          routed_scaling_factor=rsf, norm_topk_prob=norm, weight_format=fmt)
    seed = sum(map(ord, name))
    w = gen.Workload(name, cfg, tokens=S, x_dtype=xdt, seed=seed)
    dl = DeviceLayer(w, host_experts=False, mfma_min_tokens=thr, act_int8=a8)
    x = gen.tokens(w, step=3)
    xt, dt = x_device(w, x)
    idx, wt = dl.route(xt, dt)
    y = dl.ffn(xt, dt, idx, wt)
    li, lw, ly = dl.layer(xt, dt)
    torch.cuda.synchronize()
    idx, wt, y = idx.cpu().numpy(), wt.cpu().numpy(), y.cpu().numpy()
    ridx, rw = check_route(dl, x, idx, wt)
    assert np.array_equal(li.cpu().numpy(), idx) and np.array_equal(lw.cpu().numpy(), wt)
    assert np.array_equal(ly.cpu().numpy(), y, equal_nan=False)
    mfma = bool(matrix_core_experts(ridx, E, Is, thr))
    say(f"{name}: S={S}, matrix cores {'used' if mfma else 'not used'}, act_int8={a8}")
    if a8:
        check_int8act(dl, x, ridx, rw, y, np.arange(S))
    else:
        check_ffn(dl, x, ridx, rw, y, np.arange(S), TOL_BF16_SMALL if mfma else TOL_FP32,
                  mfma_min_tokens=thr if mfma else None)
