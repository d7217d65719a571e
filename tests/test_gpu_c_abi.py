"""The library driven from plain C, with no Python in the GPU path: a C11 program
(compiled here with gcc against include/moe.h, the HIP runtime's C API and
libmoe.so) reads a layer and a batch from files, packs the experts on the host,
copies them into hipMalloc'd memory, runs moe_layer on a stream of its own and
writes idx, w and y back; the test checks them against the oracle (indices
exactly, weights within 1e-6 rsf), for one token and a four-token batch of the
tiny layer (exact paths: outputs within the fp32 bar) and for a 40-token batch
(bf16 matrix cores for the experts with at least 3 tokens: outputs within the
same bar of the oracle with bf16 operands for those experts)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from gen import inputs as gen
from oracle import oracle as O
from tests.devlayer import matrix_core_experts, max_rel_err
from tests.test_gpu_parity import TOL_BF16_OPS, TOL_FP32, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SRC = r"""
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include "moe.h"

static void *slurp(const char *dir, const char *name, size_t *n) {
  char p[4096];
  snprintf(p, sizeof p, "%s/%s", dir, name);
  FILE *f = fopen(p, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", p); exit(2); }
  fseek(f, 0, SEEK_END);
  *n = (size_t)ftell(f);
  fseek(f, 0, SEEK_SET);
  void *b = malloc(*n ? *n : 1);
  if (fread(b, 1, *n, f) != *n) { fprintf(stderr, "short read %s\n", p); exit(2); }
  fclose(f);
  return b;
}
#define HIP(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_)); return 3; } } while (0)
#define MOE(x) do { int r_ = (x); if (r_ != MOE_OK) { fprintf(stderr, "%s: %s\n", #x, moe_status_string(r_)); return 4; } } while (0)

int main(int argc, char **argv) {
  if (argc != 2) return 1;
  const char *dir = argv[1];
  size_t n;
  int32_t *dims = (int32_t *)slurp(dir, "dims.bin", &n);  /* H E G Gk k I Is S */
  moe_cfg c = {0};
  c.hidden = dims[0]; c.n_experts = dims[1]; c.n_group = dims[2]; c.topk_group = dims[3]; c.top_k = dims[4];
  c.moe_inter = dims[5]; c.shared_inter = dims[6]; c.group_size = 32; c.routed_scaling_factor = 2.5f;
  c.norm_topk_prob = 1; c.mfma_min_tokens = 3; c.weight_format = MOE_WF_Q4_G32; c.act_int8 = 0;
  const int S = dims[7], H = c.hidden, E = c.n_experts, I = c.moe_inter, Is = c.shared_inter, k = c.top_k;
  MOE(moe_validate_cfg(&c));
  const int64_t sb = moe_expert_bytes(&c, I), ssb = moe_expert_bytes(&c, Is);
  uint8_t *slab_h = (uint8_t *)calloc((size_t)E, (size_t)sb), *shared_h = (uint8_t *)calloc(1, (size_t)ssb);
  for (int e = 0; e <= E; ++e) {  /* expert E is the shared one */
    char name[64];
    const int inter = e < E ? I : Is;
    void *q[6];
    for (int j = 0; j < 6; ++j) {
      snprintf(name, sizeof name, "e%d_%d.bin", e, j);
      q[j] = slurp(dir, name, &n);
    }
    MOE(moe_pack_expert(&c, inter, q[0], q[1], q[2], q[3], q[4], q[5], e < E ? slab_h + (size_t)e * sb : shared_h, 0,
                        NULL));
    for (int j = 0; j < 6; ++j) free(q[j]);
  }
  float *x_h = (float *)slurp(dir, "x.bin", &n), *W_h = (float *)slurp(dir, "W.bin", &n);
  float *b_h = (float *)slurp(dir, "bias.bin", &n);
  int32_t *table_h = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  for (int e = 0; e < E; ++e) table_h[e] = e;
  void *slab, *shared, *x, *W, *bias, *table, *idx, *w, *y, *ws;
  const size_t wsb = moe_workspace_bytes(&c, S);
  HIP(hipMalloc(&slab, (size_t)E * sb)); HIP(hipMalloc(&shared, (size_t)ssb));
  HIP(hipMalloc(&x, sizeof(float) * (size_t)S * H)); HIP(hipMalloc(&W, sizeof(float) * (size_t)E * H));
  HIP(hipMalloc(&bias, sizeof(float) * (size_t)E)); HIP(hipMalloc(&table, sizeof(int32_t) * (size_t)E));
  HIP(hipMalloc(&idx, sizeof(int32_t) * (size_t)S * k)); HIP(hipMalloc(&w, sizeof(float) * (size_t)S * k));
  HIP(hipMalloc(&y, sizeof(float) * (size_t)S * H)); HIP(hipMalloc(&ws, wsb));
  HIP(hipMemcpy(slab, slab_h, (size_t)E * sb, hipMemcpyHostToDevice));
  HIP(hipMemcpy(shared, shared_h, (size_t)ssb, hipMemcpyHostToDevice));
  HIP(hipMemcpy(x, x_h, sizeof(float) * (size_t)S * H, hipMemcpyHostToDevice));
  HIP(hipMemcpy(W, W_h, sizeof(float) * (size_t)E * H, hipMemcpyHostToDevice));
  HIP(hipMemcpy(bias, b_h, sizeof(float) * (size_t)E, hipMemcpyHostToDevice));
  HIP(hipMemcpy(table, table_h, sizeof(int32_t) * (size_t)E, hipMemcpyHostToDevice));
  hipStream_t st;
  HIP(hipStreamCreate(&st));
  MOE(moe_workspace_init(ws, wsb, st));
  moe_slot_view view = {slab, sb, (const int32_t *)table, E, NULL, NULL, 0};
  MOE(moe_layer(&c, x, MOE_F32, S, (const float *)W, (const float *)bias, (int32_t *)idx, (float *)w, &view, shared,
                (float *)y, ws, wsb, st));
  HIP(hipStreamSynchronize(st));
  int32_t *idx_h = (int32_t *)malloc(sizeof(int32_t) * (size_t)S * k);
  float *w_h = (float *)malloc(sizeof(float) * (size_t)S * k), *y_h = (float *)malloc(sizeof(float) * (size_t)S * H);
  HIP(hipMemcpy(idx_h, idx, sizeof(int32_t) * (size_t)S * k, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(w_h, w, sizeof(float) * (size_t)S * k, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(y_h, y, sizeof(float) * (size_t)S * H, hipMemcpyDeviceToHost));
  char p[4096];
  snprintf(p, sizeof p, "%s/out.bin", dir);
  FILE *f = fopen(p, "wb");
  fwrite(idx_h, sizeof(int32_t), (size_t)S * k, f);
  fwrite(w_h, sizeof(float), (size_t)S * k, f);
  fwrite(y_h, sizeof(float), (size_t)S * H, f);
  fclose(f);
  HIP(hipStreamDestroy(st));
  printf("ok\n");
  return 0;
}
"""


@pytest.fixture(scope="module")
def c_program(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    d = tmp_path_factory.mktemp("c_abi")
    src = d / "layer.c"
    src.write_text(C_SRC)
    exe = d / "layer"
    lib_dir = os.path.join(ROOT, "int4_routed_expert_amd")
    subprocess.check_call([gcc, "-std=c11", "-O1", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                           str(src), "-L", lib_dir, "-lmoe", f"-Wl,-rpath,{lib_dir}", "-L", "/opt/rocm/lib",
                           "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)])
    return exe


@pytest.mark.parametrize("S", [1, 4, 40])
def test_moe_layer_from_c(c_program, tmp_path, S):
    w = gen.WORKLOADS["tiny"].with_(tokens=S)
    c = w.cfg
    E, H, k = c.n_experts, c.hidden, c.top_k
    np.array([H, E, c.n_group, c.topk_group, k, c.moe_inter, c.shared_inter, S], np.int32).tofile(tmp_path / "dims.bin")
    x = gen.tokens(w, step=2024 + S)
    x.astype(np.float32).tofile(tmp_path / "x.bin")
    Wr, bias = gen.router_weights(w, 0), gen.router_bias(w, 0)
    Wr.astype(np.float32).tofile(tmp_path / "W.bin")
    bias.astype(np.float32).tofile(tmp_path / "bias.bin")
    experts = {}
    for e in range(E + 1):
        ex = gen.expert_weights(w, 0, e)
        experts[e] = ex
        for j, a in enumerate(ex.parts()):
            np.ascontiguousarray(a).tofile(tmp_path / f"e{e}_{j}.bin")
    r = subprocess.run([str(c_program), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = np.fromfile(tmp_path / "out.bin", np.uint8)
    idx = out[:S * k * 4].view(np.int32).reshape(S, k)
    wt = out[S * k * 4:S * k * 8].view(np.float32).reshape(S, k)
    y = out[S * k * 8:].view(np.float32).reshape(S, H)
    ridx, rw, _, flags, _ = O.route(c, x, Wr, bias)
    assert not flags.any()
    assert np.array_equal(idx, ridx)
    assert np.abs(wt - rw).max() <= 1e-6 * c.routed_scaling_factor
    mc = matrix_core_experts(ridx, E, c.shared_inter, 3)
    assert bool(mc) == (S > 4)
    ref = O.moe_ffn(c, x, ridx, rw, experts, bf16_experts=mc)
    err = max_rel_err(y, ref)
    say(f"S={S}: {len(mc)} experts on the matrix cores, max rel err {err:.3e}")
    assert err <= (TOL_BF16_OPS if mc else TOL_FP32)
