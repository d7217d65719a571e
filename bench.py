"""MoE-layer benchmark: GLM-5.2-shaped decode, one token per step, one MI355X.

A step is one pass of the whole layer (moe_route then moe_ffn through the C ABI)
for one token.  Inputs are resident in HBM before timing starts: L layer
instances (256 routed + 1 shared int4 experts each, 5.46 GB per layer) and a
pool of 1024 distinct seeded tokens; consecutive steps rotate over layers and
tokens so that no expert set is served from the 256 MB Infinity Cache.  The
timed steps are replayed from HIP graphs captured over the same C-ABI calls.

Prints one JSON line (rank 0).  --gpus above 1 is refused: this path runs on a
single GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
CHUNK = 16  # steps per captured graph


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256 over the sources of the decode kernels (counter readings go stale when they change)."""
    import hashlib
    h = hashlib.sha256()
    for f in ("ffn_gemv.hip", "dot.h", "common.h"):
        with open(os.path.join(ROOT, "int4_routed_expert_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when
    the summary is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path))
    except ValueError:
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def _pmc_means(path: str, counter: str) -> dict:
    """Mean reading (KiB) per dispatch of `counter`, by kernel name, from a rocprofv3 --pmc CSV."""
    import csv
    acc: dict = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            v = acc.setdefault(r["Kernel_Name"], [0.0, 0])
            v[0] += float(r["Counter_Value"])
            v[1] += 1
    return {k: v[0] / v[1] for k, v in acc.items()}


def summarize_pmc(fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str, copy_mib: int,
                  kernels: list) -> None:
    """Writes profiles/traffic_<kernel>.json: HBM bytes per launch from FETCH_SIZE and WRITE_SIZE,
    each scaled by what the same counter reads for a copy kernel that moves copy_mib MiB each way."""
    def one(path, counter, name_part):
        means = _pmc_means(path, counter)
        hit = [v for k, v in means.items() if name_part in k]
        if len(hit) != 1:
            raise SystemExit(f"{path}: expected one kernel matching {name_part!r}, found {len(hit)}")
        return hit[0]
    true_kib = copy_mib * 1024.0
    f_scale = true_kib / one(copy_fetch_csv, "FETCH_SIZE", "k_copy")
    w_scale = true_kib / one(copy_write_csv, "WRITE_SIZE", "k_copy")
    for short in kernels:
        fetch = one(fetch_csv, "FETCH_SIZE", f"k_{short}<")
        write = one(write_csv, "WRITE_SIZE", f"k_{short}<")
        out = {"kernel": short, "source_sha256": kernel_source_hash(),
               "fetch_kib_per_dispatch_raw": fetch, "write_kib_per_dispatch_raw": write,
               "fetch_scale": f_scale, "write_scale": w_scale,
               "bytes_per_launch": (fetch * f_scale + write * w_scale) * 1024.0,
               "calibration": f"copy kernel moving {copy_mib} MiB read + {copy_mib} MiB write"}
        path = os.path.join(ROOT, "profiles", f"traffic_{short}.json")
        with open(path, "w") as fh:
            json.dump(out, fh, indent=1)
            fh.write("\n")
        log(f"{path}: {out['bytes_per_launch'] / 1e6:.2f} MB per launch")


def main() -> int:
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        ap = argparse.ArgumentParser(prog="bench.py --summarize-pmc")
        ap.add_argument("--summarize-pmc", action="store_true")
        ap.add_argument("--fetch", required=True)
        ap.add_argument("--write", required=True)
        ap.add_argument("--copy-fetch", required=True)
        ap.add_argument("--copy-write", required=True)
        ap.add_argument("--copy-mib", type=int, default=1024)
        ap.add_argument("--kernels", default="gateup_s1,down_s1")
        a = ap.parse_args()
        summarize_pmc(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_mib, a.kernels.split(","))
        return 0
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4096)
    ap.add_argument("--warmup", type=int, default=512)
    ap.add_argument("--layers", type=int, default=4, help="resident layer instances rotated per step")
    ap.add_argument("--tokens", type=int, default=1024, help="distinct tokens rotated per step")
    ap.add_argument("--profile-steps", type=int, default=512)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this MoE-layer path runs on one GPU only; --gpus must be 1", file=sys.stderr)
        return 2

    import torch
    from gen import inputs as gen
    from int4_routed_expert_amd import moe as M

    w = gen.WORKLOADS["decode"]
    c = w.cfg
    cfg = M.make_cfg(c)
    E, H, I, k = c.n_experts, c.hidden, c.moe_inter, c.top_k
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sb = M.moe_expert_bytes(cfg, I)
    ssb = M.moe_expert_bytes(cfg, c.shared_inter)

    # ---- resident inputs ------------------------------------------------------
    layers = []
    t0 = time.time()
    stage = gen.empty_expert(c, I)
    for l in range(args.layers):
        slab = torch.empty(E * sb, dtype=torch.uint8, device=dev)
        for e in range(E + 1):
            ex = gen.expert_weights(w, l, e, out=stage if e < E else None)
            parts = [torch.from_numpy(a).to(dev, non_blocking=False) for a in ex.parts()]
            if e < E:
                M.moe_pack_expert(cfg, I, *parts, slab[e * sb:(e + 1) * sb], 1)
            else:
                shared = torch.empty(ssb, dtype=torch.uint8, device=dev)
                M.moe_pack_expert(cfg, c.shared_inter, *parts, shared, 1)
            torch.cuda.current_stream().synchronize()
        layers.append(dict(
            slab=slab, shared=shared, table=torch.arange(E, dtype=torch.int32, device=dev),
            W=torch.from_numpy(gen.router_weights(w, l)).to(dev),
            bias=torch.from_numpy(gen.router_bias(w, l)).to(dev)))
        log(f"layer {l}: {E}+1 experts packed into HBM ({(E * sb + ssb) / 1e9:.2f} GB), {time.time() - t0:.1f}s")
    xs = torch.from_numpy(np.concatenate([gen.tokens(w, layer=0, step=s) for s in range(args.tokens)])).to(dev)
    ws = M.workspace(cfg, 1, device=dev)
    n_out = CHUNK * ((args.tokens + CHUNK - 1) // CHUNK)
    idx = torch.empty((n_out, k), dtype=torch.int32, device=dev)
    wt = torch.empty((n_out, k), dtype=torch.float32, device=dev)
    y = torch.empty((n_out, H), dtype=torch.float32, device=dev)
    views = [M.slot_view(L["slab"], sb, L["table"], E) for L in layers]

    def step(j: int) -> None:
        L = layers[j % len(layers)]
        t = j % args.tokens
        o = j % n_out
        M.moe_route(cfg, xs[t:t + 1], M.MOE_F32, 1, L["W"], L["bias"], idx[o:o + 1], wt[o:o + 1], ws, ws.numel())
        M.moe_ffn(cfg, xs[t:t + 1], M.MOE_F32, 1, idx[o:o + 1], wt[o:o + 1], views[j % len(layers)], L["shared"],
                  y[o:o + 1], ws, ws.numel())

    # ---- HIP graphs over the C-ABI calls ----------------------------------------
    period = int(np.lcm(args.tokens, args.layers))
    n_graphs = (period + CHUNK - 1) // CHUNK
    n_graphs = min(n_graphs, 64)
    s = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(s):
        for j in range(CHUNK):
            step(j)
    torch.cuda.synchronize()
    for gi in range(n_graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for j in range(CHUNK):
                step(gi * CHUNK + j)
        graphs.append(g)
    torch.cuda.synchronize()
    log(f"captured {n_graphs} graphs x {CHUNK} steps")

    steps = CHUNK * ((args.steps + CHUNK - 1) // CHUNK)
    warm = CHUNK * ((args.warmup + CHUNK - 1) // CHUNK)
    for i in range(warm // CHUNK):
        graphs[i % n_graphs].replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps // CHUNK):
        graphs[i % n_graphs].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / steps
    tok_s = steps / elapsed
    layer_bytes = 9 * sb  # 8 routed + 1 shared experts streamed per token
    router_bytes = E * H * 4
    gbps = layer_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"graph replay: {ms_per_step * 1e3:.2f} us/step, {tok_s:.0f} tok/s, {gbps:.0f} GB/s expert bytes")

    # ---- eager loop (reference) and per-kernel event timing ---------------------
    torch.cuda.synchronize()
    te = time.perf_counter()
    n_eager = min(256, steps)
    for j in range(n_eager):
        step(j)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - te) * 1e6 / n_eager
    M.moe_profile_enable(True)
    M.moe_profile_report()
    for j in range(args.profile_steps):
        step(j)
    torch.cuda.synchronize()
    prof = M.moe_profile_report()
    M.moe_profile_enable(False)
    kernels = {name: {"avg_us": ms * 1e3 / n, "launches": n} for name, (ms, n) in prof.items()}
    log("per-kernel (hipEvent) averages:", json.dumps(kernels))
    gu_bytes = 9 * 2 * (I * H // 2 + I * (H // 32) * 2)  # gate+up payload and scales of 9 experts
    gu_us = kernels["gateup_s1"]["avg_us"]
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9

    traffic = measured_traffic("gateup_s1")

    # ---- CPU baseline: the fp64 oracle on a bounded sample ------------------------
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        Wh, bh = gen.router_weights(w, 0), gen.router_bias(w, 0)
        shared_h = gen.expert_weights(w, 0, E)
        done, t_cpu, n_target = 0, 0.0, 1
        while done < n_target:
            xh = gen.tokens(w, layer=0, step=done)
            experts = {E: shared_h}
            ridx, rw, _, _, _ = O.route(c, xh, Wh, bh)  # untimed: generating weights is not oracle work
            for e in ridx[0].tolist():
                experts[e] = gen.expert_weights(w, 0, e)
            tc = time.perf_counter()
            ridx, rw, _, _, _ = O.route(c, xh, Wh, bh)
            O.moe_ffn(c, xh, ridx, rw, experts)
            t_cpu += time.perf_counter() - tc
            done += 1
            if done == 1:
                n_target = int(max(1, min(64, args.cpu_seconds / max(t_cpu, 1e-3))))
        cpu = {"value": done / t_cpu, "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
               "sample": f"{done} decode tokens of layer 0 (route + 8 routed + shared experts, fp64), "
                         f"{t_cpu:.1f} s"}
        log(f"cpu oracle: {cpu['value']:.3f} tok/s on {cpu['cores']} threads")

    out = {
        "metric": "MoE-layer tokens/s and effective int4 weight GB/s (% of HBM peak), GLM-5.2",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "glm52_moe_layer_decode_S1", "hidden": H, "n_experts": E, "n_group": c.n_group,
                   "topk_group": c.topk_group, "top_k": k, "moe_inter": I, "shared_inter": c.shared_inter,
                   "quant": "int4 g32 fp16 scales", "layers_rotated": args.layers, "tokens_rotated": args.tokens,
                   "launch": "hip graphs of 16 steps"},
        "effective_gbps": gbps,
        "pct_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
        "expert_bytes_per_token": layer_bytes,
        "router_bytes_per_token": router_bytes,
        "eager_us_per_step": eager_us,
        "kernels_us": {n: round(v["avg_us"], 3) for n, v in kernels.items()},
        "roofline": {"kernel": "gateup_s1", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": gu_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
