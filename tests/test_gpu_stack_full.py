"""The 75-layer stack decode at its stated size, through the slot pool.

75 layers x 256 routed experts live in pinned host memory (the 19,200 logical
experts alias onto 1,024 distinct weight blobs; the pool still treats every
(layer, expert) as its own expert), 100 HBM slots per layer (159 GB), one token
per step for 64 steps from a cold pool, misses filled on a side stream.  The run
is made twice, without and with predictive prefetch (each next layer routed one
layer ahead on its own input and its experts prefetched while the current layer
computes), in the launch sequence the stack benchmark uses.

Checks: the router's indices on all 4,800 (step, layer) pairs equal the oracle's
(weights within 1e-6 rsf); the FFN outputs of steps 0, 1, 31 and 63 on all 75
layers are within the fp32 bar of the oracle (checking all 4,800 would take the
oracle about ten minutes); the prefetch run's outputs are bitwise those of the
plain run on every (step, layer); the pool's statistics show the cold start,
the evictions and, with prefetch, hits at every acquire after the first.
"""
import numpy as np
import pytest
import torch

from gen import inputs as gen
from int4_routed_expert_amd import moe as M
from oracle import oracle as O
from tests.devlayer import dev, max_rel_err

pytestmark = pytest.mark.gpu

CHECK_STEPS = (0, 1, 31, 63)
SLOTS_PER_LAYER = 100


def say(*a):
    print(*a, flush=True)


def run(w, cfg, host, layers, xs, prefetch: bool):
    c = w.cfg
    E, NL, steps = c.n_experts, w.layers, w.steps
    pool = M.Pool(cfg, NL, SLOTS_PER_LAYER, 0)
    for l in range(NL):
        for e in range(E):
            pool.register_host(l, e, host[gen.blob_of(w, l, e)[1]])
    compute, side = torch.cuda.current_stream(), torch.cuda.Stream()
    ws, ws2 = M.workspace(cfg, 1), M.workspace(cfg, 1)
    idx_all = np.zeros((steps, NL, c.top_k), np.int32)
    w_all = np.zeros((steps, NL, c.top_k), np.float32)
    y_all = torch.empty((steps, NL, c.hidden), dtype=torch.float32, device="cuda")
    seq = [(st, l) for st in range(steps) for l in range(NL)]
    idx = [torch.empty((1, c.top_k), dtype=torch.int32, device="cuda") for _ in range(2)]
    wt = [torch.empty((1, c.top_k), dtype=torch.float32, device="cuda") for _ in range(2)]
    misses = 0

    def route(b, st, l, buf):
        M.moe_route(cfg, xs[l][st:st + 1], M.MOE_F32, 1, layers[l]["W"], layers[l]["bias"], idx[b], wt[b], buf,
                    buf.numel())

    if prefetch:
        route(0, *seq[0], ws2)
    for j, (st, l) in enumerate(seq):
        b = j % 2 if prefetch else 0
        if not prefetch:
            route(0, st, l, ws)
        ih = idx[b].cpu().numpy()  # the host decides residency
        view, n_miss = pool.acquire(l, ih, compute, side)
        misses += n_miss
        if prefetch and j + 1 < len(seq):
            route(1 - b, *seq[j + 1], ws2)  # the next layer's routing, ahead of this layer's FFN
        M.moe_ffn(cfg, xs[l][st:st + 1], M.MOE_F32, 1, idx[b], wt[b], view, layers[l]["shared"], y_all[st, l:l + 1],
                  ws, ws.numel())
        pool.release(l, compute)
        if prefetch and j + 1 < len(seq):
            pool.prefetch(seq[j + 1][1], idx[1 - b].cpu().numpy(), side)
        idx_all[st, l] = ih[0]
        w_all[st, l] = wt[b].cpu().numpy()[0]
        if l == NL - 1 and st % 16 == 0:
            say(f"  step {st}: {misses} misses so far")
    torch.cuda.synchronize()
    st_ = pool.stats()
    pool.close()
    return idx_all, w_all, y_all.cpu().numpy(), st_


@pytest.fixture(scope="module")
def stack():
    w = gen.WORKLOADS["stack"]
    c = w.cfg
    cfg = M.make_cfg(c)
    E, I, NL = c.n_experts, c.moe_inter, w.layers
    sb = M.moe_expert_bytes(cfg, I)
    torch.cuda.empty_cache()
    say(f"packing {w.n_blobs} blobs into pinned host memory ({w.n_blobs * sb / 1e9:.1f} GB)")
    host = torch.empty((w.n_blobs, sb), dtype=torch.uint8, pin_memory=True)
    stage_d = torch.empty(sb, dtype=torch.uint8, device="cuda")
    stage = gen.empty_expert(c, I)
    done = set()
    for l in range(NL):
        for e in range(E):
            b = gen.blob_of(w, l, e)[1]
            if b not in done:
                gen.expert_weights(w, l, e, out=stage)
                M.pack_expert(cfg, I, *[dev(a) for a in stage.parts()], stage_d, 1)
                host[b].copy_(stage_d)
                done.add(b)
    layers = []
    for l in range(NL):
        sh = gen.expert_weights(w, l, E)
        shared = torch.empty(M.moe_expert_bytes(cfg, c.shared_inter), dtype=torch.uint8, device="cuda")
        M.pack_expert(cfg, c.shared_inter, *[dev(a) for a in sh.parts()], shared, 1)
        layers.append(dict(W=dev(gen.router_weights(w, l)), bias=dev(gen.router_bias(w, l)), shared=shared))
    xs = [dev(np.concatenate([gen.tokens(w, layer=l, step=s) for s in range(w.steps)])) for l in range(NL)]
    torch.cuda.synchronize()
    say("plain run")
    plain = run(w, cfg, host, layers, xs, prefetch=False)
    say("prefetch run")
    pre = run(w, cfg, host, layers, xs, prefetch=True)
    del host
    return w, plain, pre


def test_stack_router_all_pairs(stack):
    w, (idx, wts, _, st), _ = stack
    c = w.cfg
    for l in range(w.layers):
        x = np.concatenate([gen.tokens(w, layer=l, step=s) for s in range(w.steps)])
        ridx, rw, _, flags, _ = O.route(c, x, gen.router_weights(w, l), gen.router_bias(w, l))
        assert not flags.any(), l
        assert np.array_equal(idx[:, l], ridx), l
        assert np.abs(wts[:, l] - rw).max() <= 1e-6 * c.routed_scaling_factor, l
    say("pool stats (plain)", st)
    assert st["acquires"] == w.layers * w.steps
    assert st["misses"] >= w.layers * c.top_k and st["evictions"] > 0 and st["hits"] > st["misses"]


def check_outputs(stack, steps):
    w, (idx, wts, y, _), _ = stack
    c = w.cfg
    E = c.n_experts
    worst = 0.0
    for l in range(w.layers):
        x = np.concatenate([gen.tokens(w, layer=l, step=s) for s in steps])
        ridx, rw, _, _, _ = O.route(c, x, gen.router_weights(w, l), gen.router_bias(w, l))
        experts = {e: gen.expert_weights(w, l, e) for e in set(ridx.ravel().tolist())}
        experts[E] = gen.expert_weights(w, l, E)
        ref = O.moe_ffn(c, x, ridx, rw, experts)
        err = max_rel_err(y[list(steps), l], ref)
        worst = max(worst, err)
        assert err <= 2e-3, (l, err)
    say(f"steps {steps}: worst max rel err {worst:.3e} over {w.layers} layers")


def test_stack_outputs_steps_0_1(stack):
    check_outputs(stack, CHECK_STEPS[:2])


def test_stack_outputs_steps_31_63(stack):
    check_outputs(stack, CHECK_STEPS[2:])


def test_stack_prefetch_run_is_bitwise_the_plain_run(stack):
    w, (idx, wts, y, _), (idx2, wts2, y2, st2) = stack
    assert np.array_equal(idx, idx2) and np.array_equal(wts, wts2)
    assert np.array_equal(y, y2)
    assert np.isfinite(y).all()
    say("pool stats (prefetch)", st2)
    assert st2["prefetch_fills"] > 0 and st2["prefetch_hits"] > 0
    assert st2["misses"] <= w.cfg.top_k  # every acquire after the first finds its experts prefetched
