"""Slot pool on the GPU: a stack of layers decoded token by token with experts
streamed from pinned host memory into a small per-layer LRU of HBM slots.  Every
(step, layer) is checked against the fp64 oracle (indices exact, outputs within
2e-3); with poisoning on, every refilled slot is first overwritten with 0xFF
bytes on the side stream, so any read of a slot outside its published lifetime
would corrupt an output."""
import numpy as np
import pytest
import torch

from gen import inputs as gen
from int4_routed_expert_amd import moe as M
from oracle import oracle as O
from tests.devlayer import dev, max_rel_err

pytestmark = pytest.mark.gpu

MID = gen.LayerConfig(hidden=512, n_experts=32, n_group=4, topk_group=2, top_k=4, moe_inter=256, shared_inter=192)


def run_stack(w: gen.Workload, n_layers: int, steps: int, spl: int, flags: int, check_ffn_every: int = 1,
              prefetch: str | None = None, act_int8: int = 0):
    """prefetch: None; "next" (the next (step, layer)'s routing, computed ahead on
    its own input, is prefetched while the current layer's lease is open); or
    "wrong" (random experts of the next layer are prefetched instead).  act_int8:
    the layer runs with int8 activations and is checked against the oracle's
    int8-activation mode (its bar: 5e-3)."""
    c = w.cfg
    cfg = M.make_cfg(c, act_int8=act_int8)
    E, I = c.n_experts, c.moe_inter
    sb = M.moe_expert_bytes(cfg, I)
    host = torch.empty((n_layers * E, sb), dtype=torch.uint8, pin_memory=True)
    hostw = {}
    for l in range(n_layers):
        for e in range(E):
            ex = gen.expert_weights(w, l, e)
            hostw[(l, e)] = ex
            M.pack_expert(cfg, I, *ex.parts(), host[l * E + e].numpy(), 0)
    pool = M.Pool(cfg, n_layers, spl, flags)
    for l in range(n_layers):
        for e in range(E):
            pool.register_host(l, e, host[l * E + e])
    layers = []
    for l in range(n_layers):
        sh = gen.expert_weights(w, l, E)
        shared = torch.zeros(M.moe_expert_bytes(cfg, c.shared_inter), dtype=torch.uint8, device="cuda")
        M.pack_expert(cfg, c.shared_inter, *[dev(a) for a in sh.parts()], shared, 1)
        layers.append(dict(W=gen.router_weights(w, l), b=gen.router_bias(w, l), shared=shared, shared_h=sh))
    torch.cuda.synchronize()
    compute = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ws = M.workspace(cfg, 1)
    ws2 = M.workspace(cfg, 1)
    rng = np.random.default_rng(7)
    worst, n_checked = 0.0, 0
    ys = []
    for step in range(steps):
        for l in range(n_layers):
            L = layers[l]
            xh = gen.tokens(w, layer=l, step=step)
            x = dev(xh)
            idx = torch.empty((1, c.top_k), dtype=torch.int32, device="cuda")
            wt = torch.empty((1, c.top_k), dtype=torch.float32, device="cuda")
            M.moe_route(cfg, x, M.MOE_F32, 1, dev(L["W"]), dev(L["b"]), idx, wt, ws, ws.numel())
            idx_h = idx.cpu().numpy()  # the host decides residency: one sync per layer
            view, n_miss = pool.acquire(l, idx_h, compute, side)
            if prefetch:
                ns, nl = (step, l + 1) if l + 1 < n_layers else (step + 1, 0)
                if prefetch == "next":
                    L2 = layers[nl]
                    i2 = torch.empty((1, c.top_k), dtype=torch.int32, device="cuda")
                    w2 = torch.empty((1, c.top_k), dtype=torch.float32, device="cuda")
                    M.moe_route(cfg, dev(gen.tokens(w, layer=nl, step=ns)), M.MOE_F32, 1, dev(L2["W"]), dev(L2["b"]),
                                i2, w2, ws2, ws2.numel())
                    pred = i2.cpu().numpy()
                else:
                    pred = rng.choice(E, size=c.top_k, replace=False).astype(np.int32)
                pool.prefetch(nl, pred, side)
            y = torch.full((1, c.hidden), float("nan"), device="cuda")
            M.moe_ffn(cfg, x, M.MOE_F32, 1, idx, wt, view, L["shared"], y, ws, ws.numel())
            pool.release(l, compute)
            ys.append(y)
            ridx, rw, _, flags_, _ = O.route(c, xh, L["W"], L["b"])
            assert not flags_.any()
            assert np.array_equal(idx_h, ridx), (step, l)
            if (step * n_layers + l) % check_ffn_every == 0:
                experts = {e: hostw[(l, e)] for e in ridx.ravel().tolist()}
                experts[E] = L["shared_h"]
                ref = O.moe_ffn(c, xh, ridx, rw, experts, act_int8=bool(act_int8))
                err = max_rel_err(y.cpu().numpy(), ref)
                worst = max(worst, err)
                n_checked += 1
                assert err <= (5e-3 if act_int8 else 2e-3), (step, l, err)
    torch.cuda.synchronize()
    st = pool.stats()
    pool.close()
    return st, worst, n_checked, np.concatenate([y.cpu().numpy() for y in ys])


@pytest.mark.parametrize("flags", [0, M.MOE_POOL_POISON])
def test_pool_stack_mid_shape_heavy_churn(flags):
    w = gen.Workload("stack-mid", MID, tokens=1, bias_recipe="hotset", layers=6, steps=8, seed=41)
    st, worst, n, _ = run_stack(w, n_layers=6, steps=8, spl=5, flags=flags)
    print("pool stats", st, "worst", worst, "checked", n, flush=True)
    assert st["misses"] > 6 * 4 and st["evictions"] > 0 and st["hits"] > 0


def test_pool_stack_glm_shape():
    w = gen.WORKLOADS["stack"]
    st, worst, n, _ = run_stack(w, n_layers=2, steps=3, spl=12, flags=M.MOE_POOL_POISON, check_ffn_every=2)
    print("pool stats", st, "worst", worst, "checked", n, flush=True)
    assert st["evictions"] >= 0 and st["misses"] >= 16


@pytest.mark.parametrize("n_layers", [1, 3])
def test_pool_prefetch_is_value_preserving(n_layers):
    """Predictive prefetch (the next layer's routing computed ahead, or random
    mispredictions), with every refilled slot poisoned first: the outputs are
    bitwise those of the run without prefetch and match the oracle; with the
    exact prediction every routed expert is resident at its acquire.  With one
    layer the prefetch targets the layer whose lease is still open."""
    w = gen.Workload("stack-mid", MID, tokens=1, bias_recipe="hotset", layers=n_layers, steps=6, seed=43)
    base, _, _, y0 = run_stack(w, n_layers=n_layers, steps=6, spl=6, flags=M.MOE_POOL_POISON)
    nxt, _, _, y1 = run_stack(w, n_layers=n_layers, steps=6, spl=6, flags=M.MOE_POOL_POISON, prefetch="next")
    bad, _, _, y2 = run_stack(w, n_layers=n_layers, steps=6, spl=6, flags=M.MOE_POOL_POISON, prefetch="wrong")
    print("no prefetch", base, "\nnext", nxt, "\nwrong", bad, flush=True)
    assert np.array_equal(y0, y1) and np.array_equal(y0, y2)
    assert nxt["prefetch_fills"] > 0 and nxt["prefetch_hits"] > 0 and bad["prefetch_fills"] > 0
    if n_layers > 1:  # exact predictions of other layers: acquires after the first one only hit
        assert nxt["misses"] <= w.cfg.top_k


@pytest.mark.parametrize("fmt", [1, 2], ids=["q4row", "q8row"])
def test_pool_row_scaled_experts(fmt):
    """The slot pool with row-scaled experts (slots sized by the format), heavy
    churn and poisoned refills: every (step, layer) matches the oracle."""
    cfg = gen.LayerConfig(**{**MID.__dict__, "weight_format": fmt})
    w = gen.Workload("stack-mid", cfg, tokens=1, bias_recipe="hotset", layers=3, steps=5, seed=47)
    st, worst, n, _ = run_stack(w, n_layers=3, steps=5, spl=5, flags=M.MOE_POOL_POISON)
    print("pool stats", st, "worst", worst, "checked", n, flush=True)
    assert st["misses"] > 3 * 4 and st["evictions"] > 0


def test_stale_view_after_refill_is_poisoned():
    """Generation tags: a view kept after its release, used once a prefetch has
    refilled some of its slots with other experts (the device table still names
    those slots: a prefetch publishes nothing), gives NaN rows for the tokens of
    the refilled experts and bitwise the earlier rows for the others, on the
    one-token, few-token and matrix-core paths; the host check reports the view
    stale.  The same view with its tags removed reads the other experts'
    weights: finite rows that differ from the true ones."""
    c = MID
    w = gen.Workload("stale", c, tokens=1, seed=53)
    cfg = M.make_cfg(c, mfma_min_tokens=4)
    E, I, k = c.n_experts, c.moe_inter, c.top_k
    sb = M.moe_expert_bytes(cfg, I)
    host = torch.empty((E, sb), dtype=torch.uint8, pin_memory=True)
    for e in range(E):
        M.pack_expert(cfg, I, *gen.expert_weights(w, 0, e).parts(), host[e].numpy(), 0)
    sh = gen.expert_weights(w, 0, E)
    shared = torch.zeros(M.moe_expert_bytes(cfg, c.shared_inter), dtype=torch.uint8, device="cuda")
    M.pack_expert(cfg, c.shared_inter, *[dev(a) for a in sh.parts()], shared, 1)
    pool = M.Pool(cfg, 1, 2 * k + 2, M.MOE_POOL_POISON)
    for e in range(E):
        pool.register_host(0, e, host[e])
    A = np.array([3, 7, 11, 19], np.int32)   # slots 0..3 (first appearance order)
    B = np.array([5, 13, 21, 30], np.int32)  # slots 4..7
    compute, side = torch.cuda.current_stream(), torch.cuda.Stream()
    view, n_miss = pool.acquire(0, np.concatenate([A, B]), compute, side)
    assert n_miss == 2 * k
    pool.release(0, compute)
    S = 8
    x = dev(gen.tokens(w.with_(tokens=S), step=5))
    rows = np.stack([A if t % 2 == 0 else B for t in range(S)]).astype(np.int32)
    wt = dev(np.full((S, k), c.routed_scaling_factor / k, np.float32))
    ws = M.workspace(cfg, S)

    def run(v):
        out = []
        for sl in (slice(0, 1), slice(1, 2), slice(0, 2), slice(0, S)):  # one token, two tokens, matrix cores
            n = sl.stop - sl.start
            y = torch.full((n, c.hidden), 7.0, device="cuda")
            M.moe_ffn(cfg, x[sl], M.MOE_F32, n, dev(rows[sl]), wt[sl], v, shared, y, ws, ws.numel())
            out.append(y)
        torch.cuda.synchronize()
        return [y.cpu().numpy() for y in out]

    before = run(view)
    assert all(np.isfinite(y).all() for y in before)
    # a prefetch of four other experts: two free slots, then the two least recently used (ties: lowest
    # slot), i.e. slots 0 and 1 that hold A[0] and A[1]
    assert pool.prefetch(0, np.array([0, 1, 2, 4], np.int32), side) == 4
    side.synchronize()
    assert pool.check_view(0, view) == M.MOE_ESTALE
    after = run(view)
    for got, ref, sl in zip(after, before, (slice(0, 1), slice(1, 2), slice(0, 2), slice(0, S))):
        toks = np.arange(sl.start, sl.stop)
        for i, t in enumerate(toks):
            if t % 2 == 0:  # A: two of its experts were refilled
                assert np.isnan(got[i]).all(), (sl, t)
            else:
                assert np.array_equal(got[i], ref[i]), (sl, t)
    untagged = M.slot_view(view.base, view.slot_bytes, view.table, view.n_slots)
    raw = run(untagged)
    assert np.isfinite(raw[0]).all() and not np.array_equal(raw[0], before[0])
    pool.close()


@pytest.mark.parametrize("fmt", [0, 2], ids=["q4g32", "q8row"])
def test_pool_int8_activations(fmt):
    """The slot pool with int8 activations: heavy churn, poisoned refills and
    predictive prefetch; every (step, layer) against the oracle's int8 mode, and
    the prefetch run bitwise equal to the plain one."""
    cfg = gen.LayerConfig(**{**MID.__dict__, "weight_format": fmt})
    w = gen.Workload("stack-mid", cfg, tokens=1, bias_recipe="hotset", layers=3, steps=5, seed=59)
    st, worst, n, y0 = run_stack(w, n_layers=3, steps=5, spl=5, flags=M.MOE_POOL_POISON, act_int8=1)
    st2, _, _, y1 = run_stack(w, n_layers=3, steps=5, spl=5, flags=M.MOE_POOL_POISON, act_int8=1, prefetch="next")
    print("pool stats", st, st2, "worst", worst, "checked", n, flush=True)
    assert st["misses"] > 3 * 4 and st["evictions"] > 0
    assert np.array_equal(y0, y1) and st2["prefetch_hits"] > 0
