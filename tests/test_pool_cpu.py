"""Slot-pool policy on the host (no device memory): every acquire's decisions are
compared with a reference LRU written from the documented policy (hits are
leased first; a miss takes the lowest free slot, else the least recently used
unleased slot, ties to the lowest slot), plus the documented error codes."""
import numpy as np
import pytest

from gen import inputs as gen
from int4_routed_expert_amd import moe as M


class RefLRU:
    def __init__(self, n_layers, spl):
        self.spl = spl
        self.expert = [[-1] * spl for _ in range(n_layers)]
        self.last = [[0] * spl for _ in range(n_layers)]
        self.clock = 0

    def acquire(self, layer, idx):
        uniq = []
        for e in idx:
            if e not in uniq:
                uniq.append(e)
        self.clock += 1
        ex, last = self.expert[layer], self.last[layer]
        leased = set()
        out = []
        for e in uniq:
            if e in ex:
                s = ex.index(e)
                leased.add(s)
                last[s] = self.clock
                out.append((e, s, 1))
        for e in uniq:
            if e in ex:
                continue
            free = [s for s in range(self.spl) if ex[s] < 0 and s not in leased]
            if free:
                v = free[0]
            else:
                cands = [s for s in range(self.spl) if s not in leased]
                v = min(cands, key=lambda s: (last[s], s))
            ex[v] = e
            last[v] = self.clock
            leased.add(v)
            out.append((e, v, 0))
        return out


def make_pool(n_layers, spl, E=16):
    cfg = gen.LayerConfig(hidden=64, n_experts=E, n_group=4, topk_group=2, top_k=4, moe_inter=32, shared_inter=32)
    pool = M.Pool(M.make_cfg(cfg), n_layers, spl, M.MOE_POOL_NO_DEVICE)
    dummy = np.zeros(8, np.uint8)
    for l in range(n_layers):
        for e in range(E):
            pool.register_host(l, e, dummy)
    return pool


@pytest.mark.parametrize("spl", [4, 6, 9])
def test_lru_trace_matches_reference(spl):
    rng = np.random.default_rng(spl)
    n_layers, E = 3, 16
    pool = make_pool(n_layers, spl, E)
    ref = RefLRU(n_layers, spl)
    hot = [1, 5, 9]
    for it in range(400):
        layer = int(rng.integers(0, n_layers))
        n = int(rng.integers(1, spl + 1))
        # skewed: hot experts often, repeats allowed (the union is taken)
        idx = [int(rng.choice(hot)) if rng.random() < 0.5 else int(rng.integers(0, E)) for _ in range(n)]
        if len(set(idx)) > spl:
            continue
        view, n_miss = pool.acquire(layer, np.array(idx, np.int32))
        got = [tuple(int(v) for v in t) for t in pool.trace()]
        want = ref.acquire(layer, idx)
        assert got == want, (it, layer, idx)
        assert n_miss == sum(1 for t in want if t[2] == 0)
        assert view.n_slots == spl
        pool.release(layer)
    st = pool.stats()
    assert st["hits"] + st["misses"] > 0 and st["acquires"] > 0


def test_pool_errors():
    pool = make_pool(2, 3)
    pool.acquire(0, np.array([1, 2], np.int32))
    with pytest.raises(M.MoeError) as e:
        pool.acquire(0, np.array([1], np.int32))  # layer 0 still leased
    assert e.value.status == M.MOE_ESTALE
    pool.release(0)
    with pytest.raises(M.MoeError) as e:
        pool.release(0)
    assert e.value.status == M.MOE_ESTALE
    with pytest.raises(M.MoeError) as e:
        pool.acquire(1, np.array([1, 2, 3, 4], np.int32))  # union of 4 > 3 slots
    assert e.value.status == M.MOE_ENOSLOT
    with pytest.raises(M.MoeError) as e:
        pool.acquire(1, np.array([16], np.int32))
    assert e.value.status == M.MOE_EINVAL
    with pytest.raises(M.MoeError) as e:
        pool.acquire(2, np.array([1], np.int32))
    assert e.value.status == M.MOE_EINVAL
    # a miss without a registered source
    cfg = gen.LayerConfig(hidden=64, n_experts=8, n_group=2, topk_group=1, top_k=2, moe_inter=32, shared_inter=32)
    bare = M.Pool(M.make_cfg(cfg), 1, 2, M.MOE_POOL_NO_DEVICE)
    with pytest.raises(M.MoeError) as e:
        bare.acquire(0, np.array([3], np.int32))
    assert e.value.status == M.MOE_ENULL


def test_leased_slots_are_never_evicted():
    pool = make_pool(1, 4)
    pool.acquire(0, np.array([0, 1, 2, 3], np.int32))
    pool.release(0)
    pool.acquire(0, np.array([0, 1], np.int32))  # hits, leased
    pool.release(0)
    pool.acquire(0, np.array([4, 5, 0], np.int32))  # must evict 2 and 3 (least recent), not 0
    tr = pool.trace()
    evicted_slots = {int(t[1]) for t in tr if t[2] == 0}
    assert evicted_slots == {2, 3}
    pool.release(0)
