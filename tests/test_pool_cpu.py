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
        self.leased = [set() for _ in range(n_layers)]  # slots of an open acquire

    def _victim(self, layer, busy):
        ex, last = self.expert[layer], self.last[layer]
        free = [s for s in range(self.spl) if ex[s] < 0 and s not in busy]
        if free:
            return free[0]
        cands = [s for s in range(self.spl) if s not in busy]
        return min(cands, key=lambda s: (last[s], s)) if cands else -1

    def prefetch(self, layer, idx):
        """Predictive prefetch: resident experts become recently used, missing ones
        take victims like misses (never a leased slot, nor one of the prediction's
        own slots); returns the copies made."""
        uniq = []
        for e in idx:
            if e not in uniq:
                uniq.append(e)
        self.clock += 1
        ex, last = self.expert[layer], self.last[layer]
        busy = set(self.leased[layer])  # plus the prediction's own slots during the call
        for e in uniq:
            if e in ex:
                last[ex.index(e)] = self.clock
                busy.add(ex.index(e))
        fills = 0
        for e in uniq:
            if e in ex:
                continue
            v = self._victim(layer, busy)
            if v < 0:
                break
            ex[v] = e
            last[v] = self.clock
            busy.add(v)
            fills += 1
        return fills

    def release(self, layer):
        self.leased[layer] = set()

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
        self.leased[layer] = leased
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
    assert e.value.status == M.MOE_ELEASE
    pool.release(0)
    with pytest.raises(M.MoeError) as e:
        pool.release(0)
    assert e.value.status == M.MOE_ELEASE
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


@pytest.mark.parametrize("spl", [4, 6])
def test_prefetch_policy_matches_reference(spl):
    """Random acquires, releases and predictive prefetches (some while the layer
    holds a lease, some of experts that are never acquired): every acquire's
    decisions and every prefetch's copy count follow the reference policy, and a
    prefetched expert is a hit at the next acquire."""
    rng = np.random.default_rng(100 + spl)
    n_layers, E = 2, 12
    pool = make_pool(n_layers, spl, E)
    ref = RefLRU(n_layers, spl)
    open_lease = [False] * n_layers
    pf_hits_ref = 0
    pending = [set() for _ in range(n_layers)]  # prefetched, not yet acquired
    for it in range(600):
        layer = int(rng.integers(0, n_layers))
        op = rng.random()
        idx = [int(rng.integers(0, E)) for _ in range(int(rng.integers(1, spl + 1)))]
        if len(set(idx)) > spl:
            continue
        if op < 0.35:
            n_fill = pool.prefetch(layer, np.array(idx, np.int32))
            want = ref.prefetch(layer, idx)
            assert n_fill == want, (it, layer, idx)
            # a prefetched slot stays "prefetched" until an acquire leases it or it is refilled
            ex = ref.expert[layer]
            pending[layer] = {e for e in pending[layer] if e in ex} | {e for e in set(idx) if e in ex}
        elif not open_lease[layer]:
            _, n_miss = pool.acquire(layer, np.array(idx, np.int32))
            got = [tuple(int(v) for v in t) for t in pool.trace()]
            want = ref.acquire(layer, idx)
            assert got == want, (it, layer, idx)
            hits = {t[0] for t in want if t[2] == 1}
            pf_hits_ref += len(hits & pending[layer])
            pending[layer] -= hits
            pending[layer] = {e for e in pending[layer] if e in ref.expert[layer]}
            open_lease[layer] = True
        else:
            pool.release(layer)
            ref.release(layer)
            open_lease[layer] = False
    st = pool.stats()
    assert st["prefetches"] > 0 and st["prefetch_fills"] > 0


def test_prefetch_then_acquire_hits_and_leases_are_kept():
    pool = make_pool(1, 4)
    assert pool.prefetch(0, np.array([3, 7], np.int32)) == 2
    assert pool.prefetch(0, np.array([3, 7], np.int32)) == 0  # resident: no copy
    _, n_miss = pool.acquire(0, np.array([7, 3], np.int32))
    assert n_miss == 0 and pool.stats()["prefetch_hits"] == 2
    # with the lease open, a prediction can only use the two unleased slots
    assert pool.prefetch(0, np.array([1, 2, 4, 5], np.int32)) == 2
    tr_slots = {int(t[1]) for t in pool.trace()}
    pool.release(0)
    _, n_miss = pool.acquire(0, np.array([3, 7], np.int32))  # still resident in their slots
    assert n_miss == 0 and {int(t[1]) for t in pool.trace()} == tr_slots
    pool.release(0)
    with pytest.raises(M.MoeError) as e:
        pool.prefetch(0, np.array([1, 2, 3, 4, 5], np.int32))  # union of 5 > 4 slots
    assert e.value.status == M.MOE_ENOSLOT


def test_view_staleness_on_the_host():
    """moe_pool_check_view: a view is current while its lease is open and after
    its release until a slot of its layer is refilled (by an acquire miss or a
    prefetch); then it is stale.  Hits and other layers' fills leave it current."""
    pool = make_pool(2, 3)
    v1, _ = pool.acquire(0, np.array([1, 2], np.int32))
    assert pool.check_view(0, v1) == M.MOE_OK
    pool.release(0)
    assert pool.check_view(0, v1) == M.MOE_OK
    v2, n_miss = pool.acquire(0, np.array([2, 1], np.int32))  # all hits: nothing refilled
    assert n_miss == 0
    pool.release(0)
    assert pool.check_view(0, v1) == M.MOE_OK and pool.check_view(0, v2) == M.MOE_OK
    pool.acquire(1, np.array([5, 6, 7], np.int32))  # another layer's fills
    pool.release(1)
    assert pool.check_view(0, v1) == M.MOE_OK
    v3, n_miss = pool.acquire(0, np.array([3], np.int32))  # a miss: a slot of layer 0 is filled
    assert n_miss == 1
    assert pool.check_view(0, v1) == M.MOE_ESTALE and pool.check_view(0, v2) == M.MOE_ESTALE
    assert pool.check_view(0, v3) == M.MOE_OK  # its own lease is open
    pool.release(0)
    assert pool.check_view(0, v3) == M.MOE_OK
    assert pool.prefetch(0, np.array([9], np.int32)) == 1  # a prefetch refills a slot
    assert pool.check_view(0, v3) == M.MOE_ESTALE
    with pytest.raises(M.MoeError) as e:
        pool.check_view(5, v3)
    assert e.value.status == M.MOE_EINVAL
