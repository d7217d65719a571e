// HBM expert-slot pool: a per-layer LRU cache of packed experts in one device
// slab, filled from pinned host memory on a side stream.
//
// Source: "GLM-5.2 on a 32 GB Mac - native MLX port of the Colibri hierarchy",
// N3 (an explicit residency manager: a slot is resident, loading or leased; it
// is reused only after its consumer is done, and a slot whose copy is still
// running is never handed out), "G3 implementation status" (a fixed number of
// LRU slots per layer with a deterministic tie rule, the batch union, work on
// resident experts queued ahead of the reads of missing ones); the
// colibri README "What's implemented" (per-layer LRU of streamed experts); the
// strata audit's slot map (residency changes by writing one table entry).
//
// Per layer the pool owns `slots_per_layer` slots and a device table
// table[e] = slot or -1.  acquire() resolves the union of the experts named by a
// routing: hits are leased, misses take a free slot or evict the least recently
// used unleased slot (ties: the lowest slot), are copied from the registered host
// source on the side stream after the victim's last consumer has finished, and
// are published in the device table on the compute stream only after their copy
// completed (the compute stream waits on the copy's event).  release() records
// the consumer-done event of every leased slot.
//
// prefetch() (the same page, "What Colibri is actually doing", item 10,
// predictive prefetch: real loads only for a future layer, residency rechecked,
// no partially filled slot published) fills a predicted union the same way but
// leases nothing and publishes nothing: each copied slot keeps its own copy
// event and is marked pending; the next acquire of the layer makes its compute
// stream wait for the pending slots it leases and uploads the table, in which a
// pending slot that it neither leases nor finds complete is still absent (-1).
// Any later copy into a pending slot waits for the earlier copy first.
//
// Generations (N3: generation-tagged slots, so that a stale user cannot
// consume storage reused for another expert): every fill takes a new pool-wide
// number, written into the slot's device generation entry on the side stream
// before the copy; each table upload carries, next to table[e], the generation
// of e's slot.  Kernels given the view use expert e only while the two agree.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "common.h"

using namespace moe;

struct moe_pool {
  moe_cfg cfg;
  int n_layers = 0, spl = 0;  // slots per layer
  int E = 0;
  int64_t slot_bytes = 0;
  bool device = true;
  bool poison = false;
  uint8_t *slab = nullptr;        // device: n_layers * spl slots
  int32_t *d_tables = nullptr;    // device: [n_layers][2E]: table[e], then the generation of e's slot
  uint32_t *d_slot_gen = nullptr; // device: [n_layers][spl] generation of each slot's content
  int32_t *h_stage = nullptr;     // pinned: [n_layers][2E] staging for table uploads
  std::vector<hipEvent_t> table_ev;  // per layer: staging buffer's last upload
  std::vector<int32_t> table;     // host mirror [n_layers][E]
  std::vector<const void *> src;  // [n_layers][E] pinned host sources
  struct Slot {
    int expert = -1;
    uint64_t last_use = 0;  // LRU clock of the last acquire
    uint32_t gen = 0;       // pool-wide generation of the slot's content (0: never filled)
    bool leased = false;
    hipEvent_t done = nullptr;  // consumer-done event (valid when used)
    bool has_done = false;
    hipEvent_t fill_ev = nullptr;  // copy-done event of a prefetch
    bool pending = false;          // prefetched; no acquire has waited for the copy yet
  };
  std::vector<Slot> slots;  // [n_layers][spl]
  std::vector<int> leased_layer;  // per layer: number of slots leased by the open acquire, -1 none
  std::vector<std::vector<int>> lease_list;
  std::vector<hipEvent_t> ev_pool;
  std::vector<char> table_dirty;  // per layer: device table differs from the host table
  std::vector<uint64_t> lease_clock;  // per layer: clock of the open acquire
  std::vector<uint64_t> fill_clock;   // per layer: clock of the latest fill
  uint64_t clock = 0;
  uint32_t gen_counter = 0;
  // statistics
  uint64_t hits = 0, misses = 0, evictions = 0, fill_bytes = 0, acquires = 0;
  uint64_t prefetches = 0, prefetch_fills = 0, prefetch_hits = 0;
  std::vector<int32_t> trace;  // last acquire: (expert, slot, hit) triples
};

static hipEvent_t get_event(moe_pool *p) {
  if (!p->ev_pool.empty()) {
    hipEvent_t e = p->ev_pool.back();
    p->ev_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
  return e;
}

// Victim for a miss of `layer`: a free slot (lowest) first, else the least
// recently used unleased slot (ties: lowest); -1 if every slot is leased.
static int pick_victim(moe_pool *p, int layer) {
  moe_pool::Slot *base = &p->slots[(size_t)layer * p->spl];
  for (int s = 0; s < p->spl; ++s)
    if (base[s].expert < 0 && !base[s].leased) return s;
  int victim = -1;
  for (int s = 0; s < p->spl; ++s)
    if (!base[s].leased && (victim < 0 || base[s].last_use < base[victim].last_use)) victim = s;
  return victim;
}

// One 32-bit store, launched on the side stream (a kernel rather than a memset
// node, so the same sequence can sit in a captured graph).
__global__ void k_store_u32(uint32_t *dst, uint32_t v) {
  if (threadIdx.x == 0) *dst = v;
}

// Enqueues the copy of expert e into slot s of `layer` on `ss`, after the slot's
// last consumer and (for a pending prefetch) its last copy; the slot's new
// generation is stored before the copy starts.
static hipError_t enqueue_fill(moe_pool *p, int layer, int e, int s, hipStream_t ss) {
  moe_pool::Slot &sl = p->slots[(size_t)layer * p->spl + s];
  uint8_t *dst = p->slab + ((size_t)layer * p->spl + s) * (size_t)p->slot_bytes;
  hipError_t err = hipSuccess;
  if (sl.has_done) err = hipStreamWaitEvent(ss, sl.done, 0);  // previous consumer of the victim is done
  if (err == hipSuccess && sl.pending) err = hipStreamWaitEvent(ss, sl.fill_ev, 0);  // previous copy is done
  if (err == hipSuccess) {
    hipLaunchKernelGGL(k_store_u32, dim3(1), dim3(64), 0, ss, p->d_slot_gen + (size_t)layer * p->spl + s, sl.gen);
    err = hipGetLastError();
  }
  if (err == hipSuccess && p->poison) err = hipMemsetAsync(dst, 0xFF, (size_t)p->slot_bytes, ss);
  if (err == hipSuccess)
    err = hipMemcpyAsync(dst, p->src[(size_t)layer * p->E + e], (size_t)p->slot_bytes, hipMemcpyHostToDevice, ss);
  p->fill_bytes += (uint64_t)p->slot_bytes;
  return err;
}

// Union of idx[0..n) in first-appearance order, with the acquire/prefetch checks.
static int union_of(moe_pool *p, int layer, const int32_t *idx, int32_t n, std::vector<int> &uniq) {
  for (int i = 0; i < n; ++i) {
    const int e = idx[i];
    if (e < 0 || e >= p->E) return MOE_EINVAL;
    if (std::find(uniq.begin(), uniq.end(), e) == uniq.end()) uniq.push_back(e);
  }
  if ((int)uniq.size() > p->spl) return MOE_ENOSLOT;
  for (int e : uniq)
    if (p->table[(size_t)layer * p->E + e] < 0 && !p->src[(size_t)layer * p->E + e]) return MOE_ENULL;
  return MOE_OK;
}

extern "C" {

int moe_pool_create(const moe_cfg *cfg, int32_t n_layers, int32_t slots_per_layer, int32_t flags, moe_pool **out) {
  if (!out) return MOE_ENULL;
  *out = nullptr;
  int v = moe_validate_cfg(cfg);
  if (v) return v;
  if (n_layers < 1 || slots_per_layer < 1 || (flags & ~3)) return MOE_EINVAL;
  moe_pool *p = new moe_pool();
  p->cfg = *cfg;
  p->n_layers = n_layers;
  p->spl = slots_per_layer;
  p->E = cfg->n_experts;
  p->slot_bytes = moe_expert_bytes(cfg, cfg->moe_inter);
  p->device = !(flags & MOE_POOL_NO_DEVICE);
  p->poison = (flags & MOE_POOL_POISON) != 0;
  p->table.assign((size_t)n_layers * p->E, -1);
  p->src.assign((size_t)n_layers * p->E, nullptr);
  p->slots.resize((size_t)n_layers * slots_per_layer);
  p->leased_layer.assign(n_layers, -1);
  p->lease_list.resize(n_layers);
  p->table_dirty.assign(n_layers, 0);
  p->lease_clock.assign(n_layers, 0);
  p->fill_clock.assign(n_layers, 0);
  if (p->device) {
    const size_t slab = (size_t)n_layers * slots_per_layer * (size_t)p->slot_bytes;
    const size_t tab = (size_t)n_layers * 2 * p->E * sizeof(int32_t);
    hipError_t e = hipMalloc(&p->slab, slab);
    if (e == hipSuccess) e = hipMalloc(&p->d_tables, tab);
    if (e == hipSuccess) e = hipMalloc(&p->d_slot_gen, (size_t)n_layers * slots_per_layer * sizeof(uint32_t));
    if (e == hipSuccess) e = hipHostMalloc(&p->h_stage, tab, hipHostMallocDefault);
    // tables all -1 and expected generations all 0xFFFFFFFF; slot generations 0 (never filled)
    if (e == hipSuccess) e = hipMemset(p->d_tables, 0xFF, tab);
    if (e == hipSuccess) e = hipMemset(p->d_slot_gen, 0, (size_t)n_layers * slots_per_layer * sizeof(uint32_t));
    if (e == hipSuccess) {
      p->table_ev.assign(n_layers, nullptr);
      for (int l = 0; l < n_layers && e == hipSuccess; ++l) e = hipEventCreateWithFlags(&p->table_ev[l], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      moe_pool_destroy(p);
      return MOE_EHIP;
    }
  }
  *out = p;
  return MOE_OK;
}

void moe_pool_destroy(moe_pool *p) {
  if (!p) return;
  if (p->device) (void)hipDeviceSynchronize();
  for (auto &s : p->slots) {
    if (s.done) (void)hipEventDestroy(s.done);
    if (s.fill_ev) (void)hipEventDestroy(s.fill_ev);
  }
  for (auto e : p->ev_pool) (void)hipEventDestroy(e);
  for (auto e : p->table_ev)
    if (e) (void)hipEventDestroy(e);
  if (p->slab) (void)hipFree(p->slab);
  if (p->d_tables) (void)hipFree(p->d_tables);
  if (p->d_slot_gen) (void)hipFree(p->d_slot_gen);
  if (p->h_stage) (void)hipHostFree(p->h_stage);
  delete p;
}

int moe_pool_register_host(moe_pool *p, int32_t layer, int32_t expert, const void *src) {
  if (!p || !src) return MOE_ENULL;
  if (layer < 0 || layer >= p->n_layers || expert < 0 || expert >= p->E) return MOE_EINVAL;
  p->src[(size_t)layer * p->E + expert] = src;
  return MOE_OK;
}

int moe_pool_acquire(moe_pool *p, int32_t layer, const int32_t *idx, int32_t n, moe_slot_view *view,
                     int32_t *n_miss, void *compute, void *side) {
  if (!p || !view || (n > 0 && !idx)) return MOE_ENULL;
  if (layer < 0 || layer >= p->n_layers || n < 0) return MOE_EINVAL;
  if (p->leased_layer[layer] >= 0) return MOE_ELEASE;  // previous lease of this layer not released
  std::vector<int> uniq;  // union of the named experts, in first-appearance order
  const int u = union_of(p, layer, idx, n, uniq);
  if (u) return u;
  moe_pool::Slot *base = &p->slots[(size_t)layer * p->spl];
  int32_t *tab = &p->table[(size_t)layer * p->E];
  ++p->acquires;
  const uint64_t now = ++p->clock;
  p->trace.clear();
  std::vector<int> leased, waits;  // waits: prefetched slots whose copy the compute stream must wait for
  // hits first: lease them so that misses cannot evict them
  for (int e : uniq) {
    const int s = tab[e];
    if (s >= 0) {
      base[s].leased = true;
      base[s].last_use = now;
      leased.push_back(s);
      ++p->hits;
      if (base[s].pending) {
        waits.push_back(s);
        ++p->prefetch_hits;
      }
      p->trace.insert(p->trace.end(), {e, s, 1});
    }
  }
  std::vector<std::pair<int, int>> fills;  // (expert, slot)
  for (int e : uniq) {
    if (tab[e] >= 0) continue;
    const int victim = pick_victim(p, layer);
    if (victim < 0) return MOE_ENOSLOT;  // cannot happen: uniq <= spl
    if (base[victim].expert >= 0) {
      tab[base[victim].expert] = -1;
      ++p->evictions;
    }
    base[victim].expert = e;
    base[victim].leased = true;
    base[victim].last_use = now;
    base[victim].gen = ++p->gen_counter;
    tab[e] = victim;
    leased.push_back(victim);
    fills.emplace_back(e, victim);
    ++p->misses;
    p->trace.insert(p->trace.end(), {e, victim, 0});
  }
  p->leased_layer[layer] = (int)leased.size();
  p->lease_list[layer] = leased;
  p->lease_clock[layer] = now;
  if (!fills.empty()) p->fill_clock[layer] = now;
  if (n_miss) *n_miss = (int32_t)fills.size();
  view->base = p->slab + (size_t)layer * p->spl * (size_t)p->slot_bytes;
  view->slot_bytes = p->slot_bytes;
  view->table = p->d_tables ? p->d_tables + (size_t)layer * 2 * p->E : nullptr;
  view->n_slots = p->spl;
  view->gen = p->d_tables ? (const uint32_t *)(p->d_tables + (size_t)layer * 2 * p->E + p->E) : nullptr;
  view->slot_gen = p->d_slot_gen ? p->d_slot_gen + (size_t)layer * p->spl : nullptr;
  view->lease = now;
  if (!p->device) {
    for (int s : waits) base[s].pending = false;
    return MOE_OK;
  }
  hipStream_t cs = (hipStream_t)compute, ss = (hipStream_t)side;
  hipError_t err = hipSuccess;
  for (auto &f : fills) {
    err = enqueue_fill(p, layer, f.first, f.second, ss);
    base[f.second].pending = false;  // this acquire's event covers the slot from here on
    if (err != hipSuccess) break;
  }
  for (int s : waits) {  // prefetched copies: publish only complete slots
    if (err == hipSuccess) err = hipStreamWaitEvent(cs, base[s].fill_ev, 0);
    base[s].pending = false;
  }
  if (err == hipSuccess && !fills.empty()) {
    hipEvent_t filled = get_event(p);
    if (!filled) err = hipErrorOutOfMemory;
    if (err == hipSuccess) err = hipEventRecord(filled, ss);
    if (err == hipSuccess) err = hipStreamWaitEvent(cs, filled, 0);  // publish only complete slots
    if (filled) p->ev_pool.push_back(filled);  // reusable: the wait has captured its state
  }
  if (err == hipSuccess && (!fills.empty() || p->table_dirty[layer])) {  // table changed: upload on the compute stream
    p->table_dirty[layer] = 0;
    int32_t *stage = p->h_stage + (size_t)layer * 2 * p->E;
    uint32_t *stage_gen = (uint32_t *)(stage + p->E);
    err = hipEventSynchronize(p->table_ev[layer]);  // the staging buffer's previous upload is complete
    for (int e = 0; e < p->E && err == hipSuccess; ++e) {
      int s = tab[e];
      if (s >= 0 && base[s].pending) {
        // a prefetched slot this acquire did not wait for: published once its copy is complete
        const hipError_t q = hipEventQuery(base[s].fill_ev);
        if (q == hipSuccess) {
          base[s].pending = false;
        } else if (q == hipErrorNotReady) {
          s = -1;
          p->table_dirty[layer] = 1;  // the next acquire publishes it
        } else {
          err = q;
        }
      }
      stage[e] = s;
      stage_gen[e] = s >= 0 ? base[s].gen : 0xFFFFFFFFu;
    }
    if (err == hipSuccess)
      err = hipMemcpyAsync(p->d_tables + (size_t)layer * 2 * p->E, stage, sizeof(int32_t) * 2 * p->E,
                           hipMemcpyHostToDevice, cs);
    if (err == hipSuccess) err = hipEventRecord(p->table_ev[layer], cs);
  }
  if (err != hipSuccess) {
    set_hip_error(err);
    return MOE_EHIP;
  }
  return MOE_OK;
}

int moe_pool_prefetch(moe_pool *p, int32_t layer, const int32_t *idx, int32_t n, int32_t *n_fill, void *side) {
  if (!p || (n > 0 && !idx)) return MOE_ENULL;
  if (layer < 0 || layer >= p->n_layers || n < 0) return MOE_EINVAL;
  std::vector<int> uniq;
  const int u = union_of(p, layer, idx, n, uniq);
  if (u) return u;
  moe_pool::Slot *base = &p->slots[(size_t)layer * p->spl];
  int32_t *tab = &p->table[(size_t)layer * p->E];
  ++p->prefetches;
  const uint64_t now = ++p->clock;
  // residency rechecked: resident experts only become recently used; each
  // missing one takes a victim like an acquire miss (never a leased slot, nor
  // a slot of this prediction: those are held like leases during the call)
  std::vector<std::pair<int, int>> fills;
  std::vector<int> held;
  for (int e : uniq)
    if (tab[e] >= 0) {
      moe_pool::Slot &sl = base[tab[e]];
      sl.last_use = now;
      if (!sl.leased) {
        sl.leased = true;
        held.push_back(tab[e]);
      }
    }
  for (int e : uniq) {
    if (tab[e] >= 0) continue;
    const int victim = pick_victim(p, layer);
    if (victim < 0) break;  // no slot left: the rest of the prediction is dropped
    base[victim].leased = true;
    held.push_back(victim);
    if (base[victim].expert >= 0) {
      tab[base[victim].expert] = -1;
      ++p->evictions;
    }
    base[victim].expert = e;
    base[victim].last_use = now;
    base[victim].gen = ++p->gen_counter;
    tab[e] = victim;
    fills.emplace_back(e, victim);
    ++p->prefetch_fills;
  }
  for (int s : held) base[s].leased = false;
  if (n_fill) *n_fill = (int32_t)fills.size();
  if (!fills.empty()) {
    p->table_dirty[layer] = 1;
    p->fill_clock[layer] = now;
  }
  if (!p->device) {
    for (auto &f : fills) base[f.second].pending = true;
    return MOE_OK;
  }
  hipStream_t ss = (hipStream_t)side;
  hipError_t err = hipSuccess;
  for (auto &f : fills) {
    moe_pool::Slot &sl = base[f.second];
    err = enqueue_fill(p, layer, f.first, f.second, ss);
    if (err == hipSuccess && !sl.fill_ev) err = hipEventCreateWithFlags(&sl.fill_ev, hipEventDisableTiming);
    if (err == hipSuccess) err = hipEventRecord(sl.fill_ev, ss);
    if (err != hipSuccess) break;
    sl.pending = true;
  }
  if (err != hipSuccess) {
    set_hip_error(err);
    return MOE_EHIP;
  }
  return MOE_OK;
}

int moe_pool_release(moe_pool *p, int32_t layer, void *compute) {
  if (!p) return MOE_ENULL;
  if (layer < 0 || layer >= p->n_layers) return MOE_EINVAL;
  if (p->leased_layer[layer] < 0) return MOE_ELEASE;
  moe_pool::Slot *base = &p->slots[(size_t)layer * p->spl];
  hipError_t err = hipSuccess;
  for (int s : p->lease_list[layer]) {
    base[s].leased = false;
    if (p->device && err == hipSuccess) {
      if (!base[s].done) err = hipEventCreateWithFlags(&base[s].done, hipEventDisableTiming);
      if (err == hipSuccess) err = hipEventRecord(base[s].done, (hipStream_t)compute);
      base[s].has_done = err == hipSuccess;
    }
  }
  p->leased_layer[layer] = -1;
  p->lease_list[layer].clear();
  if (err != hipSuccess) {
    set_hip_error(err);
    return MOE_EHIP;
  }
  return MOE_OK;
}

int moe_pool_check_view(const moe_pool *p, int32_t layer, const moe_slot_view *v) {
  if (!p || !v) return MOE_ENULL;
  if (layer < 0 || layer >= p->n_layers) return MOE_EINVAL;
  if (p->device && (v->table != p->d_tables + (size_t)layer * 2 * p->E ||
                    v->base != p->slab + (size_t)layer * p->spl * (size_t)p->slot_bytes))
    return MOE_EINVAL;
  if (v->lease == 0 || v->lease > p->clock) return MOE_EINVAL;
  if (p->leased_layer[layer] >= 0 && v->lease == p->lease_clock[layer]) return MOE_OK;  // lease still open
  return p->fill_clock[layer] > v->lease ? MOE_ESTALE : MOE_OK;
}

int moe_pool_trace(const moe_pool *p, int32_t *out, int32_t cap) {
  if (!p || !out) return MOE_ENULL;
  const int n = (int)p->trace.size() / 3;
  if (cap < n * 3) return MOE_EINVAL;
  std::memcpy(out, p->trace.data(), sizeof(int32_t) * p->trace.size());
  return n;
}

int moe_pool_stats(const moe_pool *p, char *out, size_t cap) {
  if (!p || !out) return MOE_ENULL;
  char buf[512];
  const int len = std::snprintf(buf, sizeof buf,
                                "{\"acquires\": %llu, \"hits\": %llu, \"misses\": %llu, \"evictions\": %llu, "
                                "\"fill_bytes\": %llu, \"prefetches\": %llu, \"prefetch_fills\": %llu, "
                                "\"prefetch_hits\": %llu, \"slots_per_layer\": %d, \"layers\": %d, \"slot_bytes\": %lld}",
                                (unsigned long long)p->acquires, (unsigned long long)p->hits,
                                (unsigned long long)p->misses, (unsigned long long)p->evictions,
                                (unsigned long long)p->fill_bytes, (unsigned long long)p->prefetches,
                                (unsigned long long)p->prefetch_fills, (unsigned long long)p->prefetch_hits, p->spl,
                                p->n_layers, (long long)p->slot_bytes);
  if (len < 0 || (size_t)len + 1 > cap) return MOE_EINVAL;
  std::memcpy(out, buf, (size_t)len + 1);
  return MOE_OK;
}

}  // extern "C"
