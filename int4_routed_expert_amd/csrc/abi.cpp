// C ABI of the MoE-layer library: argument checks, workspace layout, host-side
// packing and kernel dispatch.  Declarations and contracts: include/moe.h.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "common.h"

namespace moe {

static thread_local std::string g_last_hip_error = "no error";

void set_hip_error(hipError_t e) { g_last_hip_error = hipGetErrorString(e); }

static int hip_fail(hipError_t e) {
  set_hip_error(e);
  return MOE_EHIP;
}

// ---- timing instrumentation ---------------------------------------------------
struct ProfRec {
  const char *name;
  hipEvent_t a, b;
  bool launched;
};
static bool g_prof = false;
static std::vector<ProfRec> g_recs;
static std::vector<hipEvent_t> g_pool;

static hipEvent_t pool_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  (void)hipEventCreate(&e);
  return e;
}

bool prof_on() { return g_prof; }

static thread_local long t_armed = -1;  // record awaiting its kernel

void prof_arm(const char *name) {
  g_recs.push_back(ProfRec{name, pool_event(), pool_event(), false});
  t_armed = (long)g_recs.size() - 1;
}

bool prof_take(hipEvent_t *start, hipEvent_t *stop) {
  if (t_armed < 0 || t_armed >= (long)g_recs.size()) return false;
  ProfRec &r = g_recs[(size_t)t_armed];
  t_armed = -1;
  r.launched = true;
  *start = r.a;
  *stop = r.b;
  return true;
}

// Compute units of the current device (cached per device id).
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// offset-binary nibbles (interchange) <-> two's complement nibbles (slot layout)
static void copy_flip(uint8_t *dst, const uint8_t *src, size_t n) {
  for (size_t i = 0; i < n; ++i) dst[i] = src[i] ^ 0x88u;
}

WsLayout ws_layout(const moe_cfg &c, int32_t S) {
  WsLayout L{};
  const size_t k1 = (size_t)c.top_k + 1;
  const size_t imax = (size_t)std::max(c.moe_inter, c.shared_inter);
  const size_t gh = (size_t)c.hidden / kGroup, gi = imax / kGroup;
  size_t off = 0;
  L.sync = off; off += kWsSyncBytes;
  L.logits = off; off += align256((size_t)S * c.n_experts * sizeof(double));
  L.scores = off; off += align256((size_t)S * c.n_experts * sizeof(double));
  L.keys = off; off += align256((size_t)S * c.n_experts * sizeof(float));
  L.h = off; off += align256((size_t)S * k1 * imax * sizeof(float));
  L.xl = off; off += align256((size_t)S * gh * 24 * sizeof(uint32_t));
  L.xf = off; off += align256((size_t)S * gh * sizeof(float));
  L.hl = off; off += align256((size_t)S * k1 * gi * 24 * sizeof(uint32_t));
  L.hf = off; off += align256((size_t)S * k1 * gi * sizeof(float));
  L.eptr = off; off += align256(std::max<size_t>((size_t)kMaxK * sizeof(uint64_t), kWsPlanBytes));
  L.max_items = 0;
  L.max_mtiles = 0;
  if (S >= 2) {  // per-(token, rank) expert outputs, added in route order by the combine
    L.part = off; off += align256((size_t)S * k1 * c.hidden * sizeof(float));
  }
  if (S > kSmallS) {
    L.lists = off; off += align256((size_t)c.n_experts * S * sizeof(int32_t));
    L.counts = off; off += align256((size_t)(c.n_experts + 1) * sizeof(int32_t));
    L.max_items = (int32_t)(((size_t)S * c.top_k + 3) / 4 + c.n_experts + (S + 3) / 4);
    L.items = off; off += align256((size_t)L.max_items * 3 * sizeof(int32_t));
    L.n_items = off; off += align256(4 * sizeof(int32_t));
    // a tile per kMfmaTileTokens rows of each expert's list: at most one partial tile per expert
    const size_t pairs = (size_t)S * c.top_k;
    L.max_mtiles = (int32_t)((pairs + kMfmaTileTokens - 1) / kMfmaTileTokens + std::min<size_t>(c.n_experts, pairs) +
                             (S + kMfmaTileTokens - 1) / kMfmaTileTokens);
    L.mtiles = off; off += align256((size_t)L.max_mtiles * 3 * sizeof(int32_t));
    L.xb = off; off += align256((size_t)S * c.hidden * sizeof(uint16_t));
  }
  if (c.act_int8) {
    L.xq = off; off += align256((size_t)S * c.hidden);
    L.dx = off; off += align256((size_t)S * sizeof(float));
    L.hq = off; off += align256((size_t)S * k1 * imax);
    L.dh = off; off += align256((size_t)S * k1 * sizeof(float));
  }
  L.total = std::max<size_t>(off, 256);
  return L;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_validate_cfg(const moe_cfg *c) {
  if (!c) return MOE_ENULL;
  const bool ok = c->group_size == kGroup && c->hidden >= 32 && c->hidden <= 8192 && c->hidden % 32 == 0 &&
                  c->moe_inter >= 32 && c->moe_inter <= 8192 && c->moe_inter % 32 == 0 &&
                  (c->shared_inter == 0 || (c->shared_inter >= 32 && c->shared_inter <= 8192 && c->shared_inter % 32 == 0)) &&
                  c->n_experts >= 1 && c->n_experts <= kMaxE && c->n_group >= 1 && c->n_group <= kMaxG &&
                  c->n_experts % c->n_group == 0 && c->topk_group >= 1 && c->topk_group <= c->n_group &&
                  c->top_k >= 1 && c->top_k <= kMaxK && c->top_k <= c->topk_group * (c->n_experts / c->n_group) &&
                  (c->norm_topk_prob == 0 || c->norm_topk_prob == 1) && std::isfinite(c->routed_scaling_factor) &&
                  c->mfma_min_tokens >= 0 &&
                  (c->weight_format == MOE_WF_Q4_G32 || c->weight_format == MOE_WF_Q4_ROW ||
                   c->weight_format == MOE_WF_Q8_ROW) &&
                  (c->act_int8 == 0 || c->act_int8 == 1);
  return ok ? MOE_OK : MOE_EINVAL;
}

const char *moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid configuration or shape";
    case MOE_ENULL: return "required pointer is NULL";
    case MOE_EDTYPE: return "unknown activation dtype";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_ENOSLOT: return "slot pool: expert union exceeds the layer's slots";
    case MOE_ESTALE: return "slot pool: the view's slots have been refilled since it was published";
    case MOE_ELEASE: return "slot pool: acquire of a leased layer, or release without acquire";
    case MOE_EHIP: return "HIP call failed";
    default: return "unknown status";
  }
}

const char *moe_last_hip_error(void) { return g_last_hip_error.c_str(); }

int moe_profile_enable(int on) {
  g_prof = on != 0;
  return MOE_OK;
}

int moe_profile_report(char *out, size_t cap) {
  if (!out || cap == 0) return MOE_ENULL;
  std::map<std::string, std::pair<double, long>> agg;
  for (auto &r : g_recs) {
    if (r.launched) {
      hipError_t e = hipEventSynchronize(r.b);
      if (e != hipSuccess) return hip_fail(e);
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, r.a, r.b);
      if (e != hipSuccess) return hip_fail(e);
      auto &v = agg[r.name];
      v.first += ms;
      v.second += 1;
    }
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  t_armed = -1;
  g_recs.clear();
  std::string js = "{";
  bool first = true;
  for (auto &kv : agg) {
    char buf[256];
    std::snprintf(buf, sizeof buf, "%s\"%s\": [%.6f, %ld]", first ? "" : ", ", kv.first.c_str(), kv.second.first,
                  kv.second.second);
    js += buf;
    first = false;
  }
  js += "}";
  if (js.size() + 1 > cap) return MOE_EINVAL;
  std::memcpy(out, js.c_str(), js.size() + 1);
  return MOE_OK;
}

int64_t moe_expert_bytes(const moe_cfg *c, int32_t inter) {
  const int v = moe_validate_cfg(c);
  if (v) return v;
  if (inter < 32 || inter > 8192 || inter % 32) return MOE_EINVAL;
  return slot_stride(c->hidden, inter, c->weight_format);
}

size_t moe_workspace_bytes(const moe_cfg *c, int32_t max_S) {
  if (moe_validate_cfg(c) || max_S < 0) return 0;
  return ws_layout(*c, max_S).total;
}

int moe_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  if (!ws) return MOE_ENULL;
  if (ws_bytes < (size_t)kWsSyncBytes) return MOE_EWORKSPACE;
  hipError_t e = launch_ws_init((uint32_t *)ws, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_pack_expert(const moe_cfg *c, int32_t inter, const uint8_t *qg, const uint16_t *sg, const uint8_t *qu,
                    const uint16_t *su, const uint8_t *qd, const uint16_t *sd, void *dst, int32_t where, void *stream) {
  const int64_t nb = moe_expert_bytes(c, inter);
  if (nb < 0) return (int)nb;
  if (!qg || !sg || !qu || !su || !qd || !sd || !dst) return MOE_ENULL;
  if (where != 0 && where != 1) return MOE_EINVAL;
  if (c->weight_format != MOE_WF_Q4_G32) return MOE_EINVAL;
  const int H = c->hidden, I = inter;
  const int wf = kWfQ4G32;
  if (where == 1) {
    hipError_t e = launch_pack(H, I, qg, sg, qu, su, qd, sd, (uint8_t *)dst, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
  }
  uint8_t *d = (uint8_t *)dst;
  const int ngh = H / kGroup, ngi = I / kGroup;
  for (int t = 0; t < I / kGuPairs; ++t) {
    uint8_t *tile = d + (size_t)t * gu_tile_bytes(H, wf);
    uint16_t *scl = (uint16_t *)(tile + (size_t)kGuRows * (H / 2));
    for (int i = 0; i < kGuRows; ++i) {
      const int r = kGuPairs * t + i / 2;
      const uint8_t *q = (i & 1) ? qu : qg;
      const uint16_t *s = (i & 1) ? su : sg;
      copy_flip(tile + (size_t)i * (H / 2), q + (size_t)r * (H / 2), H / 2);
      for (int g = 0; g < ngh; ++g) scl[g * kGuRows + i] = s[(size_t)r * ngh + g];
    }
  }
  for (int t = 0; t < H / kDnRows; ++t) {
    uint8_t *tile = d + down_offset(H, I, wf) + (size_t)t * dn_tile_bytes(I, wf);
    uint16_t *scl = (uint16_t *)(tile + (size_t)kDnRows * (I / 2));
    for (int i = 0; i < kDnRows; ++i) {
      const int r = kDnRows * t + i;
      copy_flip(tile + (size_t)i * (I / 2), qd + (size_t)r * (I / 2), I / 2);
      for (int g = 0; g < ngi; ++g) scl[g * kDnRows + i] = sd[(size_t)r * ngi + g];
    }
  }
  const size_t used = (size_t)packed_bytes(H, I, wf);
  std::memset(d + used, 0, (size_t)nb - used);
  return MOE_OK;
}

int moe_unpack_expert(const moe_cfg *c, int32_t inter, const void *src, uint8_t *qg, uint16_t *sg, uint8_t *qu,
                      uint16_t *su, uint8_t *qd, uint16_t *sd) {
  const int64_t nb = moe_expert_bytes(c, inter);
  if (nb < 0) return (int)nb;
  if (!src || !qg || !sg || !qu || !su || !qd || !sd) return MOE_ENULL;
  if (c->weight_format != MOE_WF_Q4_G32) return MOE_EINVAL;
  const int H = c->hidden, I = inter;
  const int wf = kWfQ4G32;
  const uint8_t *d = (const uint8_t *)src;
  const int ngh = H / kGroup, ngi = I / kGroup;
  for (int t = 0; t < I / kGuPairs; ++t) {
    const uint8_t *tile = d + (size_t)t * gu_tile_bytes(H, wf);
    const uint16_t *scl = (const uint16_t *)(tile + (size_t)kGuRows * (H / 2));
    for (int i = 0; i < kGuRows; ++i) {
      const int r = kGuPairs * t + i / 2;
      uint8_t *q = (i & 1) ? qu : qg;
      uint16_t *s = (i & 1) ? su : sg;
      copy_flip(q + (size_t)r * (H / 2), tile + (size_t)i * (H / 2), H / 2);
      for (int g = 0; g < ngh; ++g) s[(size_t)r * ngh + g] = scl[g * kGuRows + i];
    }
  }
  for (int t = 0; t < H / kDnRows; ++t) {
    const uint8_t *tile = d + down_offset(H, I, wf) + (size_t)t * dn_tile_bytes(I, wf);
    const uint16_t *scl = (const uint16_t *)(tile + (size_t)kDnRows * (I / 2));
    for (int i = 0; i < kDnRows; ++i) {
      const int r = kDnRows * t + i;
      copy_flip(qd + (size_t)r * (I / 2), tile + (size_t)i * (I / 2), I / 2);
      for (int g = 0; g < ngi; ++g) sd[(size_t)r * ngi + g] = scl[g * kDnRows + i];
    }
  }
  return MOE_OK;
}

// Row-scaled formats: rows copied whole (int4 nibbles flipped between offset
// binary and two's complement, int8 bytes as they are), 8 fp32 scales per tile.
static void pack_rows_host(int H, int I, int wf, bool unpack, uint8_t *slot, uint8_t *qg, float *sg, uint8_t *qu,
                           float *su, uint8_t *qd, float *sd) {
  auto move = [&](uint8_t *packed, uint8_t *inter, size_t n) {
    if (wf == kWfQ8Row) {
      if (unpack) std::memcpy(inter, packed, n);
      else std::memcpy(packed, inter, n);
    } else {
      if (unpack) copy_flip(inter, packed, n);
      else copy_flip(packed, inter, n);
    }
  };
  const int64_t rbh = row_bytes(H, wf), rbi = row_bytes(I, wf);
  for (int t = 0; t < I / kGuPairs; ++t) {
    uint8_t *tile = slot + (size_t)t * gu_tile_bytes(H, wf);
    float *scl = (float *)(tile + (size_t)kGuRows * rbh);
    for (int i = 0; i < kGuRows; ++i) {
      const int r = kGuPairs * t + i / 2;
      move(tile + (size_t)i * rbh, ((i & 1) ? qu : qg) + (size_t)r * rbh, (size_t)rbh);
      float *s = (i & 1) ? su : sg;
      if (unpack) s[r] = scl[i];
      else scl[i] = s[r];
    }
  }
  for (int t = 0; t < H / kDnRows; ++t) {
    uint8_t *tile = slot + down_offset(H, I, wf) + (size_t)t * dn_tile_bytes(I, wf);
    float *scl = (float *)(tile + (size_t)kDnRows * rbi);
    for (int i = 0; i < kDnRows; ++i) {
      const int r = kDnRows * t + i;
      move(tile + (size_t)i * rbi, qd + (size_t)r * rbi, (size_t)rbi);
      if (unpack) sd[r] = scl[i];
      else scl[i] = sd[r];
    }
  }
}

int moe_pack_expert_rows(const moe_cfg *c, int32_t inter, const void *qg, const float *sg, const void *qu,
                         const float *su, const void *qd, const float *sd, void *dst, int32_t where, void *stream) {
  const int64_t nb = moe_expert_bytes(c, inter);
  if (nb < 0) return (int)nb;
  if (!qg || !sg || !qu || !su || !qd || !sd || !dst) return MOE_ENULL;
  if (where != 0 && where != 1) return MOE_EINVAL;
  const int wf = c->weight_format;
  if (wf != kWfQ4Row && wf != kWfQ8Row) return MOE_EINVAL;
  const int H = c->hidden, I = inter;
  if (where == 1) {
    hipError_t e = launch_pack_rows(H, I, wf, (const uint8_t *)qg, sg, (const uint8_t *)qu, su, (const uint8_t *)qd,
                                    sd, (uint8_t *)dst, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
  }
  uint8_t *d = (uint8_t *)dst;
  pack_rows_host(H, I, wf, false, d, (uint8_t *)qg, (float *)sg, (uint8_t *)qu, (float *)su, (uint8_t *)qd,
                 (float *)sd);
  const size_t used = (size_t)packed_bytes(H, I, wf);
  std::memset(d + used, 0, (size_t)nb - used);
  return MOE_OK;
}

int moe_unpack_expert_rows(const moe_cfg *c, int32_t inter, const void *src, void *qg, float *sg, void *qu,
                           float *su, void *qd, float *sd) {
  const int64_t nb = moe_expert_bytes(c, inter);
  if (nb < 0) return (int)nb;
  if (!src || !qg || !sg || !qu || !su || !qd || !sd) return MOE_ENULL;
  const int wf = c->weight_format;
  if (wf != kWfQ4Row && wf != kWfQ8Row) return MOE_EINVAL;
  pack_rows_host(c->hidden, inter, wf, true, (uint8_t *)src, (uint8_t *)qg, sg, (uint8_t *)qu, su, (uint8_t *)qd,
                 sd);
  return MOE_OK;
}

}  // extern "C"

namespace moe {

// Argument checks and kernel arguments of moe_route and moe_ffn.
static int route_args(const moe_cfg *c, const void *x, int32_t x_dtype, int32_t S, const float *W, const float *bias,
                      int32_t *idx, float *w, void *ws, size_t ws_bytes, RouteArgs &a) {
  int v = moe_validate_cfg(c);
  if (v) return v;
  if (S < 0) return MOE_EINVAL;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EDTYPE;
  if (S == 0) return MOE_OK;
  if (!x || !W || !bias || !idx || !w || !ws) return MOE_ENULL;
  const WsLayout L = ws_layout(*c, S);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  a = RouteArgs{};
  a.H = c->hidden; a.E = c->n_experts; a.G = c->n_group; a.Gk = c->topk_group; a.k = c->top_k; a.S = S;
  a.x_bf16 = x_dtype == MOE_BF16; a.norm = c->norm_topk_prob; a.rsf = c->routed_scaling_factor;
  a.x = x; a.W = W; a.bias = bias; a.idx = idx; a.w = w;
  a.logits = (double *)((char *)ws + L.logits);
  a.scores = (double *)((char *)ws + L.scores);
  a.keys = (float *)((char *)ws + L.keys);
  a.sync = (uint32_t *)((char *)ws + L.sync);
  return MOE_OK;
}

static int ffn_args(const moe_cfg *c, const void *x, int32_t x_dtype, int32_t S, const int32_t *idx, const float *w,
                    const moe_slot_view *ex, const void *shared, float *y, void *ws, size_t ws_bytes, FfnArgs &a) {
  int v = moe_validate_cfg(c);
  if (v) return v;
  if (S < 0) return MOE_EINVAL;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EDTYPE;
  if (S == 0) return MOE_OK;
  if (!x || !idx || !w || !ex || !y || !ws || !ex->base || !ex->table) return MOE_ENULL;
  if (ex->gen && !ex->slot_gen) return MOE_ENULL;
  if (c->shared_inter > 0 && !shared) return MOE_ENULL;
  if (ex->n_slots < 1 || ex->slot_bytes < slot_stride(c->hidden, c->moe_inter, c->weight_format) ||
      ex->slot_bytes % 256)
    return MOE_EINVAL;
  const WsLayout L = ws_layout(*c, S);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  a = FfnArgs{};
  a.H = c->hidden; a.E = c->n_experts; a.k = c->top_k; a.I = c->moe_inter; a.Is = c->shared_inter; a.S = S;
  a.x_bf16 = x_dtype == MOE_BF16;
  a.wf = c->weight_format;
  a.act_q = c->act_int8;
  a.x = x; a.idx = idx; a.w = w;
  a.base = (const uint8_t *)ex->base; a.slot_bytes = ex->slot_bytes; a.table = ex->table; a.n_slots = ex->n_slots;
  a.gen = ex->gen; a.slot_gen = ex->gen ? ex->slot_gen : nullptr;
  a.shared = (const uint8_t *)shared;
  a.y = y;
  char *b = (char *)ws;
  a.h = (float *)(b + L.h);
  a.xl = (uint32_t *)(b + L.xl);
  a.xf = (float *)(b + L.xf);
  a.hl = (uint32_t *)(b + L.hl);
  a.hf = (float *)(b + L.hf);
  a.eptr = (uint64_t *)(b + L.eptr);
  a.n_cu = device_cus();
  if (S >= 2) a.part = (float *)(b + L.part);
  if (a.act_q) {
    a.xq = (int8_t *)(b + L.xq);
    a.dx = (float *)(b + L.dx);
    a.hq = (int8_t *)(b + L.hq);
    a.dh = (float *)(b + L.dh);
  }
  if (S <= kSmallS) {
    // one-token down kernel: about one row block per compute unit, at most 8 tiles each
    const int nt = c->hidden / kDnRows;
    a.tb = std::min(8, std::max(1, (nt + a.n_cu - 1) / a.n_cu));
    a.n_blk = (nt + a.tb - 1) / a.tb;
  } else {
    a.lists = (int32_t *)(b + L.lists);
    a.counts = (int32_t *)(b + L.counts);
    a.items = (int32_t *)(b + L.items);
    a.n_items = (int32_t *)(b + L.n_items);
    a.max_items = L.max_items;
    a.mtiles = (int32_t *)(b + L.mtiles);
    a.xb = (uint16_t *)(b + L.xb);
    a.max_mtiles = L.max_mtiles;
    a.mfma_thr = c->mfma_min_tokens;
  }
  return MOE_OK;
}

static hipError_t run_ffn(const FfnArgs &a, hipStream_t st) {
  return a.S <= kSmallS ? launch_ffn_decode(a, st) : launch_ffn_batch(a, st);
}

}  // namespace moe

extern "C" {

int moe_route(const moe_cfg *c, const void *x, int32_t x_dtype, int32_t S, const float *W, const float *bias,
              int32_t *idx, float *w, void *ws, size_t ws_bytes, void *stream) {
  RouteArgs a;
  const int v = route_args(c, x, x_dtype, S, W, bias, idx, w, ws, ws_bytes, a);
  if (v || S == 0) return v;
  hipError_t e = launch_route(a, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_ffn(const moe_cfg *c, const void *x, int32_t x_dtype, int32_t S, const int32_t *idx, const float *w,
            const moe_slot_view *ex, const void *shared, float *y, void *ws, size_t ws_bytes, void *stream) {
  FfnArgs a;
  const int v = ffn_args(c, x, x_dtype, S, idx, w, ex, shared, y, ws, ws_bytes, a);
  if (v || S == 0) return v;
  hipError_t e = run_ffn(a, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

}  // extern "C"

namespace moe {

// One layer forward on a workspace; write_header: the workspace header is
// written first (by a kernel on the stream) when the call reads it (S > 1).
static int layer_impl(const moe_cfg *c, const void *x, int32_t x_dtype, int32_t S, const float *W, const float *bias,
                      int32_t *idx, float *w, const moe_slot_view *ex, const void *shared, float *y, void *ws,
                      size_t ws_bytes, hipStream_t st, bool write_header) {
  RouteArgs r;
  int v = route_args(c, x, x_dtype, S, W, bias, idx, w, ws, ws_bytes, r);
  if (v || S == 0) return v;
  FfnArgs f;
  v = ffn_args(c, x, x_dtype, S, idx, w, ex, shared, y, ws, ws_bytes, f);
  if (v) return v;
  hipError_t e = hipSuccess;
  if (write_header && S > 1) e = launch_ws_init(r.sync, st);
  if (e != hipSuccess) return hip_fail(e);
  if (S == 1) {  // the router kernel stores scores and keys; the gate/up kernel selects
    f.sel = 1;
    f.G = r.G; f.Gk = r.Gk; f.norm = r.norm; f.rsf = r.rsf;
    f.keys = r.keys; f.scores = r.scores;
    f.idx_out = idx; f.w_out = w;
    e = launch_route_scores(r, st);
    if (e == hipSuccess) e = launch_ffn_decode(f, st);
  } else {
    e = launch_route(r, st);
    if (e == hipSuccess) e = run_ffn(f, st);
  }
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

// ---- workspace of the entry point that allocates nothing -----------------------
// A fixed array in the library's code object: every device the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: only the address hipGetSymbolAddress
// returns for the current device is ever passed to a kernel.
constexpr int kScratchDevices = 64;
static __device__ __align__(256) uint8_t scratch[MOE_SCRATCH_BYTES];

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
static int scratch_ptr(void **out) {
  static std::mutex mu;
  static void *ptrs[kScratchDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kScratchDevices) return MOE_EINVAL;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p) return MOE_EHIP;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return MOE_OK;
}

}  // namespace moe

extern "C" {

int moe_layer(const moe_cfg *c, const void *x, int32_t x_dtype, int32_t S, const float *W, const float *bias,
              int32_t *idx, float *w, const moe_slot_view *ex, const void *shared, float *y, void *ws, size_t ws_bytes,
              void *stream) {
  return layer_impl(c, x, x_dtype, S, W, bias, idx, w, ex, shared, y, ws, ws_bytes, (hipStream_t)stream, false);
}

int moe_layer_noalloc(const moe_cfg *c, const void *x, int32_t x_dtype, int32_t S, const float *W, const float *bias,
                      int32_t *idx, float *w, const moe_slot_view *ex, const void *shared, float *y, void *stream) {
  const int v = moe_validate_cfg(c);
  if (v) return v;
  if (S < 0) return MOE_EINVAL;
  if (S == 0) return MOE_OK;
  if (ws_layout(*c, S).total > MOE_SCRATCH_BYTES) return MOE_EWORKSPACE;
  void *ws = nullptr;
  const int p = scratch_ptr(&ws);
  if (p) return p;
  return layer_impl(c, x, x_dtype, S, W, bias, idx, w, ex, shared, y, ws, MOE_SCRATCH_BYTES, (hipStream_t)stream,
                    true);
}

}  // extern "C"

// ---- recorded chains of layer calls ----------------------------------------------
// The calls are recorded by stream capture on a private stream, so the graph
// holds exactly the kernels (and kernel arguments) that the same moe_layer calls
// would enqueue one by one.
struct moe_chain {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int device = -1;
};

namespace moe {

static int check_call(const moe_layer_call &c) {
  if (!c.cfg) return MOE_ENULL;
  RouteArgs r;
  int v = route_args(c.cfg, c.x, c.x_dtype, c.S, c.W_gate, c.bias, c.idx, c.w, c.ws, c.ws_bytes, r);
  if (v) return v;
  FfnArgs f;
  return ffn_args(c.cfg, c.x, c.x_dtype, c.S, c.idx, c.w, c.experts, c.shared, c.y, c.ws, c.ws_bytes, f);
}

}  // namespace moe

extern "C" {

int moe_chain_create(const moe_layer_call *calls, int32_t n, moe_chain **out) {
  using namespace moe;
  if (!out) return MOE_ENULL;
  *out = nullptr;
  if (n < 1) return MOE_EINVAL;
  if (!calls) return MOE_ENULL;
  if (prof_on()) return MOE_EINVAL;
  for (int32_t i = 0; i < n; ++i) {
    const int v = check_call(calls[i]);
    if (v) return v;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  hipStream_t s = nullptr;
  e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e);
  e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    hipStreamDestroy(s);
    return hip_fail(e);
  }
  int v = MOE_OK;
  for (int32_t i = 0; i < n && v == MOE_OK; ++i) {
    const moe_layer_call &c = calls[i];
    v = layer_impl(c.cfg, c.x, c.x_dtype, c.S, c.W_gate, c.bias, c.idx, c.w, c.experts, c.shared, c.y, c.ws,
                   c.ws_bytes, s, false);
  }
  hipGraph_t g = nullptr;
  const hipError_t ec = hipStreamEndCapture(s, &g);
  hipStreamDestroy(s);
  if (v != MOE_OK || ec != hipSuccess) {
    if (g) hipGraphDestroy(g);
    return v != MOE_OK ? v : hip_fail(ec);
  }
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    hipGraphDestroy(g);
    return hip_fail(e);
  }
  moe_chain *ch = new (std::nothrow) moe_chain;
  if (!ch) {
    hipGraphExecDestroy(x);
    hipGraphDestroy(g);
    return MOE_EINVAL;
  }
  ch->graph = g;
  ch->exec = x;
  ch->device = dev;
  *out = ch;
  return MOE_OK;
}

int moe_chain_launch(const moe_chain *chain, void *stream) {
  using namespace moe;
  if (!chain) return MOE_ENULL;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev != chain->device) return MOE_EINVAL;
  e = hipGraphLaunch(chain->exec, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

void moe_chain_destroy(moe_chain *chain) {
  if (!chain) return;
  if (chain->exec) hipGraphExecDestroy(chain->exec);
  if (chain->graph) hipGraphDestroy(chain->graph);
  delete chain;
}

}  // extern "C"
