// Expert FFN for decode batches (S <= 4 tokens): gate/up projection, SwiGLU,
// down projection and the route-order combine with the shared expert.
//
// Method: "GLM-5.2 on a 32 GB Mac - native MLX port of the Colibri hierarchy",
// N1 and "G2 implementation status": routed experts are SwiGLU FFNs over int4
// weights with a scale per group; the weighted expert outputs are composed in
// route order and the shared expert is added unweighted.  colibri README
// "What's implemented" (batch-union MoE): the experts named by the whole batch
// are de-duplicated, so each is streamed a single time for all of its tokens.
//
// Every weight group is contracted with the exact integer dot product of dot.h,
// for each weight format (template parameter WF: int4 with fp16 scales per 32,
// int4 or int8 with one fp32 scale per row).  With int8 activations
// (k_quant_rows) the quantised integers take the activations' place and the
// row scale folds into each group's factor.  All paths use the same per-token
// arithmetic in the same order (lane groups in order, then one fixed wave
// reduction, then the route-order combine), so a token's output does not depend
// on which other tokens share its batch.
//
// One token (the decode step): two streaming kernels.
//  * k_gateup_s1: the work is the list of features (gate row r and up row r of
//    one expert).  Each wave takes an equal share of the shared expert's
//    features first (their weights do not depend on the routing, so they stream
//    while the wave resolves idx -> slot), then an equal share of the routed
//    experts' features, with two features in flight while one is computed.
//    x is converted to limbs once per workgroup in LDS and kept in registers.
//  * k_down_s1: one workgroup per block of output rows; its waves take the
//    experts (routed in rank order, then shared), stream that expert's down tiles
//    for the block and leave the dot products in LDS; the workgroup then adds them
//    in route order into y: deterministic, no atomics, no cross-workgroup sync.
// Two to four tokens: the batch union is derived in every workgroup from idx (at
// most 64 entries), activations are converted to limbs by a small pass, and the
// same tile math runs over (unique expert, tile) pairs.
#include <algorithm>

#include "gemv_dev.h"
#include "route_dev.h"

namespace moe {
namespace {

// ---- activations -> limbs (global), one thread per (row, group) ---------------
// q != null: int8 activations, the rows' quantised integers q (same layout as
// src) and their scales dq.
template <int WF>
__global__ __launch_bounds__(256) void k_to_limbs(const void *src, int bf16, int rows, int K, int stride,
                                                  uint32_t *limbs, float *factors, const int8_t *q,
                                                  const float *dq) {
  const int ng = K / kGroup;
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)rows * ng) return;
  const int r = (int)(i / ng), g = (int)(i - (long)r * ng);
  float v[32];
  const size_t off = (size_t)r * stride + (size_t)g * kGroup;
  if (q) load32_i8(q + off, v);
  else load32(src, bf16, off, v);
  Limbs L;
  to_limbs_wf<WF>(v, L);
  if (q) L.f *= ldg<float>(dq + r);
  uint4 *d = (uint4 *)(limbs + (size_t)i * 24);
#pragma unroll
  for (int l = 0; l < 6; ++l) stg<uint4>(d + l, make_uint4(L.L[l][0], L.L[l][1], L.L[l][2], L.L[l][3]));
  stg<float>(factors + i, L.f);
}

// EPT > 0 (the one-token layer call): the workgroup first selects the token's
// experts from the router's scores and keys (EPT experts per thread); the
// loads of the selection inputs go first, then the activations and the first
// two shared-expert features, so that the selection overlaps them.
#ifndef MOE_GU_RING
#define MOE_GU_RING 3
#endif
constexpr int kGuRing = MOE_GU_RING;  // feature slots of the one-token gate/up ring (kGuRing - 1 in flight)

template <int NG, int WF, int EPT>
__global__ __launch_bounds__(256, 2) void k_gateup_s1(FfnArgs a) {
  extern __shared__ uint32_t lds[];  // x limbs [H/32][24], then factors [H/32]
  const int lane = threadIdx.x & 63;
  const int W = gridDim.x * 4, wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int ng = a.H / kGroup, Imax = max(a.I, a.Is);
  const long Is = a.Is, Fr = (long)a.k * a.I;
  const int s0 = (int)(wid * Is / W), s1 = (int)((wid + 1) * Is / W);
  const int r0 = (int)(wid * Fr / W), r1 = (int)((wid + 1) * Fr / W);
  const int ns = s1 - s0, n = ns + (r1 - r0);
  const bool has_x = (int)threadIdx.x < ng;
  GuFeat<NG, WF> b[kGuRing];
  GuFeat<NG, WF> &b0 = b[0];
  uint64_t my_ptr = 0;
  float v[32];
  float *lf = (float *)(lds + (size_t)ng * 24);
  // x becomes limbs right after its loads and one feature's request: behind
  // the full ring's requests (a long queue while every wave streams) the
  // staging, and the barrier after it, would start late.
  auto stage_x = [&]() {
    if (has_x) {
      Limbs L;
      to_limbs_wf<WF>(v, L);
      L.f *= act_scale(a, true, 0);
      store_limbs(lds + (size_t)threadIdx.x * 24, lf + threadIdx.x, L);
    }
  };
  if constexpr (EPT > 0) {
    __shared__ SelLds sel;
    const SelCfg c{a.E, a.G, a.Gk, a.k, a.norm, a.rsf};
    SelIn<EPT> in;
    sel_load<EPT, true>(c, a.keys, a.scores, a.table, in);
    load_act32(a, true, (size_t)min((int)threadIdx.x, ng - 1) * kGroup, v);
    const bool early = n > 0 && ns >= 1;  // a first feature of the shared expert needs no selection
    if (early) gu_feat_load(b0, a, 0, n, ns, s0, r0, 0, lane);
    stage_x();
    select_block<EPT, true>(c, 0, in, sel, blockIdx.x == 0 ? a.idx_out : nullptr, a.w_out);
    if (lane < a.k) {
      const int slot = sel.out_slot[lane];
      if (slot_ok(a, sel.out_e[lane], slot)) my_ptr = (uint64_t)(uintptr_t)(a.base + (size_t)slot * (size_t)a.slot_bytes);
    }
    if (blockIdx.x == 0 && threadIdx.x < 64 && lane < a.k) a.eptr[lane] = my_ptr;  // for the down kernel
    if (n > 0 && !early) gu_feat_load(b0, a, 0, n, ns, s0, r0, my_ptr, lane);
#pragma unroll
    for (int r = 1; r < kGuRing - 1; ++r)
      if (n > 0) gu_feat_load(b[r], a, r, n, ns, s0, r0, my_ptr, lane);
  } else {
    // Order (loads return in order): lane j's expert id, the activations, then
    // the expert's slot; all unconditional (clamped) so the waits are exact.
    const int e_raw = ldg<int>(a.idx + min(lane, a.k - 1));
    load_act32(a, true, (size_t)min((int)threadIdx.x, ng - 1) * kGroup, v);
    const bool e_ok = lane < a.k && e_raw >= 0 && e_raw < a.E;
    const int slot = ldg<int>(a.table + (e_ok ? e_raw : 0));
    my_ptr = e_ok && slot_ok(a, e_raw, slot) ? (uint64_t)(uintptr_t)(a.base + (size_t)slot * (size_t)a.slot_bytes) : 0;
    if (blockIdx.x == 0 && threadIdx.x < 64 && lane < a.k) a.eptr[lane] = my_ptr;  // for the down kernel
    // kGuRing-slot ring, kGuRing - 1 features in flight while one is computed.
    // Loads are unconditional (indices clamped; repeats at the tail hit in
    // cache) so the load counter order is fixed.
    if (n > 0) gu_feat_load(b0, a, 0, n, ns, s0, r0, my_ptr, lane);
    stage_x();
#pragma unroll
    for (int r = 1; r < kGuRing - 1; ++r)
      if (n > 0) gu_feat_load(b[r], a, r, n, ns, s0, r0, my_ptr, lane);
  }
  __syncthreads();
  if (n <= 0) return;
  Limbs xv[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int g = lane + 64 * j;
    if (g < ng) {
      load_limbs_lds(lds + (size_t)g * 24, lf + g, xv[j]);
    } else {
#pragma unroll
      for (int l = 0; l < 6; ++l)
#pragma unroll
        for (int m = 0; m < 4; ++m) xv[j].L[l][m] = 0u;
      xv[j].f = 0.f;
    }
  }
  float hout = 0.f;
  for (int i = 0; i < n; i += kGuRing) {
    // step r requests feature i + r + kGuRing - 1 into the slot computed at step r - 1
#pragma unroll
    for (int r = 0; r < kGuRing; ++r) {
      gu_feat_load(b[(r + kGuRing - 1) % kGuRing], a, i + r + kGuRing - 1, n, ns, s0, r0, my_ptr, lane);
      if (r == 0 || i + r < n) hout = gu_feat_compute(b[r], xv, i + r, hout);
    }
  }
  if (lane < n) {
    int hrow;
    if (lane < ns) {
      hrow = a.k * Imax + s0 + lane;
    } else {
      const int f = r0 + lane - ns, j = f / a.I;
      hrow = j * Imax + (f - j * a.I);
    }
    stg<float>(a.h + hrow, hout);
  }
}

// HLDS: h of every expert is converted to limbs into LDS by the workgroup;
// otherwise the limbs come from global memory (converted by k_to_limbs).
//
// Work of a workgroup: the (expert, tile) units of its row block, unit u =
// expert u / nb, tile t0 + u % nb (nb tiles in the block); wave w takes units
// w, w + nw, ... .  Each wave requests its first tile, then converts its share
// of h (staging that waits behind a long queue of weight requests would hold
// the whole workgroup at the barrier), and after the barrier requests unit
// m + 1 before it computes unit m.
template <int NGD, int WF, bool HLDS>
__global__ __launch_bounds__(dn_s1_waves(WF) * 64) void k_down_s1(FfnArgs a) {
  constexpr int MU = 3;  // units per wave per round
  __shared__ float part[kMaxK + 1][kDnRows * kDnMaxTb];
  __shared__ int s_idx[kMaxK];  // [0]: the token's idx row is invalid (combine poisons y)
  __shared__ float s_w[kMaxK];
  extern __shared__ uint32_t hlds[];  // HLDS: [NE][Imax/32][24] limbs, then [NE][Imax/32] factors
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int NE = a.k + (a.Is > 0 ? 1 : 0);
  const int Imax = max(a.I, a.Is), ngm = Imax / kGroup, nt = a.H / kDnRows;
  const int t0 = blockIdx.x * a.tb, t1 = min(nt, t0 + a.tb), nb = t1 - t0, U = NE * nb;
  float *hf_lds = (float *)(hlds + (size_t)NE * ngm * 24);
  auto h_group = [&](int i, bool &use, float (&v)[32]) {
    const int e2 = i / ngm, g = i - e2 * ngm;
    use = HLDS && i < NE * ngm && g * kGroup < (e2 == a.k ? a.Is : a.I);
    // unconditional (a group that is not used reads group 0 and is dropped), so
    // that the waits for the loads issued before it can be exact
    load_act32(a, false, use ? (size_t)e2 * Imax + (size_t)g * kGroup : 0, v);
  };
  // unit -> expert, tile, weights (clamped: units past U repeat the last unit and are not computed)
  struct Unit {
    int j, t, inter;
    bool valid;
    const uint8_t *dn;
  };
  auto ex_of = [&](int jj) -> const uint8_t * {  // the load is unconditional (exact waits)
    const uint8_t *p = (const uint8_t *)(uintptr_t)ldg<uint64_t>(a.eptr + min(jj, a.k - 1));
    return jj == a.k ? a.shared : p;
  };
  auto unit_of = [&](int u, const uint8_t *ex) {
    Unit r;
    u = min(u, U - 1);
    r.j = u / nb;
    r.t = t0 + (u - r.j * nb);
    r.valid = ex != nullptr;
    r.inter = (r.j == a.k && r.valid) ? a.Is : a.I;
    r.dn = uniform_ptr((r.valid ? ex : a.base) + down_offset(a.H, r.inter, WF));
    return r;
  };
  auto unit_expert = [&](int u) { return min(u, U - 1) / nb; };
  DnTile<NGD, WF> q[2];
  Unit un[2];
  // order of the first loads: the units' expert pointers, this thread's first
  // group of h, the first unit's tile, idx and w for the combine
  const uint8_t *ex[MU];
#pragma unroll
  for (int m = 0; m < MU; ++m) ex[m] = ex_of(unit_expert(wave + nw * m));
  bool use_h;
  float hv0[32];
  h_group(threadIdx.x, use_h, hv0);
  un[0] = unit_of(wave, ex[0]);
  dn_tile_load(q[0], un[0].dn, un[0].inter, un[0].t, un[0].t + 1, lane);
  int my_idx = 0;
  float my_w = 0.f;
  if ((int)threadIdx.x < a.k) {
    my_idx = ldg<int>(a.idx + threadIdx.x);
    my_w = ldg<float>(a.w + threadIdx.x);
  }
  if (use_h) {
    Limbs L;
    to_limbs_wf<WF>(hv0, L);
    L.f *= act_scale(a, false, (int)threadIdx.x / ngm);
    store_limbs(hlds + (size_t)threadIdx.x * 24, hf_lds + threadIdx.x, L);
  }
  for (int i = threadIdx.x + blockDim.x; HLDS && i < NE * ngm; i += blockDim.x) {
    float v[32];
    h_group(i, use_h, v);
    if (use_h) {
      Limbs L;
      to_limbs_wf<WF>(v, L);
      L.f *= act_scale(a, false, i / ngm);
      store_limbs(hlds + (size_t)i * 24, hf_lds + i, L);
    }
  }
  __syncthreads();
  auto compute = [&](const DnTile<NGD, WF> &b, const Unit &uu) {
    const int ng = uu.inter / kGroup;
    Limbs hv[NGD];
#pragma unroll
    for (int g2 = 0; g2 < NGD; ++g2) {
      const int g = min(lane + 64 * g2, ng - 1);
      if (HLDS) load_limbs_lds(hlds + ((size_t)uu.j * ngm + g) * 24, hf_lds + (size_t)uu.j * ngm + g, hv[g2]);
      else load_limbs_global(a.hl + ((size_t)uu.j * ngm + g) * 24, a.hf + (size_t)uu.j * ngm + g, hv[g2]);
      if (lane + 64 * g2 >= ng) hv[g2].f = 0.f;  // clamped duplicate group contributes zero
    }
    float acc[kDnRows];
    dn_tile_dots(b, hv, acc);
    if (lane == 63) {
      float *dst = &part[uu.j][(uu.t - t0) * kDnRows];
#pragma unroll
      for (int i = 0; i < kDnRows; ++i) dst[i] = uu.valid ? acc[i] : __builtin_nanf("");
    }
  };
#pragma unroll
  for (int m = 0; m < MU; ++m) {
    if (m + 1 < MU) {
      un[(m + 1) & 1] = unit_of(wave + nw * (m + 1), ex[m + 1]);
      dn_tile_load(q[(m + 1) & 1], un[(m + 1) & 1].dn, un[(m + 1) & 1].inter, un[(m + 1) & 1].t,
                   un[(m + 1) & 1].t + 1, lane);
    }
    if (wave + nw * m < U) compute(q[m & 1], un[m & 1]);
  }
  // further rounds (more units than MU per wave), same pipeline
  for (int base = nw * MU; base < U; base += nw * MU) {
    un[0] = unit_of(base + wave, ex_of(unit_expert(base + wave)));
    dn_tile_load(q[0], un[0].dn, un[0].inter, un[0].t, un[0].t + 1, lane);
#pragma unroll
    for (int m = 0; m < MU; ++m) {
      if (m + 1 < MU) {
        const int u = base + wave + nw * (m + 1);
        un[(m + 1) & 1] = unit_of(u, ex_of(unit_expert(u)));
        dn_tile_load(q[(m + 1) & 1], un[(m + 1) & 1].dn, un[(m + 1) & 1].inter, un[(m + 1) & 1].t,
                     un[(m + 1) & 1].t + 1, lane);
      }
      if (base + wave + nw * m < U) compute(q[m & 1], un[m & 1]);
    }
  }
  if ((int)threadIdx.x < a.k) {
    s_w[threadIdx.x] = my_w;
  }
  if (wave == 0) {  // the token's idx row: every entry in [0, E) and no entry twice (lane j < k holds entry j)
    bool bad_j = lane < a.k && (my_idx < 0 || my_idx >= a.E);
    for (int ii = 0; ii < a.k; ++ii) {
      const int e = __builtin_amdgcn_readlane(my_idx, ii);
      bad_j |= ii < lane && lane < a.k && e == my_idx;
    }
    const bool bad = __ballot(bad_j) != 0;
    if (lane == 0) s_idx[0] = bad;
  }
  __syncthreads();
  const int rows = nb * kDnRows;
  if ((int)threadIdx.x < rows) {
    const bool bad = s_idx[0] != 0;
    const int i = threadIdx.x;
    float acc = 0.f;
    for (int jj = 0; jj < a.k; ++jj) acc = fmaf(s_w[jj], part[jj][i], acc);
    if (a.Is > 0) acc += part[a.k][i];
    stg<float>(a.y + t0 * kDnRows + i, bad ? __builtin_nanf("") : acc);
  }
}

// ---- two to four tokens ---------------------------------------------------------
// Batch union in LDS.  uniq[0..U) ascending expert ids; for unique slot u:
// ntok[u] tokens tok[u][a] (ascending) with pair index pair[u][a] =
// token * (k+1) + rank.  Slot U is the shared expert with every token.
struct SmallPlan {
  int U;
  int tokbad[kSmallS];          // token's idx row names an expert outside [0, E) or twice
  int sidx[kSmallS * kMaxK];    // idx with invalid and repeated entries as -1
  int sfirst[kSmallS * kMaxK];  // entry is the first occurrence of its expert
  int uniq[kSmallS * kMaxK];
  int ntok[kSmallS * kMaxK + 1];
  int tok[kSmallS * kMaxK + 1][kSmallS];
  int pair[kSmallS * kMaxK + 1][kSmallS];
};

// Needs blockDim.x > S * k.  idx: the batch's [S, k] rows (global or LDS).
__device__ void build_small_plan(const FfnArgs &a, SmallPlan &p, const int32_t *idx) {
  const int n = a.S * a.k, tid = threadIdx.x;
  if (tid == 0) p.U = 0;
  if (tid < a.S) p.tokbad[tid] = 0;
  __syncthreads();
  if (tid < n) {
    const int e = idx[tid];
    const int t = tid / a.k;
    bool ok = e >= 0 && e < a.E;
    for (int j = t * a.k; j < tid && ok; ++j) ok = idx[j] != e;
    p.sidx[tid] = ok ? e : -1;
    if (!ok) atomicOr(&p.tokbad[t], 1);
  }
  __syncthreads();
  if (tid < n) {
    const int e = p.sidx[tid];
    int first = e >= 0;
    for (int j = 0; j < tid; ++j) first &= (p.sidx[j] != e);
    p.sfirst[tid] = first;
  }
  __syncthreads();
  if (tid < n && p.sfirst[tid]) {
    const int e = p.sidx[tid];
    int pos = 0;
    for (int j = 0; j < n; ++j) pos += (p.sfirst[j] && p.sidx[j] < e) ? 1 : 0;
    p.uniq[pos] = e;
    atomicAdd(&p.U, 1);
  }
  __syncthreads();
  const int U = p.U;
  if (tid <= U) {
    int c = 0;
    for (int t = 0; t < a.S; ++t) {
      if (tid == U) {  // shared expert: every token, rank k
        p.tok[tid][c] = t; p.pair[tid][c] = t * (a.k + 1) + a.k; ++c;
      } else {
        for (int j = 0; j < a.k; ++j)
          if (p.sidx[t * a.k + j] == p.uniq[tid]) { p.tok[tid][c] = t; p.pair[tid][c] = t * (a.k + 1) + j; ++c; }
      }
    }
    p.ntok[tid] = c;
  }
  __syncthreads();
}


// One gate/up tile (4 features) for a set of tokens; x limbs from global.  The
// tile's rows are taken RC at a time (int8: 4, so that the weights of a chunk
// stay within the register file next to the activation limbs).
template <int NG, int WF>
__device__ inline void gateup_tile(const FfnArgs &a, const uint8_t *tile, int ntok, const int *toks, const int *pairs,
                                   int feat0, int inter_stride) {
  constexpr int RC = WF == kWfQ8Row ? 4 : kGuRows;
  const int lane = threadIdx.x & 63, H = a.H, ng = H / kGroup;
  const int64_t rb = row_bytes(H, WF);
  const uint8_t *scp = tile + (size_t)kGuRows * rb;
#pragma unroll 1
  for (int r0 = 0; r0 < kGuRows; r0 += RC) {
    QGroup<WF> q[RC][NG];
    uint4 sc[NG];
    float rs[RC];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int g = min(lane + 64 * j, ng - 1);
#pragma unroll
      for (int i = 0; i < RC; ++i) load_group(q[i][j], tile + (size_t)(r0 + i) * rb, g);
      if constexpr (WF == kWfQ4G32) sc[j] = ldg<uint4>(scp + g * 16);
    }
    if constexpr (WF != kWfQ4G32) {
#pragma unroll
      for (int i = 0; i < RC; ++i) rs[i] = ldg<float>(scp + 4 * (r0 + i));
    }
    for (int tt = 0; tt < ntok; ++tt) {
      Limbs xv[NG];
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const int g = min(lane + 64 * j, ng - 1);
        load_limbs_global(a.xl + ((size_t)toks[tt] * ng + g) * 24, a.xf + (size_t)toks[tt] * ng + g, xv[j]);
        if (lane + 64 * j >= ng) xv[j].f = 0.f;
      }
      float acc[RC];
#pragma unroll
      for (int i = 0; i < RC; ++i) acc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < NG; ++j)
#pragma unroll
        for (int i = 0; i < RC; ++i) {
          if constexpr (WF == kWfQ4G32)
            acc[i] = group_fma(qdot(q[i][j], xv[j]), scale_of(sc[j], r0 + i), xv[j].f, acc[i]);
          else acc[i] = fmaf(qdot(q[i][j], xv[j]), xv[j].f, acc[i]);
        }
#pragma unroll
      for (int i = 0; i < RC; ++i) {
        acc[i] = wave_sum_to63(acc[i]);
        if constexpr (WF != kWfQ4G32) acc[i] *= rs[i];
      }
      if (lane == 63) {
        float *dst = a.h + (size_t)pairs[tt] * inter_stride + feat0 + r0 / 2;
        if constexpr (RC == 8)
          stg<float4>(dst, make_float4(silu_mul(acc[0], acc[1]), silu_mul(acc[2], acc[3]), silu_mul(acc[4], acc[5]),
                                       silu_mul(acc[6], acc[7])));
        else
          stg<float2>(dst, make_float2(silu_mul(acc[0], acc[1]), silu_mul(acc[2], acc[3])));
      }
    }
  }
}

__device__ inline void poison_h(const FfnArgs &a, int ntok, const int *pairs, int feat0, int inter_stride) {
  const int lane = threadIdx.x & 63;
  if (lane < kGuPairs)
    for (int tt = 0; tt < ntok; ++tt) a.h[(size_t)pairs[tt] * inter_stride + feat0 + lane] = __builtin_nanf("");
}

// The union and its experts' packed weights, as the gate/up kernel's first
// workgroup derived them, handed to the down kernel of the same call through
// the workspace (the eptr region): the plan's words, then one pointer per
// unique expert.  The down kernel then needs one round of loads instead of
// the plan's dependent loads and barriers and the slot-table lookups.
constexpr int kPlanWords = (int)(sizeof(SmallPlan) / 4);
constexpr int kPlanPtrOff = (kPlanWords + 1) / 2;  // in 64-bit words
static_assert((kPlanPtrOff + kSmallS * kMaxK) * 8 <= kWsPlanBytes, "the plan record fits its workspace region");

__device__ inline void store_small_plan(const FfnArgs &a, const SmallPlan &p, const uint8_t *const *ptr) {
  const uint32_t *src = (const uint32_t *)&p;
  for (int i = threadIdx.x; i < kPlanWords; i += blockDim.x) stg<uint32_t>((uint32_t *)a.eptr + i, src[i]);
  if ((int)threadIdx.x < p.U) stg<uint64_t>(a.eptr + kPlanPtrOff + threadIdx.x, (uint64_t)(uintptr_t)ptr[threadIdx.x]);
}

// Ends with a barrier.  ptr[u] for u < U; the entries past U hold stale words.
__device__ inline void load_small_plan(const FfnArgs &a, SmallPlan &p, const uint8_t **ptr) {
  uint32_t *dst = (uint32_t *)&p;
  for (int i = threadIdx.x; i < kPlanWords; i += blockDim.x) dst[i] = ldg<uint32_t>((const uint32_t *)a.eptr + i);
  if ((int)threadIdx.x < kSmallS * kMaxK)
    ptr[threadIdx.x] = (const uint8_t *)(uintptr_t)ldg<uint64_t>(a.eptr + kPlanPtrOff + threadIdx.x);
  __syncthreads();
}

constexpr int kGuSmallWaves = 8;  // waves per small-batch gate/up workgroup (one workgroup per CU)

// Two to four tokens, gate/up: the batch's (feature, token) pairs stream
// through the waves token-major, so that a wave's activation limbs stay in
// registers as in the one-token kernel (reloading them from LDS for every
// (feature, token) pair would put two dependent LDS round trips in front of
// every pair's dot products).  Pair order: the shared expert's features for
// token 0, 1, ... (S * Is pairs), then each unique expert u (ascending) in
// blocks of 32 features, each block once for every token that chose u
// (ascending).  Each wave takes an equal share of the shared pairs (they need
// no routing, so they stream while the union is built) and of the others; the
// limbs are reloaded from LDS only when the token changes (at most every 32
// pairs).  An expert chosen by several tokens is read once per token, by the
// same or the next wave right after (four tokens' limbs would not fit in the
// registers next to the prefetch ring).  The per-pair arithmetic is the
// one-token kernel's, so a token's h does not depend on the other tokens of
// its batch.  Results park in lanes (value and h row) and are stored 64 at a
// time.
template <int NG, int WF>
__global__ __launch_bounds__(kGuSmallWaves * 64) void k_gateup_small(FfnArgs a) {
  __shared__ SmallPlan plan;
  __shared__ const uint8_t *s_ptr[kSmallS * kMaxK];
  __shared__ int seg_start[kSmallS * kMaxK + 1];  // first union pair of unique expert u; [U]: all
  // [S][H/32] groups of 24 limb words at a stride of kXs words (conflict-free
  // 16-byte reads across lanes), then [S][H/32] factors; H <= 8192
  constexpr int kXs = 28;
  __shared__ __align__(16) uint32_t xlds[kSmallS * 256 * (kXs + 1)];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ng = a.H / kGroup, Imax = max(a.I, a.Is), nx = a.S * ng;
  float *xf_lds = (float *)(xlds + (size_t)nx * kXs);
  // activations of group threadIdx.x (and + blockDim.x) of the S tokens, loaded first
  float v0[32], v1[32];
  const int i0 = threadIdx.x, i1 = threadIdx.x + blockDim.x;
  load_act32(a, true, (size_t)min(i0, nx - 1) * kGroup, v0);
  load_act32(a, true, (size_t)min(i1, nx - 1) * kGroup, v1);
  const int W = gridDim.x * (blockDim.x >> 6), wid = blockIdx.x * (blockDim.x >> 6) + wave;
  const long Ps = (long)a.S * a.Is;
  const int sp0 = (int)(wid * Ps / W), ns = (int)((wid + 1) * Ps / W) - sp0;
  GuFeat<NG, WF> b0, b1, b2;
  int row0 = 0, row1 = 0, row2 = 0, tok0 = 0, tok1 = 0, tok2 = 0;  // slot tags: h row and token
  auto shared_item = [&](GuFeat<NG, WF> &b, int i, int &row, int &tok) {
    const int p = sp0 + i, t = p / a.Is, f = p - t * a.Is;
    gu_row_load(b, a, a.shared, f, lane);
    tok = t;
    row = (t * (a.k + 1) + a.k) * Imax + f;
  };
  if (ns >= 1) shared_item(b0, 0, row0, tok0);
  if (ns >= 2) shared_item(b1, 1, row1, tok1);
  build_small_plan(a, plan, a.idx);
  const int U = plan.U;
  if (threadIdx.x == 0) {
    int start = 0;
    for (int u = 0; u < U; ++u) {
      seg_start[u] = start;
      start += plan.ntok[u] * a.I;
    }
    seg_start[U] = start;
  }
  if ((int)threadIdx.x < U) s_ptr[threadIdx.x] = expert_ptr(a, plan.uniq[threadIdx.x]);
  if (i0 < nx) {
    Limbs L;
    to_limbs_wf<WF>(v0, L);
    L.f *= act_scale(a, true, i0 / ng);
    store_limbs(xlds + (size_t)i0 * kXs, xf_lds + i0, L);
  }
  if (i1 < nx) {
    Limbs L;
    to_limbs_wf<WF>(v1, L);
    L.f *= act_scale(a, true, i1 / ng);
    store_limbs(xlds + (size_t)i1 * kXs, xf_lds + i1, L);
  }
  for (int i = threadIdx.x + 2 * blockDim.x; i < nx; i += blockDim.x) {  // S * H/32 > 2 * blockDim
    float v[32];
    load_act32(a, true, (size_t)i * kGroup, v);
    Limbs L;
    to_limbs_wf<WF>(v, L);
    L.f *= act_scale(a, true, i / ng);
    store_limbs(xlds + (size_t)i * kXs, xf_lds + i, L);
  }
  __syncthreads();
  if (blockIdx.x == 0) store_small_plan(a, plan, s_ptr);  // for the down kernel
  const long Pu = seg_start[U];
  const int up0 = (int)(wid * Pu / W), n = ns + (int)((wid + 1) * Pu / W) - up0;
  if (n <= 0) return;
  int lc = 0;  // unique expert of the last union pair requested (a wave's pairs increase)
  // item i of the wave (clamped to its last one, so that loads are unconditional)
  auto load_item = [&](GuFeat<NG, WF> &b, int i, int &row, int &tok) {
    i = min(i, n - 1);
    if (i < ns) {
      shared_item(b, i, row, tok);
      return;
    }
    const int p = up0 + (i - ns);
    while (p >= seg_start[lc + 1]) ++lc;
    const int u = lc, nt = plan.ntok[u], q = p - seg_start[u];
    const int blk = q / (kGroup * nt), r = q - blk * kGroup * nt, tt = r / kGroup;
    const int f = blk * kGroup + (r - tt * kGroup);
    gu_row_load(b, a, uniform_ptr(s_ptr[u]), f, lane);
    tok = plan.tok[u][tt];
    row = plan.pair[u][tt] * Imax + f;
  };
  if (ns < 1) load_item(b0, 0, row0, tok0);
  if (ns < 2) load_item(b1, 1, row1, tok1);
  Limbs xv[NG];
  int xt = -1;  // token whose limbs are in xv
  float hout = 0.f;
  int prow = 0, c = 0;
  auto finish = [&](const GuFeat<NG, WF> &b, int row, int tok) {
    if (tok != xt) {
      xt = tok;
#pragma unroll
      for (int j = 0; j < NG; ++j) {  // lanes past the last group repeat it with a zero factor
        const int g = min(lane + 64 * j, ng - 1);
        load_limbs_lds(xlds + ((size_t)tok * ng + g) * kXs, xf_lds + (size_t)tok * ng + g, xv[j]);
        if (lane + 64 * j >= ng) xv[j].f = 0.f;
      }
    }
    hout = gu_feat_compute(b, xv, c, hout);
    if (lane == c) prow = row;
    if (++c == 64) {
      stg<float>(a.h + prow, hout);
      c = 0;
    }
  };
  if constexpr (WF != kWfQ8Row) {
    for (int i = 0; i < n; i += 3) {
      load_item(b2, i + 2, row2, tok2);
      finish(b0, row0, tok0);
      load_item(b0, i + 3, row0, tok0);
      if (i + 1 < n) finish(b1, row1, tok1);
      load_item(b1, i + 4, row1, tok1);
      if (i + 2 < n) finish(b2, row2, tok2);
    }
  } else {  // int8 features are twice as large: two slots, one in flight while one is computed
    for (int i = 0; i < n; i += 2) {
      finish(b0, row0, tok0);
      load_item(b0, i + 2, row0, tok0);
      if (i + 1 < n) finish(b1, row1, tok1);
      load_item(b1, i + 3, row1, tok1);
    }
  }
  if (lane < c) stg<float>(a.h + prow, hout);
}

// Two to four tokens, down projection: (expert, token, tile) units stream
// through the waves, and each unit's 8 row dots are stored as per-(token, rank)
// partial rows; k_combine then adds them in route order with the shared expert.
// Each wave takes an equal share of the units, with two tiles in flight while
// one is computed; the per-unit arithmetic is the one-token kernel's.
//   HLDS: units in tile order, the expert's tokens innermost, so the tokens that
//   share a tile request it back to back from the same wave (the repeats are
//   served by the caches instead of being fetched again); the h rows of the
//   (token, expert) pairs that the workgroup's units touch are converted to limbs
//   once, into LDS (at most dn_slots pairs; a pair beyond that is converted in
//   registers when it changes, as below).
//   Otherwise: for each unique expert, blocks of B tiles, each block once for
//   every token of the expert, with the pair's h converted to limbs in registers
//   whenever the pair changes.
// Unique experts ascend, then the shared expert with every token.  The union
// and the experts' weights are the ones the gate/up kernel stored.
constexpr int kDnSmallWaves = 8;
template <int NGD, int WF, bool HLDS>
__global__ __launch_bounds__(kDnSmallWaves * 64) void k_down_small(FfnArgs a) {
  __shared__ SmallPlan plan;
  __shared__ const uint8_t *s_ptr[kSmallS * kMaxK + 1];
  __shared__ int seg_start[kSmallS * kMaxK + 2];  // first unit of unique expert u (U: shared); [U + 1]: all
  __shared__ int s_slot0[kSmallS * kMaxK + 1];    // HLDS: LDS slot of unique expert u's first token (-1: none)
  __shared__ int s_nslots;
  extern __shared__ uint32_t hl[];  // HLDS: [slot][Imax/32][24] limbs, then [slot][Imax/32] factors
  load_small_plan(a, plan, s_ptr);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwb = blockDim.x >> 6;
  const int U = plan.U, Imax = max(a.I, a.Is), nt = a.H / kDnRows, ngm = Imax / kGroup;
  const int B = (nt % 16 == 0) ? 16 : 4;  // tiles per block (nt is a multiple of 4)
  auto ntok_of = [&](int u) { return u == U ? (a.Is > 0 ? a.S : 0) : plan.ntok[u]; };
  if (threadIdx.x == 0) {
    int start = 0;
    for (int u = 0; u <= U; ++u) {
      seg_start[u] = start;
      start += ntok_of(u) * nt;
    }
    seg_start[U + 1] = start;
  }
  if ((int)threadIdx.x == U) s_ptr[U] = a.shared;
  __syncthreads();
  const int W = gridDim.x * nwb, wid = blockIdx.x * nwb + wave;
  const long P = seg_start[U + 1];
  float *hf = (float *)(hl + (size_t)max(a.dn_slots, 0) * ngm * 24);
  auto pair_of = [&](int u, int tt) { return u == U ? tt * (a.k + 1) + a.k : plan.pair[u][tt]; };
  if constexpr (HLDS) {
    // LDS slots for the pairs of the unique experts whose units meet this
    // workgroup's share
    if (threadIdx.x == 0) {
      const long q0 = (long)blockIdx.x * nwb * P / W, q1 = (long)(blockIdx.x + 1) * nwb * P / W;
      int slots = 0;
      for (int u = 0; u <= U; ++u) {
        const int ntu = ntok_of(u);
        const bool meets = ntu > 0 && seg_start[u] < q1 && seg_start[u + 1] > q0;
        if (meets && slots + ntu <= a.dn_slots) {
          s_slot0[u] = slots;
          slots += ntu;
        } else {
          s_slot0[u] = -1;
        }
      }
      s_nslots = slots;
    }
    __syncthreads();
  }
  Limbs hv[NGD];
  int hp = -1;  // pair whose h limbs are in hv
  // h limbs of a pair: from LDS, or converted in registers (only when the pair changes)
  auto stage_h = [&](int pair, int slot, int ngi) {
    if (pair == hp) return;
    hp = pair;
#pragma unroll
    for (int g2 = 0; g2 < NGD; ++g2) {  // lanes past the last group repeat it with a zero factor
      const int g = min(lane + 64 * g2, ngi - 1);
      if (HLDS && slot >= 0) {
        const size_t i = (size_t)slot * ngm + g;
        load_limbs_lds(hl + i * 24, hf + i, hv[g2]);
      } else {
        float v[32];
        load_act32(a, false, (size_t)pair * Imax + (size_t)g * kGroup, v);
        to_limbs_wf<WF>(v, hv[g2]);
        hv[g2].f *= act_scale(a, false, pair);
      }
      if (lane + 64 * g2 >= ngi) hv[g2].f = 0.f;
    }
  };
  auto dots_out = [&](const DnTile<NGD, WF> &b, int pair, int t, bool valid) {
    float acc[kDnRows];
    dn_tile_dots(b, hv, acc);
    if (lane == 63) {
      const float nan = __builtin_nanf("");
      float4 *d = (float4 *)(a.part + (size_t)pair * a.H + (size_t)t * kDnRows);
      stg<float4>(d, valid ? make_float4(acc[0], acc[1], acc[2], acc[3]) : make_float4(nan, nan, nan, nan));
      stg<float4>(d + 1, valid ? make_float4(acc[4], acc[5], acc[6], acc[7]) : make_float4(nan, nan, nan, nan));
    }
  };
  const int p0 = (int)(wid * P / W), n = (int)((wid + 1) * P / W) - p0;
  int lc = 0;  // unique expert of the last unit taken (a wave's units increase)
  if constexpr (HLDS) {
    // The wave's units, in tile order, grouped by tile: each tile is loaded once
    // and its tokens (those in this wave's share) are computed one after another.
    struct TileW {
      int u, t, tt0, cnt, inter;
      bool valid;
      const uint8_t *dn;
    };
    int cur = p0;
    const int end = p0 + max(n, 0);
    TileW last{};
    auto next_tile = [&]() {
      if (cur >= end) {  // past the share: repeat the last tile (the load stays unconditional), compute nothing
        TileW r = last;
        r.cnt = 0;
        return r;
      }
      while (cur >= seg_start[lc + 1]) ++lc;
      TileW r;
      r.u = lc;
      const int ntu = ntok_of(lc), q = cur - seg_start[lc];
      r.t = q / ntu;
      r.tt0 = q - r.t * ntu;
      r.cnt = min(ntu - r.tt0, end - cur);
      cur += r.cnt;
      const uint8_t *ex = uniform_ptr(s_ptr[lc]);
      r.valid = ex != nullptr;
      r.inter = (lc == U && r.valid) ? a.Is : a.I;
      r.dn = uniform_ptr((r.valid ? ex : a.base) + down_offset(a.H, r.inter, WF));
      last = r;
      return r;
    };
    // the first two tiles are requested before the workgroup stages h
    DnTile<NGD, WF> q0, q1, q2;
    TileW w0{}, w1{}, w2{};
    if (n > 0) {
      w0 = next_tile();
      dn_tile_load(q0, w0.dn, w0.inter, w0.t, w0.t + 1, lane);
      w1 = next_tile();
      dn_tile_load(q1, w1.dn, w1.inter, w1.t, w1.t + 1, lane);
    }
    for (int i = threadIdx.x; i < s_nslots * ngm; i += blockDim.x) {
      const int slot = i / ngm, g = i - slot * ngm;
      int u = 0;
      while (s_slot0[u] < 0 || slot >= s_slot0[u] + ntok_of(u)) ++u;
      const int pair = pair_of(u, slot - s_slot0[u]);
      if (g * kGroup < (u == U ? a.Is : a.I)) {
        float v[32];
        load_act32(a, false, (size_t)pair * Imax + (size_t)g * kGroup, v);
        Limbs L;
        to_limbs_wf<WF>(v, L);
        L.f *= act_scale(a, false, pair);
        store_limbs(hl + (size_t)i * 24, hf + i, L);
      }
    }
    __syncthreads();
    if (n <= 0) return;
    auto compute = [&](const DnTile<NGD, WF> &b, const TileW &tw) {
      for (int j = 0; j < tw.cnt; ++j) {
        const int tt = tw.tt0 + j;
        stage_h(pair_of(tw.u, tt), s_slot0[tw.u] < 0 ? -1 : s_slot0[tw.u] + tt, tw.inter / kGroup);
        dots_out(b, pair_of(tw.u, tt), tw.t, tw.valid);
      }
    };
    if constexpr (NGD == 1 && WF != kWfQ8Row) {  // three tiles: two in flight while one is computed
      while (w0.cnt > 0) {
        w2 = next_tile();
        dn_tile_load(q2, w2.dn, w2.inter, w2.t, w2.t + 1, lane);
        compute(q0, w0);
        w0 = next_tile();
        dn_tile_load(q0, w0.dn, w0.inter, w0.t, w0.t + 1, lane);
        compute(q1, w1);
        w1 = next_tile();
        dn_tile_load(q1, w1.dn, w1.inter, w1.t, w1.t + 1, lane);
        compute(q2, w2);
      }
    } else {  // wider tiles: two, to stay within the register file
      while (w0.cnt > 0) {
        compute(q0, w0);
        w0 = next_tile();
        dn_tile_load(q0, w0.dn, w0.inter, w0.t, w0.t + 1, lane);
        compute(q1, w1);
        w1 = next_tile();
        dn_tile_load(q1, w1.dn, w1.inter, w1.t, w1.t + 1, lane);
      }
    }
  } else {
    if (n <= 0) return;
    struct Unit {
      int pair, t, inter;
      bool valid;
      const uint8_t *dn;
    };
    auto unit_of = [&](int i) {
      const int p = p0 + min(i, n - 1);
      while (p >= seg_start[lc + 1]) ++lc;
      const int u = lc, ntu = ntok_of(u), q = p - seg_start[u];
      const int blk = q / (B * ntu), r = q - blk * B * ntu, tt = r / B;
      Unit un;
      un.t = blk * B + (r - tt * B);
      un.pair = pair_of(u, tt);
      const uint8_t *ex = uniform_ptr(s_ptr[u]);
      un.valid = ex != nullptr;
      un.inter = (u == U && un.valid) ? a.Is : a.I;
      un.dn = uniform_ptr((un.valid ? ex : a.base) + down_offset(a.H, un.inter, WF));
      return un;
    };
    auto finish = [&](const DnTile<NGD, WF> &b, const Unit &uu) {
      stage_h(uu.pair, -1, uu.inter / kGroup);
      dots_out(b, uu.pair, uu.t, uu.valid);
    };
    DnTile<NGD, WF> q0, q1;
    Unit u0 = unit_of(0), u1 = unit_of(1);
    dn_tile_load(q0, u0.dn, u0.inter, u0.t, u0.t + 1, lane);
    dn_tile_load(q1, u1.dn, u1.inter, u1.t, u1.t + 1, lane);
    if constexpr (NGD == 1 && WF != kWfQ8Row) {  // three tiles: two in flight while one is computed
      DnTile<NGD, WF> q2;
      Unit u2;
      for (int i = 0; i < n; i += 3) {
        u2 = unit_of(i + 2);
        dn_tile_load(q2, u2.dn, u2.inter, u2.t, u2.t + 1, lane);
        finish(q0, u0);
        u0 = unit_of(i + 3);
        dn_tile_load(q0, u0.dn, u0.inter, u0.t, u0.t + 1, lane);
        if (i + 1 < n) finish(q1, u1);
        u1 = unit_of(i + 4);
        dn_tile_load(q1, u1.dn, u1.inter, u1.t, u1.t + 1, lane);
        if (i + 2 < n) finish(q2, u2);
      }
    } else {  // wider tiles (inter > 2048, or int8 weights): two, to stay within the register file
      for (int i = 0; i < n; i += 2) {
        finish(q0, u0);
        u0 = unit_of(i + 2);
        dn_tile_load(q0, u0.dn, u0.inter, u0.t, u0.t + 1, lane);
        if (i + 1 < n) finish(q1, u1);
        u1 = unit_of(i + 3);
        dn_tile_load(q1, u1.dn, u1.inter, u1.t, u1.t + 1, lane);
      }
    }
  }
}


// ---- large batches (S > 4) -------------------------------------------------------
// Per-expert token lists (k_bucket), work items of up to 4 tokens (k_schedule),
// the same tile math over (item, tile) pairs writing per-(token, rank) expert
// outputs, and a combine in route order.
constexpr int kTB = 4;  // tokens per work item

// Per-expert token list in token order: block e scans idx in order and compacts
// the entries equal to e (each token names an expert at most once).
__global__ __launch_bounds__(256) void k_bucket(FfnArgs a) {
  // Entries i of idx in blocks of 64 rows x 256; per (row, wave) a ballot of the
  // entries equal to e; an exclusive scan over (row, wave) in order gives each
  // wave's offset, so the list keeps the order of i.
  __shared__ unsigned long long s_mask[64][4];
  __shared__ int s_off[64 * 4];
  __shared__ int s_wsum[4];
  const int e = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = a.S * a.k;
  const bool lane_tok = 64 % a.k == 0;  // entries i of one token share a wave (i % k == lane % k)
  const unsigned long long lt = (1ull << lane) - 1ull;
  const unsigned long long seg_lo = (1ull << (lane - lane % a.k)) - 1ull;  // lanes before this token's segment
  int base = 0;
  for (int b0 = 0; b0 < n; b0 += 64 * 256) {
    const int rows = min(64, (n - b0 + 255) / 256);
    for (int r0 = 0; r0 < rows; r0 += 16) {
      int v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {  // loads of 16 rows in flight together
        const int i = b0 + (r0 + r) * 256 + tid;
        v[r] = ldg<int>(a.idx + min(i, n - 1));
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = b0 + (r0 + r) * 256 + tid;
        bool m = r0 + r < rows && i < n && v[r] == e;
        // a token that names e twice contributes once (the combine poisons it)
        if (lane_tok) {  // the token's entries are k consecutive lanes: an earlier match in the segment
          const unsigned long long hits = __ballot(m);
          m = m && (hits & lt & ~seg_lo) == 0ull;
        } else if (m) {
          const int t0 = i / a.k * a.k;
          for (int j = t0; j < i; ++j) m = m && ldg<int>(a.idx + j) != e;
        }
        const unsigned long long bal = __ballot(m);
        if (lane == 0 && r0 + r < rows) s_mask[r0 + r][wave] = bal;
      }
    }
    __syncthreads();
    // exclusive scan of the (row, wave) counts; thread tid holds entry tid = row * 4 + wave
    const int cnt = (tid >> 2) < rows ? __popcll(s_mask[tid >> 2][tid & 3]) : 0;
    int inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(inc, o);
      if (lane >= o) inc += u;
    }
    if (lane == 63) s_wsum[wave] = inc;
    __syncthreads();
    int pre = base;
    for (int w2 = 0; w2 < wave; ++w2) pre += s_wsum[w2];
    s_off[tid] = pre + inc - cnt;
    const int block_total = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    __syncthreads();
    for (int r = 0; r < rows; ++r) {
      const unsigned long long msk = s_mask[r][wave];
      if ((msk >> lane) & 1ull) {
        const int i = b0 + r * 256 + tid;
        const int t = i / a.k, j = i - t * a.k;
        a.lists[(size_t)e * a.S + s_off[r * 4 + wave] + __popcll(msk & lt)] = t * (a.k + 1) + j;
      }
    }
    base += block_total;
    __syncthreads();  // the next block reuses s_mask, s_off and s_wsum
  }
  if (tid == 0) a.counts[e] = base;
}

// Work items {expert, first list position, n tokens}: routed experts in id order,
// then the shared expert (id E) over all tokens.  An expert with at least
// mfma_thr tokens (mfma_thr > 0) gets matrix-core tiles of up to
// kMfmaTileTokens rows instead.  The tile list is ordered for the GEMMs' block
// scheduling, longest first: every full tile (the shared expert's, then the
// routed experts' in id order), then the experts' last, partial tiles by
// decreasing rows (ties in no fixed order: the order changes which workgroup
// computes a tile, never a result), so that the last workgroups to start are
// the short ones.
__global__ __launch_bounds__(1024) void k_schedule(FfnArgs a) {
  constexpr int MT = kMfmaTileTokens;
  __shared__ int pre[kMaxE + 1], pmt[kMaxE + 1];
  __shared__ int cur[MT];  // partial tiles per row count, then the next position of each
  __shared__ int s_np;     // routed experts with a partial tile
  const int tid = threadIdx.x, E = a.E;
  const int thr = a.mfma_thr;
  auto is_mfma = [&](int c) { return thr > 0 && c >= thr; };
  const bool sh_mfma = a.Is > 0 && is_mfma(a.S);
  const int sh_full = sh_mfma ? a.S / MT : 0, sh_part = sh_mfma ? a.S % MT : 0;
  for (int r = tid; r < MT; r += blockDim.x) cur[r] = 0;
  if (tid == 0) s_np = 0;
  for (int e = tid; e < E; e += blockDim.x) {
    const int c = a.counts[e];
    pre[e] = is_mfma(c) ? 0 : (c + kTB - 1) / kTB;
    pmt[e] = is_mfma(c) ? c / MT : 0;  // full tiles
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    const int c = a.counts[e];
    if (is_mfma(c) && c % MT) {
      atomicAdd(&cur[c % MT], 1);
      atomicAdd(&s_np, 1);
    }
  }
  if (tid == 0 && sh_part) atomicAdd(&cur[sh_part], 1);
  __syncthreads();
  if (tid == 0) {
    int s = 0, m = sh_full;
    const int np = s_np;
    for (int e = 0; e < E; ++e) {
      const int c = pre[e], d = pmt[e];
      pre[e] = s;
      pmt[e] = m;
      s += c;
      m += d;
    }
    pre[E] = s;
    pmt[E] = m + np;  // routed tiles end here (their full tiles, then the partial tiles of every expert)
    a.n_items[2] = m - sh_full + np;    // routed tiles
    a.n_items[3] = sh_full + (sh_part ? 1 : 0);  // shared tiles
  }
  __syncthreads();
  if (tid < 64) {
    // partial tiles start after every full tile (pmt[E] - np of them), by decreasing rows: lane l owns
    // the row counts MT - 1 - 4 l .. MT - 4 - 4 l; a wave scan gives each lane its first position
    static_assert(MT == 256, "four row counts per lane");
    int n[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = MT - 1 - 4 * tid - j;
      n[j] = r > 0 ? cur[r] : 0;
      sum += n[j];
    }
    int inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(inc, o);
      if (tid >= o) inc += u;
    }
    int q = pmt[E] - s_np + inc - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = MT - 1 - 4 * tid - j;
      if (r > 0) cur[r] = q;
      q += n[j];
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    const int c = a.counts[e];
    if (is_mfma(c)) {
      for (int s = 0; s < c / MT; ++s) {
        int *mt = a.mtiles + 3 * (size_t)(pmt[e] + s);
        mt[0] = e; mt[1] = s * MT; mt[2] = MT;
      }
      if (c % MT) {
        int *mt = a.mtiles + 3 * (size_t)atomicAdd(&cur[c % MT], 1);
        mt[0] = e; mt[1] = c - c % MT; mt[2] = c % MT;
      }
    } else {
      for (int s = 0; s * kTB < c; ++s) {
        int *it = a.items + 3 * (size_t)(pre[e] + s);
        it[0] = e; it[1] = s * kTB; it[2] = min(kTB, c - s * kTB);
      }
    }
  }
  const int nr = pre[E];
  const int nsh = a.Is > 0 && !sh_mfma ? (a.S + kTB - 1) / kTB : 0;
  for (int s = tid; s < nsh; s += blockDim.x) {
    int *it = a.items + 3 * (size_t)(nr + s);
    it[0] = E; it[1] = s * kTB; it[2] = min(kTB, a.S - s * kTB);
  }
  for (int s = tid; s < sh_full; s += blockDim.x) {
    int *mt = a.mtiles + 3 * (size_t)s;
    mt[0] = E; mt[1] = s * MT; mt[2] = MT;
  }
  if (tid == 0) {
    if (sh_part) {
      int *mt = a.mtiles + 3 * (size_t)atomicAdd(&cur[sh_part], 1);
      mt[0] = E; mt[1] = a.S - sh_part; mt[2] = sh_part;
    }
    a.n_items[0] = nr;
    a.n_items[1] = nsh;
  }
}

__device__ inline int item_tokens(const FfnArgs &a, const int *it, int *toks, int *pairs) {
  const int e = it[0], s0 = it[1], n = it[2];
  for (int tt = 0; tt < n; ++tt) {
    if (e == a.E) { toks[tt] = s0 + tt; pairs[tt] = (s0 + tt) * (a.k + 1) + a.k; }
    else { const int p = a.lists[(size_t)e * a.S + s0 + tt]; pairs[tt] = p; toks[tt] = p / (a.k + 1); }
  }
  return n;
}

// Limb form of just the rows the GEMV items read (most of a large batch goes to
// the matrix cores): X: the items' tokens' x (H/32 groups); else the items'
// (token, rank) rows of h (inter/32 groups).  A token or row named by several
// items is converted more than once, to the same values.  Grid-stride over
// (item, token slot, group).
template <bool X, int WF>
__global__ __launch_bounds__(256) void k_item_limbs(FfnArgs a) {
  const int Imax = max(a.I, a.Is), ng = X ? a.H / kGroup : Imax / kGroup;
  const long n_it = a.n_items[0] + a.n_items[1], total = n_it * kTB * ng;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
    const int item = (int)(i / (kTB * ng)), r = (int)(i - (long)item * kTB * ng), tt = r / ng, g = r - tt * ng;
    const int *it = a.items + 3 * (size_t)item;
    const int e = it[0];
    if (tt >= it[2] || (!X && g * kGroup >= (e == a.E ? a.Is : a.I))) continue;
    const int pair = e == a.E ? (it[1] + tt) * (a.k + 1) + a.k : a.lists[(size_t)e * a.S + it[1] + tt];
    const int row = X ? pair / (a.k + 1) : pair;
    float v[32];
    load_act32(a, X, X ? (size_t)row * a.H + (size_t)g * kGroup : (size_t)row * Imax + (size_t)g * kGroup, v);
    Limbs L;
    to_limbs_wf<WF>(v, L);
    L.f *= act_scale(a, X, row);
    uint32_t *dl = (X ? a.xl : a.hl) + ((size_t)row * ng + g) * 24;
#pragma unroll
    for (int l = 0; l < 6; ++l) stg<uint4>((uint4 *)dl + l, make_uint4(L.L[l][0], L.L[l][1], L.L[l][2], L.L[l][3]));
    stg<float>((X ? a.xf : a.hf) + (size_t)row * ng + g, L.f);
  }
}

template <int NG, int WF>
__global__ __launch_bounds__(256) void k_gateup_items(FfnArgs a) {
  const int wave = threadIdx.x >> 6;
  const int nr = a.n_items[0], nsh = a.n_items[1];
  const int Imax = max(a.I, a.Is);
  const int tr = a.I / kGuPairs, ts = a.Is / kGuPairs;
  const long total = (long)nr * tr + (long)nsh * ts;
  for (long w = (long)blockIdx.x * 4 + wave; w < total; w += (long)gridDim.x * 4) {
    int item, t;
    if (w < (long)nr * tr) { item = (int)(w / tr); t = (int)(w - (long)item * tr); }
    else { const long r = w - (long)nr * tr; item = nr + (int)(r / ts); t = (int)(r - (long)(item - nr) * ts); }
    const int *it = a.items + 3 * (size_t)item;
    int toks[kTB], pairs[kTB];
    const int n = item_tokens(a, it, toks, pairs);
    const uint8_t *ex = it[0] == a.E ? a.shared : expert_ptr(a, it[0]);
    if (!ex) { poison_h(a, n, pairs, t * kGuPairs, Imax); continue; }
    gateup_tile<NG, WF>(a, uniform_ptr(ex + (size_t)t * gu_tile_bytes(a.H, WF)), n, toks, pairs, t * kGuPairs, Imax);
  }
}

template <int NGD, int WF>
__global__ __launch_bounds__(256) void k_down_items(FfnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nr = a.n_items[0], nsh = a.n_items[1];
  const int Imax = max(a.I, a.Is), ngm = Imax / kGroup;
  const int nt = a.H / kDnRows;
  const long total = (long)(nr + nsh) * nt;
  for (long w = (long)blockIdx.x * 4 + wave; w < total; w += (long)gridDim.x * 4) {
    const int item = (int)(w / nt), rt = (int)(w - (long)item * nt);
    const int *it = a.items + 3 * (size_t)item;
    int toks[kTB], pairs[kTB];
    const int n = item_tokens(a, it, toks, pairs);
    const bool sh = it[0] == a.E;
    const uint8_t *ex = sh ? a.shared : expert_ptr(a, it[0]);
    const int inter = sh ? a.Is : a.I;
    if (!ex) {
      if (lane < kDnRows)
        for (int tt = 0; tt < n; ++tt) a.part[(size_t)pairs[tt] * a.H + rt * kDnRows + lane] = __builtin_nanf("");
      continue;
    }
    DnTile<NGD, WF> q;
    dn_tile_load(q, uniform_ptr(ex + down_offset(a.H, inter, WF)), inter, rt, rt + 1, lane);
    const int ng = inter / kGroup;
    for (int tt = 0; tt < n; ++tt) {
      const int pr = pairs[tt];
      Limbs hv[NGD];
#pragma unroll
      for (int g2 = 0; g2 < NGD; ++g2) {
        const int g = min(lane + 64 * g2, ng - 1);
        load_limbs_global(a.hl + ((size_t)pr * ngm + g) * 24, a.hf + (size_t)pr * ngm + g, hv[g2]);
        if (lane + 64 * g2 >= ng) hv[g2].f = 0.f;
      }
      float acc[kDnRows];
      dn_tile_dots(q, hv, acc);
      if (lane == 63) {
        float4 *d = (float4 *)(a.part + (size_t)pr * a.H + rt * kDnRows);
        stg<float4>(d, make_float4(acc[0], acc[1], acc[2], acc[3]));
        stg<float4>(d + 1, make_float4(acc[4], acc[5], acc[6], acc[7]));
      }
    }
  }
}

// y[t, c] = sum_j w[t, j] * part[t, j, c] (route order) + part[t, k, c]; a token
// whose idx row is out of range or repeats an expert gets NaN.
__global__ __launch_bounds__(256) void k_combine(FfnArgs a) {
  const int t = blockIdx.y, lane = threadIdx.x & 63;
  // the token's idx row: every entry in [0, E) and no entry twice (lane j < k holds entry j)
  const int my_idx = lane < a.k ? ldg<int>(a.idx + (size_t)t * a.k + lane) : 0;
  const float my_w = lane < a.k ? ldg<float>(a.w + (size_t)t * a.k + lane) : 0.f;
  bool bad_j = lane < a.k && (my_idx < 0 || my_idx >= a.E);
  for (int ii = 0; ii < a.k; ++ii) {
    const int e = __builtin_amdgcn_readlane(my_idx, ii);
    bad_j |= ii < lane && lane < a.k && e == my_idx;
  }
  const bool bad = __ballot(bad_j) != 0;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;  // four columns per thread (H is a multiple of 32)
  if (c >= a.H) return;
  const float *pt = a.part + (size_t)t * (a.k + 1) * a.H + c;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int j = 0; j < a.k; ++j) {
    const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
    const float4 p = ldg<float4>(pt + (size_t)j * a.H);
    acc = make_float4(fmaf(wj, p.x, acc.x), fmaf(wj, p.y, acc.y), fmaf(wj, p.z, acc.z), fmaf(wj, p.w, acc.w));
  }
  if (a.Is > 0) {
    const float4 p = ldg<float4>(pt + (size_t)a.k * a.H);
    acc = make_float4(acc.x + p.x, acc.y + p.y, acc.z + p.z, acc.w + p.w);
  }
  const float nan = __builtin_nanf("");
  stg<float4>(a.y + (size_t)t * a.H + c, bad ? make_float4(nan, nan, nan, nan) : acc);
}

// int8 activations: one workgroup per row.  Row r (elements r * stride ...) has
// `len` elements, or `len_last` when kp1 > 0 and r % kp1 == kp1 - 1 (the shared
// expert's hidden row of a token); d = fp32(amax / 127) and q = rint(fp32(v / d)),
// with IEEE divisions; a row holding a NaN gets d = NaN (its outputs stay NaN).
__global__ __launch_bounds__(256) void k_quant_rows(const void *src, int bf16, int stride, int len, int len_last,
                                                    int kp1, int8_t *q, float *d) {
  __shared__ float s_max[4];
  __shared__ int s_nan[4];
  const int r = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = (kp1 > 0 && r % kp1 == kp1 - 1) ? len_last : len;
  const size_t base = (size_t)r * stride;
  auto load4 = [&](int c, float *v) {
    if (bf16) {
      const uint2 w = ldg<uint2>((const uint16_t *)src + base + c);
      v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xFFFF0000u);
      v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xFFFF0000u);
    } else {
      const float4 f = ldg<float4>((const float *)src + base + c);
      v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    }
  };
  // the row (at most 8192 elements, 32 per thread) stays in registers between
  // the two passes, so it is read from memory once
  constexpr int kIt = 8;
  float v[kIt][4];
  float m = 0.f;
  int nan = 0;
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int c = threadIdx.x * 4 + it * 1024;  // n is a multiple of 32
    if (c < n) {
      load4(c, v[it]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        nan |= v[it][j] != v[it][j];
        m = fmaxf(m, fabsf(v[it][j]));
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    m = fmaxf(m, __shfl_xor(m, o));
    nan |= __shfl_xor(nan, o);
  }
  if (lane == 0) {
    s_max[wave] = m;
    s_nan[wave] = nan;
  }
  __syncthreads();
  const float amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const bool any_nan = (s_nan[0] | s_nan[1] | s_nan[2] | s_nan[3]) != 0;
  const float dd = any_nan ? __builtin_nanf("") : __fdiv_rn(amax, 127.0f);
  if (threadIdx.x == 0) stg<float>(d + r, dd);
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int c = threadIdx.x * 4 + it * 1024;
    if (c < n) {
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int qi = dd > 0.f ? (int)rintf(__fdiv_rn(v[it][j], dd)) : 0;
        w |= ((uint32_t)qi & 0xFFu) << (8 * j);
      }
      stg<uint32_t>(q + base + c, w);
    }
  }
}

int ceil_groups(int K) { return (K / kGroup + 63) / 64; }

}  // namespace

hipError_t launch_to_limbs(const void *src, int src_bf16, int rows, int K, int src_stride, uint32_t *limbs,
                           float *factors, int wf, const int8_t *q, const float *dq, hipStream_t st) {
  const long n = (long)rows * (K / kGroup);
  if (n == 0) return hipSuccess;
  const dim3 g((unsigned)((n + 255) / 256)), b(256);
  if (wf == kWfQ8Row)
    MOE_LAUNCH(k_to_limbs<kWfQ8Row>, g, b, 0, st, src, src_bf16, rows, K, src_stride, limbs, factors, q, dq);
  else
    MOE_LAUNCH(k_to_limbs<kWfQ4G32>, g, b, 0, st, src, src_bf16, rows, K, src_stride, limbs, factors, q, dq);
  return hipGetLastError();
}

hipError_t launch_quant_x(const FfnArgs &a, hipStream_t st) {
  if (!a.act_q || a.S == 0) return hipSuccess;
  ProfScope ps("quant_x", st);
  MOE_LAUNCH(k_quant_rows, dim3((unsigned)a.S), dim3(256), 0, st, a.x, a.x_bf16, a.H, a.H, a.H, 0, a.xq, a.dx);
  return hipGetLastError();
}

hipError_t launch_quant_h(const FfnArgs &a, hipStream_t st) {
  if (!a.act_q || a.S == 0) return hipSuccess;
  ProfScope ps("quant_h", st);
  const int Imax = std::max(a.I, a.Is), kp1 = a.k + 1;
  MOE_LAUNCH(k_quant_rows, dim3((unsigned)(a.S * kp1)), dim3(256), 0, st, (const void *)a.h, 0, Imax, a.I,
             a.Is > 0 ? a.Is : a.I, kp1, a.hq, a.dh);
  return hipGetLastError();
}

// KERNEL<NG, WF, extra...> for NG = 1..4 groups per lane and the weight format.
#define MOE_NG_CASES(NG_, WFV, KERNEL, GRID, BLOCK, LDS, ST, ...)                                       \
  switch (NG_) {                                                                                      \
    case 1: MOE_LAUNCH((KERNEL<1, WFV __VA_OPT__(, ) __VA_ARGS__>), GRID, BLOCK, LDS, ST, a); break;   \
    case 2: MOE_LAUNCH((KERNEL<2, WFV __VA_OPT__(, ) __VA_ARGS__>), GRID, BLOCK, LDS, ST, a); break;   \
    case 3: MOE_LAUNCH((KERNEL<3, WFV __VA_OPT__(, ) __VA_ARGS__>), GRID, BLOCK, LDS, ST, a); break;   \
    default: MOE_LAUNCH((KERNEL<4, WFV __VA_OPT__(, ) __VA_ARGS__>), GRID, BLOCK, LDS, ST, a); break;  \
  }
#define MOE_NG_CASES_ARGS(ARGS, NG_, WFV, KERNEL, GRID, BLOCK, LDS, ST, ...)                              \
  switch (NG_) {                                                                                         \
    case 1: MOE_LAUNCH((KERNEL<1, WFV __VA_OPT__(, ) __VA_ARGS__>), GRID, BLOCK, LDS, ST, ARGS); break;   \
    case 2: MOE_LAUNCH((KERNEL<2, WFV __VA_OPT__(, ) __VA_ARGS__>), GRID, BLOCK, LDS, ST, ARGS); break;   \
    case 3: MOE_LAUNCH((KERNEL<3, WFV __VA_OPT__(, ) __VA_ARGS__>), GRID, BLOCK, LDS, ST, ARGS); break;   \
    default: MOE_LAUNCH((KERNEL<4, WFV __VA_OPT__(, ) __VA_ARGS__>), GRID, BLOCK, LDS, ST, ARGS); break;  \
  }
#define MOE_DISPATCH_NG_ARGS(ARGS, ng, KERNEL, GRID, BLOCK, LDS, ST, ...)                                 \
  do {                                                                                                   \
    const int ng_ = (ng);                                                                                \
    switch ((ARGS).wf) {                                                                                 \
      case kWfQ4Row: MOE_NG_CASES_ARGS(ARGS, ng_, kWfQ4Row, KERNEL, GRID, BLOCK, LDS, ST, __VA_ARGS__); break; \
      case kWfQ8Row: MOE_NG_CASES_ARGS(ARGS, ng_, kWfQ8Row, KERNEL, GRID, BLOCK, LDS, ST, __VA_ARGS__); break; \
      default: MOE_NG_CASES_ARGS(ARGS, ng_, kWfQ4G32, KERNEL, GRID, BLOCK, LDS, ST, __VA_ARGS__); break;        \
    }                                                                                                    \
  } while (0)
#define MOE_DISPATCH_NG(ng, KERNEL, GRID, BLOCK, LDS, ST, ...)                                       \
  do {                                                                                               \
    const int ng_ = (ng);                                                                            \
    switch (a.wf) {                                                                                  \
      case kWfQ4Row: MOE_NG_CASES(ng_, kWfQ4Row, KERNEL, GRID, BLOCK, LDS, ST, __VA_ARGS__); break;  \
      case kWfQ8Row: MOE_NG_CASES(ng_, kWfQ8Row, KERNEL, GRID, BLOCK, LDS, ST, __VA_ARGS__); break;  \
      default: MOE_NG_CASES(ng_, kWfQ4G32, KERNEL, GRID, BLOCK, LDS, ST, __VA_ARGS__); break;        \
    }                                                                                                \
  } while (0)
hipError_t launch_gateup_s1(const FfnArgs &a, hipStream_t st) {
  ProfScope ps("gateup_s1", st);
  const long feats = (long)a.k * a.I + a.Is;
  const long waves = std::max<long>((long)a.n_cu * 8, (feats + kGuMaxPerWave - 1) / kGuMaxPerWave);
  const dim3 g((unsigned)((waves + 3) / 4)), blk(256);
  const size_t lds = (size_t)(a.H / kGroup) * 25 * sizeof(uint32_t);
  if (!a.sel) {
    MOE_DISPATCH_NG(ceil_groups(a.H), k_gateup_s1, g, blk, lds, st, 0);
  } else if (a.E <= 256) {
    MOE_DISPATCH_NG(ceil_groups(a.H), k_gateup_s1, g, blk, lds, st, 1);
  } else {
    MOE_DISPATCH_NG(ceil_groups(a.H), k_gateup_s1, g, blk, lds, st, 4);
  }
  return hipGetLastError();
}

hipError_t launch_down_s1(const FfnArgs &a, hipStream_t st) {
  const int Imax = std::max(a.I, a.Is);
  hipError_t e = launch_quant_h(a, st);
  if (e != hipSuccess) return e;
  const int NE = a.k + (a.Is > 0 ? 1 : 0);
  const size_t hlds = (size_t)NE * (Imax / kGroup) * 25 * sizeof(uint32_t);
  const bool in_lds = hlds <= 64 * 1024;
  if (!in_lds) {
    ProfScope ps("h_limbs", st);
    e = launch_to_limbs(a.h, 0, NE, Imax, Imax, a.hl, a.hf, a.wf, a.act_q ? a.hq : nullptr, a.dh, st);
    if (e != hipSuccess) return e;
  }
  ProfScope ps("down_s1", st);
  const dim3 g((unsigned)a.n_blk), blk(64 * std::min(NE * a.tb, dn_s1_waves(a.wf)));
  if (in_lds) {
    MOE_DISPATCH_NG(ceil_groups(Imax), k_down_s1, g, blk, hlds, st, true);
  } else {
    MOE_DISPATCH_NG(ceil_groups(Imax), k_down_s1, g, blk, 0, st, false);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_decode(const FfnArgs &a, hipStream_t st) {
  hipError_t e = launch_quant_x(a, st);
  if (e != hipSuccess) return e;
  if (a.S == 1) {
    e = launch_gateup_s1(a, st);
    return e == hipSuccess ? launch_down_s1(a, st) : e;
  }
  const int Imax = std::max(a.I, a.Is);
  {
    ProfScope ps("gateup_small", st);
    const dim3 g((unsigned)a.n_cu), blk(kGuSmallWaves * 64);
    MOE_DISPATCH_NG(ceil_groups(a.H), k_gateup_small, g, blk, 0, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  e = launch_quant_h(a, st);
  if (e != hipSuccess) return e;
  {
    ProfScope ps("down_small", st);
    const dim3 g2((unsigned)a.n_cu), b2(kDnSmallWaves * 64);
    // (token, expert) pairs a workgroup's share of the units can meet: the share
    // spans at most ceil(share / nt) + 1 unique experts, each with at most S tokens
    const long nt = a.H / kDnRows, units_max = (long)a.S * (a.k + 1) * nt;
    const long share = (units_max + a.n_cu - 1) / a.n_cu + 1;
    FfnArgs b = a;
    b.dn_slots = (int)std::min<long>((long)a.S * ((share + nt - 1) / nt + 1), (long)a.S * (a.k + 1));
    const size_t hlds = (size_t)b.dn_slots * (Imax / kGroup) * 25 * sizeof(uint32_t);
    // one group of h per lane (I <= 2048): wider rows leave too few registers for the tile ring
    if (hlds <= 64 * 1024 && ceil_groups(Imax) == 1) {
      MOE_DISPATCH_NG_ARGS(b, ceil_groups(Imax), k_down_small, g2, b2, hlds, st, true);
    } else {
      b.dn_slots = 0;
      MOE_DISPATCH_NG_ARGS(b, ceil_groups(Imax), k_down_small, g2, b2, 0, st, false);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ProfScope ps("combine", st);
  MOE_LAUNCH(k_combine, dim3((a.H + 1023) / 1024, a.S), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_ffn_batch(const FfnArgs &a, hipStream_t st) {
  const int Imax = std::max(a.I, a.Is);
  hipError_t e = launch_quant_x(a, st);
  if (e != hipSuccess) return e;
  {
    ProfScope ps("bucket", st);
    MOE_LAUNCH(k_bucket, dim3(a.E), dim3(256), 0, st, a);
  }
  {
    ProfScope ps("schedule", st);
    MOE_LAUNCH(k_schedule, dim3(1), dim3(1024), 0, st, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("x_limbs", st);
    if (a.wf == kWfQ8Row) MOE_LAUNCH((k_item_limbs<true, kWfQ8Row>), dim3((unsigned)a.n_cu * 4), dim3(256), 0, st, a);
    else MOE_LAUNCH((k_item_limbs<true, kWfQ4G32>), dim3((unsigned)a.n_cu * 4), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("gateup_items", st);
    const long tiles_max = (long)a.max_items * (Imax / kGuPairs);
    const dim3 g((unsigned)std::min<long>((tiles_max + 3) / 4, 8192)), blk(256);
    MOE_DISPATCH_NG(ceil_groups(a.H), k_gateup_items, g, blk, 0, st);
  }
  e = launch_gu_mfma(a, st);
  if (e != hipSuccess) return e;
  e = launch_quant_h(a, st);
  if (e != hipSuccess) return e;
  {
    ProfScope ps("h_limbs", st);
    if (a.wf == kWfQ8Row) MOE_LAUNCH((k_item_limbs<false, kWfQ8Row>), dim3((unsigned)a.n_cu * 4), dim3(256), 0, st, a);
    else MOE_LAUNCH((k_item_limbs<false, kWfQ4G32>), dim3((unsigned)a.n_cu * 4), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("down_items", st);
    const long dtiles = (long)a.max_items * (a.H / kDnRows);
    const dim3 g((unsigned)std::min<long>((dtiles + 3) / 4, 8192)), blk(256);
    MOE_DISPATCH_NG(ceil_groups(Imax), k_down_items, g, blk, 0, st);
  }
  e = launch_dn_mfma(a, st);
  if (e != hipSuccess) return e;
  {
    ProfScope ps("combine", st);
    MOE_LAUNCH(k_combine, dim3((a.H + 1023) / 1024, a.S), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace moe
